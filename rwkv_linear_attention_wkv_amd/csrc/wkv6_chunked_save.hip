// The chunked v6 forward that also saves the state at every chunk boundary, for the chunked
// backward (its own translation unit, so the plain forward's code object is unchanged).
#include "wkv56_chunked.hpp"

namespace wkv {

hipError_t launch_wkv6_chunked_save(const ScanParams &p, hipStream_t s) {
  return p.y_bf16 ? launch<true, true, true>(p, s) : launch<true, false, true>(p, s);
}

}  // namespace wkv
