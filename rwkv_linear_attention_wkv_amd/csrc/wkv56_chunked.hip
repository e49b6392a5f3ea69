// Launches of the 64-token chunked WKV v5 / v6 forward (the kernel and its design are in
// wkv56_chunked.hpp).
#include "wkv56_chunked.hpp"

namespace wkv {

hipError_t launch_wkv56_chunked(const ScanParams &p, bool v6, bool bf16, hipStream_t s) {
  if (!bf16) return hipErrorInvalidValue;  // the ABI layer routes fp32 inputs to the scan
  if (p.y_bf16) return v6 ? launch<true, true, false>(p, s) : launch<false, true, false>(p, s);
  return v6 ? launch<true, false, false>(p, s) : launch<false, false, false>(p, s);
}

}  // namespace wkv
