// 64-token chunked WKV v5 / v6 with MFMA contractions (not built yet).
#include "kernels.hpp"

namespace wkv {
hipError_t launch_wkv56_chunked(const ScanParams &, bool, bool, hipStream_t) { return hipErrorNotSupported; }
}  // namespace wkv
