// Prefill-path expert FFN (grouped GEMM on bf16 MFMA).  Not yet provided:
// the launcher reports hipErrorNotSupported, which the C ABI returns as
// MOE_ERR_UNSUPPORTED.
#include "common.h"
#include "launch.h"

namespace moe {

size_t ffn_prefill_workspace(int T, int k, int f, bool has_shared) {
  return static_cast<size_t>(T) * (k + (has_shared ? 1 : 0)) * f * sizeof(uint16_t);
}

hipError_t launch_ffn_prefill(const FfnProblem&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace moe
