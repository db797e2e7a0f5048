// FP16/BF16 MFMA GEMM (placeholder until the kernel lands: reports no support,
// so dispatch falls back to the general kernel).
#include "common.h"

namespace mgemm {
bool h_mfma_supports(const Problem&, int) { return false; }
hipError_t launch_h_mfma(const Problem&, int, hipStream_t) { return hipErrorInvalidValue; }
bool skinny_supports(const Problem&) { return false; }
hipError_t launch_skinny(const Problem&, hipStream_t) { return hipErrorInvalidValue; }
}  // namespace mgemm
