// The register-staged FP16/BF16 kernel (h_mfma_body.h) for operands whose
// base address or leading dimension is not a multiple of 8 elements: each run
// of 8 elements is read with one 16-byte buffer load when the operands are
// dword-aligned (every tile form), else with eight 2-byte loads (the 128x128
// form only); the rest of the kernel is unchanged.  Compiled apart from the
// 16-byte forms so that the two sources build in parallel.
#include "h_mfma_body.h"

namespace mgemm {

hipError_t launch_h_mfma_narrow(const Problem& p, int variant, int aw, hipStream_t s) {
    if (aw >= 4) {
        switch (variant) {
        case 3: return dispatch_layout<256, 256, 4>(p, s);
        case 4: return dispatch_layout<256, 192, 4>(p, s);
        case 5: return dispatch_layout<128, 128, 4>(p, s);
        }
    } else if (aw == 2 && variant == 5) {
        return dispatch_layout<128, 128, 2>(p, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace mgemm
