// FP16/BF16 GEMM on the gfx950 matrix cores (v_mfma_f32_32x32x16_{f16,bf16}),
// FP32 accumulation, one rounding to the output type at the end.
//
// Prior art on the pages, retargeted to CDNA4:
//  * a large output tile per workgroup for reuse, BM*BN/(BM+BN) flop per
//    staged byte (MTT S4000 FP16 GEMM write-up, sections 1 and 15; tiled
//    traffic V = 2MK*N/n + 2KN*M/m + 2MN of "Chapter 5: Operators and
//    Runtime", section 5.2.2);
//  * global -> register prefetch of the next K slice while the matrix cores
//    work on the current one, then a write into the other of two LDS slots
//    (the write-up's section 4 pipeline; Chapter 5, section 5.3.2, two slots);
//  * LDS rows padded so the column-wise operand reads spread over all banks
//    (Chapter 5, section 5.2.3; the write-up's stride-33 fix, section 13);
//  * an M-grouped, XCD-aware tile order (common.h);
//  * masked edge tiles (Chapter 5, section 5.4.2).
//
// Layout.  Both operand tiles live in LDS K-contiguous: row r of the A tile
// is A'(m0+r, k0..k0+63), row c of the B tile is B'(k0..k0+63, n0+c), each
// row 64 elements + 8 of padding (144 bytes).  A K-contiguous global operand
// is copied 16 bytes at a time.  An MN-contiguous one (e.g. a row-major B,
// N-contiguous) is read as 8x8 element blocks, transposed in registers, and
// written as 8 K-runs -- the layout change happens on the way into LDS, never
// in HBM.
//
// Contraction.  A 256-thread workgroup has 2x2 waves; a wave owns a
// (BM/2) x (BN/2) sub-tile of 32x32 blocks.  Each MFMA is issued with the B
// fragment as its first operand, so the accumulator holds the transposed
// block: lane l has column-of-C index n = 8q + 4(l/32) + {0..3} and row
// m = l%32 -- four consecutive outputs of one row per register quad, stored
// as one 8-byte write.  Which k each lane's 8 fragment elements stand for is
// irrelevant as long as A and B use the same assignment, which they do.
//
// Operands that are not 16-byte aligned (a base address or leading dimension
// that is not a multiple of 8 elements) are read with buffer loads
// (k_h_mfma_u.hip): one 16-byte load per run of 8 elements when they are
// dword-aligned (every tile form), eight 2-byte loads when not (the 128x128
// form).  Same tiles, LDS layout and contraction; only the global loads differ.
#include "h_mfma_body.h"

namespace mgemm {

// Alignment (bytes, at most 16) shared by every run of 8 elements of A and B:
// the largest power of two dividing both base addresses and both leading
// dimensions in bytes (tile and slice origins add multiples of 16 bytes).
static int h_mfma_load_width(const Problem& p) {
    const uint64_t bits = (uint64_t)(uintptr_t)p.A | (uint64_t)(uintptr_t)p.B |
                          (uint64_t)(2 * p.lda) | (uint64_t)(2 * p.ldb) | 16u;
    return (int)(bits & (~bits + 1));
}

// Variant ids follow mgemm_kernel_t: 3 = 256x256, 4 = 256x192, 5 = 128x128.
bool h_mfma_supports(const Problem& p, int variant) {
    if (p.dtype != F16 && p.dtype != BF16) return false;
    if (variant < 3 || variant > 5) return false;
    const int aw = h_mfma_load_width(p);
    // Buffer loads for operands that are not 16-byte aligned: dword-aligned
    // ones in every form, 2-byte aligned ones in the 128x128 form.  Offsets
    // within a K slice stay below 2^31 bytes while the leading dimensions
    // stay below 2^22.
    if (aw < 16 && (aw < 2 || (aw < 4 && variant != 5) || p.lda >= (1 << 22) ||
                    p.ldb >= (1 << 22)))
        return false;
    const int bm = variant == 5 ? 128 : 256, bn = variant == 3 ? 256 : variant == 4 ? 192 : 128;
    const int64_t tiles = ((p.M + bm - 1) / bm) * ((p.N + bn - 1) / bn);
    return tiles > 0 && tiles <= 0x7fffffff;
}

hipError_t launch_h_mfma(const Problem& p, int variant, hipStream_t s) {
    const int aw = h_mfma_load_width(p);
    if (aw < 16) return launch_h_mfma_narrow(p, variant, aw, s);
    switch (variant) {
    case 3: return dispatch_layout<256, 256, 16>(p, s);
    case 4: return dispatch_layout<256, 192, 16>(p, s);
    case 5: return dispatch_layout<128, 128, 16>(p, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace mgemm
