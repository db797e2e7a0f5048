// Internal definitions shared by the libmgemm kernels and host dispatch.
//
// Every kernel works on ONE canonical problem: a row-major C (M x N, ldc)
//     C(m,n) = alpha * sum_k A'(m,k) B'(k,n) + beta * C(m,n)
// where A' and B' are each either K-contiguous or MN-contiguous in memory.
// The host reaches this form from any (layoutA, layoutB) pair with the
// transpose identity of the SGEMM report ("SGEMM measurements and three
// ledgers", section "how the cuBLAS denominator was fixed"): a column-major C
// is the row-major C^T = B^T A^T of the same bytes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mgemm {

enum DType : int { F32 = 0, F16 = 1, BF16 = 2 };

struct Problem {
    int64_t M, N, K;
    float alpha, beta;
    const void* A;   // A'(m,k) = a_kc ? A[m*lda + k] : A[k*lda + m]
    int64_t lda;
    const void* B;   // B'(k,n) = b_kc ? B[n*ldb + k] : B[k*ldb + n]
    int64_t ldb;
    void* C;         // C(m,n) = C[m*ldc + n]
    int64_t ldc;
    int a_kc, b_kc;
    int dtype;
    int num_cu;
    int epilogue;    // Epilogue below, applied to alpha*acc + beta*C before the final rounding
    const void* B2;  // gated pair only: second B' (N-contiguous, leading dimension ldb2)
    int64_t ldb2;
    // Clock stamps (measurement hook, off when null): workgroup b < stamps_cap
    // of a kernel that records them stores 4 values at stamps[4b]: shader-clock
    // cycles (s_memtime) at its start and end, and 100 MHz real-time ticks
    // (s_memrealtime) at its start and end, taken by its first wave.
    unsigned long long* stamps = nullptr;
    int64_t stamps_cap = 0;
};

// Global -> LDS copy of 16 bytes per lane (lane l lands at lds + 16*l), the
// direct-to-LDS staging of the streaming kernels.  Issued through inline asm
// (m0 set in the same statement) so that the compiler does not treat the LDS
// reads that follow as dependent on it: it would otherwise wait for every
// copy in flight before each such read.  Completion is tracked by hand with
// the vmcnt waits of each kernel's schedule.  Naming m0 as clobbered draws a
// warning because m0 is reserved to the compiler; this is sound only while
// the compiler keeps no value of its own in m0 in these kernels, which
// tests/test_codegen.py checks on the generated code.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy_to_lds(const void* src, unsigned lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(src), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

struct ClockStamp {
    unsigned long long cycles, ticks;
};
__device__ __forceinline__ ClockStamp clock_stamp_begin() {
    ClockStamp s;
    s.ticks = __builtin_amdgcn_s_memrealtime();
    s.cycles = __builtin_amdgcn_s_memtime();
    return s;
}
// Thread 0 of the workgroup stores its stamps if the hook is on.
__device__ __forceinline__ void clock_stamp_end(const Problem& p, const ClockStamp& s0) {
    if (p.stamps == nullptr || (int64_t)blockIdx.x >= p.stamps_cap || threadIdx.x != 0) return;
    const unsigned long long c1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    unsigned long long* o = p.stamps + 4 * (int64_t)blockIdx.x;
    o[0] = s0.cycles;
    o[1] = c1;
    o[2] = s0.ticks;
    o[3] = r1;
}

// Device workspace of a handle: FP32 partial results and per-block arrival
// counters (zero between calls) for kernels that split K over workgroups.
struct Workspace {
    void* part;
    int64_t part_bytes;
    unsigned* counters;
    int64_t ncounters;
};

// Exchange of FP32 partial results between workgroups of one launch (split
// K and stream-K).  Device-coherent 16-byte store and load: buffer accesses
// with the device-scope cache policy (sc1), so the store writes through this
// XCD's L2 and the load does not hit a stale line there.  A partial written on
// one XCD and counted with a device-scope atomic is thus read correctly on
// another, with no whole-L2 write-back or invalidation.  The compiler sees
// both (it resolves the store's register hazards and keeps many loads in
// flight); offsets past the buffer's size read as zero and drop stores.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int CPOL_DEVICE = 16;   // sc1
__device__ __forceinline__ void store_coherent(__amdgpu_buffer_rsrc_t ws, unsigned off, f32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ws, off, 0, CPOL_DEVICE);
}
__device__ __forceinline__ f32x4 load_coherent(__amdgpu_buffer_rsrc_t ws, unsigned off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ws, off, 0, CPOL_DEVICE));
}

// ---------------------------------------------------------------------------
// Workgroup -> output tile.
//
// gfx950 hands consecutive workgroup ids to its 8 XCDs in turn (id % 8 picks
// the XCD), and each XCD has its own L2.  We first renumber ids so that the
// workgroups sharing an XCD get consecutive tile numbers, then walk tiles in
// groups of `group_m` tile-rows (all tile-columns of a group before the next
// group), so that workgroups resident at the same time on one XCD share A rows
// and B columns in that XCD's L2.  This is the M-grouped order of the K1 GEMM
// resource model (GROUP_SIZE_M) and the M-first CTA order of the MTT S4000
// write-up (section 14), made XCD-aware.
// ---------------------------------------------------------------------------
// Workgroup id -> position in an order where each XCD's workgroups are consecutive.
__device__ __forceinline__ int xcd_linear(int bid, int nblocks) {
    constexpr int NXCD = 8;
    int xcd = bid % NXCD;
    int local = bid / NXCD;
    int q = nblocks / NXCD, r = nblocks % NXCD;
    return xcd * q + (xcd < r ? xcd : r) + local;
}
// Position t -> (tm, tn) in the M-grouped order.
__device__ __forceinline__ void tile_from_linear(int t, int tiles_m, int tiles_n, int group_m,
                                                 int& tm, int& tn) {
    int per_group = group_m * tiles_n;
    int g = t / per_group;
    int first_m = g * group_m;
    int gsize = tiles_m - first_m < group_m ? tiles_m - first_m : group_m;
    int within = t - g * per_group;
    tm = first_m + within % gsize;
    tn = within / gsize;
}
__device__ __forceinline__ void tile_of_block(int bid, int nblocks, int tiles_m, int tiles_n,
                                              int group_m, int& tm, int& tn) {
    tile_from_linear(xcd_linear(bid, nblocks), tiles_m, tiles_n, group_m, tm, tn);
}

// ---------------------------------------------------------------------------
// Element conversions.  16-bit types travel as raw uint16_t bit patterns.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
    // v_cvt_f16_f32 rounds to nearest even under the default float mode.
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    // v_cvt_pk_bf16_f32: round to nearest even under the default float mode,
    // NaN stays a NaN (gfx950 converts in hardware; the parity tests check
    // the ties against the oracle's own RNE).
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// ---------------------------------------------------------------------------
// Output epilogue.  EPI_SILU stores SiLU(round(v)) for v = alpha*acc + beta*C:
// the value is first rounded to the output format (as if C were written), then
// SiLU(x) = x / (1 + e^-x) is evaluated in FP32 and the result is rounded
// once more on store ("Chapter 5: Operators and Runtime", sections 5.4.2 and
// 5.4.3: the activation follows the complete K sum and its rounding).
// ---------------------------------------------------------------------------
enum Epilogue : int { EPI_NONE = 0, EPI_SILU = 1 };

template <int DT>
__device__ __forceinline__ float round_trip(float v) {
    if constexpr (DT == F32) return v;
    else if constexpr (DT == F16) return f16_bits_to_f32(f32_to_f16_bits(v));
    else return bf16_bits_to_f32(f32_to_bf16_bits(v));
}
// 16-bit storage <-> FP32 for the two 16-bit formats.
template <int DT>
__device__ __forceinline__ uint16_t to_bits(float v) {
    if constexpr (DT == F16) return f32_to_f16_bits(v);
    else return f32_to_bf16_bits(v);
}
template <int DT>
__device__ __forceinline__ float from_bits(uint16_t b) {
    if constexpr (DT == F16) return f16_bits_to_f32(b);
    else return bf16_bits_to_f32(b);
}
// SiLU(c) = c / (1 + e^-c) in FP32.  In the far negative tail (c < -87 for
// FP32 outputs, c < -20 for 16-bit ones) it is evaluated as c * e^c, equal
// to it within 2e-9 relative there, so neither the overflowing e^-c nor a
// denormal reciprocal is ever formed.
template <int DT>
__device__ __forceinline__ float silu_f32(float c) {
    constexpr float LOG2E = 1.44269504088896341f;
    if constexpr (DT == F32) {
        if (!(c >= -87.0f)) return c * expf(c);           // also NaN in, NaN out
        return c / (1.0f + expf(-c));
    } else {
        // 16-bit outputs: the hardware exp2 and reciprocal (relative errors
        // near 1e-6) are far below the final rounding (2^-9 or 2^-12) and
        // much cheaper than the IEEE forms.  The hardware exp2 has no
        // denormal results, so the tail takes e^c * 2^64 (normal down to
        // c = -131; below that the result is under half the smallest BF16
        // denormal anyway) and scales the product back by 2^-64, a multiply
        // that rounds into the denormal range correctly.  Both branches share
        // one exp2 and end in a select, so the unrolled store loops stay
        // straight-line code.
        const bool tail = !(c >= -20.0f);                 // also NaN in, NaN out
        const float e = __builtin_amdgcn_exp2f(tail ? fmaf(c, LOG2E, 64.0f) : -c * LOG2E);
        const float head = c * __builtin_amdgcn_rcpf(1.0f + e);
        return tail ? (c * e) * 0x1p-64f : head;
    }
}
template <int DT, int EPI>
__device__ __forceinline__ float epilogue_op(float v) {
    if constexpr (EPI == EPI_SILU) return silu_f32<DT>(round_trip<DT>(v));
    else return v;
}
template <int DT>
__device__ __forceinline__ float apply_epilogue(float v, int epi) {
    return epi == EPI_SILU ? epilogue_op<DT, EPI_SILU>(v) : v;
}
// Calls f(E) with E an integral_constant holding the epilogue, so each store
// loop is compiled once per epilogue and the plain path carries no
// activation code between its stores.
template <class F>
__device__ __forceinline__ void with_epilogue(int epi, F&& f) {
    if (epi == EPI_SILU) f(std::integral_constant<int, EPI_SILU>{});
    else f(std::integral_constant<int, EPI_NONE>{});
}
// Gated pair ("Chapter 5: Operators and Runtime", section 5.3.1): from the
// FP32 sums g = (X W_g)(m,n) and u = (X W_u)(m,n), Z = round(T * round(u)) with
// T = round(SiLU(round(g))): G, U and T keep the rounding they would get as
// stored tensors; the caller rounds the returned value once on store.
template <int DT>
__device__ __forceinline__ float swiglu_out(float g, float u) {
    const float t = round_trip<DT>(silu_f32<DT>(round_trip<DT>(g)));
    return t * round_trip<DT>(u);
}

// Writes the four 16-bit outputs crow[ni .. ni+3] (those below nlim) from
// v = alpha * acc: adds beta * C, applies the epilogue once, rounds, and
// stores 8 bytes at once when all four are in range and aligned (vec_ok).
template <int DT, int EPI>
__device__ __forceinline__ void store_out4(uint16_t* crow, int ni, int nlim, bool vec_ok,
                                           float beta, float (&v)[4]) {
    const bool full = vec_ok && ni + 4 <= nlim;
    if (beta != 0.f) {
        float c[4] = {0.f, 0.f, 0.f, 0.f};
        if (full) {
            const uint2 cw = *(const uint2*)(crow + ni);
            c[0] = from_bits<DT>((uint16_t)cw.x);
            c[1] = from_bits<DT>((uint16_t)(cw.x >> 16));
            c[2] = from_bits<DT>((uint16_t)cw.y);
            c[3] = from_bits<DT>((uint16_t)(cw.y >> 16));
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (ni + e < nlim) c[e] = from_bits<DT>(crow[ni + e]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = fmaf(beta, c[e], v[e]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = epilogue_op<DT, EPI>(v[e]);
    if (full) {
        const uint32_t w0 = (uint32_t)to_bits<DT>(v[0]) | ((uint32_t)to_bits<DT>(v[1]) << 16);
        const uint32_t w1 = (uint32_t)to_bits<DT>(v[2]) | ((uint32_t)to_bits<DT>(v[3]) << 16);
        *(uint2*)(crow + ni) = make_uint2(w0, w1);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (ni + e < nlim) crow[ni + e] = to_bits<DT>(v[e]);
    }
}

template <int DT> struct Elem;
template <> struct Elem<F32> {
    using T = float;
    static __device__ __forceinline__ float load(const T* p, int64_t i) { return p[i]; }
    static __device__ __forceinline__ void store(T* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<F16> {
    using T = uint16_t;
    static __device__ __forceinline__ float load(const T* p, int64_t i) { return f16_bits_to_f32(p[i]); }
    static __device__ __forceinline__ void store(T* p, int64_t i, float v) { p[i] = f32_to_f16_bits(v); }
};
template <> struct Elem<BF16> {
    using T = uint16_t;
    static __device__ __forceinline__ float load(const T* p, int64_t i) { return bf16_bits_to_f32(p[i]); }
    static __device__ __forceinline__ void store(T* p, int64_t i, float v) { p[i] = f32_to_bf16_bits(v); }
};

// Raises a kernel's dynamic LDS limit once per device (the attribute is held
// per device).  done[] is the caller's per-kernel flag array; two threads
// that race on a first call both set the same value, which is harmless.
constexpr int MAX_DEVICES = 64;
inline hipError_t set_lds_limit_once(const void* kern, int lds, bool (&done)[MAX_DEVICES]) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const bool track = dev >= 0 && dev < MAX_DEVICES;
    if (track && done[dev]) return hipSuccess;
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e == hipSuccess && track) done[dev] = true;
    return e;
}

// ---------------------------------------------------------------------------
// Launchers (each kernel file defines its own).  They return a HIP error of
// the launch; shape/alignment eligibility is checked by the *_supports calls.
// ---------------------------------------------------------------------------
hipError_t launch_general(const Problem& p, hipStream_t s);
hipError_t launch_scale(const Problem& p, hipStream_t s);
hipError_t launch_f32_mfma(const Problem& p, hipStream_t s);
bool f32_mfma_supports(const Problem& p);
hipError_t launch_f32_fast(const Problem& p, bool big, hipStream_t s);
bool f32_fast_supports(const Problem& p, bool big);
bool f32_unaligned_supports(const Problem& p);
hipError_t launch_f32_unaligned(const Problem& p, hipStream_t s);
// Stream-K form of the f32_fast_u kernel (same support); it needs two partial
// tiles per CU and one counter per tile in the workspace.
bool f32_sk_fits(const Problem& p, const Workspace& ws);
hipError_t launch_f32_sk(const Problem& p, const Workspace& ws, hipStream_t s);
hipError_t launch_h_mfma(const Problem& p, int variant, hipStream_t s);
bool h_mfma_supports(const Problem& p, int variant);
hipError_t launch_skinny(const Problem& p, hipStream_t s);
// Direct-to-LDS FP16/BF16 kernel.  ksplit > 1 cuts K into that many ranges
// (two launches, partials in ws); h_dma_splits gives the number of ranges a
// request for at most `requested` turns into (whole 32-slices per range; 1
// for requests <= 1), 0 when the partials would not fit the workspace.
constexpr int MAX_KSPLIT = 32;
int h_dma_splits(const Problem& p, int bn, bool dual, int requested, const Workspace& ws,
                 int bm = 256);
hipError_t launch_h_dma(const Problem& p, int bn, int ksplit, const Workspace& ws, hipStream_t s,
                        int bm = 256);
// alpha * the FP32 accumulators of the 256-row direct-to-LDS kernel (one K
// range) into p.C as FP32 with leading dimension p.ldc.
hipError_t launch_h_dma_acc32(const Problem& p, int bn, hipStream_t s);
bool h_gated_supports(const Problem& p);
hipError_t launch_h_gated(const Problem& p, int ksplit, const Workspace& ws, hipStream_t s,
                          int bm = 256);
bool skinny_sk_supports(const Problem& p);
int skinny_sk_splits(const Problem& p, const Workspace& ws, int requested);
hipError_t launch_skinny_sk(const Problem& p, const Workspace& ws, int ksplit, hipStream_t s);
bool h_dma_supports(const Problem& p, int bn, int bm = 256);
// FP8 E4M3: per-row quantisation of an M x K matrix of xtype (codes Q with
// row stride ldq, FP32 dequantisation scales), and the FP8 GEMM on codes:
// p.A = A codes (M x K, stride lda), p.B = B codes one output column per row
// (N x K, stride ldb), p.dtype = C's type; sa/sb = the row scales of A and B.
hipError_t launch_quantize_fp8(int64_t M, int64_t K, const void* X, int64_t ldx, int xtype, void* Q,
                               int64_t ldq, float* scales, hipStream_t s);
bool f8_mfma_supports(const Problem& p, int bn);          // bn = 256 or 192
bool f8_general_supports(const Problem& p);
// bn: the MFMA kernel's tile width (256 or 192), 0 for the scalar kernel.
// ksplit > 1 (MFMA kernel only) cuts K into ranges of whole 64-slices (two
// launches, partials in ws); f8_splits turns a request into the number of
// ranges used (0 when the partials do not fit the workspace).
int f8_splits(const Problem& p, int bn, int requested, const Workspace& ws);
hipError_t launch_f8_gemm(const Problem& p, const float* sa, const float* sb, int bn, int ksplit,
                          const Workspace& ws, hipStream_t s);
// n elements of dtype at p get small exact values (a hash of the index and seed).
hipError_t launch_fill_pattern(void* p, int64_t n, int dtype, uint32_t seed, hipStream_t s);
bool skinny_supports(const Problem& p);

}  // namespace mgemm
