"""Python binding of libmgemm (dense GEMM for MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libmgemm.so``.  The functions carry the names of the C entry
points declared in ``include/mgemm.h``.  Operands are passed as device
pointers (ints) or as torch tensors on the GPU, whose ``data_ptr()`` is
taken; torch is used for device memory and streams only.

There is no fallback: if ``libmgemm.so`` is missing or fails to load, every
entry point raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmgemm.so")

(MGEMM_SUCCESS, MGEMM_ERR_INVALID_ARG, MGEMM_ERR_UNSUPPORTED, MGEMM_ERR_HIP, MGEMM_ERR_ALLOC,
 MGEMM_ERR_SCRATCH) = range(6)
MGEMM_ROW_MAJOR, MGEMM_COL_MAJOR = 0, 1
MGEMM_F32, MGEMM_F16, MGEMM_BF16 = 0, 1, 2
KERNELS = ["auto", "general", "f32_mfma", "h_mfma_256x256", "h_mfma_256x192", "h_mfma_128x128",
           "skinny", "reserved_7", "f32_fast", "f32_fast_128",
           "h_dma_256x256", "skinny_sk", "h_dma_256x192", "f32_fast_u",
           "f8_mfma_256x256", "f8_general", "f8_mfma_256x192", "f32_sk", "h_dma_128x192",
           "h_dma_64x192", "f8_mfma_128x192"]
MGEMM_KERNEL_AUTO = 0
MGEMM_EPILOGUE_NONE, MGEMM_EPILOGUE_SILU = 0, 1
_EPILOGUE = {"none": MGEMM_EPILOGUE_NONE, "silu": MGEMM_EPILOGUE_SILU}

_LAYOUT = {"row": MGEMM_ROW_MAJOR, "col": MGEMM_COL_MAJOR}
_DTYPE = {"f32": MGEMM_F32, "f16": MGEMM_F16, "bf16": MGEMM_BF16}

EXPORTED = ["mgemm_create", "mgemm_destroy", "mgemm_run", "mgemm_run_kernel", "mgemm_run_ex",
            "mgemm_run_variant", "mgemm_run_gated", "mgemm_run_gated_ex", "mgemm_select_kernel",
            "mgemm_select_variant", "mgemm_tune", "mgemm_table_export", "mgemm_table_import",
            "mgemm_table_clear", "mgemm_weighted_choice", "mgemm_quantize_fp8", "mgemm_run_fp8",
            "mgemm_status_string",
            "mgemm_kernel_name", "mgemm_num_cu", "mgemm_run_noalloc", "mgemm_set_clock_stamps",
            "mgemm_run_acc32"]


class MgemmError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s failed: %s (status %d)" % (what, _status_str(status), status))
        self.status = status


_lib = None

MGEMM_MAX_KSPLIT = 32


class MgemmVariant(ctypes.Structure):
    """mgemm_variant_t: a kernel (mgemm_kernel_t) and its number of K ranges."""
    _fields_ = [("kernel", ctypes.c_int32), ("ksplit", ctypes.c_int32)]


class MgemmTuneResult(ctypes.Structure):
    """mgemm_tune_result_t."""
    _fields_ = [("chosen", MgemmVariant), ("chosen_us", ctypes.c_float), ("model", MgemmVariant),
                ("model_us", ctypes.c_float)]


def load(path: str | None = None):
    """Load libmgemm.so (raises OSError if it is not built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise OSError("libmgemm.so is not built (%s); run `python -m dense_gemm_mgemm_amd.build`" % p)
    lib = ctypes.CDLL(p)
    i64, f32, vp, ci = ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_int
    run_args = [ci, ci, i64, i64, i64, f32, vp, i64, vp, i64, f32, vp, i64, ci, vp]
    lib.mgemm_create.argtypes = [ctypes.POINTER(vp)]
    lib.mgemm_destroy.argtypes = [vp]
    lib.mgemm_run.argtypes = [vp] + run_args
    lib.mgemm_run_kernel.argtypes = [vp, ci] + run_args
    lib.mgemm_run_ex.argtypes = [vp, ci] + run_args[:-1] + [ci, vp]
    lib.mgemm_run_gated.argtypes = [vp, i64, i64, i64, vp, i64, vp, vp, i64, vp, i64, ci, vp]
    lib.mgemm_run_gated_ex.argtypes = [vp, ctypes.c_int32, i64, i64, i64, vp, i64, vp, vp, i64, vp,
                                       i64, ci, vp]
    lib.mgemm_run_variant.argtypes = [vp, ctypes.POINTER(MgemmVariant)] + run_args[:-1] + [ci, vp]
    lib.mgemm_select_variant.argtypes = [vp] + run_args[:-1] + [ctypes.POINTER(MgemmVariant)]
    lib.mgemm_run_noalloc.argtypes = [ctypes.POINTER(MgemmVariant)] + run_args[:-1] + [ci, vp]
    pi64, pdbl = ctypes.POINTER(i64), ctypes.POINTER(ctypes.c_double)
    lib.mgemm_tune.argtypes = [vp, ci, ci, ci, ctypes.c_int32, pi64, pi64, pi64, pdbl,
                               ctypes.POINTER(MgemmTuneResult), vp]
    lib.mgemm_table_export.argtypes = [vp, ctypes.c_char_p, ctypes.c_size_t,
                                       ctypes.POINTER(ctypes.c_size_t)]
    lib.mgemm_table_import.argtypes = [vp, ctypes.c_char_p]
    lib.mgemm_table_clear.argtypes = [vp]
    lib.mgemm_weighted_choice.argtypes = [ctypes.c_int32, ctypes.c_int32, pdbl, pdbl]
    lib.mgemm_weighted_choice.restype = ctypes.c_int32
    lib.mgemm_quantize_fp8.argtypes = [vp, i64, i64, vp, i64, ci, vp, i64, vp, vp]
    lib.mgemm_run_fp8.argtypes = [vp, ci, ctypes.c_int32, i64, i64, i64, f32, vp, i64, vp, vp, i64,
                                  vp, f32, vp, i64, ci, vp]
    lib.mgemm_select_kernel.argtypes = [vp] + run_args[:-1] + [ctypes.POINTER(ci)]
    for name in ("mgemm_create", "mgemm_destroy", "mgemm_run", "mgemm_run_kernel", "mgemm_run_ex",
                 "mgemm_run_gated", "mgemm_run_gated_ex", "mgemm_run_variant",
                 "mgemm_select_variant", "mgemm_select_kernel", "mgemm_tune", "mgemm_table_export",
                 "mgemm_table_import", "mgemm_table_clear", "mgemm_quantize_fp8",
                 "mgemm_run_fp8", "mgemm_run_noalloc", "mgemm_run_acc32"):
        getattr(lib, name).restype = ci
    lib.mgemm_run_acc32.argtypes = [vp, ci, ci, ci, i64, i64, i64, f32, vp, i64, vp, i64, vp, i64,
                                    ci, vp]
    lib.mgemm_status_string.argtypes = [ci]
    lib.mgemm_status_string.restype = ctypes.c_char_p
    lib.mgemm_kernel_name.argtypes = [ci]
    lib.mgemm_kernel_name.restype = ctypes.c_char_p
    lib.mgemm_num_cu.argtypes = [vp]
    lib.mgemm_num_cu.restype = ci
    lib.mgemm_set_clock_stamps.argtypes = [vp, vp, i64]
    lib.mgemm_set_clock_stamps.restype = ci
    if path is None:
        _lib = lib
    return lib


def _status_str(s: int) -> str:
    try:
        return load().mgemm_status_string(s).decode()
    except OSError:
        return "status %d" % s


def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _enum(x, table):
    return table[x] if isinstance(x, str) else int(x)


def _stream(s) -> int | None:
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def mgemm_create() -> int:
    """Handle bound to the current HIP device."""
    h = ctypes.c_void_p()
    st = load().mgemm_create(ctypes.byref(h))
    if st != MGEMM_SUCCESS:
        raise MgemmError(st, "mgemm_create")
    return h.value


def mgemm_destroy(h: int) -> None:
    load().mgemm_destroy(h)


def _args(layoutA, layoutB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, dtype):
    return (_enum(layoutA, _LAYOUT), _enum(layoutB, _LAYOUT), int(M), int(N), int(K), float(alpha),
            _ptr(A), int(lda), _ptr(B), int(ldb), float(beta), _ptr(C), int(ldc),
            _enum(dtype, _DTYPE))


def mgemm_run(h, layoutA, layoutB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, dtype,
              stream=None) -> None:
    """Enqueue C = alpha*op(A)op(B) + beta*C on `stream` (torch's current by default)."""
    st = load().mgemm_run(h, *_args(layoutA, layoutB, M, N, K, alpha, A, lda, B, ldb, beta, C,
                                    ldc, dtype), _stream(stream))
    if st != MGEMM_SUCCESS:
        raise MgemmError(st, "mgemm_run")


def mgemm_run_kernel(h, kernel, layoutA, layoutB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                     dtype, stream=None) -> None:
    """As mgemm_run with one kernel variant forced (name or number)."""
    k = KERNELS.index(kernel) if isinstance(kernel, str) else int(kernel)
    st = load().mgemm_run_kernel(h, k, *_args(layoutA, layoutB, M, N, K, alpha, A, lda, B, ldb,
                                              beta, C, ldc, dtype), _stream(stream))
    if st != MGEMM_SUCCESS:
        raise MgemmError(st, "mgemm_run_kernel(%s)" % KERNELS[k] if 0 <= k < len(KERNELS) else k)


def mgemm_run_acc32(h, kernel, layoutA, layoutB, M, N, K, alpha, A, lda, B, ldb, C32, ldc, dtype,
                    stream=None) -> None:
    """C32 (FP32, layoutA's order) = alpha*op(A)op(B): the 16-bit direct-to-LDS
    kernel's sums before the output rounding ("auto", "h_dma_256x256" or
    "h_dma_256x192")."""
    k = KERNELS.index(kernel) if isinstance(kernel, str) else int(kernel)
    st = load().mgemm_run_acc32(h, k, _enum(layoutA, _LAYOUT), _enum(layoutB, _LAYOUT), int(M),
                                int(N), int(K), float(alpha), _ptr(A), int(lda), _ptr(B), int(ldb),
                                _ptr(C32), int(ldc), _enum(dtype, _DTYPE), _stream(stream))
    if st != MGEMM_SUCCESS:
        raise MgemmError(st, "mgemm_run_acc32")


def mgemm_run_ex(h, kernel, layoutA, layoutB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, dtype,
                 epilogue="none", stream=None) -> None:
    """As mgemm_run ("auto") or mgemm_run_kernel, with an output epilogue ("none" or "silu")."""
    k = KERNELS.index(kernel) if isinstance(kernel, str) else int(kernel)
    st = load().mgemm_run_ex(h, k, *_args(layoutA, layoutB, M, N, K, alpha, A, lda, B, ldb, beta,
                                          C, ldc, dtype), _enum(epilogue, _EPILOGUE), _stream(stream))
    if st != MGEMM_SUCCESS:
        raise MgemmError(st, "mgemm_run_ex(%s, %s)" % (kernel, epilogue))


def mgemm_run_gated(h, M, N, K, X, ldx, Wg, Wu, ldw, Z, ldz, dtype, stream=None) -> None:
    """Enqueue Z = SiLU(X W_g) * (X W_u) (row-major, 16-bit) on `stream`."""
    st = load().mgemm_run_gated(h, int(M), int(N), int(K), _ptr(X), int(ldx), _ptr(Wg), _ptr(Wu),
                                int(ldw), _ptr(Z), int(ldz), _enum(dtype, _DTYPE), _stream(stream))
    if st != MGEMM_SUCCESS:
        raise MgemmError(st, "mgemm_run_gated")


def mgemm_run_variant(h, kernel, ksplit, layoutA, layoutB, M, N, K, alpha, A, lda, B, ldb, beta, C,
                      ldc, dtype, epilogue="none", stream=None) -> None:
    """As mgemm_run_ex with a split of K (0: the library's choice, 1: none, n: at most n ranges)."""
    k = KERNELS.index(kernel) if isinstance(kernel, str) else int(kernel)
    v = MgemmVariant(k, int(ksplit))
    st = load().mgemm_run_variant(h, ctypes.byref(v), *_args(layoutA, layoutB, M, N, K, alpha, A,
                                                             lda, B, ldb, beta, C, ldc, dtype),
                                  _enum(epilogue, _EPILOGUE), _stream(stream))
    if st != MGEMM_SUCCESS:
        raise MgemmError(st, "mgemm_run_variant(%s, %d)" % (kernel, ksplit))


def mgemm_run_noalloc(kernel, ksplit, layoutA, layoutB, M, N, K, alpha, A, lda, B, ldb, beta, C,
                      ldc, dtype, epilogue="none", stream=None) -> None:
    """mgemm_run_variant without a handle or any allocation (the library's
    static scratch array on the current device)."""
    k = KERNELS.index(kernel) if isinstance(kernel, str) else int(kernel)
    v = MgemmVariant(k, int(ksplit))
    st = load().mgemm_run_noalloc(ctypes.byref(v), *_args(layoutA, layoutB, M, N, K, alpha, A, lda,
                                                          B, ldb, beta, C, ldc, dtype),
                                  _enum(epilogue, _EPILOGUE), _stream(stream))
    if st != MGEMM_SUCCESS:
        raise MgemmError(st, "mgemm_run_noalloc(%s, %d)" % (kernel, ksplit))


def mgemm_run_gated_ex(h, ksplit, M, N, K, X, ldx, Wg, Wu, ldw, Z, ldz, dtype, stream=None) -> None:
    """mgemm_run_gated with a split of K (0: the library's choice)."""
    st = load().mgemm_run_gated_ex(h, int(ksplit), int(M), int(N), int(K), _ptr(X), int(ldx),
                                   _ptr(Wg), _ptr(Wu), int(ldw), _ptr(Z), int(ldz),
                                   _enum(dtype, _DTYPE), _stream(stream))
    if st != MGEMM_SUCCESS:
        raise MgemmError(st, "mgemm_run_gated_ex(%d)" % ksplit)


def mgemm_select_variant(h, layoutA, layoutB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                         dtype) -> tuple:
    """(kernel name, K ranges) that mgemm_run would launch (("auto", 0): scale-only or nothing)."""
    out = MgemmVariant()
    st = load().mgemm_select_variant(h, *_args(layoutA, layoutB, M, N, K, alpha, A, lda, B, ldb,
                                               beta, C, ldc, dtype), ctypes.byref(out))
    if st != MGEMM_SUCCESS:
        raise MgemmError(st, "mgemm_select_variant")
    return load().mgemm_kernel_name(out.kernel).decode(), int(out.ksplit)


def mgemm_tune(h, dtype, layoutA, layoutB, shapes, calls=None, stream=None) -> list:
    """Measure every variant on each (M, N, K) and fill the handle's dispatch
    table (blocking).  Returns, per shape, the fastest variant and the model's
    choice with their measured times."""
    n = len(shapes)
    arr = lambda vals, t: (t * n)(*vals)
    Ms = arr([int(s[0]) for s in shapes], ctypes.c_int64)
    Ns = arr([int(s[1]) for s in shapes], ctypes.c_int64)
    Ks = arr([int(s[2]) for s in shapes], ctypes.c_int64)
    cw = None if calls is None else arr([float(c) for c in calls], ctypes.c_double)
    res = (MgemmTuneResult * n)()
    st = load().mgemm_tune(h, _enum(dtype, _DTYPE), _enum(layoutA, _LAYOUT), _enum(layoutB, _LAYOUT),
                           n, Ms, Ns, Ks, cw, res, _stream(stream))
    if st != MGEMM_SUCCESS:
        raise MgemmError(st, "mgemm_tune")
    name = lambda v: (load().mgemm_kernel_name(v.kernel).decode(), int(v.ksplit))
    return [{"shape": tuple(shapes[i]), "chosen": name(r.chosen), "chosen_us": r.chosen_us,
             "model": name(r.model), "model_us": r.model_us} for i, r in enumerate(res)]


def mgemm_table_export(h) -> str:
    """The handle's dispatch table as text."""
    n = ctypes.c_size_t()
    st = load().mgemm_table_export(h, None, 0, ctypes.byref(n))
    if st != MGEMM_SUCCESS:
        raise MgemmError(st, "mgemm_table_export")
    buf = ctypes.create_string_buffer(n.value + 1)
    st = load().mgemm_table_export(h, buf, n.value + 1, ctypes.byref(n))
    if st != MGEMM_SUCCESS:
        raise MgemmError(st, "mgemm_table_export")
    return buf.value.decode()


def mgemm_table_import(h, text: str) -> None:
    st = load().mgemm_table_import(h, text.encode())
    if st != MGEMM_SUCCESS:
        raise MgemmError(st, "mgemm_table_import")


def mgemm_table_clear(h) -> None:
    st = load().mgemm_table_clear(h)
    if st != MGEMM_SUCCESS:
        raise MgemmError(st, "mgemm_table_clear")


def mgemm_weighted_choice(times, calls=None) -> int:
    """Index of the variant (column of `times`, one row per shape) with the
    smallest call-weighted total time; -1 if none runs every called shape."""
    rows = [list(map(float, r)) for r in times]
    ns, nv = len(rows), len(rows[0]) if rows else 0
    flat = (ctypes.c_double * (ns * nv))(*[t for r in rows for t in r])
    cw = None if calls is None else (ctypes.c_double * ns)(*map(float, calls))
    return int(load().mgemm_weighted_choice(ns, nv, flat, cw))


def mgemm_quantize_fp8(h, M, K, X, ldx, xtype, Q, ldq, scales, stream=None) -> None:
    """Per-row E4M3 quantisation of X (M x K) into codes Q and FP32 scales."""
    st = load().mgemm_quantize_fp8(h, int(M), int(K), _ptr(X), int(ldx), _enum(xtype, _DTYPE),
                                   _ptr(Q), int(ldq), _ptr(scales), _stream(stream))
    if st != MGEMM_SUCCESS:
        raise MgemmError(st, "mgemm_quantize_fp8")


def mgemm_run_fp8(h, kernel, M, N, K, alpha, A, lda, sa, B, ldb, sb, beta, C, ldc, ctype,
                  stream=None, ksplit=0) -> None:
    """C = alpha * sa[m] * sb[n] * sum_k A[m,k] B[n,k] + beta * C on E4M3 codes
    (ksplit: 0 = the library's choice, 1 = no split, n = at most n K ranges)."""
    k = KERNELS.index(kernel) if isinstance(kernel, str) else int(kernel)
    st = load().mgemm_run_fp8(h, k, int(ksplit), int(M), int(N), int(K), float(alpha), _ptr(A),
                              int(lda), _ptr(sa), _ptr(B), int(ldb), _ptr(sb), float(beta),
                              _ptr(C), int(ldc), _enum(ctype, _DTYPE), _stream(stream))
    if st != MGEMM_SUCCESS:
        raise MgemmError(st, "mgemm_run_fp8(%s, %d)" % (kernel, ksplit))


def mgemm_select_kernel(h, layoutA, layoutB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                        dtype) -> str:
    """Name of the variant mgemm_run would launch ("auto": scale-only or nothing)."""
    out = ctypes.c_int()
    st = load().mgemm_select_kernel(h, *_args(layoutA, layoutB, M, N, K, alpha, A, lda, B, ldb,
                                              beta, C, ldc, dtype), ctypes.byref(out))
    if st != MGEMM_SUCCESS:
        raise MgemmError(st, "mgemm_select_kernel")
    return load().mgemm_kernel_name(out.value).decode()


def mgemm_status_string(s: int) -> str:
    return load().mgemm_status_string(s).decode()


def mgemm_kernel_name(k: int) -> str:
    return load().mgemm_kernel_name(k).decode()


def mgemm_num_cu(h) -> int:
    return load().mgemm_num_cu(h)


def mgemm_set_clock_stamps(h, buf, nblocks: int) -> None:
    """Measurement hook: buf (device, 4*nblocks int64, or None) receives each
    workgroup's (cycles at start, at end, 100 MHz ticks at start, at end)."""
    st = load().mgemm_set_clock_stamps(h, _ptr(buf), int(nblocks))
    if st != MGEMM_SUCCESS:
        raise MgemmError(st, "mgemm_set_clock_stamps")
