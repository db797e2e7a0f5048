"""CPU oracle for dense GEMM -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never links, loads or
calls it, and it shares no code, header, table or helper with that library.

The arithmetic lives in ``mgemm_oracle.c`` (plain C, FP64 accumulation, one
final IEEE round-to-nearest-even into the output format).  This module only
compiles that file with gcc and marshals numpy arrays into it.

Definition implemented (see the header of ``mgemm_oracle.c`` for the page
citations):  C = round_out(alpha * op(A) @ op(B) + beta * C), with FP32, FP16 or
BF16 storage, row- or column-major operands and C stored in A's order.

The SiLU epilogue (``silu_epilogue``) and the gated pair (``swiglu``) are
plain numpy in FP64 on top of those results: Y = round_out(SiLU(round_out(C)))
and Z = round_out(round_out(SiLU(round_out(G))) * round_out(U)).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mgemm_oracle.c")
_LIB = os.path.join(_HERE, "libmgemm_oracle.so")

F32, F16, BF16 = 0, 1, 2
ROW, COL = 0, 1
DTYPES = {"f32": F32, "f16": F16, "bf16": BF16}
LAYOUTS = {"row": ROW, "col": COL}
_ITEMSIZE = {F32: 4, F16: 2, BF16: 2}
_STORAGE = {F32: np.uint32, F16: np.uint16, BF16: np.uint16}

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle into a shared library next to its source."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        i64, dbl, vp, ci = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_int
        lib.orc_gemm_rows.argtypes = [ci, ci, i64, i64, i64, dbl, vp, i64, vp, i64, dbl, vp, vp,
                                      i64, ci, i64, vp, vp, ci]
        lib.orc_gemm_rows.restype = ci
        lib.orc_gemm_points.argtypes = [ci, ci, i64, i64, i64, dbl, vp, i64, vp, i64, dbl, vp,
                                        i64, ci, i64, vp, vp, vp, ci]
        lib.orc_gemm_points.restype = ci
        for name in ("orc_decode_array", "orc_round_array"):
            getattr(lib, name).argtypes = [ci, vp, i64, vp]
            getattr(lib, name).restype = None
        lib.orc_encode_array.argtypes = [ci, vp, i64, vp]
        lib.orc_encode_array.restype = None
        lib.orc_max_threads.argtypes = []
        lib.orc_max_threads.restype = ci
        _lib = lib
    return _lib


def _dt(dtype) -> int:
    return DTYPES[dtype] if isinstance(dtype, str) else int(dtype)


def _lay(layout) -> int:
    return LAYOUTS[layout] if isinstance(layout, str) else int(layout)


def _buf(x):
    """Return (pointer, keepalive) for a contiguous numpy/torch CPU buffer or None."""
    if x is None:
        return None, None
    if hasattr(x, "data_ptr"):              # torch CPU tensor
        if x.device.type != "cpu" or not x.is_contiguous():
            raise ValueError("oracle takes contiguous CPU tensors")
        return x.data_ptr(), x
    a = np.ascontiguousarray(x)
    return a.ctypes.data, a


def max_threads() -> int:
    return _load().orc_max_threads()


def decode(dtype, bits) -> np.ndarray:
    """Storage bits (uint32 for f32, uint16 for f16/bf16) -> exact float64."""
    d = _dt(dtype)
    b = np.ascontiguousarray(bits, dtype=_STORAGE[d])
    out = np.empty(b.shape, np.float64)
    _load().orc_decode_array(d, b.ctypes.data, b.size, out.ctypes.data)
    return out


def encode(dtype, x) -> np.ndarray:
    """float64 -> storage bits, IEEE round-to-nearest-even."""
    d = _dt(dtype)
    a = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(a.shape, _STORAGE[d])
    _load().orc_encode_array(d, a.ctypes.data, a.size, out.ctypes.data)
    return out


def round_to(dtype, x) -> np.ndarray:
    """float64 -> float64 value of the nearest representable element (RNE)."""
    d = _dt(dtype)
    a = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(a.shape, np.float64)
    _load().orc_round_array(d, a.ctypes.data, a.size, out.ctypes.data)
    return out


def silu_epilogue(dtype, c_exact) -> np.ndarray:
    """Unrounded FP64 value of the fused projection Y = SiLU(round(C)).

    "Chapter 5: Operators and Runtime" (ai-infra-book), section 5.4.2 (the
    loop nest for Y = SiLU(AW): the FP32 sum is rounded to the output format,
    then the activation is applied) and section 5.4.3 (the activation must
    come after the whole K reduction and after that rounding).  SiLU(x) is
    x * sigmoid(x) = x / (1 + e^-x).  ``c_exact`` holds the unrounded GEMM
    results (as returned by ``gemm``); the stored Y is round_to(dtype, result).
    """
    c = round_to(dtype, c_exact)
    with np.errstate(over="ignore"):
        return c / (1.0 + np.exp(-c))


def swiglu(dtype, g_exact, u_exact) -> np.ndarray:
    """Unrounded FP64 value of the gated FFN pair Z = SiLU(G) * U.

    "Chapter 5: Operators and Runtime", section 5.3.1 (G = X W_g and
    U = X W_u, Z = SiLU(G) elementwise-times U, every tensor stored in the
    output format) and Figure 5-14 (fusing keeps the rounding of the
    intermediate results): G and U are rounded as stored tensors, T = SiLU(G)
    is rounded as the stored intermediate, and Z = T * U is rounded on store.
    ``g_exact`` and ``u_exact`` are the unrounded GEMM results from ``gemm``.
    """
    t = round_to(dtype, silu_epilogue(dtype, g_exact))
    return t * round_to(dtype, u_exact)


def gemm(layoutA, layoutB, M, N, K, alpha, A, lda, B, ldb, beta, C_in, C_out, ldc, dtype,
         rows=None, want_exact=True, nthreads=0):
    """C_out <- round(alpha*op(A)op(B) + beta*C_in) for all rows or the listed rows.

    A, B, C_in, C_out are flat storage buffers (numpy arrays of the storage
    type, or contiguous CPU torch tensors) addressed with the given leading
    dimensions.  Returns the unrounded float64 values as a (len(rows) or M, N)
    array when want_exact, else None.  C_out may be None.
    """
    lib = _load()
    pa, ka = _buf(A)
    pb, kb = _buf(B)
    pc, kc = _buf(C_in)
    po, ko = _buf(C_out)
    if rows is not None:
        rows_a = np.ascontiguousarray(rows, dtype=np.int64)
        nrows, prow = rows_a.size, rows_a.ctypes.data
    else:
        rows_a, nrows, prow = None, M, None
    exact = np.empty((nrows, N), np.float64) if want_exact else None
    rc = lib.orc_gemm_rows(_lay(layoutA), _lay(layoutB), M, N, K, float(alpha), pa, lda, pb,
                           ldb, float(beta), pc, po, ldc, _dt(dtype), nrows if rows is not None
                           else 0, prow, exact.ctypes.data if want_exact else None, nthreads)
    del ka, kb, kc, ko, rows_a
    if rc != 0:
        raise ValueError("oracle gemm rejected its arguments (code %d)" % rc)
    return exact


def gemm_points(layoutA, layoutB, M, N, K, alpha, A, lda, B, ldb, beta, C_in, ldc, dtype,
                pi, pj, nthreads=0):
    """Unrounded float64 value of the listed outputs (i, j), each summed on its own."""
    lib = _load()
    pa, ka = _buf(A)
    pb, kb = _buf(B)
    pc, kc = _buf(C_in)
    pi = np.ascontiguousarray(pi, dtype=np.int64)
    pj = np.ascontiguousarray(pj, dtype=np.int64)
    out = np.empty(pi.size, np.float64)
    rc = lib.orc_gemm_points(_lay(layoutA), _lay(layoutB), M, N, K, float(alpha), pa, lda, pb,
                             ldb, float(beta), pc, ldc, _dt(dtype), pi.size, pi.ctypes.data,
                             pj.ctypes.data, out.ctypes.data, nthreads)
    del ka, kb, kc
    if rc != 0:
        raise ValueError("oracle gemm_points rejected its arguments (code %d)" % rc)
    return out


def _use_library(path: str | None):
    """Point this module at another build of the oracle (None restores the
    default).  Only the mutation test uses this, to show the pins catch
    planted mistakes in copies of the oracle source."""
    global _lib
    _lib = None
    if path is not None:
        global _LIB
        saved = _LIB
        _LIB = path
        try:
            _load()
        finally:
            _LIB = saved
