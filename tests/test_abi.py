"""The C ABI: libmgemm.so loads, exports every function include/mgemm.h
declares, and the header compiles as plain C.  No compute call is made (no
GPU is needed)."""
import ctypes
import os
import re
import subprocess

import pytest

import dense_gemm_mgemm_amd as mg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mgemm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mgemm_[a-z0-9_]+)\s*\(", text)))


def test_library_is_built():
    assert os.path.exists(mg.LIB_PATH), "run `python -m dense_gemm_mgemm_amd.build`"


def test_exports_every_declared_symbol():
    lib = ctypes.CDLL(mg.LIB_PATH)
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), "libmgemm.so does not export %s" % n
    assert sorted(mg.EXPORTED) == names


def test_nm_shows_c_linkage():
    out = subprocess.run(["nm", "-D", "--defined-only", mg.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    syms = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for n in declared_functions():
        assert n in syms          # unmangled: extern "C"


def test_header_compiles_as_c(tmp_path):
    src = tmp_path / "use.c"
    src.write_text('#include "mgemm.h"\n'
                   "int main(void) {\n"
                   "  mgemm_handle_t h = 0;\n"
                   "  mgemm_kernel_t k = MGEMM_KERNEL_AUTO;\n"
                   "  (void)h; (void)k;\n"
                   "  return mgemm_status_string(MGEMM_SUCCESS) == 0;\n"
                   "}\n")
    exe = tmp_path / "use"
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe), "-L", os.path.dirname(mg.LIB_PATH), "-lmgemm",
                    "-Wl,-rpath," + os.path.dirname(mg.LIB_PATH)], check=True)


def test_strings_and_kernel_names():
    assert mg.mgemm_status_string(0) == "success"
    assert mg.mgemm_status_string(99) == "unknown"
    for i, name in enumerate(mg.KERNELS):
        assert mg.mgemm_kernel_name(i) == name
    assert mg.mgemm_kernel_name(1234) == "unknown"


def test_null_handle_is_rejected_without_touching_a_gpu():
    lib = mg.load()
    st = lib.mgemm_run(None, 0, 0, 4, 4, 4, 1.0, None, 4, None, 4, 0.0, None, 4, 0, None)
    assert st == mg.MGEMM_ERR_INVALID_ARG
    out = ctypes.c_int()
    st = lib.mgemm_select_kernel(None, 0, 0, 4, 4, 4, 1.0, None, 4, None, 4, 0.0, None, 4, 0,
                                 ctypes.byref(out))
    assert st == mg.MGEMM_ERR_INVALID_ARG
    assert lib.mgemm_num_cu(None) == 0
    assert lib.mgemm_destroy(None) == mg.MGEMM_SUCCESS


def test_create_without_gpu_fails_cleanly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    h = ctypes.c_void_p()
    st = mg.load().mgemm_create(ctypes.byref(h))
    assert st in (mg.MGEMM_ERR_HIP, mg.MGEMM_ERR_UNSUPPORTED)
    assert h.value is None


def test_set_clock_stamps_needs_a_handle():
    assert mg.load().mgemm_set_clock_stamps(None, None, 0) == mg.MGEMM_ERR_INVALID_ARG


def test_acc32_needs_a_handle():
    assert mg.load().mgemm_run_acc32(None, 0, 0, 0, 4, 4, 32, 1.0, None, 32, None, 4, None, 4, 1,
                                     None) == mg.MGEMM_ERR_INVALID_ARG
