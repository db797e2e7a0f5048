"""Checks on the generated gfx950 code that the source relies on.

The direct-to-LDS copies are issued through inline asm that sets m0 and
declares it clobbered.  m0 is a reserved register for the compiler, so that
is only sound if the compiler itself keeps no value in m0 in these kernels:
every m0 access in their code must be one of ours.  Also checks that the
kernels that must not spill registers do not.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dense_gemm_mgemm_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"


_BUILT = {}


def _compile(name, out_dir):
    out = os.path.join(out_dir, name + ".s")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "--offload-device-only", "-S", "-O3",
                        "-std=c++17", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                        "-Rpass-analysis=kernel-resource-usage",
                        "-I" + os.path.join(ROOT, "include"), os.path.join(CSRC, name),
                        "-o", out], check=True, capture_output=True, text=True)
    with open(out) as f:
        return f.read(), r.stderr


def device_build(name, tmp_path):
    """gfx950 assembly of one source and the compiler's per-kernel resource
    remarks, from a single compile shared by every test of this module.  The
    first call compiles every kernel source at once, a few at a time."""
    if not _BUILT:
        from concurrent.futures import ThreadPoolExecutor
        names = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
        with ThreadPoolExecutor(max_workers=max(1, min(8, os.cpu_count() or 1))) as ex:
            for n, res in zip(names, ex.map(lambda n: _compile(n, str(tmp_path)), names)):
                _BUILT[n] = res
    if name not in _BUILT:
        _BUILT[name] = _compile(name, str(tmp_path))
    return _BUILT[name]


def device_asm(src, tmp_path):
    return device_build(os.path.basename(src), tmp_path)[0]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("name", ["k_skinny.hip", "k_h_dma.hip", "k_skinny_sk.hip",
                                  "k_f8.hip"])
def test_m0_only_written_by_our_copies(name, tmp_path):
    text = device_asm(os.path.join(CSRC, name), tmp_path)
    lines = [l.strip() for l in text.splitlines() if re.search(r"\bm0\b", l) and not l.strip().startswith(";")]
    assert lines, "expected the direct-to-LDS copies to set m0"
    body = [l.strip() for l in text.splitlines()]
    for idx, l in enumerate(body):
        if re.search(r"\bm0\b", l) and not l.startswith(";"):
            assert l.startswith("s_mov_b32 m0,"), "unexpected m0 use: " + l
            # our asm: s_mov_b32 m0 / s_nop 0 / global_load_lds_dwordx4
            assert body[idx + 1] == "s_nop 0" and body[idx + 2].startswith("global_load_lds_dwordx4"), l


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
# k_h_mfma.hip and k_h_mfma_u.hip are left out: their 256x256 register-staged
# instantiations hold 256 accumulators plus a full slice of prefetch
# registers and spill a few VGPRs outside the main loop (as does the 2-byte
# load form for two MN-contiguous operands, one VGPR).  Scratch memory also appears when a store loop
# over the accumulators is too large to unroll fully (the array then lives in
# memory), so the per-lane scratch size must be zero as well.
@pytest.mark.parametrize("name", ["k_skinny.hip", "k_f32_mfma.hip", "k_skinny_sk.hip",
                                  "k_h_dma.hip", "k_general.hip", "k_f8.hip", "k_util.hip"])
def test_no_register_spills(name, tmp_path):
    remarks = device_build(name, tmp_path)[1]
    spills = [int(x) for x in re.findall(r"VGPRs Spill: (\d+)", remarks)]
    assert spills and max(spills) == 0, remarks[-2000:]
    scratch = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", remarks)]
    assert len(scratch) == len(spills) and max(scratch) == 0, remarks[-2000:]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("name", sorted(f for f in os.listdir(CSRC) if f.endswith(".hip")))
def test_no_scalar_cache_writes(name, tmp_path):
    """No kernel may write through the scalar data cache: no scalar stores or
    scalar atomics, no scalar-cache write-back or discard.  The split-K
    kernel's fences must come out as vector L2 write-back/invalidate."""
    text = device_asm(os.path.join(CSRC, name), tmp_path)
    bad = [l.strip() for l in text.splitlines()
           if re.match(r"\s*s_(store|buffer_store|atomic|buffer_atomic|dcache_wb|dcache_discard|scratch_store)", l)]
    assert not bad, bad[:5]
