"""The input generators (CPU): the counter-hashed operands that large tests
fill on the device agree with the host's recomputation of any element,
including counters past 2^32, and take only the values -1, 0, 1."""
import numpy as np
import torch

import workloads as W


def test_hashed_operand_matches_host_values():
    nr, nc = 37, 1000
    for dtype in ("f32", "f16", "bf16"):
        t = W.hashed_operand(nr, nc, 77, dtype, "cpu", chunk=4096).float().reshape(nr, nc).numpy()
        h = W.hashed_values(np.arange(nr), np.arange(nc), nc, 77)
        assert np.array_equal(t, h)
    vals, counts = np.unique(h, return_counts=True)
    assert list(vals) == [-1.0, 0.0, 1.0] and counts.min() > 0.3 * h.size


def test_hashed_values_use_the_whole_counter():
    # Counters past 2^32 (elements of operands with more than 2^32 entries):
    # the host formula agrees with the device formula on them, and the high
    # word matters (rows 2^32 apart differ).
    nc = 7
    rows = np.array([2 ** 33 // nc, 2 ** 33 // nc + 1])
    n = torch.tensor(rows)[:, None] * nc + torch.arange(nc)[None, :]
    hh = W._fmix32_torch((n & W._M32) ^ 5)
    hh = W._fmix32_torch(hh ^ (n >> 32))
    assert np.array_equal(((hh % 3) - 1).double().numpy(), W.hashed_values(rows, np.arange(nc), nc, 5))
    lo = W.hashed_values(np.arange(64), np.array([0]), 1, 3)
    hi = W.hashed_values(np.arange(64) + 2 ** 32, np.array([0]), 1, 3)
    assert not np.array_equal(lo, hi)
