"""The oracle still reproduces its stored outputs on the tiny workload (regression anchor).

tests/golden/tiny_oracle.npz is written by tests/golden/make_tiny_golden.py,
which calls only the oracle and the seeded generator.  Also checks properties
that tie the stored chain together (window-score mass, recent window kept,
selection consistent with the stored scores).
"""

import os
import sys

import numpy as np

import oracle

sys.path.insert(0, os.path.join(os.path.dirname(__file__), "golden"))
import make_tiny_golden  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tiny_oracle.npz")


def test_tiny_golden_reproduces():
    stored = np.load(GOLDEN, allow_pickle=False)
    now = make_tiny_golden.compute()
    for key, val in now.items():
        ref = stored[key]
        if val.dtype.kind in "iu" or val.dtype == np.float16:
            assert np.array_equal(val, ref), key
        else:
            assert np.allclose(val, ref, rtol=1e-12, atol=1e-15), key


def test_tiny_golden_properties():
    g = np.load(GOLDEN, allow_pickle=False)
    assert np.allclose(g["scores"].sum(-1), 16.0)
    idx = g["idx"]
    assert idx.shape == (1, 2, 64)
    for h in range(2):
        assert set(range(240, 256)) <= set(idx[0, h].tolist())
        assert np.all(np.diff(idx[0, h]) > 0)
    assert np.array_equal(oracle.select_ref(g["scores"], 48, 16), idx)
    assert g["k_codes"].shape == (1, 2, 64, 16) and g["k_scale"].shape == (1, 2, 2, 64)
    # decode output is a convex combination of dequantised values
    _, vh = oracle.dequant_ref({k: g[k] for k in ("k_codes", "k_scale", "k_zero",
                                                   "v_codes", "v_scale", "v_zero")})
    out = g["decode_out"]
    assert np.all(out <= vh.max(axis=2) + 1e-12) and np.all(out >= vh.min(axis=2) - 1e-12)
