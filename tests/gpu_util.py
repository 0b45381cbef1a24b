"""Helpers for the GPU parity tests: device tensors <-> oracle arrays, tolerances."""

import numpy as np
import torch

import oracle


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def to_np(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def packed_to_np(cache):
    """PackedCache tensors -> the oracle's packed dict (codes, fp16 scale / zero)."""
    ksz = cache.k_sz.cpu().numpy().view(np.uint32)
    vsz = cache.v_sz.cpu().numpy().view(np.uint32)
    half = lambda w: (w & 0xFFFF).astype(np.uint16).view(np.float16)  # noqa: E731
    return {
        "k_codes": cache.k_codes.cpu().numpy(),
        "k_scale": half(ksz),
        "k_zero": half(ksz >> 16),
        "v_codes": cache.v_codes.cpu().numpy(),
        "v_scale": half(vsz),
        "v_zero": half(vsz >> 16),
    }


def assert_packed_equal(got, ref):
    for key in ("k_codes", "v_codes"):
        g, r = got[key], ref[key]
        assert g.shape == r.shape, key
        bad = np.count_nonzero(g != r)
        assert bad == 0, f"{key}: {bad} of {g.size} bytes differ"
    for key in ("k_scale", "k_zero", "v_scale", "v_zero"):
        g = got[key].view(np.uint16)
        r = np.asarray(ref[key], dtype=np.float16).view(np.uint16)
        assert g.shape == r.shape, key
        bad = np.count_nonzero(g != r)
        assert bad == 0, f"{key}: {bad} of {g.size} fp16 words differ"


def pack_parity(got, ref, what="pack"):
    """Packed cache against the oracle's (quant_pack_ref with return_u).

    Codes first, with near-ties (|u - (m + 1/2)| < 1e-6 on the oracle's fp32
    ratio) excluded and counted: no code may differ elsewhere.  Then every
    byte and fp16 word bit for bit (both sides decide in fp32 with the same
    rule, so near-tie flips are expected to be 0 as well).  Prints and returns
    the counts {"k": (near_ties, flips), "v": (...)}.
    """
    n = ref["k_u"].shape[2]
    counts = {}
    for name, g, r, u in (
            ("k", oracle.unpack_codes_ref(got["k_codes"]), oracle.unpack_codes_ref(ref["k_codes"]), ref["k_u"]),
            ("v", oracle.unpack_value_codes_ref(got["v_codes"], n), oracle.unpack_value_codes_ref(ref["v_codes"], n),
             ref["v_u"])):
        off, near, flips = oracle.code_parity(g, r, u)
        assert off == 0, f"{what}: {off} {name} codes differ away from near-ties"
        counts[name] = (near, flips)
    print(f"{what}: code near-ties (count, flipped) keys {counts['k']}, values {counts['v']}", flush=True)
    assert_packed_equal(got, ref)
    return counts


def check_selection(idx_gpu, sc_gpu, sc_ref, n_heavy, n_recent, what="select"):
    """Selection exact against the oracle on the GPU's own fp32 scores, and
    different from the oracle on its fp64 scores only inside the near-tie set.
    Returns (index differences against fp64, near-tie set size)."""
    assert np.array_equal(idx_gpu, oracle.select_ref(sc_gpu, n_heavy, n_recent)), f"{what}: not exact"
    idx_ref = oracle.select_ref(sc_ref, n_heavy, n_recent)
    near = oracle.index_near_ties(sc_ref, n_heavy, n_recent)
    flat_g = idx_gpu.reshape(-1, idx_gpu.shape[-1])
    flat_r = idx_ref.reshape(-1, idx_ref.shape[-1])
    n_diff = n_near = 0
    for row in range(flat_g.shape[0]):
        sym = set(flat_g[row].tolist()) ^ set(flat_r[row].tolist())
        assert sym <= set(near[row].tolist()), f"{what} row {row}: {sorted(sym)[:8]} not near-ties"
        n_diff += len(sym)
        n_near += len(near[row])
    print(f"{what}: index near-ties {n_near}, differences against fp64 {n_diff}", flush=True)
    return n_diff, n_near


def assert_attn_close(got, ref, what):
    """|got - ref| <= max(2e-3, 1 bf16 ulp of ref), elementwise (bf16 outputs, fp32 math)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape
    err = np.abs(got - ref)
    tol = oracle.attn_tolerance(ref)
    bad = err > tol
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} beyond tolerance; "
                           f"max err {err.max():.3g}, max err/tol {(err / tol).max():.3g}")
    return float(err.max())
