"""Helpers for the GPU parity tests: device tensors <-> oracle arrays, tolerances."""

import numpy as np
import torch


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


def ulp_bf16(x):
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def assert_attn_close(got, ref, what):
    """|got - ref| <= max(2e-3, 1 bf16 ulp of ref), elementwise (bf16 outputs, fp32 math)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape
    err = np.abs(got - ref)
    tol = np.maximum(2e-3, ulp_bf16(ref))
    bad = err > tol
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} beyond tolerance; "
                           f"max err {err.max():.3g}, max err/tol {(err / tol).max():.3g}")
    return float(err.max())
