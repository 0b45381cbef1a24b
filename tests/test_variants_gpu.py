"""GPU parity of the comparison-table policies: compress() through the C ABI vs the oracle.

Each policy runs pass 1, pass 2 with its window (every prompt row for the
cumulative, H2O-like policy), the selection and the 2-bit pack on the GPU; the
oracle recomputes each step from the GPU's inputs to it.  Same bars as the
chain tests: scores within 1e-4 relative, selection exact on the GPU's scores
and different from the fp64 oracle only on near-ties, packed bytes exact,
decode within max(2e-3, 1 bf16 ulp).
"""

import numpy as np
import pytest
import torch

import oracle
import bit_quantized_kv_quant_amd as mk
from gpu_util import assert_attn_close, check_selection, pack_parity, packed_to_np, require_gpu, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _inputs(dev, B, Hq, Hkv, T, D, seed):
    g = torch.Generator(device=dev).manual_seed(seed)
    q = torch.randn((B, Hq, T, D), generator=g, device=dev).to(torch.bfloat16)
    k = torch.randn((B, Hkv, T, D), generator=g, device=dev)
    k[..., :4] *= 8
    k = k.to(torch.bfloat16)
    v = torch.randn((B, Hkv, T, D), generator=g, device=dev).to(torch.bfloat16)
    qd = torch.randn((B, Hq, D), generator=g, device=dev).to(torch.bfloat16)
    return q, k, v, qd


@pytest.mark.parametrize("policy,B,Hq,Hkv,T,n_layers,layer", [
    ("h2o_like", 2, 8, 2, 700, 1, 0),
    ("h2o_like", 1, 4, 4, 161, 1, 0),
    ("minikv", 2, 8, 2, 700, 1, 0),
    ("kivi_like", 1, 4, 2, 333, 1, 0),
    ("kivi_like", 2, 2, 2, 64, 1, 0),
    ("minikv_pyramid", 1, 4, 2, 1000, 32, 0),
    ("minikv_pyramid", 1, 4, 2, 1000, 32, 31),
])
def test_policy_matches_oracle(dev, policy, B, Hq, Hkv, T, n_layers, layer):
    print("policy", policy, "B", B, "Hq", Hq, "Hkv", Hkv, "T", T, "layer", layer, flush=True)
    D = 128
    q, k, v, qd = _inputs(dev, B, Hq, Hkv, T, D, seed=T + layer)
    W, n_keep, nh, nr = mk.layer_plan(policy, T, n_layers, layer)
    o, idx, cache = mk.compress(q, k, v, policy, n_layers, layer)
    out = mk.decode_attn(qd, cache)
    torch.cuda.synchronize()
    qn, kn, vn = to_np(q), to_np(k), to_np(v)
    # pass 1 output on a few rows (the full check lives with the prefill tests)
    rows = np.array(sorted({0, 1, T // 2, T - 1}))
    o_ref, _ = oracle.prefill_ref(qn, kn, vn, rows=rows)
    assert_attn_close(to_np(o)[:, :, rows], o_ref, f"{policy} o")
    if idx is None:
        assert n_keep == T
        ref_pack = oracle.quant_pack_ref(kn, vn, None, return_u=True)
    else:
        _, lse, sc = mk.prefill_attn_scores(q, k, v, W, with_o=False)
        sc_np = to_np(sc)
        sc_ref = oracle.window_scores_ref(qn, kn, W)
        rel = np.abs(sc_np - sc_ref) / np.maximum(np.abs(sc_ref), 1e-6)
        assert rel.max() < 1e-4, f"scores rel err {rel.max()}"
        idx_np = idx.cpu().numpy()
        assert idx_np.shape == (B, Hkv, n_keep)
        check_selection(idx_np, sc_np, sc_ref, nh, nr, f"{policy} select")
        ref_pack = oracle.quant_pack_ref(kn, vn, idx_np, return_u=True)
    got = packed_to_np(cache)
    pack_parity(got, ref_pack, f"{policy} pack")
    assert cache.nbytes() == oracle.packed_bytes_ref(B, Hkv, n_keep, D)
    assert_attn_close(to_np(out), oracle.decode_ref(to_np(qd), got), f"{policy} decode")
