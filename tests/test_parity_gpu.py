"""GPU parity: every step of the HIP path against the CPU oracle on the same inputs.

Integer / byte outputs (codes, fp16 scale / zero words, selected indices) must
be bit-exact; attention outputs within max(2e-3, 1 bf16 ulp) elementwise of
the fp64 oracle; window scores within a relative 1e-4 (fp32 logits vs fp64).
"""

import numpy as np
import pytest
import torch

import oracle
import synth
import bit_quantized_kv_quant_amd as mk
from gpu_util import (assert_attn_close, check_selection, pack_parity, packed_to_np, require_gpu, to_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def say(*a):
    print(*a, flush=True)


# ---------------------------------------------------------------------------
# quantise + pack
# ---------------------------------------------------------------------------

def _pack_and_compare(k, v, idx, dev, what="pack"):
    kd = torch.from_numpy(k).to(dev) if isinstance(k, np.ndarray) else k
    vd = torch.from_numpy(v).to(dev) if isinstance(v, np.ndarray) else v
    idd = None if idx is None else torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).to(dev)
    cache = mk.quant_pack(kd, vd, idd)
    torch.cuda.synchronize()
    got = packed_to_np(cache)
    ref = oracle.quant_pack_ref(to_np(kd), to_np(vd), idx, return_u=True)
    pack_parity(got, ref, what)
    return cache


def test_quant_pack_tiny_all_tokens(dev):
    say("quant_pack tiny fp32 D64 T256 all tokens")
    d = synth.tiny_inputs(0)
    _pack_and_compare(d["k"], d["v"], None, dev)


@pytest.mark.parametrize("n", [1, 31, 32, 33, 77, 256])
def test_quant_pack_bf16_ragged(dev, n):
    say("quant_pack bf16 D128 B2 Hkv3 T300 n", n)
    rng = np.random.default_rng(n)
    k = synth.bf16_round(rng.standard_normal((2, 3, 300, 128)).astype(np.float32) * 3)
    v = synth.bf16_round(rng.standard_normal((2, 3, 300, 128)).astype(np.float32))
    idx = np.sort(np.stack([[rng.choice(300, n, replace=False) for _ in range(3)] for _ in range(2)]), -1)
    kd = torch.from_numpy(k).to(dev).to(torch.bfloat16)
    vd = torch.from_numpy(v).to(dev).to(torch.bfloat16)
    _pack_and_compare(kd, vd, idx, dev)


@pytest.mark.parametrize("dtype,D", [("f32", 64), ("f32", 128), ("bf16", 64), ("bf16", 128)])
@pytest.mark.parametrize("n,T,with_idx", [(5, 40, True), (70, 70, False), (161, 500, True)])
def test_quant_pack_each_tile_shape(dev, dtype, D, n, T, with_idx):
    """Every load tile of the pack kernel: fp32 and bf16 rows of 64 and 128
    channels (16-byte chunks of 4 or 8 channels, 2 to 8 rows per load
    instruction), full and partial groups, gathered and identity rows."""
    say("quant_pack tile", dtype, "D", D, "n", n, "T", T, "idx", with_idx)
    rng = np.random.default_rng(1000 * D + n)
    k = rng.standard_normal((2, 3, T, D)).astype(np.float32) * 2
    k[..., 5] *= 30.0                                     # an outlier channel
    v = rng.standard_normal((2, 3, T, D)).astype(np.float32)
    idx = (np.sort(np.stack([[rng.choice(T, n, replace=False) for _ in range(3)] for _ in range(2)]), -1)
           if with_idx else None)
    kd, vd = torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev)
    if dtype == "bf16":
        kd, vd = kd.to(torch.bfloat16), vd.to(torch.bfloat16)
    _pack_and_compare(kd, vd, idx, dev, f"tile {dtype} D{D} n{n}")


def test_quant_pack_special_groups(dev):
    """Constant groups, exact ties, fp16 zero rounding up, subnormal and vanishing scales."""
    say("quant_pack special groups fp32 D64")
    T, D = 64, 64
    k = np.zeros((1, 2, T, D), np.float32)
    v = np.zeros((1, 2, T, D), np.float32)
    k[0, 0, :, 0] = 1.25                                       # constant key group
    k[0, 0, :, 1] = np.tile([0, 0.5, 1.5, 2.5, 3.0, 1.0, 2.0, 0.25], 8)  # ties at 0.5, 1.5, 2.5
    k[0, 0, :, 2] = np.tile([1000.75, 1001.0], 32)             # z rounds up past the range
    k[0, 0, :, 3] = np.tile([0.0, 2.0 ** -20], 32)             # subnormal fp16 scale
    k[0, 0, :, 4] = np.tile([0.0, 2.0 ** -26], 32)             # scale underflows to 0
    k[0, 0, :, 5] = np.tile([1 + 2.0 ** -11, 4.0], 32)         # z ties down to even
    k[0, 1] = np.random.default_rng(3).standard_normal((T, D)).astype(np.float32) * 1e-6
    v[0, 0, :, :32] = np.tile([-3.0, -2.5, -1.5, -0.5, 0.0, -1.0, -2.0, -0.75], 4)
    v[0, 0, :, 32:] = 7.5                                      # constant value group
    v[0, 1] = np.random.default_rng(4).standard_normal((T, D)).astype(np.float32) * 100
    _pack_and_compare(k, v, None, dev)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quant_pack_signed_zero_groups(dev, dtype):
    """Groups whose minimum is zero with -0 and +0 mixed in both orders, all -0,
    all +0, and zero maxima of non-positive groups: the stored zero point takes
    -0 below +0 (its fp16 sign bit), bit for bit with the oracle; full and
    partial key groups."""
    say("quant_pack signed zeros", dtype)
    T, D = 40, 64
    k = np.zeros((1, 2, T, D), np.float32)
    v = np.zeros((1, 2, T, D), np.float32)
    k[0, 0, 1::2, 0] = -0.0                      # +0, -0, +0, ...
    k[0, 0, 0::2, 1] = -0.0                      # -0, +0, -0, ...
    k[0, 0, :, 2] = -0.0                         # all -0
    k[0, 0, ::3, 4] = 1.5                        # +0 minimum with a positive maximum
    k[0, 0, 1::3, 5] = -0.0
    k[0, 0, ::3, 5] = 1.5                        # -0 minimum with a positive maximum
    k[0, 0, ::2, 6] = -1.5
    k[0, 0, 1::4, 6] = -0.0                      # zero maximum of a non-positive group
    k[0, 0, 39, 7] = -0.0                        # a -0 only in the partial last group
    rng = np.random.default_rng(17)
    k[0, 1] = np.where(rng.random((T, D)) < 0.5, np.float32(-0.0), np.float32(0.0))
    k[0, 1, :, ::3] += rng.integers(0, 4, (T, (D + 2) // 3)).astype(np.float32) * 0.5
    v[0, 0, 0, 1::2] = -0.0                      # token 0: +0, -0, ... in both value groups
    v[0, 0, 1, 0::2] = -0.0                      # token 1: -0, +0, ...
    v[0, 0, 2, :] = -0.0
    v[0, 0, 3, ::5] = 0.75
    v[0, 0, 3, 1::5] = -0.0
    v[0, 1] = np.where(rng.random((T, D)) < 0.5, np.float32(-0.0), np.float32(0.0))
    v[0, 1, ::2] -= rng.integers(0, 3, ((T + 1) // 2, D)).astype(np.float32) * 0.25
    kd, vd = torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev)
    if dtype == "bf16":
        kd, vd = kd.to(torch.bfloat16), vd.to(torch.bfloat16)
        assert (kd.view(torch.int16) == -32768).any()   # the -0 survives the cast
    cache = _pack_and_compare(kd, vd, None, dev, f"signed zeros {dtype}")
    kz = (cache.k_sz.cpu().numpy().view(np.uint32) >> 16)[0, 0, 0]
    assert kz[0] == 0x8000 and kz[1] == 0x8000 and kz[2] == 0x8000 and kz[4] == 0


def test_quant_pack_llama7b_shape(dev):
    """8 x 32 heads x 4096 tokens, 614 kept (bf16), every byte compared."""
    wl = synth.WORKLOADS["llama7b_decode"]
    say("quant_pack llama7b B8 H32 T4096 n614")
    _, k, v, _ = synth.make_qkv(wl, dev, q_rows=1)
    g = torch.Generator(device="cpu").manual_seed(5)
    idx = torch.sort(torch.rand((wl.B, wl.Hkv, wl.T), generator=g).argsort(-1)[..., :614], -1).values
    _pack_and_compare(k, v, idx.numpy().astype(np.int32), dev)


# ---------------------------------------------------------------------------
# selection
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T,n_heavy,n_recent,levels", [
    (256, 48, 16, 0), (256, 48, 16, 5), (4096, 492, 122, 0), (4096, 492, 122, 64),
    (1000, 0, 10, 0), (1000, 990, 10, 0), (16384, 1966, 491, 0), (44000, 5280, 1320, 0),
    (44000, 5280, 1320, 1000), (65000, 100, 7, 0), (33, 32, 1, 3),
])
def test_select_matches_oracle(dev, T, n_heavy, n_recent, levels):
    say("select T", T, "heavy", n_heavy, "recent", n_recent, "levels", levels)
    rng = np.random.default_rng(T + n_heavy)
    rows = 3
    if levels:
        s = (rng.integers(0, levels, (1, rows, T)) / levels).astype(np.float32)
    else:
        s = rng.random((1, rows, T), dtype=np.float32) * 0.01
    s[0, 0, : T // 3] = 0.0 if levels else s[0, 0, : T // 3]
    got = mk.select_topk(torch.from_numpy(s).to(dev), n_heavy, n_recent)
    torch.cuda.synchronize()
    ref = oracle.select_ref(s, n_heavy, n_recent)
    assert np.array_equal(got.cpu().numpy(), ref)


def test_select_all_equal_and_negative_zero(dev):
    say("select all-equal / signed zeros")
    T = 500
    s = np.zeros((2, 2, T), np.float32)
    s[0, 1, ::2] = -0.0
    s[1] = 0.125
    got = mk.select_topk(torch.from_numpy(s).to(dev), 40, 10).cpu().numpy()
    ref = oracle.select_ref(s, 40, 10)
    assert np.array_equal(got, ref)
    assert np.array_equal(got[0, 0, :40], np.arange(40))


# ---------------------------------------------------------------------------
# decode over the packed cache
# ---------------------------------------------------------------------------

def _decode_case(dev, B, Hq, Hkv, n, D, seed, kmul=3.0, vstd=1.0):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, Hkv, n, D)).astype(np.float32) * kmul
    k[..., :4] *= 8
    v = rng.standard_normal((B, Hkv, n, D)).astype(np.float32) * vstd
    q = synth.bf16_round(rng.standard_normal((B, Hq, D)).astype(np.float32))
    kd = torch.from_numpy(k).to(dev).to(torch.bfloat16)
    vd = torch.from_numpy(v).to(dev).to(torch.bfloat16)
    cache = mk.quant_pack(kd, vd)
    qd = torch.from_numpy(q).to(dev).to(torch.bfloat16)
    out = mk.decode_attn(qd, cache)
    torch.cuda.synchronize()
    ref = oracle.decode_ref(q, packed_to_np(cache))
    return to_np(out), ref


@pytest.mark.parametrize("B,Hq,Hkv,n,D", [
    (1, 2, 2, 64, 64), (1, 1, 1, 1, 128), (2, 4, 4, 45, 128), (3, 8, 4, 300, 128), (2, 8, 2, 1000, 128),
    (1, 4, 1, 6600, 128), (4, 2, 1, 129, 64), (8, 32, 32, 614, 128),
    # more token ranges than merge threads: 157 ranges at D = 64, 129 at D = 128
    (1, 2, 1, 20000, 64), (1, 2, 1, 33000, 128),
    # heads merged inside the launch: one 4-wave or one 8-wave workgroup per
    # head (LDS merge), and two, three and four 8-wave workgroups per head
    # (ticket handover; some with empty ranges)
    (3, 8, 4, 300, 128), (2, 8, 2, 1000, 128), (1, 4, 4, 1500, 128), (2, 8, 2, 2000, 64),
    (1, 4, 4, 2900, 128), (2, 8, 2, 4000, 64),
])
def test_decode_matches_oracle(dev, B, Hq, Hkv, n, D):
    say("decode B", B, "Hq", Hq, "Hkv", Hkv, "n", n, "D", D)
    got, ref = _decode_case(dev, B, Hq, Hkv, n, D, seed=B * 1000 + n)
    assert_attn_close(got, ref, "decode out")


def test_decode_single_token_is_vhat(dev):
    say("decode single token")
    rng = np.random.default_rng(1)
    k = torch.from_numpy(rng.standard_normal((2, 2, 1, 128)).astype(np.float32)).to(dev)
    v = torch.from_numpy(rng.standard_normal((2, 2, 1, 128)).astype(np.float32)).to(dev)
    cache = mk.quant_pack(k, v)
    q = torch.randn((2, 4, 128), device=dev).to(torch.bfloat16)
    out = to_np(mk.decode_attn(q, cache))
    _, vh = oracle.dequant_ref(packed_to_np(cache))
    for h in range(4):
        assert_attn_close(out[:, h], vh[:, h // 2, 0], "single-token decode")


# ---------------------------------------------------------------------------
# selective flash attention: pass 1 (o, lse) and pass 2 (window scores)
# ---------------------------------------------------------------------------

def _prefill_case(dev, q, k, v, W, rows=None, with_o=True):
    qd, kd, vd = (torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (q, k, v))
    o, lse, sc = mk.prefill_attn_scores(qd, kd, vd, W, with_o=with_o)
    torch.cuda.synchronize()
    qb, kb, vb = (to_np(x) for x in (qd, kd, vd))
    o_ref, lse_ref = oracle.prefill_ref(qb, kb, vb, rows=rows)
    sc_ref = oracle.window_scores_ref(qb, kb, W)
    sel = slice(None) if rows is None else rows
    lse_g = to_np(lse)[:, :, sel]
    assert np.abs(lse_g - lse_ref).max() < 2e-5 * max(1.0, np.abs(lse_ref).max())
    if with_o:
        assert_attn_close(to_np(o)[:, :, sel], o_ref, "prefill o")
    scg = to_np(sc)
    rel = np.abs(scg - sc_ref) / np.maximum(np.abs(sc_ref), 1e-6)
    assert rel.max() < 1e-4, f"scores rel err {rel.max()}"
    r = q.shape[1] // k.shape[1]
    assert np.allclose(scg.sum(-1), W * r, rtol=1e-4)
    return o, lse, sc


def test_prefill_tiny(dev):
    say("prefill tiny T256 H2 D64 W16")
    d = synth.tiny_inputs(0)
    _prefill_case(dev, d["q"], d["k"], d["v"], 16)


@pytest.mark.parametrize("B,Hq,Hkv,T,D,W", [
    (2, 4, 2, 333, 128, 40), (1, 2, 2, 1, 64, 1), (1, 8, 2, 200, 128, 32), (1, 1, 1, 129, 128, 129),
    (2, 4, 4, 1000, 128, 32), (1, 2, 2, 300, 64, 32), (3, 2, 2, 33, 128, 7), (64, 4, 4, 97, 64, 32),
    (16, 16, 16, 270, 128, 13),
])
def test_prefill_ragged_gqa(dev, B, Hq, Hkv, T, D, W):
    say("prefill B", B, "Hq", Hq, "Hkv", Hkv, "T", T, "D", D, "W", W)
    rng = np.random.default_rng(T)
    q = rng.standard_normal((B, Hq, T, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, T, D)).astype(np.float32)
    k[..., :4] *= 8
    v = rng.standard_normal((B, Hkv, T, D)).astype(np.float32)
    _prefill_case(dev, q, k, v, W)


@pytest.mark.parametrize("B,H,T,D,W", [
    (4, 64, 256, 64, 16), (32, 8, 1000, 128, 32), (64, 4, 300, 64, 32), (256, 1, 1, 128, 1), (128, 2, 33, 128, 32),
    (16, 16, 4100, 128, 4), (8, 32, 4096, 128, 32), (86, 3, 520, 128, 8),
])
@pytest.mark.parametrize("with_o", [True, False])
def test_single_pass_scores_equal_two_passes(dev, B, H, T, D, W, with_o):
    """Scores from inside pass 1 are the second pass's bits; o and lse are pass 1's alone."""
    say("single-pass scores B", B, "H", H, "T", T, "D", D, "W", W, "o", with_o)
    assert mk.prefill_fuses_scores(B, T, H, H, W), "needs at least one head per compute unit"
    g = torch.Generator(device=dev).manual_seed(T * 7 + W)
    q = torch.randn((B, H, T, D), generator=g, device=dev).to(torch.bfloat16)
    k = torch.randn((B, H, T, D), generator=g, device=dev)
    k[..., :3] *= 6
    k = k.to(torch.bfloat16)
    v = torch.randn((B, H, T, D), generator=g, device=dev).to(torch.bfloat16)
    o1, l1, s1 = mk.prefill_attn_scores(q, k, v, W, with_o=with_o)
    o2, l2 = mk.prefill_attn(q, k, v, with_o=with_o)
    s2 = mk.window_scores(q, k, l2, W)
    torch.cuda.synchronize()
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    if with_o:
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32))
    r = torch.allclose(s1.sum(-1).double(), torch.full((B, H), float(W), dtype=torch.float64, device=dev), rtol=1e-4)
    assert r


def test_prefill_lse_only_matches(dev):
    say("prefill without o")
    rng = np.random.default_rng(9)
    q, k, v = (rng.standard_normal((1, 2, 300, 128)).astype(np.float32) for _ in range(3))
    _, lse1, sc1 = _prefill_case(dev, q, k, v, 32, with_o=True)
    _, lse2, sc2 = _prefill_case(dev, q, k, v, 32, with_o=False)
    assert torch.equal(lse1, lse2) and torch.equal(sc1, sc2)


def test_prefill_16k_chain(dev):
    """The 16k prefill-and-compress workload end to end at its own sizes (1 x 32
    heads x 16384 causal tokens, W = 32, 15 % budget): o / lse on sampled rows,
    every window score; then selection of 1966 heavy + 491 recent tokens on those
    scores (exact on the GPU's scores, near-ties only against fp64), the 2-bit
    pack of the 2457 kept tokens x 32 heads (codes with near-ties counted, every
    byte), and one decode query over the packed cache."""
    wl = synth.WORKLOADS["prefill_16k"]
    say("prefill 16k H32 D128: prefill + scores")
    q, k, v, _ = synth.make_qkv(wl, dev)
    o, lse, sc = mk.prefill_attn_scores(q, k, v, wl.window)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 63, 64, 127, 128, 129, 4095, 8191, 8192, 12345, 16256, 16383])
    qb, kb, vb = (to_np(x) for x in (q, k, v))
    o_ref, lse_ref = oracle.prefill_ref(qb, kb, vb, rows=rows)
    assert_attn_close(to_np(o)[:, :, rows], o_ref, "prefill 16k o")
    assert np.abs(to_np(lse)[:, :, rows] - lse_ref).max() < 1e-4
    sc_ref = oracle.window_scores_ref(qb, kb, wl.window)
    sc_np = to_np(sc)
    rel = np.abs(sc_np - sc_ref) / np.maximum(sc_ref, 1e-6)
    assert rel.max() < 1e-4
    del o, q, o_ref
    say("prefill 16k: select 1966 + 491, pack 2457 x 32 heads, decode")
    n_keep = oracle.keep_count(wl.T, wl.budget_pct)
    nh, nr = oracle.split_heavy_recent(n_keep)
    assert (n_keep, nh, nr) == (2457, 1966, 491)
    idx = mk.select_topk(sc, nh, nr)
    cache = mk.quant_pack(k, v, idx)
    qdec = synth.make_decode_q(wl, dev)
    out = mk.decode_attn(qdec, cache)
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    check_selection(idx_np, sc_np, sc_ref, nh, nr, "16k select")
    got = packed_to_np(cache)
    pack_parity(got, oracle.quant_pack_ref(kb, vb, idx_np, return_u=True), "16k pack")
    assert_attn_close(to_np(out), oracle.decode_ref(to_np(qdec), got), "16k decode")


# ---------------------------------------------------------------------------
# the whole chain
# ---------------------------------------------------------------------------

def _chain(dev, q, k, v, qdec, W, n_heavy, n_recent, k_pack=None, v_pack=None):
    """GPU chain; each step compared with the oracle fed the GPU's own inputs to that step."""
    qd, kd, vd = (torch.from_numpy(x).to(dev).to(torch.bfloat16) if isinstance(x, np.ndarray) else x
                  for x in (q, k, v))
    _, _, sc = mk.prefill_attn_scores(qd, kd, vd, W, with_o=False)
    idx = mk.select_topk(sc, n_heavy, n_recent)
    kp = kd if k_pack is None else torch.from_numpy(k_pack).to(dev)
    vp = vd if v_pack is None else torch.from_numpy(v_pack).to(dev)
    cache = mk.quant_pack(kp, vp, idx)
    qdd = torch.from_numpy(qdec).to(dev).to(torch.bfloat16) if isinstance(qdec, np.ndarray) else qdec
    out = mk.decode_attn(qdd, cache)
    torch.cuda.synchronize()
    # selection: exact against the oracle run on the GPU's fp32 scores, and
    # against the oracle's own fp64 scores different only on near-ties
    sc_np = to_np(sc)
    idx_np = idx.cpu().numpy()
    sc_ref = oracle.window_scores_ref(to_np(qd), to_np(kd), W)
    n_diff, _ = check_selection(idx_np, sc_np, sc_ref, n_heavy, n_recent, "chain select")
    # packing of the GPU's selection: codes with near-ties counted, then bit-exact
    ref_pack = oracle.quant_pack_ref(to_np(kp), to_np(vp), idx_np, return_u=True)
    got_pack = packed_to_np(cache)
    pack_parity(got_pack, ref_pack, "chain pack")
    # decode on the packed cache
    ref_out = oracle.decode_ref(to_np(qdd), got_pack)
    err = assert_attn_close(to_np(out), ref_out, "chain decode")
    return n_diff, err


def test_chain_tiny(dev):
    say("chain tiny")
    d = synth.tiny_inputs(0)
    _chain(dev, synth.bf16_round(d["q"]), synth.bf16_round(d["k"]), synth.bf16_round(d["v"]),
           synth.bf16_round(d["q_dec"]), 16, 48, 16, k_pack=d["k"], v_pack=d["v"])


def test_chain_llama7b(dev):
    wl = synth.WORKLOADS["llama7b_decode"]
    say("chain llama7b B8 H32 T4096")
    q, k, v, _ = synth.make_qkv(wl, dev)
    qdec = synth.make_decode_q(wl, dev)
    n_keep = oracle.keep_count(wl.T, wl.budget_pct)
    nh, nr = oracle.split_heavy_recent(n_keep)
    n_diff, err = _chain(dev, q, k, v, qdec, wl.window, nh, nr)
    say("near-tie index differences:", n_diff, "decode max err:", err)


# ---------------------------------------------------------------------------
# determinism (races show up as run-to-run differences)
# ---------------------------------------------------------------------------

def test_repeat_runs_bit_identical(dev):
    say("determinism")
    wl = synth.WORKLOADS["llama7b_decode"]
    q, k, v, _ = synth.make_qkv(wl, dev, seed=11)
    qdec = synth.make_decode_q(wl, dev, seed=11)
    res = []
    for _ in range(2):
        o, lse, sc = mk.prefill_attn_scores(q, k, v, wl.window)
        idx = mk.select_topk(sc, 492, 122)
        cache = mk.quant_pack(k, v, idx)
        out = mk.decode_attn(qdec, cache)
        torch.cuda.synchronize()
        res.append([o.clone(), lse.clone(), sc.clone(), idx.clone(), cache.k_codes.clone(), cache.v_sz.clone(),
                    out.clone()])
    for a, b in zip(*res):
        assert torch.equal(a, b)


# ---------------------------------------------------------------------------
# full-size configurations, checked on sampled outputs
# ---------------------------------------------------------------------------

def _slice_cache(cache, bsel):
    """The packed cache of the sequences bsel (device copies)."""
    ix = torch.as_tensor(bsel, device=cache.k_codes.device)
    return mk.PackedCache(cache.k_codes[ix].contiguous(), cache.k_sz[ix].contiguous(),
                          cache.v_codes[ix].contiguous(), cache.v_sz[ix].contiguous(),
                          len(bsel), cache.Hkv, cache.n_keep, cache.D)


@pytest.mark.parametrize("B", [64, 256, 1133])
@pytest.mark.parametrize("layer", [0, 39])
def test_decode_pyramid_layer_sampled(dev, B, layer):
    """LLaMA2-13B-shaped pyramid layer (40 heads, context 8192, budget 30 % -> 5 %): the
    whole batch decoded (several work items per wave; at B = 64 each KV head is split
    into token ranges; B = 1133 is the headline's batch and launch, 11 or 12 KV heads per
    wave, the last sequence in the twelfth round), sampled sequences against the oracle."""
    wl = synth.WORKLOADS["llama13b_pyramid"]
    n = oracle.pyramid_keep(wl.T, wl.layers, layer, *wl.pyramid)
    say("pyramid decode layer", layer, "n", n, "B", B)
    cache = mk.PackedCache.alloc(B, wl.Hkv, n, wl.D, dev)
    for b0 in range(0, B, 64):
        b1 = min(B, b0 + 64)
        k, v = synth.make_kept_kv(wl, n, dev, seed=wl.seed * 100000 + layer * 1000 + b0, B=b1 - b0)
        sub = mk.PackedCache(cache.k_codes[b0:b1], cache.k_sz[b0:b1], cache.v_codes[b0:b1], cache.v_sz[b0:b1],
                             b1 - b0, wl.Hkv, n, wl.D)
        mk.quant_pack(k, v, out=sub)
        del k, v
    q = synth.make_decode_q(wl, dev, B=B)
    out = mk.decode_attn(q, cache)
    torch.cuda.synchronize()
    bsel = sorted({0, 1, B // 2, B - 1})
    ref = oracle.decode_ref(to_np(q)[bsel], packed_to_np(_slice_cache(cache, bsel)))
    assert_attn_close(to_np(out)[bsel], ref, "pyramid decode")


def test_gqa_44k_chain_sampled(dev):
    """Mistral-7B-shaped long context (GQA 32 / 8, prompt 44000, batch 4, 15 % budget):
    the whole chain at full size; o / lse on sampled rows and window scores for the
    first KV heads of sequence 0, selection exact on the GPU's scores, packing
    bit-exact, decode of every head against the oracle."""
    wl = synth.WORKLOADS["mistral_44k"]
    say("gqa 44k: prefill")
    q, k, v, _ = synth.make_qkv(wl, dev)
    o, lse, sc = mk.prefill_attn_scores(q, k, v, wl.window)
    torch.cuda.synchronize()
    hq = slice(0, 8)   # query heads 0..7 = KV heads 0, 1
    hk = slice(0, 2)
    qb = to_np(q[0:1, hq])
    kb = to_np(k[0:1, hk])
    vb = to_np(v[0:1, hk])
    rows = np.array([0, 1, 127, 128, 4095, 22000, 43967, 43968, 43999])
    o_ref, lse_ref = oracle.prefill_ref(qb, kb, vb, rows=rows)
    assert_attn_close(to_np(o[0:1, hq])[:, :, rows], o_ref, "gqa prefill o")
    assert np.abs(to_np(lse[0:1, hq])[:, :, rows] - lse_ref).max() < 1e-4
    say("gqa 44k: window scores")
    sc_ref = oracle.window_scores_ref(qb, kb, wl.window)
    sc_np = to_np(sc)
    rel = np.abs(sc_np[0:1, hk] - sc_ref) / np.maximum(sc_ref, 1e-6)
    assert rel.max() < 1e-4
    say("gqa 44k: select / pack / decode")
    n_keep = oracle.keep_count(wl.T, wl.budget_pct)
    nh, nr = oracle.split_heavy_recent(n_keep)
    idx = mk.select_topk(sc, nh, nr)
    cache = mk.quant_pack(k, v, idx)
    qdec = synth.make_decode_q(wl, dev)
    out = mk.decode_attn(qdec, cache)
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    assert np.array_equal(idx_np, oracle.select_ref(sc_np, nh, nr))
    del o, q
    got = packed_to_np(cache)
    pack_parity(got, oracle.quant_pack_ref(to_np(k), to_np(v), idx_np, return_u=True), "gqa 44k pack")
    assert_attn_close(to_np(out), oracle.decode_ref(to_np(qdec), got), "gqa decode")


def test_decode_graph_replay_matches_eager(dev):
    """Decode through several layers captured as one HIP graph: every replay,
    with eager work on the stream between replays, equals the eager result."""
    say("decode: graph capture of 4 layers, 3 replays")
    rng = np.random.default_rng(21)
    B, Hq, Hkv, D = 2, 8, 2, 128
    caches = []
    for n in (300, 257, 64, 1000):
        k = torch.from_numpy(synth.bf16_round(rng.standard_normal((B, Hkv, n, D)).astype(np.float32))).to(dev)
        v = torch.from_numpy(synth.bf16_round(rng.standard_normal((B, Hkv, n, D)).astype(np.float32))).to(dev)
        caches.append(mk.quant_pack(k.to(torch.bfloat16), v.to(torch.bfloat16)))
    q = torch.from_numpy(synth.bf16_round(rng.standard_normal((B, Hq, D)).astype(np.float32))).to(dev).to(torch.bfloat16)
    outs = [torch.empty_like(q) for _ in caches]
    ws = torch.zeros(max(mk.decode_ws_bytes(B, Hq, Hkv, c.n_keep, D) for c in caches) + 16, dtype=torch.uint8, device=dev)
    for c, o in zip(caches, outs):
        mk.decode_attn(q, c, out=o, ws=ws)
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for c, o in zip(caches, outs):
            mk.decode_attn(q, c, out=o, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(graph):
        for c, o in zip(caches, outs):
            mk.decode_attn(q, c, out=o, ws=ws)
    for rep in range(3):
        for o in outs:
            o.zero_()
        mk.decode_attn(q, caches[3], out=torch.empty_like(q), ws=torch.zeros_like(ws))  # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(o, e), f"replay {rep}, layer {i}"
