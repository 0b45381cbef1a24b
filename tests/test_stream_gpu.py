"""GPU parity of streaming decode (generated tokens joining the cache) against the oracle.

A selection starts the cache (whole 32-token groups packed, the rest in the
exact residual window); generated tokens are appended one per step and every
32nd packs the window as the next group.  Packed bytes must equal the oracle's
bit for bit after every flush; decode over packed + residual tokens is within
max(2e-3, 1 bf16 ulp) of the fp64 oracle at every step.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
import bit_quantized_kv_quant_amd as mk
from gpu_util import assert_attn_close, assert_packed_equal, require_gpu, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def say(*a):
    print(*a, flush=True)


def stream_packed_np(c):
    """The valid packed region of a StreamCache as the oracle's packed dict."""
    n, G = c.n_packed, c.n_packed // 32
    ksz = c.k_sz[:, :, :G].cpu().numpy().view(np.uint32)
    vsz = c.v_sz[:, :, :n].cpu().numpy().view(np.uint32)
    half = lambda w: (w & 0xFFFF).astype(np.uint16).view(np.float16)  # noqa: E731
    return {"k_codes": c.k_codes[:, :, :n].cpu().numpy(), "k_scale": half(ksz), "k_zero": half(ksz >> 16),
            "v_codes": c.v_codes[:, :, :G].cpu().numpy(), "v_scale": half(vsz), "v_zero": half(vsz >> 16)}


def _inputs(seed, B, Hkv, T, D):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, Hkv, T, D)).astype(np.float32)
    k[..., :: D // 4] *= 8.0  # outlier key channels
    v = rng.standard_normal((B, Hkv, T, D)).astype(np.float32) * 0.5
    return rng, synth.bf16_round(k), synth.bf16_round(v)


def _check_state(c, st):
    assert c.n_packed == st["packed"]["k_codes"].shape[2] and c.n_res == st["k_res"].shape[2]
    if c.n_packed:
        assert_packed_equal(stream_packed_np(c), st["packed"])
    if c.n_res:
        assert np.array_equal(to_np(c.k_res[:, :, :c.n_res]), st["k_res"])
        assert np.array_equal(to_np(c.v_res[:, :, :c.n_res]), st["v_res"])


@pytest.mark.parametrize("Hq,Hkv,D,n_sel,steps", [(2, 2, 128, 150, 45), (8, 2, 128, 614, 40), (4, 4, 64, 20, 50)])
def test_stream_generation_matches_oracle(dev, Hq, Hkv, D, n_sel, steps):
    say("stream Hq", Hq, "Hkv", Hkv, "D", D, "selection", n_sel, "steps", steps)
    B, T = 2, 700
    rng, k, v = _inputs(n_sel, B, Hkv, T, D)
    idx = np.sort(np.stack([[rng.choice(T, n_sel, replace=False) for _ in range(Hkv)] for _ in range(B)]), -1)
    kd = torch.from_numpy(k).to(dev).to(torch.bfloat16)
    vd = torch.from_numpy(v).to(dev).to(torch.bfloat16)
    idd = torch.from_numpy(idx.astype(np.int32)).to(dev)
    cap = 32 * ((n_sel + steps) // 32 + 1)
    c = mk.StreamCache.alloc(B, Hkv, cap, D, dev).init(kd, vd, idd)
    st = oracle.stream_init_ref(k, v, idx)
    torch.cuda.synchronize()
    _check_state(c, st)
    flushes = 0
    for step in range(steps):
        kn = synth.bf16_round(rng.standard_normal((B, Hkv, D)).astype(np.float32))
        vn = synth.bf16_round(rng.standard_normal((B, Hkv, D)).astype(np.float32) * 0.5)
        before = c.n_packed
        c.append(torch.from_numpy(kn).to(dev).to(torch.bfloat16), torch.from_numpy(vn).to(dev).to(torch.bfloat16))
        st = oracle.stream_append_ref(st, kn, vn)
        q = synth.bf16_round(rng.standard_normal((B, Hq, D)).astype(np.float32))
        out = c.decode(torch.from_numpy(q).to(dev).to(torch.bfloat16))
        torch.cuda.synchronize()
        if c.n_packed != before:
            flushes += 1
            _check_state(c, st)
        assert_attn_close(to_np(out), oracle.stream_decode_ref(q, st), f"stream decode step {step}")
    _check_state(c, st)
    assert flushes == (n_sel % 32 + steps) // 32


def test_stream_decode_without_residual_equals_packed_decode(dev):
    say("stream decode, whole groups only, vs decode_attn")
    B, Hq, Hkv, T, D = 4, 8, 2, 1000, 128
    rng, k, v = _inputs(3, B, Hkv, T, D)
    idx = np.sort(np.stack([[rng.choice(T, 256, replace=False) for _ in range(Hkv)] for _ in range(B)]), -1)
    kd = torch.from_numpy(k).to(dev).to(torch.bfloat16)
    vd = torch.from_numpy(v).to(dev).to(torch.bfloat16)
    idd = torch.from_numpy(idx.astype(np.int32)).to(dev)
    c = mk.StreamCache.alloc(B, Hkv, 512, D, dev).init(kd, vd, idd)
    assert c.n_res == 0 and c.n_packed == 256
    q = torch.from_numpy(synth.bf16_round(rng.standard_normal((B, Hq, D)).astype(np.float32))).to(dev).to(torch.bfloat16)
    a = c.decode(q)
    b = mk.decode_attn(q, mk.quant_pack(kd, vd, idd))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_stream_residual_only(dev):
    say("stream decode, residual tokens only")
    B, Hq, Hkv, T, D = 3, 4, 4, 100, 128
    rng, k, v = _inputs(4, B, Hkv, T, D)
    idx = np.sort(np.stack([[rng.choice(T, 17, replace=False) for _ in range(Hkv)] for _ in range(B)]), -1)
    kd = torch.from_numpy(k).to(dev).to(torch.bfloat16)
    vd = torch.from_numpy(v).to(dev).to(torch.bfloat16)
    c = mk.StreamCache.alloc(B, Hkv, 64, D, dev).init(kd, vd, torch.from_numpy(idx.astype(np.int32)).to(dev))
    assert c.n_packed == 0 and c.n_res == 17
    q = synth.bf16_round(rng.standard_normal((B, Hq, D)).astype(np.float32))
    out = c.decode(torch.from_numpy(q).to(dev).to(torch.bfloat16))
    torch.cuda.synchronize()
    assert_attn_close(to_np(out), oracle.stream_decode_ref(q, oracle.stream_init_ref(k, v, idx)), "residual only")


@pytest.mark.parametrize("D", [64, 128])
def test_stream_decode_many_ranges(dev, D):
    """A long packed region (more token ranges than merge threads) plus a window: host-side
    and device-side counts against the oracle."""
    say("stream decode, many ranges and a window, D", D)
    B, Hq, Hkv, T, n_sel = 1, 2, 1, 33100, 33013
    rng, c, st = _start(dev, 5 + D, B, Hkv, T, D, n_sel, 32 * (n_sel // 32 + 2))
    assert c.n_packed == 32 * (n_sel // 32) and c.n_res == n_sel % 32  # 32992 packed, 21 in the window
    q = synth.bf16_round(rng.standard_normal((B, Hq, D)).astype(np.float32))
    qd = torch.from_numpy(q).to(dev).to(torch.bfloat16)
    ref = oracle.stream_decode_ref(q, st)
    assert_attn_close(to_np(c.decode(qd)), ref, "host counts")
    c.to_device_counts()
    assert_attn_close(to_np(c.step_decode(qd)), ref, "device counts")


# ---------------------------------------------------------------------------
# device-side generation step (counts in device memory) and its graph replays
# ---------------------------------------------------------------------------

def _start(dev, seed, B, Hkv, T, D, n_sel, cap):
    rng, k, v = _inputs(seed, B, Hkv, T, D)
    idx = np.sort(np.stack([[rng.choice(T, n_sel, replace=False) for _ in range(Hkv)] for _ in range(B)]), -1)
    kd = torch.from_numpy(k).to(dev).to(torch.bfloat16)
    vd = torch.from_numpy(v).to(dev).to(torch.bfloat16)
    c = mk.StreamCache.alloc(B, Hkv, cap, D, dev).init(kd, vd, torch.from_numpy(idx.astype(np.int32)).to(dev))
    return rng, c, oracle.stream_init_ref(k, v, idx)


def _token(rng, B, H, D, scale=1.0):
    return synth.bf16_round(rng.standard_normal((B, H, D)).astype(np.float32) * scale)


@pytest.mark.parametrize("Hq,Hkv,D,n_sel,steps", [(8, 2, 128, 150, 70), (4, 4, 64, 20, 45), (2, 2, 128, 64, 33)])
def test_device_step_matches_oracle(dev, Hq, Hkv, D, n_sel, steps):
    """step_append / step_decode (counts read on the device) against the oracle at every step."""
    say("device step Hq", Hq, "Hkv", Hkv, "D", D, "selection", n_sel, "steps", steps)
    B, T = 2, 600
    cap = 32 * ((n_sel + steps) // 32 + 2)
    rng, c, st = _start(dev, n_sel + 1, B, Hkv, T, D, n_sel, cap)
    c.to_device_counts()
    ws = torch.zeros(c.step_ws_bytes(Hq), dtype=torch.uint8, device=dev)
    for step in range(steps):
        kn, vn = _token(rng, B, Hkv, D), _token(rng, B, Hkv, D, 0.5)
        c.step_append(torch.from_numpy(kn).to(dev).to(torch.bfloat16), torch.from_numpy(vn).to(dev).to(torch.bfloat16))
        st = oracle.stream_append_ref(st, kn, vn)
        q = _token(rng, B, Hq, D)
        out = c.step_decode(torch.from_numpy(q).to(dev).to(torch.bfloat16), ws=ws)
        torch.cuda.synchronize()
        assert_attn_close(to_np(out), oracle.stream_decode_ref(q, st), f"device step {step}")
        if step % 16 == 15 or step == steps - 1:
            c.from_device_counts()
            _check_state(c, st)


@pytest.mark.parametrize("Hq,Hkv,D,n_sel", [(8, 2, 128, 3001), (4, 4, 64, 2097), (2, 1, 128, 4010)])
def test_stream_split_heads_with_window(dev, Hq, Hkv, D, n_sel):
    """KV heads whose packed tokens span several workgroups of the one-launch plan, plus a
    window: the head's last workgroup computes the window's exact part and merges it with its
    ranges before the cross-workgroup merge.  Host-side counts, then 40 device-side steps
    (plans over the whole capacity, whose last ranges are empty) against the oracle."""
    say("stream split heads + window, Hq", Hq, "Hkv", Hkv, "D", D, "selection", n_sel)
    B, T, steps = 1, n_sel + 300, 40
    cap = 32 * ((n_sel + steps) // 32 + 2)
    rng, c, st = _start(dev, 3 * n_sel + D, B, Hkv, T, D, n_sel, cap)
    assert c.n_res == n_sel % 32 > 0
    # the plan has two to eight workgroup parts per head (a one-launch plan split over workgroups)
    parts = (mk.decode_ws_bytes(B, Hq, Hkv, c.n_packed, D) - 16384) // (B * Hq * (D + 2) * 4)
    assert 2 <= parts <= 8, parts
    q = _token(rng, B, Hq, D)
    assert_attn_close(to_np(c.decode(torch.from_numpy(q).to(dev).to(torch.bfloat16))),
                      oracle.stream_decode_ref(q, st), "host counts")
    c.to_device_counts()
    ws = torch.zeros(c.step_ws_bytes(Hq), dtype=torch.uint8, device=dev)
    for step in range(steps):
        kn, vn = _token(rng, B, Hkv, D), _token(rng, B, Hkv, D, 0.5)
        c.step_append(torch.from_numpy(kn).to(dev).to(torch.bfloat16), torch.from_numpy(vn).to(dev).to(torch.bfloat16))
        st = oracle.stream_append_ref(st, kn, vn)
        q = _token(rng, B, Hq, D)
        out = c.step_decode(torch.from_numpy(q).to(dev).to(torch.bfloat16), ws=ws)
        torch.cuda.synchronize()
        assert_attn_close(to_np(out), oracle.stream_decode_ref(q, st), f"device step {step}")
    assert ws[:16384].count_nonzero().item() == 0  # every call leaves the tickets zero
    c.from_device_counts()
    _check_state(c, st)


# (B, Hq, Hkv, D, selection): query heads per KV head 1, 2 and 4 at D = 64 and 128; windows of 1,
# 5, 9, 13 and 31 tokens; plans of one 4-wave or 8-wave workgroup per KV head and of 2, 3, 5 and 8
# workgroups per head (the device-side plans cover the capacity, one more group than is packed)
_PLAN_SWEEP = [(1, 4, 1, 64, 7917), (1, 2, 1, 64, 4543), (2, 4, 1, 128, 1505), (3, 2, 2, 64, 325),
               (2, 8, 2, 64, 2057), (1, 4, 2, 128, 1055)]


@pytest.mark.parametrize("B,Hq,Hkv,D,n_sel", _PLAN_SWEEP)
def test_stream_window_plan_sweep(dev, B, Hq, Hkv, D, n_sel):
    """The window part in every kind of one-launch plan: one decode with host-side counts and one
    with the counts on the device, each against the oracle; the ticket area is zero afterwards."""
    say("stream window plan sweep B", B, "Hq", Hq, "Hkv", Hkv, "D", D, "selection", n_sel)
    cap = 32 * (n_sel // 32 + 2)
    rng, c, st = _start(dev, 7 * n_sel + B, B, Hkv, n_sel + 100, D, n_sel, cap)
    assert c.n_res == n_sel % 32
    q = _token(rng, B, Hq, D)
    qd = torch.from_numpy(q).to(dev).to(torch.bfloat16)
    ref = oracle.stream_decode_ref(q, st)
    ws = torch.zeros(c.ws_bytes(Hq), dtype=torch.uint8, device=dev)
    assert_attn_close(to_np(c.decode(qd, ws=ws)), ref, "host counts")
    c.to_device_counts()
    ws_d = torch.zeros(c.step_ws_bytes(Hq), dtype=torch.uint8, device=dev)
    assert_attn_close(to_np(c.step_decode(qd, ws=ws_d)), ref, "device counts")
    torch.cuda.synchronize()
    assert ws[:16384].count_nonzero().item() == 0 and ws_d[:16384].count_nonzero().item() == 0


def test_device_step_graph_replays(dev):
    """One captured generation step over two layers (append + decode each), replayed 40 times with
    new inputs copied in and eager work between replays; every replay against the oracle."""
    say("device step in a HIP graph")
    B, Hq, Hkv, T, D, n_sel = 2, 8, 2, 500, 128, 90
    cap = 256
    layers = []
    for l in range(2):
        rng, c, st = _start(dev, 50 + l, B, Hkv, T, D, n_sel, cap)
        c.to_device_counts()
        layers.append([rng, c, st, torch.zeros(c.step_ws_bytes(Hq), dtype=torch.uint8, device=dev)])
    # one eager step on a scratch cache of the same shapes (host-side launch set-up happens outside the capture)
    _, scratch, _ = _start(dev, 99, B, Hkv, T, D, n_sel, cap)
    scratch.to_device_counts()
    scratch.step_append(torch.zeros((B, Hkv, D), dtype=torch.bfloat16, device=dev),
                        torch.zeros((B, Hkv, D), dtype=torch.bfloat16, device=dev))
    scratch.step_decode(torch.zeros((B, Hq, D), dtype=torch.bfloat16, device=dev))
    k_in = torch.empty((B, Hkv, D), dtype=torch.bfloat16, device=dev)
    v_in = torch.empty_like(k_in)
    q_in = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    outs = [torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev) for _ in layers]
    torch.cuda.synchronize()
    # capture on a side stream; the capture itself runs nothing
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for (rng, c, st, ws), out in zip(layers, outs):
                c.step_append(k_in, v_in)
                c.step_decode(q_in, out=out, ws=ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    for rep in range(40):
        kn, vn, q = _token(rng, B, Hkv, D), _token(rng, B, Hkv, D, 0.5), _token(rng, B, Hq, D)
        k_in.copy_(torch.from_numpy(kn).to(torch.bfloat16))
        v_in.copy_(torch.from_numpy(vn).to(torch.bfloat16))
        q_in.copy_(torch.from_numpy(q).to(torch.bfloat16))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, layer in enumerate(layers):
            layer[2] = oracle.stream_append_ref(layer[2], kn, vn)
            assert_attn_close(to_np(outs[i]), oracle.stream_decode_ref(q, layer[2]), f"replay {rep} layer {i}")
        _ = (q_in.float() * 2).sum().item()  # eager work between replays
    for rng_, c, st, ws in layers:
        c.from_device_counts()
        _check_state(c, st)
        assert c.n_packed == 32 * ((n_sel + 40) // 32) and c.n_res == (n_sel + 40) % 32


def test_device_step_overflow_sets_flag(dev):
    """A full window that does not fit the capacity sets the flag; nothing is written out of bounds."""
    say("device step overflow")
    B, Hq, Hkv, T, D = 1, 2, 2, 200, 128
    rng, c, st = _start(dev, 7, B, Hkv, T, D, 63, 64)   # 32 packed + 31 in the window
    c.to_device_counts()
    kn, vn = _token(rng, B, Hkv, D), _token(rng, B, Hkv, D)   # fills the window: packed at 32 (cap 64 reached)
    c.step_append(torch.from_numpy(kn).to(dev).to(torch.bfloat16), torch.from_numpy(vn).to(dev).to(torch.bfloat16))
    st = oracle.stream_append_ref(st, kn, vn)
    c.from_device_counts()
    _check_state(c, st)
    assert c.n_packed == 64 and c.n_res == 0
    packed0 = [t.clone() for t in (c.k_codes, c.k_sz, c.v_codes, c.v_sz)]
    for _ in range(32):  # 31 fill the window again, the 32nd cannot be packed
        kn, vn = _token(rng, B, Hkv, D), _token(rng, B, Hkv, D)
        c.step_append(torch.from_numpy(kn).to(dev).to(torch.bfloat16), torch.from_numpy(vn).to(dev).to(torch.bfloat16))
    torch.cuda.synchronize()
    counts = c.counts.cpu().tolist()
    assert counts[:3] == [64, 31, 1]
    with pytest.raises(ValueError):
        c.from_device_counts()
    # the packed region is untouched after the overflow
    for a, b in zip((c.k_codes, c.k_sz, c.v_codes, c.v_sz), packed0):
        assert torch.equal(a, b)
