"""Pins of the CPU oracle against things other than itself.

Closed forms, hand-derived cases (tests/golden/quant_cases.json), IEEE rounding
from first principles (exact rationals), invariants and brute force on tiny
inputs.  CPU only.
"""

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# IEEE round-to-nearest-even from first principles (exact rationals)
# ---------------------------------------------------------------------------

def round_ieee(x, p, emin):
    """Nearest binary float with p significant bits (min normal exponent emin), ties to even."""
    x = Fraction(x)
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - p + 1)
    q = a / ulp
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * ulp


def f32(x):
    return round_ieee(x, 24, -126)


def f16(x):
    return round_ieee(x, 11, -14)


def rint_half_even(x):
    x = Fraction(x)
    n = math.floor(x)
    rem = x - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n


def quant_group_exact(xs):
    """The quantisation rule evaluated with exact rationals and explicit roundings."""
    xs = [Fraction(float(x)) for x in xs]
    mn, mx = min(xs), max(xs)
    s = f16(f32(f32(mx - mn) / 3))
    z = f16(mn)
    if s == 0:
        return [0] * len(xs), s, z
    codes = [min(3, max(0, rint_half_even(f32(f32(x - z) / s)))) for x in xs]
    return codes, s, z


def test_round_ieee_self_check():
    # sanity of the reference rounding itself on textbook values
    assert f16(1 + Fraction(1, 2 ** 11)) == 1
    assert f16(1 + Fraction(3, 2 ** 11)) == 1 + Fraction(1, 2 ** 9)
    assert f16(Fraction(65504)) == 65504
    assert f16(Fraction(1, 2 ** 25)) == 0          # half of the smallest subnormal ties to 0
    assert f16(Fraction(3, 2 ** 26)) == Fraction(1, 2 ** 24)
    assert f32(Fraction(1, 3)) == Fraction(11184811, 2 ** 25)


# ---------------------------------------------------------------------------
# Quantiser: hand-derived cases, first-principles rounding, error bound
# ---------------------------------------------------------------------------

def _cases():
    with open(os.path.join(GOLDEN, "quant_cases.json")) as fh:
        return json.load(fh)


@pytest.mark.parametrize("case", _cases()["cases"], ids=lambda c: c["name"])
def test_quant_hand_derived(case):
    x = np.array([float.fromhex(h) for h in case["x"]], dtype=np.float32)
    codes, s, z, _ = oracle.quant_group_ref(x)
    # compared as fp16 bit patterns, so the sign of a zero counts
    assert np.float16(s).view(np.uint16) == np.float16(float.fromhex(case["scale"])).view(np.uint16)
    assert np.float16(z).view(np.uint16) == np.float16(float.fromhex(case["zero"])).view(np.uint16)
    assert codes.tolist() == case["codes"]
    # the same case evaluated with exact rationals agrees
    ce, se, ze = quant_group_exact(x)
    assert ce == case["codes"] and se == Fraction(float(s)) and ze == Fraction(float(z))


@pytest.mark.parametrize("case", _cases()["pack"])
def test_pack_hand_derived(case):
    c = np.array(case["codes"], dtype=np.uint8)
    assert oracle.pack_codes_ref(c).tolist() == [case["byte"]]
    assert oracle.unpack_codes_ref(np.array([case["byte"]], np.uint8)).tolist() == case["codes"]


def _random_groups(rng, n, size):
    kinds = []
    for i in range(n):
        kind = i % 5
        if kind == 0:
            x = rng.standard_normal(size)
        elif kind == 1:
            x = rng.standard_normal(size) * 10.0 + 3.0
        elif kind == 2:
            x = rng.uniform(-1e-3, 1e-3, size)
        elif kind == 3:
            x = rng.standard_normal(size) * 1e-6     # subnormal fp16 scales
        else:
            # half-integer multiples of an fp16-exact step: exercises exact ties
            step = 2.0 ** rng.integers(-6, 3)
            x = rng.integers(0, 7, size) * 0.5 * step + rng.integers(-8, 8) * step
        kinds.append(x.astype(np.float32))
    return kinds


def test_quant_matches_first_principles_rounding():
    rng = np.random.default_rng(123)
    for x in _random_groups(rng, 250, 32):
        codes, s, z, _ = oracle.quant_group_ref(x)
        ce, se, ze = quant_group_exact(x)
        assert codes.tolist() == ce
        assert Fraction(float(s)) == se
        assert Fraction(float(z)) == ze


def test_scale_division_near_fp16_midpoints():
    """s = fp16(fl32(range / 3)) where range / 3 sits next to an fp16 rounding midpoint.

    A divide that is not correctly rounded (e.g. a multiply by fl32(1/3)) picks
    the other fp16 neighbour on some of these.
    """
    rng = np.random.default_rng(99)
    mism = 0
    for _ in range(400):
        s16 = np.float16(abs(rng.standard_normal()) * 2.0 ** int(rng.integers(-10, 6)))
        if not np.isfinite(s16) or float(s16) == 0:
            continue
        nxt = np.nextafter(s16, np.float16(np.inf))
        mid = (Fraction(float(s16)) + Fraction(float(nxt))) / 2
        base = np.float32(float(3 * mid))
        for d in range(-3, 4):
            r32 = base
            for _ in range(abs(d)):
                r32 = np.nextafter(r32, np.float32(np.inf if d > 0 else -np.inf))
            x = np.array([0.0, r32], dtype=np.float32)
            _, s, _, _ = oracle.quant_group_ref(x)
            exact = f16(f32(Fraction(float(r32)) / 3))
            assert Fraction(float(s)) == exact
            mism += f16(f32(Fraction(float(r32)) * f32(Fraction(1, 3)))) != exact
    assert mism > 0  # the set does separate the two divides


def test_quant_error_bound():
    """|x - x_hat| <= s/2 + cover slack (+ fp32 ratio rounding), slack from fp16 rounding of z, s."""
    rng = np.random.default_rng(7)
    for x in _random_groups(rng, 400, 32):
        codes, s, z, _ = oracle.quant_group_ref(x)
        s64, z64 = float(s), float(z)
        xh = codes.astype(np.float64) * s64 + z64
        mn, mx = float(x.min()), float(x.max())
        slack = max(0.0, z64 - mn) + max(0.0, mx - (z64 + 3 * s64))
        bound = s64 / 2 + slack + 4e-7 * s64 + 1e-45
        assert np.all(np.abs(x.astype(np.float64) - xh) <= bound)
        if s64 == 0:
            assert np.all(xh == z64)


def test_quant_exact_groups_reconstruct():
    rng = np.random.default_rng(11)
    for _ in range(50):
        a = float(np.float16(rng.standard_normal()))
        sigma = 2.0 ** int(rng.integers(-8, 4))
        # constant group (fp16-exact) reconstructs exactly
        codes, s, z, _ = oracle.quant_group_ref(np.full(32, a, np.float32))
        assert float(s) == 0 and float(z) == a and not codes.any()
        # two-level group {a, a + 3 sigma}: codes {0, 3}, exact
        lv = rng.integers(0, 2, 32)
        lv[0], lv[1] = 0, 1
        x = (a + 3 * sigma * lv).astype(np.float32)
        if float(np.float16(a + 3 * sigma)) != a + 3 * sigma:
            continue
        codes, s, z, _ = oracle.quant_group_ref(x)
        assert sorted(set(codes.tolist())) == [0, 3]
        xh = codes * float(s) + float(z)
        assert np.array_equal(xh, x.astype(np.float64))


def _total_order_key(x):
    """IEEE 754 totalOrder as an integer key of fp32 values (-0 below +0)."""
    b = np.asarray(x, np.float32).view(np.int32).astype(np.int64)
    return np.where(b < 0, -(b & 0x7FFFFFFF) - 1, b)


def test_group_min_max_follow_total_order():
    """Every group of 1..4 elements from {-0, +0, 0.5, -0.5, 2}: the oracle's
    minimum / maximum are the totalOrder extremes (so -0 < +0), the stored
    zero point z = fp16(min) carries that sign, and no permutation of a group
    changes its fp16 words or codes."""
    vals = np.array([-0.0, 0.0, 0.5, -0.5, 2.0], np.float32)
    seen = 0
    for size in range(1, 5):
        for combo in itertools.product(range(len(vals)), repeat=size):
            x = vals[list(combo)]
            key = _total_order_key(x)
            want_mn, want_mx = x[np.argmin(key)], x[np.argmax(key)]
            mn, mx = oracle.group_min_max(x[None])
            assert mn.view(np.uint32)[0, 0] == np.float32(want_mn).view(np.uint32)
            assert mx.view(np.uint32)[0, 0] == np.float32(want_mx).view(np.uint32)
            codes, s, z, _ = oracle.quant_group_ref(x)
            assert np.float16(z).view(np.uint16) == np.float16(want_mn).view(np.uint16)
            for perm in itertools.permutations(range(size)):
                c2, s2, z2, _ = oracle.quant_group_ref(x[list(perm)])
                assert np.float16(s2).view(np.uint16) == np.float16(s).view(np.uint16)
                assert np.float16(z2).view(np.uint16) == np.float16(z).view(np.uint16)
                assert c2.tolist() == codes[list(perm)].tolist()
            seen += 1
    assert seen == 5 + 25 + 125 + 625


def test_signed_zero_groups_in_the_packed_cache():
    """A key channel of alternating +0 / -0 and a value group starting with +0
    then -0 store z = -0; all-+0 groups store +0 (fp16 bits)."""
    k = np.zeros((1, 1, 32, 32), np.float32)
    v = np.zeros((1, 1, 32, 32), np.float32)
    k[0, 0, 1::2, 0] = -0.0       # channel 0: +0, -0, +0, ...
    k[0, 0, 0::2, 1] = -0.0       # channel 1: -0, +0, ...
    v[0, 0, 0, 1] = -0.0          # token 0: +0, -0, +0, ...
    v[0, 0, 1, 0] = -0.0          # token 1: -0, +0, ...
    p = oracle.quant_pack_ref(k, v)
    kz = p["k_zero"].view(np.uint16)[0, 0, 0]
    vz = p["v_zero"].view(np.uint16)[0, 0, :, 0]
    assert kz[0] == 0x8000 and kz[1] == 0x8000 and not kz[2:].any()
    assert vz[0] == 0x8000 and vz[1] == 0x8000 and not vz[2:].any()
    assert not p["k_scale"].view(np.uint16).any() and not p["v_scale"].view(np.uint16).any()


def test_code_near_ties_hand_cases():
    """Near-ties are |u - (m + 1/2)| < 1e-6 for m = 0, 1, 2 on the fp32 ratio u.
    fp32 spacing is 2^-24 below 0.5 ... 2^-22 near 2.5, so the cases step by ulps."""
    f = np.float32
    cases = [
        (f(0.5), True), (f(1.5), True), (f(2.5), True),
        (f(0.5) + f(2 ** -20), True),            # 9.5e-7 above 0.5
        (f(0.5) + f(2 ** -19), False),           # 1.9e-6 above
        (f(1.5) - f(2 ** -20), True),            # 9.5e-7 below 1.5
        (f(1.5) - f(2 ** -19), False),
        (f(2.5) + f(4 * 2 ** -22), True),        # 4 ulps (9.5e-7) above 2.5
        (f(2.5) + f(5 * 2 ** -22), False),       # 5 ulps (1.19e-6)
        (f(3.5), False), (f(-0.5), False),       # past the clamp: not a boundary
        (f(1.0), False), (f(0.0), False), (f(3.0), False),
        (f(np.nan), False),                      # a group with s == 0
    ]
    u = np.array([c[0] for c in cases], np.float32)
    assert oracle.code_near_ties(u).tolist() == [c[1] for c in cases]
    # a group whose second element lands exactly on u = 1.5: x = 0, 1.5, 3 (s = 1, z = 0)
    p = oracle.quant_pack_ref(np.array([0.0, 1.5, 3.0] + [0.0] * 29, np.float32).reshape(1, 1, 32, 1)
                              .repeat(32, axis=3), np.zeros((1, 1, 32, 32), np.float32), return_u=True)
    near = oracle.code_near_ties(p["k_u"])
    assert near[0, 0, 1].all() and near.sum() == 32
    assert not oracle.code_near_ties(p["v_u"]).any()
    # parity counting: a flipped code on a near-tie is counted apart from other mismatches
    ref = np.array([0, 2, 3, 1])
    uu = np.array([0.1, 1.5, 2.9, 0.9], np.float32)
    assert oracle.code_parity(np.array([0, 1, 3, 1]), ref, uu) == (0, 1, 1)
    assert oracle.code_parity(np.array([1, 2, 3, 1]), ref, uu) == (1, 1, 0)
    assert oracle.code_parity(ref, ref, uu) == (0, 1, 0)


# ---------------------------------------------------------------------------
# Packed layout and bit accounting
# ---------------------------------------------------------------------------

def test_pack_roundtrip():
    rng = np.random.default_rng(3)
    c = rng.integers(0, 4, size=(5, 7, 128)).astype(np.uint8)
    p = oracle.pack_codes_ref(c)
    assert p.shape == (5, 7, 32)
    assert np.array_equal(oracle.unpack_codes_ref(p), c)


def test_value_code_layout_by_hand():
    # one code 3 at kept token 37 (block 1, token 5 of the block), channel 5:
    # byte (37 - 32) // 4 = 1 of (block 1, channel 5), bits 2 * ((37 - 32) % 4) = 2..3
    c = np.zeros((1, 1, 40, 8), np.uint8)
    c[0, 0, 37, 5] = 3
    p = oracle.pack_value_codes_ref(c)
    assert p.shape == (1, 1, 2, 8, 8)
    want = np.zeros_like(p)
    want[0, 0, 1, 5, 1] = 3 << 2
    assert np.array_equal(p, want)
    # every token of a 32-token block in its own bit pair, tail tokens zero
    rng = np.random.default_rng(4)
    c = rng.integers(0, 4, size=(2, 3, 45, 64)).astype(np.uint8)
    p = oracle.pack_value_codes_ref(c)
    for (b, h, t, ch) in [(0, 0, 0, 0), (1, 2, 44, 63), (0, 1, 31, 7), (1, 0, 32, 40)]:
        byte = int(p[b, h, t // 32, ch, (t % 32) // 4])
        assert (byte >> (2 * (t % 4))) & 3 == c[b, h, t, ch]
    assert not p[:, :, 1, :, 4:].any()          # tokens 45..63 of block 1 are padding
    assert not (p[:, :, 1, :, 3] >> 2).any()    # tokens 45..47 in byte 3
    assert np.array_equal(oracle.unpack_value_codes_ref(p, 45), c)


def test_sz_words_layout():
    w = oracle.sz_words_ref(np.float16(1.0), np.float16(-2.0))
    assert int(w) == (0xC000 << 16) | 0x3C00


def test_bit_accounting_closed_form():
    # tiny workload: 64 kept of 256 tokens, D = 64
    assert oracle.packed_bytes_ref(1, 1, 64, 64) == 3072
    assert oracle.compression_ratio_ref(256, 64, 64) == 0.953125
    assert oracle.compression_ratio_ref(256, 256, 64) == 0.8125     # 2-bit alone: 81.25 %
    # LLaMA2-7B-shaped: 614 kept of 4096, D = 128, 20 blocks:
    # 614*32 + 20*512 + 20*1024 + 614*16 = 60,192 B per head
    assert oracle.packed_bytes_ref(1, 1, 614, 128) == 60192
    assert abs(oracle.compression_ratio_ref(4096, 614, 128) - (1 - 60192 / 2097152)) < 1e-15
    # prefill 16k: 2457 kept, 77 blocks: 2457*32 + 77*512 + 77*1024 + 2457*16 = 236,208 B
    assert oracle.packed_bytes_ref(1, 1, 2457, 128) == 236208
    # the arrays the oracle produces have exactly that many bytes
    d = synth.tiny_inputs()
    idx = np.broadcast_to(np.arange(64, dtype=np.int32) * 4, (1, 2, 64))
    p = oracle.quant_pack_ref(d["k"], d["v"], idx)
    nbytes = p["k_codes"].nbytes + p["v_codes"].nbytes + 2 * (
        p["k_scale"].nbytes + p["v_scale"].nbytes)  # scale + zero each fp16
    assert nbytes == oracle.packed_bytes_ref(1, 2, 64, 64)


def test_partial_last_key_group_uses_valid_tokens_only():
    rng = np.random.default_rng(5)
    k = rng.standard_normal((1, 1, 40, 32)).astype(np.float32)
    v = rng.standard_normal((1, 1, 40, 32)).astype(np.float32)
    p = oracle.quant_pack_ref(k, v)  # n = 40: groups of 32 and 8 tokens
    assert p["k_scale"].shape == (1, 1, 2, 32)
    for c in range(32):
        _, s, z, _ = oracle.quant_group_ref(k[0, 0, 32:40, c])
        assert p["k_scale"][0, 0, 1, c] == s and p["k_zero"][0, 0, 1, c] == z
        _, s, z, _ = oracle.quant_group_ref(k[0, 0, 0:32, c])
        assert p["k_scale"][0, 0, 0, c] == s


def test_quant_pack_gathers_in_index_order():
    rng = np.random.default_rng(9)
    k = rng.standard_normal((1, 2, 64, 32)).astype(np.float32)
    v = rng.standard_normal((1, 2, 64, 32)).astype(np.float32)
    idx = np.stack([np.sort(rng.choice(64, 33, replace=False)) for _ in range(2)])[None].astype(np.int32)
    p = oracle.quant_pack_ref(k, v, idx)
    q = oracle.quant_pack_ref(np.take_along_axis(k, idx[..., None], 2),
                              np.take_along_axis(v, idx[..., None], 2))
    for key in ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero"):
        assert np.array_equal(p[key], q[key])


# ---------------------------------------------------------------------------
# Budgets
# ---------------------------------------------------------------------------

def test_budgets():
    assert oracle.keep_count(4096, 15) == 614
    assert oracle.keep_count(16384, 15) == 2457
    assert oracle.keep_count(44000, 15) == 6600
    assert oracle.split_heavy_recent(614) == (492, 122)
    assert oracle.split_heavy_recent(2457) == (1966, 491)
    assert oracle.split_heavy_recent(6600) == (5280, 1320)
    assert oracle.keep_count(256, 100) == 256
    ks = [oracle.pyramid_keep(8192, 40, l) for l in range(40)]
    assert ks[0] == 2457 and ks[-1] == 409
    # brute force with exact rationals: pct(l) = 30 - 25 l / 39
    for l, kl in enumerate(ks):
        pct = Fraction(30) - Fraction(25 * l, 39)
        assert kl == math.floor(pct * 8192 / 100)
    assert sum(ks) == 57324
    assert all(a >= b for a, b in zip(ks, ks[1:]))


# ---------------------------------------------------------------------------
# Attention: brute force on tiny shapes, special cases
# ---------------------------------------------------------------------------

def _attn_loops(q, k, v, scale):
    """Pure-Python causal attention for one head (lists of floats)."""
    T, D = len(q), len(q[0])
    out, lse = [], []
    for i in range(T):
        logits = [sum(q[i][d] * k[j][d] for d in range(D)) * scale for j in range(i + 1)]
        m = max(logits)
        den = sum(math.exp(x - m) for x in logits)
        lse.append(m + math.log(den))
        out.append([sum(math.exp(logits[j] - m) / den * v[j][d] for j in range(i + 1))
                    for d in range(D)])
    return out, lse


def test_prefill_bruteforce_gqa():
    rng = np.random.default_rng(21)
    B, Hq, Hkv, T, D = 1, 4, 2, 9, 8
    q = rng.standard_normal((B, Hq, T, D))
    k = rng.standard_normal((B, Hkv, T, D)) * 2
    v = rng.standard_normal((B, Hkv, T, D))
    o, lse = oracle.prefill_ref(q, k, v)
    for h in range(Hq):
        g = h // 2
        ol, ll = _attn_loops(q[0, h].tolist(), k[0, g].tolist(), v[0, g].tolist(), 1 / math.sqrt(D))
        assert np.allclose(o[0, h], ol, rtol=1e-12, atol=1e-12)
        assert np.allclose(lse[0, h], ll, rtol=1e-12, atol=1e-12)
    # rows= gives the same rows
    o2, l2 = oracle.prefill_ref(q, k, v, rows=np.array([0, 5, 8]))
    assert np.allclose(o2, o[:, :, [0, 5, 8]]) and np.allclose(l2, lse[:, :, [0, 5, 8]])


def test_prefill_first_row_is_v0():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 2, 5, 16))
    k = rng.standard_normal((1, 2, 5, 16))
    v = rng.standard_normal((1, 2, 5, 16))
    o, lse = oracle.prefill_ref(q, k, v)
    assert np.allclose(o[:, :, 0], v[:, :, 0], atol=1e-15)
    assert np.allclose(lse[:, :, 0], (q[:, :, 0] * k[:, :, 0]).sum(-1) / 4)


def test_window_scores_bruteforce_and_sum():
    rng = np.random.default_rng(4)
    B, Hq, Hkv, T, D, W = 1, 4, 2, 11, 8, 4
    q = rng.standard_normal((B, Hq, T, D))
    k = rng.standard_normal((B, Hkv, T, D))
    sc = oracle.window_scores_ref(q, k, W)
    ref = np.zeros((Hkv, T))
    for h in range(Hq):
        g = h // 2
        for i in range(T - W, T):
            logits = [float(q[0, h, i] @ k[0, g, j]) / math.sqrt(D) for j in range(i + 1)]
            m = max(logits)
            den = sum(math.exp(x - m) for x in logits)
            for j in range(i + 1):
                ref[g, j] += math.exp(logits[j] - m) / den
    assert np.allclose(sc[0], ref, rtol=1e-12, atol=1e-14)
    assert np.allclose(sc.sum(-1), W * 2, rtol=1e-12)


def test_window_scores_sum_tiny_workload():
    d = synth.tiny_inputs()
    sc = oracle.window_scores_ref(d["q"], d["k"], 16)
    assert np.allclose(sc.sum(-1), 16.0, rtol=1e-12)
    assert (sc >= 0).all()



@pytest.mark.parametrize("T,W", [(40, 40), (40, 9), (1, 1), (17, 1)])
def test_window_scores_uniform_logits_closed_form(T, W):
    """q = 0 makes every causal row uniform: row i gives each key j <= i exactly 1/(i+1).

    Key j then collects, per query head, sum_{i = max(j, T-W)}^{T-1} 1/(i+1); with
    W = T (every prompt row, the cumulative mass) that is H_T - H_j in harmonic
    numbers.  Two query heads share each KV head here.
    """
    rng = np.random.default_rng(T * 100 + W)
    q = np.zeros((1, 4, T, 8))
    k = rng.standard_normal((1, 2, T, 8)) * 3
    sc = oracle.window_scores_ref(q, k, W)
    harmonic = [Fraction(0)]
    for n in range(1, T + 1):
        harmonic.append(harmonic[-1] + Fraction(1, n))
    for j in range(T):
        lo = max(j, T - W)
        expect = 2 * (harmonic[T] - harmonic[lo])
        assert sc[0, 0, j] == pytest.approx(float(expect), rel=1e-13, abs=1e-15)
        assert sc[0, 1, j] == pytest.approx(float(expect), rel=1e-13, abs=1e-15)


# ---------------------------------------------------------------------------
# Selection: brute force over subsets, special cases
# ---------------------------------------------------------------------------

def _valid_topk(scores, subset, cand):
    """Exchange property of top-k with lower-position tie-break."""
    for j in subset:
        for jp in cand:
            if jp in subset:
                continue
            if not (scores[j] > scores[jp] or (scores[j] == scores[jp] and j < jp)):
                return False
    return True


@pytest.mark.parametrize("seed", range(6))
def test_select_bruteforce(seed):
    rng = np.random.default_rng(seed)
    T, n_heavy, n_recent = 10, 3, 2
    # few distinct values so that ties occur
    s = rng.integers(0, 4, T).astype(np.float32) / 4
    idx = oracle.select_ref(s[None], n_heavy, n_recent)[0].tolist()
    cand = list(range(T - n_recent))
    valid = [set(c) for c in itertools.combinations(cand, n_heavy) if _valid_topk(s, set(c), cand)]
    assert len(valid) == 1
    expect = sorted(valid[0] | set(range(T - n_recent, T)))
    assert idx == expect


def test_select_special_cases():
    T = 50
    eq = np.ones((2, 3, T), np.float32)
    idx = oracle.select_ref(eq, 10, 5)
    assert np.array_equal(idx[1, 2], np.r_[np.arange(10), np.arange(45, 50)])
    full = oracle.select_ref(np.random.default_rng(0).random((1, T)), T - 7, 7)
    assert np.array_equal(full[0], np.arange(T))
    only_recent = oracle.select_ref(np.zeros((1, T)), 0, 4)
    assert only_recent[0].tolist() == [46, 47, 48, 49]
    # a huge score in the recent window does not take a heavy slot
    s = np.zeros(T)
    s[-1] = 100
    s[3] = 1
    assert oracle.select_ref(s[None], 1, 2)[0].tolist() == [3, 48, 49]


def test_select_decides_in_given_precision():
    # two scores equal in fp32 but not in fp64: fp32 input keeps the lower position
    a = 0.1
    b = np.nextafter(0.1, 1.0)
    s64 = np.array([a, b, 0.0, 0.0])
    assert oracle.select_ref(s64[None], 1, 1)[0].tolist() == [1, 3]
    s32 = s64.astype(np.float32)
    assert s32[0] == s32[1]
    assert oracle.select_ref(s32[None], 1, 1)[0].tolist() == [0, 3]


def test_index_near_ties():
    s = np.array([0.5, 0.3, 0.3 + 5e-7, 0.1, 0.0])
    n = oracle.index_near_ties(s[None], 2, 1)[0].tolist()
    assert n == [1, 2]


# ---------------------------------------------------------------------------
# Decode over the packed cache
# ---------------------------------------------------------------------------

def _packed_from(k, v, idx=None):
    return oracle.quant_pack_ref(k, v, idx)


def test_decode_single_token_is_v_hat():
    rng = np.random.default_rng(8)
    k = rng.standard_normal((1, 2, 1, 64)).astype(np.float32)
    v = rng.standard_normal((1, 2, 1, 64)).astype(np.float32)
    p = _packed_from(k, v)
    _, vh = oracle.dequant_ref(p)
    out = oracle.decode_ref(rng.standard_normal((1, 4, 64)), p)
    for h in range(4):
        assert np.allclose(out[0, h], vh[0, h // 2, 0], atol=1e-15)


def test_decode_constant_keys_is_mean():
    rng = np.random.default_rng(10)
    k = np.full((1, 1, 37, 32), 0.75, np.float32)
    v = rng.standard_normal((1, 1, 37, 32)).astype(np.float32)
    p = _packed_from(k, v)
    _, vh = oracle.dequant_ref(p)
    out = oracle.decode_ref(rng.standard_normal((1, 1, 32)), p)
    assert np.allclose(out[0, 0], vh[0, 0].mean(0), atol=1e-14)


def test_decode_bruteforce_loops():
    rng = np.random.default_rng(12)
    n, D = 45, 64
    k = rng.standard_normal((1, 1, n, D)).astype(np.float32) * 3
    v = rng.standard_normal((1, 1, n, D)).astype(np.float32)
    p = _packed_from(k, v)
    q = rng.standard_normal((1, 1, D))
    out = oracle.decode_ref(q, p)
    # rebuild x_hat by hand from the packed bytes, scalar by scalar
    kb, vb = p["k_codes"][0, 0], p["v_codes"][0, 0]
    khat = [[((int(kb[t, c // 4]) >> (2 * (c % 4))) & 3) * float(p["k_scale"][0, 0, t // 32, c])
             + float(p["k_zero"][0, 0, t // 32, c]) for c in range(D)] for t in range(n)]
    vhat = [[((int(vb[t // 32, c, (t % 32) // 4]) >> (2 * (t % 4))) & 3) * float(p["v_scale"][0, 0, t, c // 32])
             + float(p["v_zero"][0, 0, t, c // 32]) for c in range(D)] for t in range(n)]
    logits = [sum(q[0, 0, c] * khat[t][c] for c in range(D)) / math.sqrt(D) for t in range(n)]
    m = max(logits)
    w = [math.exp(x - m) for x in logits]
    den = sum(w)
    ref = [sum(w[t] / den * vhat[t][c] for t in range(n)) for c in range(D)]
    assert np.allclose(out[0, 0], ref, rtol=1e-12, atol=1e-13)
