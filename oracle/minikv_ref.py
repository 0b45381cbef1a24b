"""CPU oracle: each step of the 2-bit layer-discriminative KV-cache path, spelled out.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Shares no code with the
HIP library; imports numpy only.

Notation: B batch, T context, Hq / Hkv query / key-value heads (r = Hq / Hkv query
heads share one KV head, head h uses KV head h // r), D head dim, W observation
window (the last W query rows), n_keep kept tokens = n_heavy + n_recent,
GROUP = 32.

Layouts (all row-major):
  q, o        [B, Hq, T, D]      k, v      [B, Hkv, T, D]
  lse         [B, Hq, T]         scores    [B, Hkv, T]
  idx         [B, Hkv, n_keep]   int32, ascending token positions
  k_codes     [B, Hkv, n_keep, D/4] uint8         k_scale/k_zero [B, Hkv, ceil(n_keep/32), D] fp16
  v_codes     [B, Hkv, ceil(n_keep/32), D, 8] uint8  v_scale/v_zero [B, Hkv, n_keep, D/32]  fp16
Keys are packed along channels: byte m of a token's row holds channels
4m..4m+3, channel 4m+j in bits 2j..2j+1.  Values are packed along tokens, in
blocks of 32 kept tokens: the 8 bytes of (block, channel) hold the channel's
32 codes, byte m holding tokens 4m..4m+3 of the block, token 4m+j in bits
2j..2j+1; tokens past n_keep in the last block have code 0.
"""

import math

import numpy as np

GROUP = 32  # quantisation group: 32 kept tokens (keys) or 32 channels (values)


# ---------------------------------------------------------------------------
# Budgets: adaptive KV keeps a fixed share of the tokens, and the "Pyramid"
# variant gives each layer its own share.
# ---------------------------------------------------------------------------

def keep_count(T, pct):
    """Tokens kept at a budget of ``pct`` percent of a T-token context.

    Glossary of the gptget.net summary (adaptive KV: keep KV states by
    importance).  Reading: n_keep = floor(pct * T / 100) in exact integer
    arithmetic, at least 1.
    """
    if T <= 0:
        raise ValueError("T must be positive")
    num = int(round(pct * 1000))  # pct given with at most 3 decimals
    n = (num * T) // 100000
    return max(1, min(T, n))


def pyramid_keep(T, n_layers, layer, first_pct=30, last_pct=5):
    """Kept tokens for ``layer`` of a layer-discriminative ("Pyramid") cache.

    notesum.ai LongBench table, "MiniKV Pyramid" rows; paper-listing abstract
    ("layer-discriminative").  The pages give no schedule.  Reading: the budget
    falls linearly from ``first_pct`` percent at layer 0 to ``last_pct`` percent at
    the last layer, n = floor(pct(layer) * T / 100), exact in integers:
    n = floor((first*(L-1) + (last-first)*layer) * T / (100*(L-1))).
    """
    if not 0 <= layer < n_layers:
        raise ValueError("layer out of range")
    if n_layers == 1:
        return max(1, (first_pct * T) // 100)
    L1 = n_layers - 1
    num = (first_pct * L1 + (last_pct - first_pct) * layer) * T
    return max(1, num // (100 * L1))


def split_heavy_recent(n_keep, recent_num=1, recent_den=5):
    """Split a budget into (n_heavy, n_recent).

    Reading (pages silent on the split): recent = floor(n_keep * 1/5) (a 20 %
    recent window), heavy = the rest.
    """
    n_recent = (n_keep * recent_num) // recent_den
    return n_keep - n_recent, n_recent


# ---------------------------------------------------------------------------
# Selective flash attention: pass 1 (attention + per-row log-sum-exp) and the
# second kernel's quantity (per-key probability sums over the window rows).
# gptget.net summary, 方法详解: selective flash attention realised with a second
# kernel, keeping memory low (no T x T probability matrix is stored).
# ---------------------------------------------------------------------------

def _softmax_rows(q_rows, k_keys, row_pos, scale):
    """fp64 causal softmax rows: returns (P [n_rows, T], lse [n_rows])."""
    s = (q_rows @ k_keys.T) * scale
    T = k_keys.shape[0]
    mask = np.arange(T)[None, :] > row_pos[:, None]
    s = np.where(mask, -np.inf, s)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    den = e.sum(axis=1, keepdims=True)
    lse = (m + np.log(den))[:, 0]
    return e / den, lse


def prefill_ref(q, k, v, sm_scale=None, rows=None):
    """Causal attention O = softmax(Q K^T * scale + mask) V and per-row LSE (fp64).

    Paper-listing abstract (attention kept FlashAttention-compatible); gptget.net
    summary, 方法详解 (selective flash attention, first pass).  Readings: scale
    1/sqrt(D); keys already position-encoded (no rotary step in the path); query
    head h attends KV head h // (Hq/Hkv).

    ``rows`` (optional, 1-D int array) restricts the computation to those query
    positions; O and LSE are then [B, Hq, len(rows), D] and [B, Hq, len(rows)].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    r = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.empty((B, Hq, len(rows), D))
    lse = np.empty((B, Hq, len(rows)))
    for b in range(B):
        for h in range(Hq):
            g = h // r
            p, l_ = _softmax_rows(q[b, h, rows], k[b, g], rows, scale)
            o[b, h] = p @ v[b, g]
            lse[b, h] = l_
    return o, lse


def window_scores_ref(q, k, window, sm_scale=None):
    """Per-key importance: probability mass each key receives from the window rows.

    gptget.net summary, 方法详解 (the second kernel of selective flash
    attention) and 术语表 "adaptive KV" (importance-based retention).  Readings:
    the importance of key j is the sum over the last ``window`` query rows i
    (i >= j, causal) of softmax probability P[h, i, j], summed again over the r
    query heads that share KV head g:

        score[b, g, j] = sum_{h: h // r = g} sum_{i = T-W}^{T-1} P[b, h, i, j]

    fp64.  Each softmax row sums to one, so sum_j score[b, g, j] = W * r.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    r = Hq // Hkv
    W = int(window)
    if not 1 <= W <= T:
        raise ValueError("window must be in [1, T]")
    scale = 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)
    rows = np.arange(T - W, T)
    scores = np.zeros((B, Hkv, T))
    for b in range(B):
        for h in range(Hq):
            p, _ = _softmax_rows(q[b, h, rows], k[b, h // r], rows, scale)
            scores[b, h // r] += p.sum(axis=0)
    return scores


# ---------------------------------------------------------------------------
# Heavy-hitter + recent-window selection (adaptive KV policy).
# ---------------------------------------------------------------------------

def select_ref(scores, n_heavy, n_recent):
    """Kept token positions: the last n_recent tokens plus the n_heavy highest scores.

    gptget.net summary, 方法论 / 术语表 (adaptive KV: keep the important states).
    Readings: the recent window is positions T-n_recent .. T-1; heavy hitters are
    the n_heavy largest scores among positions < T - n_recent; equal scores go to
    the lower position; the result is sorted ascending.  Comparisons are made in
    the dtype of ``scores`` (pass fp32 scores to decide exactly as an fp32 kernel
    does).  Returns int32 [..., n_heavy + n_recent].
    """
    s = np.asarray(scores)
    T = s.shape[-1]
    if n_heavy < 0 or n_recent < 0 or n_heavy + n_recent > T or n_heavy + n_recent < 1:
        raise ValueError("bad budget")
    flat = s.reshape(-1, T)
    out = np.empty((flat.shape[0], n_heavy + n_recent), dtype=np.int32)
    n_cand = T - n_recent
    for row in range(flat.shape[0]):
        cand = flat[row, :n_cand]
        # stable sort of the negated scores: larger score first, ties keep the
        # lower position first
        order = np.argsort(-cand, kind="stable")
        heavy = order[:n_heavy]
        recent = np.arange(n_cand, T)
        out[row] = np.sort(np.concatenate([heavy, recent])).astype(np.int32)
    return out.reshape(s.shape[:-1] + (n_heavy + n_recent,))


def index_near_ties(scores, n_heavy, n_recent, tol=1e-6):
    """Candidate positions whose score lies within ``tol`` of the selection threshold.

    The threshold tau is the n_heavy-th largest candidate score.  Two correct
    implementations whose scores differ by rounding may disagree only on these
    positions.  Returns a list (one entry per row) of int arrays.
    """
    s = np.asarray(scores, dtype=np.float64)
    T = s.shape[-1]
    flat = s.reshape(-1, T)
    res = []
    for row in range(flat.shape[0]):
        cand = flat[row, : T - n_recent]
        if n_heavy == 0:
            res.append(np.zeros(0, dtype=np.int64))
            continue
        tau = np.sort(cand)[::-1][n_heavy - 1]
        res.append(np.nonzero(np.abs(cand - tau) <= tol)[0])
    return res


# ---------------------------------------------------------------------------
# 2-bit asymmetric min/max quantisation and the packed layout.
# gptget.net summary, 方法论 / 方法详解: 2-bit quantisation, keys per channel,
# values per token, compact layout.
# ---------------------------------------------------------------------------

def group_min_max(x):
    """Minimum and maximum along the last axis, with -0 ordered below +0.

    Reading (the pages do not say which zero a group's minimum is): the IEEE
    754-2019 minimum / maximum operations, which rank -0 below +0, so the
    result does not depend on the order of the elements.  A group whose
    smallest value is zero has minimum -0 if it holds a -0, else +0; a group
    whose largest value is zero has maximum +0 if it holds a +0, else -0.
    Only the sign of the stored zero point z = fp16(min) can change; codes and
    the scale cannot (x - z and max - min are the same for either zero).
    """
    x = np.asarray(x, dtype=np.float32)
    mn = x.min(axis=-1, keepdims=True)
    mx = x.max(axis=-1, keepdims=True)
    zero = x == 0
    has_neg0 = (zero & np.signbit(x)).any(axis=-1, keepdims=True)
    has_pos0 = (zero & ~np.signbit(x)).any(axis=-1, keepdims=True)
    mn = np.where(mn == 0, np.where(has_neg0, np.float32(-0.0), np.float32(0.0)), mn).astype(np.float32)
    mx = np.where(mx == 0, np.where(has_pos0, np.float32(0.0), np.float32(-0.0)), mx).astype(np.float32)
    return mn, mx


def _quant_groups(x):
    """Quantise groups laid along the last axis of fp32 ``x`` (see quant_group_ref)."""
    x = np.asarray(x, dtype=np.float32)
    mn, mx = group_min_max(x)
    s32 = (mx - mn) / np.float32(3.0)          # fp32 subtract, fp32 divide
    s16 = s32.astype(np.float16)               # round-half-even to fp16
    z16 = mn.astype(np.float16)
    s = s16.astype(np.float32)
    z = z16.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        u = (x - z) / s                        # fp32 subtract, fp32 divide
    zero = s == 0
    codes = np.where(zero, 0.0, np.clip(np.rint(u), 0.0, 3.0)).astype(np.uint8)
    u = np.where(zero, np.float32(np.nan), u).astype(np.float32)
    return codes, s16[..., 0], z16[..., 0], u


def quant_group_ref(x):
    """Quantise one group (1-D fp32 values) to 2-bit codes with fp16 scale / zero.

    Readings (pages give only "2-bit, asymmetric, per-channel K / per-token V"):
      mn, mx = min, max of the group (exact; -0 below +0, see group_min_max)
      s = fp16( fl32( fl32(mx - mn) / 3 ) )      four levels 0..3
      z = fp16( mn )                             a float offset, not an integer zero point
      u = fl32( fl32(x - z) / s )                with the *stored* fp16 s, z
      code = 0 if s == 0 else clamp(round_half_even(u), 0, 3)
    fl32 is IEEE fp32 with round-half-even; fp16 is IEEE half, round-half-even,
    subnormals kept.  Returns (codes uint8, s fp16, z fp16, u fp32; u is NaN
    where s == 0).
    """
    codes, s16, z16, u = _quant_groups(np.asarray(x, dtype=np.float32)[None, :])
    return codes[0], s16[0], z16[0], u[0]


def pack_codes_ref(codes):
    """Pack 2-bit codes [..., D] into bytes [..., D/4]: channel 4m+j -> bits 2j..2j+1."""
    c = np.asarray(codes, dtype=np.uint8)
    D = c.shape[-1]
    if D % 4:
        raise ValueError("D must be a multiple of 4")
    c4 = c.reshape(c.shape[:-1] + (D // 4, 4)).astype(np.uint32)
    b = c4[..., 0] | (c4[..., 1] << 2) | (c4[..., 2] << 4) | (c4[..., 3] << 6)
    return b.astype(np.uint8)


def unpack_codes_ref(packed):
    """Inverse of pack_codes_ref: bytes [..., D/4] -> codes [..., D]."""
    p = np.asarray(packed, dtype=np.uint8)
    parts = [(p >> (2 * j)) & 3 for j in range(4)]
    return np.stack(parts, axis=-1).reshape(p.shape[:-1] + (p.shape[-1] * 4,)).astype(np.uint8)


def pack_value_codes_ref(codes):
    """Value codes [B, Hkv, n, D] -> token-packed blocks [B, Hkv, ceil(n/32), D, 8] (zero padded)."""
    c = np.asarray(codes, dtype=np.uint8)
    B, Hkv, n, D = c.shape
    G = -(-n // GROUP)
    pad = np.zeros((B, Hkv, G * GROUP, D), np.uint8)
    pad[:, :, :n, :] = c
    blocks = pad.reshape(B, Hkv, G, GROUP, D)
    return pack_codes_ref(np.swapaxes(blocks, 3, 4))  # pack the 32 tokens of each (block, channel)


def unpack_value_codes_ref(packed, n):
    """Inverse of pack_value_codes_ref for the first n tokens: -> codes [B, Hkv, n, D]."""
    p = np.asarray(packed, dtype=np.uint8)
    B, Hkv, G, D, _ = p.shape
    c = np.swapaxes(unpack_codes_ref(p), 3, 4)  # [B, Hkv, G, 32, D]
    return c.reshape(B, Hkv, G * GROUP, D)[:, :, :n, :]


def sz_words_ref(scale, zero):
    """Interleave fp16 scale / zero into 32-bit words: scale in bits 0..15, zero in 16..31."""
    s = np.asarray(scale, dtype=np.float16).view(np.uint16).astype(np.uint32)
    z = np.asarray(zero, dtype=np.float16).view(np.uint16).astype(np.uint32)
    return (s | (z << 16)).astype(np.uint32)


def quant_pack_ref(k, v, idx=None, return_u=False):
    """Gather the kept tokens and quantise / pack them (fp32 inputs, exact).

    Keys: groups of GROUP consecutive kept tokens (in ascending position order)
    per channel; the last group may be partial and uses its valid tokens only.
    Values: groups of GROUP consecutive channels per kept token.  ``idx`` None
    keeps every token (n_keep = T).

    Returns a dict with k_codes, k_scale, k_zero, v_codes, v_scale, v_zero (and
    the fp32 ratios k_u, v_u [B, Hkv, n, D], for near-tie accounting, when
    return_u is set).
    """
    k = np.asarray(k, dtype=np.float32)
    v = np.asarray(v, dtype=np.float32)
    B, Hkv, T, D = k.shape
    if D % GROUP:
        raise ValueError("D must be a multiple of 32")
    if idx is None:
        idx = np.broadcast_to(np.arange(T, dtype=np.int64), (B, Hkv, T))
    idx = np.asarray(idx, dtype=np.int64)
    if idx.min() < 0 or idx.max() >= T:
        raise ValueError("idx out of range")
    n = idx.shape[-1]
    G = -(-n // GROUP)
    xk = np.take_along_axis(k, idx[..., None], axis=2)  # [B, Hkv, n, D]
    xv = np.take_along_axis(v, idx[..., None], axis=2)

    k_codes = np.zeros((B, Hkv, n, D), np.uint8)
    k_scale = np.zeros((B, Hkv, G, D), np.float16)
    k_zero = np.zeros((B, Hkv, G, D), np.float16)
    k_u = np.zeros((B, Hkv, n, D), np.float32)
    for gi in range(G):  # one key group = up to 32 tokens x 1 channel
        t0, t1 = gi * GROUP, min(n, (gi + 1) * GROUP)
        grp = np.swapaxes(xk[:, :, t0:t1, :], 2, 3)  # [B, Hkv, D, tokens]
        c, s16, z16, u = _quant_groups(grp)
        k_codes[:, :, t0:t1, :] = np.swapaxes(c, 2, 3)
        k_u[:, :, t0:t1, :] = np.swapaxes(u, 2, 3)
        k_scale[:, :, gi, :] = s16
        k_zero[:, :, gi, :] = z16

    grp = xv.reshape(B, Hkv, n, D // GROUP, GROUP)  # one value group = 1 token x 32 channels
    c, s16, z16, u = _quant_groups(grp)
    out = {
        "k_codes": pack_codes_ref(k_codes),
        "k_scale": k_scale,
        "k_zero": k_zero,
        "v_codes": pack_value_codes_ref(c.reshape(B, Hkv, n, D)),
        "v_scale": s16,
        "v_zero": z16,
    }
    if return_u:
        out["k_u"] = k_u
        out["v_u"] = u.reshape(B, Hkv, n, D)
    return out


def code_near_ties(u, tol=1e-6):
    """Elements whose fp32 ratio u sits within tol of a rounding boundary m + 1/2.

    The code of an element is rint(u) clamped to 0..3, so it changes only at
    u = 0.5, 1.5 and 2.5; an element with |u - (m + 1/2)| < tol for m in
    {0, 1, 2} is a near-tie, whose code a differently rounded evaluation of u
    could flip.  u is NaN for groups with s == 0 (never a near-tie); values past
    the clamp (u near 3.5 or -0.5) are not boundaries.  Returns a bool array.
    """
    u = np.asarray(u, dtype=np.float64)
    near = np.zeros(u.shape, dtype=bool)
    for m in (0, 1, 2):
        near |= np.abs(u - (m + 0.5)) < tol
    return near


def code_parity(got_codes, ref_codes, u, tol=1e-6):
    """Compare 2-bit codes with near-ties excluded and counted.

    got_codes, ref_codes: unpacked codes of the same shape; u: the oracle's fp32
    ratios.  Returns (mismatches outside near-ties, near-ties, mismatches among
    near-ties).
    """
    got = np.asarray(got_codes)
    ref = np.asarray(ref_codes)
    near = code_near_ties(u, tol)
    diff = got != ref
    return int(np.count_nonzero(diff & ~near)), int(np.count_nonzero(near)), int(np.count_nonzero(diff & near))


def dequant_ref(packed, D=None):
    """Dequantised keys / values x = code * s + z in fp64 (exact for fp16 s, z).

    Returns (k_hat [B, Hkv, n, D], v_hat [B, Hkv, n, D]).
    """
    kc = unpack_codes_ref(packed["k_codes"]).astype(np.float64)
    B, Hkv, n, Dk = kc.shape
    vc = unpack_value_codes_ref(packed["v_codes"], n).astype(np.float64)
    ks = np.asarray(packed["k_scale"], np.float64)
    kz = np.asarray(packed["k_zero"], np.float64)
    tok_group = np.arange(n) // GROUP
    k_hat = kc * ks[:, :, tok_group, :] + kz[:, :, tok_group, :]
    vs = np.asarray(packed["v_scale"], np.float64)
    vz = np.asarray(packed["v_zero"], np.float64)
    ch_group = np.arange(Dk) // GROUP
    v_hat = vc * vs[:, :, :, ch_group] + vz[:, :, :, ch_group]
    return k_hat, v_hat


def decode_ref(q, packed, sm_scale=None):
    """Single-query attention over the packed cache, dequantised (fp64).

    out[b, h] = sum_t softmax_t(q[b, h] . k_hat[b, g, t] * scale) v_hat[b, g, t],
    g = h // r, over exactly the kept tokens.  Paper-listing abstract (the
    compressed cache serves inference); reading: no new token is appended, the
    query attends only the packed tokens.
    """
    q = np.asarray(q, dtype=np.float64)
    k_hat, v_hat = dequant_ref(packed)
    B, Hq, D = q.shape
    Hkv = k_hat.shape[1]
    r = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)
    out = np.empty((B, Hq, D))
    for b in range(B):
        for h in range(Hq):
            g = h // r
            logits = (k_hat[b, g] @ q[b, h]) * scale
            m = logits.max()
            p = np.exp(logits - m)
            p /= p.sum()
            out[b, h] = p @ v_hat[b, g]
    return out


def attn_tolerance(ref):
    """Elementwise bound for a bf16 attention output against the fp64 oracle.

    The target is a max-abs error of 2e-3 with bf16 outputs and fp32
    accumulation; a bf16 output alone is off by up to half an ulp, which
    exceeds 2e-3 once |o| >= 0.5.  Reading: pass where
    |o - o_ref| <= max(2e-3, 1 bf16 ulp of o_ref).
    """
    ax = np.abs(np.asarray(ref, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return np.maximum(2e-3, 2.0 ** (e - 7))


# ---------------------------------------------------------------------------
# Streaming decode: generated tokens join the cache.  Keys are quantised per
# channel over groups of 32 tokens (gptget.net summary, 方法论 / 方法详解), so a
# key group can only be formed once 32 tokens exist.  Reading (the pages are
# silent on generation): the packed region holds whole 32-token groups only;
# the remaining kept tokens and the generated ones wait, unquantised (their
# 16-bit values), in a residual window of at most 31 tokens, and every 32nd
# residual token packs the window as the next group.  Decode attends to the
# packed tokens and the residual ones.
# ---------------------------------------------------------------------------

def stream_split_ref(n_keep):
    """(packed, residual) token counts of an n_keep-token selection: whole groups are packed."""
    n_pk = GROUP * (int(n_keep) // GROUP)
    return n_pk, int(n_keep) - n_pk


def _empty_packed(B, Hkv, D):
    return {
        "k_codes": np.zeros((B, Hkv, 0, D // 4), np.uint8),
        "k_scale": np.zeros((B, Hkv, 0, D), np.float16),
        "k_zero": np.zeros((B, Hkv, 0, D), np.float16),
        "v_codes": np.zeros((B, Hkv, 0, D, 8), np.uint8),
        "v_scale": np.zeros((B, Hkv, 0, D // GROUP), np.float16),
        "v_zero": np.zeros((B, Hkv, 0, D // GROUP), np.float16),
    }


def concat_packed_ref(a, b):
    """Packed cache of a's tokens followed by b's; a must hold whole groups."""
    if a["k_codes"].shape[2] % GROUP:
        raise ValueError("the first cache must end on a group boundary")
    return {key: np.concatenate([a[key], b[key]], axis=2) for key in a}


def stream_init_ref(k, v, idx):
    """Streaming state from a selection idx [B, Hkv, n]: the first whole groups of
    kept tokens packed (quant_pack_ref), the rest kept as they are (fp32 values)."""
    k = np.asarray(k, dtype=np.float32)
    v = np.asarray(v, dtype=np.float32)
    idx = np.asarray(idx, dtype=np.int64)
    B, Hkv, _, D = k.shape
    n_pk, _ = stream_split_ref(idx.shape[-1])
    packed = quant_pack_ref(k, v, idx[..., :n_pk]) if n_pk else _empty_packed(B, Hkv, D)
    rest = idx[..., n_pk:, None]
    return {"packed": packed, "k_res": np.take_along_axis(k, rest, axis=2),
            "v_res": np.take_along_axis(v, rest, axis=2)}


def stream_append_ref(state, k_new, v_new):
    """One generated token per (sequence, KV head), k_new / v_new [B, Hkv, D], joins
    the residual; when the residual reaches 32 tokens it is packed as the next group."""
    k_res = np.concatenate([state["k_res"], np.asarray(k_new, np.float32)[:, :, None]], axis=2)
    v_res = np.concatenate([state["v_res"], np.asarray(v_new, np.float32)[:, :, None]], axis=2)
    packed = state["packed"]
    if k_res.shape[2] == GROUP:
        packed = concat_packed_ref(packed, quant_pack_ref(k_res, v_res))
        k_res, v_res = k_res[:, :, :0], v_res[:, :, :0]
    return {"packed": packed, "k_res": k_res, "v_res": v_res}


def stream_decode_ref(q, state, sm_scale=None):
    """Single-query attention over the packed tokens (dequantised) followed by the
    residual tokens (exact), fp64: the softmax runs over both sets together."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    k_res = np.asarray(state["k_res"], np.float64)
    v_res = np.asarray(state["v_res"], np.float64)
    Hkv = k_res.shape[1]
    if state["packed"]["k_codes"].shape[2]:
        k_hat, v_hat = dequant_ref(state["packed"])
        keys = np.concatenate([k_hat, k_res], axis=2)
        vals = np.concatenate([v_hat, v_res], axis=2)
    else:
        keys, vals = k_res, v_res
    r = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)
    out = np.empty((B, Hq, D))
    for b in range(B):
        for h in range(Hq):
            g = h // r
            logits = (keys[b, g] @ q[b, h]) * scale
            p = np.exp(logits - logits.max())
            out[b, h] = (p / p.sum()) @ vals[b, g]
    return out


# ---------------------------------------------------------------------------
# Bit accounting of the compact layout.
# ---------------------------------------------------------------------------

def packed_bytes_ref(B, Hkv, n_keep, D):
    """Bytes of the packed cache: codes, per-group K scale/zero, per-token V scale/zero.

    Per (sequence, KV head), with G = ceil(n/32): K codes n*D/4 + K scale/zero
    G*D*4 + V codes G*32*D/4 (whole 32-token blocks) + V scale/zero n*(D/32)*4.
    """
    n = int(n_keep)
    G = -(-n // GROUP)
    per = n * D // 4 + G * D * 4 + G * GROUP * D // 4 + n * (D // GROUP) * 4
    return B * Hkv * per


def compression_ratio_ref(T, n_keep, D):
    """1 - packed bytes / 16-bit bytes of the full T-token K and V (per head)."""
    full = 2 * T * D * 2
    return 1.0 - packed_bytes_ref(1, 1, n_keep, D) / full
