"""Cache policies of the pages' comparison tables, run on this library's kernels.

The LongBench table of the notesum.ai summary of "MiniKV: Pushing the Limits of
LLM Inference via 2-Bit Layer-Discriminative KV Cache" sets MiniKV and MiniKV
Pyramid beside the uncompressed model, KIVI (2-bit quantisation of every token),
H2O and SnapKV (15 % of the tokens kept, chosen by attention mass).  The
"experiment design" section of the same summary names the same comparison.
Each policy here is a choice of the three knobs that the hot path exposes:

  window  which prompt rows score a key: the last W rows (observation window,
          as MiniKV and SnapKV) or every row (W = T: the cumulative mass that
          H2O accumulates);
  budget  tokens kept per layer: every token (KIVI), a uniform share, or a
          share falling linearly over the layers (Pyramid);
  storage the kept tokens are always packed at 2 bits here; 16-bit storage of
          a selection (H2O and SnapKV as published) has no kernel in this
          library and is only ever an error reference.

compress() runs pass 1 (o, lse), pass 2 (scores), the heavy-hitter + recent
selection and the 2-bit pack of one layer; a policy that keeps every token
skips scoring and selection and packs the whole prompt.
"""

from dataclasses import dataclass

from . import api


@dataclass(frozen=True)
class Policy:
    """One row of the comparison.

    window: rows of the prompt that score a key; 0 = every row (W = T).
    schedule: "full" (every token), "uniform" (pct of T per layer) or
      "pyramid" (first_pct at layer 0 falling linearly to last_pct).
    """

    name: str
    window: int
    schedule: str
    pct: float = 15.0
    first_pct: int = 30
    last_pct: int = 5


POLICIES = {
    # MiniKV: observation window of 32 rows, 15 % of the tokens, 2-bit
    "minikv": Policy("minikv", window=32, schedule="uniform", pct=15.0),
    # MiniKV Pyramid: same selection, budget 30 % at the first layer to 5 % at the last
    "minikv_pyramid": Policy("minikv_pyramid", window=32, schedule="pyramid", first_pct=30, last_pct=5),
    # H2O-like: cumulative mass from every prompt row, 15 % of the tokens
    "h2o_like": Policy("h2o_like", window=0, schedule="uniform", pct=15.0),
    # KIVI-like: no eviction, every token at 2 bits
    "kivi_like": Policy("kivi_like", window=0, schedule="full"),
}


def layer_plan(policy, T, n_layers=1, layer=0):
    """(window rows, kept tokens, heavy hitters, recent tokens) of one layer.

    The window is resolved to a row count in [1, T]; a policy that keeps every
    token returns n_keep = T with no heavy / recent split (0, 0).
    """
    if isinstance(policy, str):
        policy = POLICIES[policy]
    if T < 1 or not 0 <= layer < n_layers:
        raise ValueError("need T >= 1 and 0 <= layer < n_layers")
    W = T if policy.window <= 0 else min(policy.window, T)
    if policy.schedule == "full":
        return W, T, 0, 0
    if policy.schedule == "uniform":
        n_keep = api.keep_count(T, policy.pct)
    elif policy.schedule == "pyramid":
        n_keep = api.pyramid_keep(T, n_layers, layer, policy.first_pct, policy.last_pct)
    else:
        raise ValueError(f"unknown schedule {policy.schedule!r}")
    n_heavy, n_recent = api.split_heavy_recent(n_keep)
    return W, n_keep, n_heavy, n_recent


def compress(q, k, v, policy, n_layers=1, layer=0, with_o=True):
    """Prefill-side compression of one layer under ``policy``.

    q [B, Hq, T, D], k, v [B, Hkv, T, D] bf16 on the GPU.  Returns
    (o or None, idx or None, PackedCache); idx is None when every token is kept.
    """
    T = q.shape[2]
    W, n_keep, n_heavy, n_recent = layer_plan(policy, T, n_layers, layer)
    if n_keep == T and n_heavy == 0 and n_recent == 0:
        o = api.prefill_attn(q, k, v)[0] if with_o else None
        return o, None, api.quant_pack(k, v, None)
    o, _, scores = api.prefill_attn_scores(q, k, v, W, with_o=with_o)
    idx = api.select_topk(scores, n_heavy, n_recent)
    return o, idx, api.quant_pack(k, v, idx)
