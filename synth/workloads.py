"""Workload shapes and seeded generators (random draws only; no method arithmetic)."""

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    """Shape and distribution of one synthetic workload.

    budget_pct: share of the T tokens kept (None when n_heavy / n_recent are
    given explicitly); pyramid: (first_pct, last_pct) per-layer budget.
    """

    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    T: int
    window: int
    layers: int = 1
    budget_pct: float = None
    n_heavy: int = None
    n_recent: int = None
    pyramid: tuple = None
    n_outlier: int = 4
    outlier_mult: float = 8.0
    v_std: float = 1.0
    in_dtype: str = "bf16"
    decode_steps: int = 1
    seed: int = 0


WORKLOADS = {
    # Tiny CPU-checkable case: 1 layer, 2 heads, head dim 64, batch 1, context 256,
    # fp32 K/V ~N(0,1) with 2 outlier key channels per head at x10, keep 48 heavy
    # hitters (16-query window) + 16 recent, one decode query, seed 0.
    "tiny": Workload("tiny", B=1, Hq=2, Hkv=2, D=64, T=256, window=16,
                     n_heavy=48, n_recent=16, n_outlier=2, outlier_mult=10.0,
                     v_std=1.0, in_dtype="f32", seed=0),
    # LLaMA2-7B-shaped single layer: 32 MHA heads, D 128, batch 8, context 4096,
    # 4 outlier key channels per head at x8, V ~N(0, 0.5), 15 % budget.
    "llama7b_decode": Workload("llama7b_decode", B=8, Hq=32, Hkv=32, D=128, T=4096,
                               window=32, budget_pct=15, n_outlier=4, outlier_mult=8.0,
                               v_std=0.5, seed=1),
    # Prefill selective attention + compress: 32 heads, D 128, batch 1, causal 16384.
    "prefill_16k": Workload("prefill_16k", B=1, Hq=32, Hkv=32, D=128, T=16384,
                            window=32, budget_pct=15, n_outlier=4, outlier_mult=8.0,
                            v_std=1.0, seed=2),
    # LLaMA2-13B-shaped pyramid decode: 40 layers x 40 heads, D 128, context 8192,
    # per-layer budget 30 % -> 5 %; batch is swept by the caller.
    "llama13b_pyramid": Workload("llama13b_pyramid", B=1, Hq=40, Hkv=40, D=128, T=8192,
                                 window=32, layers=40, pyramid=(30, 5), n_outlier=4,
                                 outlier_mult=8.0, v_std=0.5, seed=3),
    # Mistral-7B-shaped long context: GQA 32 / 8, D 128, 32 layers, prompt 44000,
    # batch 4, 15 % budget, 256 decode steps.
    "mistral_44k": Workload("mistral_44k", B=4, Hq=32, Hkv=8, D=128, T=44000,
                            window=32, layers=32, budget_pct=15, n_outlier=4,
                            outlier_mult=8.0, v_std=1.0, decode_steps=256, seed=4),
}


def outlier_channels(rng, n_heads, D, n_outlier):
    """Distinct outlier key channels per head, drawn from a numpy Generator."""
    return np.stack([np.sort(rng.choice(D, size=n_outlier, replace=False))
                     for _ in range(n_heads)]).astype(np.int64)


def tiny_inputs(seed=0, B=1, H=2, T=256, D=64, n_outlier=2, outlier_mult=10.0):
    """fp32 numpy inputs of the tiny workload.

    Draw order (numpy default_rng(seed)): q [B,H,T,D], k, v, decode query [B,H,D],
    then the outlier channels per head; outlier key channels are multiplied by
    ``outlier_mult``.
    """
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, T, D), dtype=np.float32)
    k = rng.standard_normal((B, H, T, D), dtype=np.float32)
    v = rng.standard_normal((B, H, T, D), dtype=np.float32)
    q_dec = rng.standard_normal((B, H, D), dtype=np.float32)
    outl = outlier_channels(rng, H, D, n_outlier)
    for h in range(H):
        k[:, h, :, outl[h]] *= np.float32(outlier_mult)
    return {"q": q, "k": k, "v": v, "q_dec": q_dec, "outliers": outl}


def torch_generator(device, seed):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _outlier_mask(torch, Hkv, D, n_outlier, mult, seed, device, dtype):
    rng = np.random.default_rng(seed + 7919)
    outl = outlier_channels(rng, Hkv, D, n_outlier)
    mask = np.ones((Hkv, D), dtype=np.float32)
    for h in range(Hkv):
        mask[h, outl[h]] = mult
    return torch.from_numpy(mask).to(device=device, dtype=torch.float32)[None, :, None, :], outl


def make_qkv(wl, device, seed=None, layer=0, q_rows=None, dtype=None):
    """Seeded torch tensors q [B,Hq,Tq,D], k, v [B,Hkv,T,D] on ``device``.

    q_rows: number of trailing query rows to draw (None = all T).  K gets the
    outlier channels, V has std ``wl.v_std``.  Drawn in fp32 and cast (round to
    nearest even) to ``dtype`` (default bf16).
    """
    import torch

    dtype = torch.bfloat16 if dtype is None else dtype
    s = (wl.seed if seed is None else seed) * 1000 + layer
    g = torch_generator(device, s)
    Tq = wl.T if q_rows is None else int(q_rows)
    q = torch.randn((wl.B, wl.Hq, Tq, wl.D), generator=g, device=device, dtype=torch.float32)
    k = torch.randn((wl.B, wl.Hkv, wl.T, wl.D), generator=g, device=device, dtype=torch.float32)
    v = torch.randn((wl.B, wl.Hkv, wl.T, wl.D), generator=g, device=device, dtype=torch.float32)
    mask, outl = _outlier_mask(torch, wl.Hkv, wl.D, wl.n_outlier, wl.outlier_mult, s, device, dtype)
    k.mul_(mask)
    v.mul_(wl.v_std)
    return q.to(dtype), k.to(dtype), v.to(dtype), outl


def make_decode_q(wl, device, seed=None, step=0, B=None):
    """Seeded decode queries [B, Hq, D] (bf16, ~N(0,1))."""
    import torch

    s = (wl.seed if seed is None else seed) * 1000 + 500 + step
    g = torch_generator(device, s)
    B = wl.B if B is None else B
    q = torch.randn((B, wl.Hq, wl.D), generator=g, device=device, dtype=torch.float32)
    return q.to(torch.bfloat16)


def make_kept_kv(wl, n_keep, device, seed, B=None):
    """Seeded bf16 kept-token K/V [B, Hkv, n_keep, D] drawn directly (no full context).

    Used where the full T-token cache of every sequence would not fit in memory:
    the tokens that survive selection are drawn from the same distributions.
    """
    import torch

    B = wl.B if B is None else B
    g = torch_generator(device, seed)
    k = torch.randn((B, wl.Hkv, n_keep, wl.D), generator=g, device=device, dtype=torch.float32)
    v = torch.randn((B, wl.Hkv, n_keep, wl.D), generator=g, device=device, dtype=torch.float32)
    mask, _ = _outlier_mask(torch, wl.Hkv, wl.D, wl.n_outlier, wl.outlier_mult, seed, device, torch.bfloat16)
    k.mul_(mask)
    v.mul_(wl.v_std)
    return k.to(torch.bfloat16), v.to(torch.bfloat16)



def make_heavy_qkv(wl, device, heavy_frac=0.05, strength=7.0, seed=None):
    """Seeded bf16 q [B,Hq,T,D], k, v [B,Hkv,T,D] and decode queries [B,Hq,D] whose
    attention concentrates on a few positions (heavy hitters).

    As make_qkv, plus: per (sequence, KV head) a random unit direction u and a
    random ``heavy_frac`` share of the positions.  Those keys and every query
    row (prompt and decode) of the heads that share the KV head get
    ``strength * u`` added, so the marked keys draw a large share of every
    row's attention.  Random draws only; which positions are marked is not an
    input of the method.
    """
    import torch

    s = (wl.seed if seed is None else seed) * 1000 + 900
    q, k, v, _ = make_qkv(wl, device, seed=s, dtype=torch.float32)
    g = torch_generator(device, s + 1)
    B, Hkv, T, D = k.shape
    r = wl.Hq // Hkv
    u = torch.randn((B, Hkv, D), generator=g, device=device, dtype=torch.float32)
    u = u / u.norm(dim=-1, keepdim=True)
    n_heavy = max(1, int(heavy_frac * T))
    pos = torch.rand((B, Hkv, T), generator=g, device=device).argsort(-1)[..., :n_heavy]
    mark = torch.zeros((B, Hkv, T), device=device, dtype=torch.float32).scatter_(-1, pos, 1.0)
    k = k + strength * mark[..., None] * u[:, :, None, :]
    uq = u.repeat_interleave(r, 1)
    q = q + strength * uq[:, :, None, :]
    qd = torch.randn((B, wl.Hq, D), generator=g, device=device, dtype=torch.float32) + strength * uq
    bf = torch.bfloat16
    return q.to(bf), k.to(bf), v.to(bf), qd.to(bf)

def bf16_round(x):
    """Round fp32 numpy values to bf16 (nearest even) and return them as fp32."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()
