"""Benchmark of the 2-bit layer-discriminative KV-cache hot path on one MI355X.

Headline (the JSON line's value): decode attention over the LLaMA2-13B-shaped
layer-discriminative cache - 40 layers x 40 heads, head dim 128, context 8192,
per-layer budget falling linearly from 30 % (2457 kept tokens) to 5 % (409),
2-bit packed - at the batch that fills about 250 GB of HBM (1133 sequences,
249.8 GB packed).  A step is one decode query per sequence through all 40
layers (40 launches of the decode kernel); value = batch / step time in
tokens/s, beside the achieved HBM GB/s and its fraction of 8 TB/s.  Kept-token
K/V are drawn directly from the workload's distributions (bf16, 4 outlier key
channels per head x 8, V ~ N(0, 0.5)) and packed by the library before the
timed region, so the cache is resident in HBM when timing starts.  Each
launch is bracketed by HIP events on the stream it runs on; the roofline
object reports the decode kernel's algorithmic bytes per launch over its
average launch time.  cpu_baseline times the oracle's decode of the same
cache on a bounded sample of sequences.

Extra objects in the same line:
  chain            the whole path on the LLaMA2-7B-shaped workload (8 x 32 heads x
                   4096 tokens, 15 % budget): selective flash attention with the
                   window scores, selection, quantise-and-pack, decode; per-stage
                   HIP-event times and the prefill kernel's bf16 MFMA roofline
                   (prefill_roofline)
  decode           the chain's single-layer decode alone, rotating over >= 1 GB of
                   distinct packed caches (Infinity Cache excluded), eager and as a
                   HIP graph replay
  decode_gqa       the Mistral-7B-shaped 32-layer GQA cache (32 / 8 heads, 6600
                   kept of 44000, batch 4), 256 steps of fresh queries, eager and
                   as a HIP graph replay
  decode_stream    the same cache as generation (append + decode per layer)
  prefill_16k, prefill_gqa_44k   single-layer prefill lines
  variants         the comparison tables' cache policies on the chain's prompt
  decode_pyramid_sweep (--pyramid-sweep) the pyramid decode over a batch sweep

    python bench.py [--gpus 1] [--steps 20] [--warmup 5]
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "2-bit KV decode-attn tokens/s + achieved HBM GB/s (% peak); prefill MFMA %"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 / fp16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=25)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--decode-rotation-gb", type=float, default=1.2)
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="after the timed region, run one device copy of this size (counter calibration)")
    ap.add_argument("--pyramid-batch", type=int, default=1133,
                    help="batch of the headline 40-layer pyramid decode (1133 fills about 250 GB)")
    ap.add_argument("--headline-only", action="store_true",
                    help="run the headline decode only (e.g. under a counter profiler)")
    ap.add_argument("--only", choices=["prefill_16k", "chain", "decode_gqa", "decode_stream"], default=None,
                    help="run one extra alone and print it (no headline; e.g. under a counter profiler)")
    ap.add_argument("--chain-warmup", type=int, default=25,
                    help="warm-up steps of the chain extra (a fresh process runs its first chain steps slow)")
    ap.add_argument("--pyramid-sweep", default="",
                    help="comma-separated batches for a max-throughput sweep of the 40-layer pyramid decode "
                         "(e.g. 1,64,256,512,1024,1133; 1133 fills about 250 GB); off by default")
    ap.add_argument("--no-gqa-sweep", action="store_true", help="skip the 32-layer GQA decode sweep")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the comparison of cache policies (KIVI-like, H2O-like, MiniKV, Pyramid)")
    ap.add_argument("--no-prefill-sweep", action="store_true",
                    help="skip the single-layer prefill lines (1 x 32 x 16384 and the 44k-token GQA layer)")
    return ap.parse_args()


def decode_layers(torch, mk, synth, wl, B, budgets, reps=3, chunk=64, n_queries=1):
    """Pack one cache per layer (kept-token K/V drawn directly), then time `reps`
    decode steps through all layers: one query per sequence per step, step i
    using seeded query set i % n_queries (fresh queries each step when
    n_queries >= reps)."""
    dev = torch.device("cuda:0")
    caches = build_layer_caches(torch, mk, synth, wl, B, budgets, chunk)
    qs = [synth.make_decode_q(wl, dev, B=B, step=i) for i in range(max(1, n_queries))]
    q = qs[0]
    out = torch.empty_like(q)
    ws = torch.zeros(max(16, max(mk.decode_ws_bytes(B, wl.Hq, wl.Hkv, c.n_keep, wl.D) for c in caches)),
                     dtype=torch.uint8, device=dev)
    for c in caches:  # warm-up pass
        mk.decode_attn(q, c, out=out, ws=ws)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(reps):
        qi = qs[i % len(qs)]
        for c in caches:
            mk.decode_attn(qi, c, out=out, ws=ws)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / reps
    # The same steps replayed as one HIP graph (how a serving loop issues it): no
    # per-call host work between the layers' launches; each step's queries are
    # copied into the captured query buffer first.
    q_buf = q.clone()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for c in caches:
            mk.decode_attn(q_buf, c, out=out, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(graph):
        for c in caches:
            mk.decode_attn(q_buf, c, out=out, ws=ws)
    graph.replay()
    torch.cuda.synchronize()
    ev0.record()
    for i in range(reps):
        if len(qs) > 1:
            q_buf.copy_(qs[i % len(qs)])
        graph.replay()
    ev1.record()
    torch.cuda.synchronize()
    gms = ev0.elapsed_time(ev1) / reps
    del graph
    cache_bytes = sum(c.nbytes() for c in caches)
    qo_bytes = 2 * B * wl.Hq * wl.D * 2 * len(caches)
    gbs = (cache_bytes + qo_bytes) / (ms * 1e-3) / 1e9
    ggbs = (cache_bytes + qo_bytes) / (gms * 1e-3) / 1e9
    del caches
    torch.cuda.empty_cache()
    return {"workload": wl.name, "batch": B, "layers": len(budgets), "q_heads": wl.Hq, "kv_heads": wl.Hkv,
            "kept_tokens_first_last": [int(budgets[0]), int(budgets[-1])], "packed_GB": cache_bytes / 1e9,
            "ms_per_step": ms, "tokens_per_s": B / (ms * 1e-3), "achieved_GBs": gbs,
            "hbm_frac": gbs / PEAK_HBM_GBS,
            "graph_ms_per_step": gms, "graph_tokens_per_s": B / (gms * 1e-3), "graph_achieved_GBs": ggbs,
            "graph_hbm_frac": ggbs / PEAK_HBM_GBS, "steps": reps, "distinct_queries": len(qs)}


def build_layer_caches(torch, mk, synth, wl, B, budgets, chunk=64):
    """One packed cache per layer, kept-token K/V drawn directly per chunk of
    sequences and packed by the library into the layer's cache."""
    dev = torch.device("cuda:0")
    caches = []
    t0 = time.perf_counter()
    for l, n in enumerate(budgets):
        if l and l % 8 == 0:
            torch.cuda.synchronize()
            print(f"# building {wl.name} caches: {l} of {len(budgets)} layers, {time.perf_counter() - t0:.1f} s",
                  file=sys.stderr, flush=True)
        c = mk.PackedCache.alloc(B, wl.Hkv, n, wl.D, dev)
        for b0 in range(0, B, chunk):
            b1 = min(B, b0 + chunk)
            k, v = synth.make_kept_kv(wl, n, dev, seed=wl.seed * 100000 + l * 1000 + b0, B=b1 - b0)
            sub = mk.PackedCache(c.k_codes[b0:b1], c.k_sz[b0:b1], c.v_codes[b0:b1], c.v_sz[b0:b1],
                                 b1 - b0, wl.Hkv, n, wl.D)
            mk.quant_pack(k, v, out=sub)
            del k, v
        caches.append(c)
    return caches


def pyramid_headline(torch, mk, synth, B, steps, warmup, sample_seqs=0):
    """The headline: decode over the 40-layer pyramid cache at batch B.

    Returns the step time (HIP events around the K timed steps, bracketed by
    device synchronisation), the per-launch durations of the decode kernel
    (one launch per layer; events on the launch stream) and the algorithmic
    bytes: each layer's packed cache plus the bf16 query read and output
    written."""
    dev = torch.device("cuda:0")
    pw = synth.WORKLOADS["llama13b_pyramid"]
    budgets = [mk.pyramid_keep(pw.T, pw.layers, l, *pw.pyramid) for l in range(pw.layers)]
    t0 = time.perf_counter()
    caches = build_layer_caches(torch, mk, synth, pw, B, budgets)
    torch.cuda.synchronize()
    build_s = time.perf_counter() - t0
    n_q = 4  # distinct seeded query sets, cycled step by step
    qs = [synth.make_decode_q(pw, dev, B=B, step=i) for i in range(n_q)]
    out = torch.empty_like(qs[0])
    ws = torch.zeros(max(16, max(mk.decode_ws_bytes(B, pw.Hq, pw.Hkv, c.n_keep, pw.D) for c in caches)),
                     dtype=torch.uint8, device=dev)
    cache_bytes = [c.nbytes() for c in caches]
    print(f"# pyramid cache: batch {B}, {sum(cache_bytes) / 1e9:.1f} GB packed, built in {build_s:.1f} s",
          file=sys.stderr, flush=True)
    for i in range(warmup):
        for c in caches:
            mk.decode_attn(qs[i % n_q], c, out=out, ws=ws)
    torch.cuda.synchronize()
    L = len(caches)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(L + 1)] for _ in range(steps)]
    e_all = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    wall0 = time.perf_counter()
    e_all[0].record()
    for s_ in range(steps):
        q = qs[s_ % n_q]
        for l, c in enumerate(caches):
            ev[s_][l].record()
            mk.decode_attn(q, c, out=out, ws=ws)
        ev[s_][L].record()
    e_all[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = e_all[0].elapsed_time(e_all[1]) / steps
    launch_ms = [[ev[s_][l].elapsed_time(ev[s_][l + 1]) for l in range(L)] for s_ in range(steps)]
    layer_ms = [sum(launch_ms[s_][l] for s_ in range(steps)) / steps for l in range(L)]
    qo_bytes = 2 * B * pw.Hq * pw.D * 2
    alg_bytes = [cb + qo_bytes for cb in cache_bytes]
    step_bytes = sum(alg_bytes)
    kernel_ms = sum(layer_ms)
    # the kernel plan: one token range per KV head at this batch, so the decode
    # call is exactly one decode_partial_kernel launch per layer (no merge)
    splits = [mk.decode_ws_bytes(B, pw.Hq, pw.Hkv, c.n_keep, pw.D) for c in caches]
    # host copies of a bounded sample of the same cache and queries, for the
    # oracle's timing (cpu_baseline)
    sample = None
    if sample_seqs:
        sel = torch.arange(sample_seqs, device=dev)
        sample = {"q": qs[0][sel].float().cpu().numpy(), "layers": [], "seqs": sample_seqs}
        for c in caches:
            ksz = c.k_sz[sel].cpu().numpy().view("uint32")
            vsz = c.v_sz[sel].cpu().numpy().view("uint32")
            sample["layers"].append({"k_codes": c.k_codes[sel].cpu().numpy(), "v_codes": c.v_codes[sel].cpu().numpy(),
                                     "k_sz": ksz, "v_sz": vsz})
    del caches, ws, out, qs
    torch.cuda.empty_cache()
    gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    return {
        "workload": "llama13b_pyramid", "batch": B, "layers": L, "q_heads": pw.Hq, "kv_heads": pw.Hkv,
        "head_dim": pw.D, "context": pw.T, "kept_tokens_first_last": [int(budgets[0]), int(budgets[-1])],
        "kept_tokens_per_seq_head": int(sum(budgets)), "packed_GB": sum(cache_bytes) / 1e9,
        "cache_build_s": build_s, "ms_per_step": ms_per_step, "host_ms_per_step": wall * 1e3 / steps,
        "tokens_per_s": B / (ms_per_step * 1e-3), "achieved_GBs": gbs, "hbm_frac": gbs / PEAK_HBM_GBS,
        "step_bytes": step_bytes, "kernel_ms_per_step": kernel_ms,
        "launch_ms_avg": kernel_ms / L, "bytes_per_launch_avg": step_bytes / L,
        "single_range_per_head": all(x == splits[0] for x in splits),
        "layer_ms_first_last": [layer_ms[0], layer_ms[-1]], "distinct_queries": n_q,
    }, sample


def prefill_layer(torch, mk, synth, wl, reps, warm=5):
    """One layer of a prefill workload through the chain's first four steps,
    each timed alone (HIP events, `reps` calls after `warm` warm-up calls), and
    the single-pass call (window scores from inside pass 1) where it applies.
    The prefill's first launches in a process run up to a quarter slower while
    the clock settles under the matrix cores' load, so a few are run first."""
    dev = torch.device("cuda:0")
    q, k, v, _ = synth.make_qkv(wl, dev)
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    n_keep = mk.keep_count(T, wl.budget_pct)
    n_heavy, n_recent = mk.split_heavy_recent(n_keep)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
    scores = torch.empty((B, Hkv, T), dtype=torch.float32, device=dev)
    idx = torch.empty((B, Hkv, n_keep), dtype=torch.int32, device=dev)
    cache = mk.PackedCache.alloc(B, Hkv, n_keep, D, dev)
    calls = {
        "prefill_attn": lambda: mk.prefill_attn(q, k, v, o=o, lse=lse),
        "window_scores": lambda: mk.window_scores(q, k, lse, wl.window, scores=scores),
        "select_topk": lambda: mk.select_topk(scores, n_heavy, n_recent, idx=idx),
        "quant_pack": lambda: mk.quant_pack(k, v, idx, out=cache),
    }
    if mk.prefill_fuses_scores(B, T, Hq, Hkv, wl.window):  # single pass: both in one launch
        calls["prefill_attn_scores"] = lambda: mk.prefill_attn_scores(q, k, v, wl.window, o=o, lse=lse,
                                                                      scores=scores)
    ms = {}
    for name, fn in calls.items():
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms[name] = e0.elapsed_time(e1) / reps
    flops = 2.0 * D * T * (T + 1) * Hq * B
    tf = flops / (ms["prefill_attn"] * 1e-3) / 1e12
    k_bytes = k.numel() * k.element_size()
    pack_bytes = 2 * B * Hkv * n_keep * D * k.element_size() + cache.nbytes()
    res = {"workload": wl.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "context": T, "head_dim": D,
           "window": wl.window, "n_keep": n_keep, "warmup_calls": warm, "timed_calls": reps, "stages_ms": ms,
           "prefill_TFLOPs": tf, "prefill_mfma_frac": tf / PEAK_BF16_TFLOPS,
           "window_scores_GBs": k_bytes / (ms["window_scores"] * 1e-3) / 1e9,
           "quant_pack_GBs": pack_bytes / (ms["quant_pack"] * 1e-3) / 1e9}
    del q, k, v, o, lse, scores, idx, cache
    torch.cuda.empty_cache()
    return res


def decode_stream(torch, mk, synth, wl, steps):
    """Generation over a streaming cache per layer: each step appends one token per
    (sequence, KV head) to every layer (packing every 32nd) and decodes one query per
    sequence through all layers.  Kept-token K/V of the prompt are drawn directly.
    Timed twice: with host-side counts (Python decides each pack), and with the
    counts on the device, one step of all layers captured in a HIP graph and
    replayed per token (graph_*)."""
    dev = torch.device("cuda:0")
    B, n = wl.B, mk.keep_count(wl.T, wl.budget_pct)
    cap = 32 * ((n + steps) // 32 + 1)
    caches = []
    for l in range(wl.layers):
        k, v = synth.make_kept_kv(wl, n, dev, seed=wl.seed * 100000 + l * 1000 + 7, B=B)
        idx = torch.arange(n, dtype=torch.int32, device=dev).expand(B, wl.Hkv, n).contiguous()
        caches.append(mk.StreamCache.alloc(B, wl.Hkv, cap, wl.D, dev).init(k, v, idx))
        del k, v, idx
    g = torch.Generator(device=dev).manual_seed(wl.seed * 31 + 5)
    pool = 8  # distinct new tokens / queries, cycled
    kn = [torch.randn((B, wl.Hkv, wl.D), generator=g, device=dev).to(torch.bfloat16) for _ in range(pool)]
    vn = [torch.randn((B, wl.Hkv, wl.D), generator=g, device=dev).to(torch.bfloat16) for _ in range(pool)]
    qs = [synth.make_decode_q(wl, dev, step=i, B=B) for i in range(pool)]
    out = torch.empty_like(qs[0])
    # the largest streaming workspace: the whole capacity packed and a full window
    ws = torch.zeros(max(16, caches[0].step_ws_bytes(wl.Hq)), dtype=torch.uint8, device=dev)
    res0 = caches[0].n_res
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    e0.record()
    for s in range(steps):
        for c in caches:
            c.append(kn[s % pool], vn[s % pool])
            c.decode(qs[s % pool], out=out, ws=ws)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = e0.elapsed_time(e1) / steps
    packed_bytes = sum(mk.packed_bytes(B, wl.Hkv, c.n_packed, wl.D) for c in caches)
    flushes = (res0 + steps) // 32

    # ---- the same generation with device-side counts: one step (all layers) is a
    # fixed launch sequence, captured once in a HIP graph and replayed per token ----
    for l, c in enumerate(caches):  # back to the prompt's state
        k, v = synth.make_kept_kv(wl, n, dev, seed=wl.seed * 100000 + l * 1000 + 7, B=B)
        idx = torch.arange(n, dtype=torch.int32, device=dev).expand(B, wl.Hkv, n).contiguous()
        c.init(k, v, idx).to_device_counts()
        del k, v, idx
    k_in, v_in, q_in = kn[0].clone(), vn[0].clone(), qs[0].clone()
    ws_g = torch.zeros(max(16, caches[0].step_ws_bytes(wl.Hq)), dtype=torch.uint8, device=dev)
    scratch = mk.StreamCache.alloc(B, wl.Hkv, cap, wl.D, dev)
    scratch.n_packed, scratch.n_res = 0, 0
    scratch.to_device_counts()
    scratch.step_append(k_in, v_in)  # launch set-up outside the capture
    scratch.step_decode(q_in, out=out, ws=ws_g)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for c in caches:
                c.step_append(k_in, v_in)
                c.step_decode(q_in, out=out, ws=ws_g)
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    g0.record()
    for s in range(steps):
        k_in.copy_(kn[s % pool])  # the step's new token and query
        v_in.copy_(vn[s % pool])
        q_in.copy_(qs[s % pool])
        graph.replay()
    g1.record()
    torch.cuda.synchronize()
    gwall = time.perf_counter() - wall0
    gms = g0.elapsed_time(g1) / steps
    caches[0].from_device_counts()  # raises if a window could not be packed
    g_packed = caches[0].n_packed
    del caches, graph, scratch
    torch.cuda.empty_cache()
    return {"workload": wl.name, "batch": B, "layers": wl.layers, "q_heads": wl.Hq, "kv_heads": wl.Hkv,
            "prompt_kept_tokens": n, "steps": steps, "packs_per_layer": flushes,
            "packed_GB_at_end": packed_bytes / 1e9, "ms_per_step": ms, "tokens_per_s": B / (ms * 1e-3),
            "host_ms_per_step": wall * 1e3 / steps,
            "graph_ms_per_step": gms, "graph_tokens_per_s": B / (gms * 1e-3),
            "graph_host_ms_per_step": gwall * 1e3 / steps, "graph_packed_tokens_at_end": g_packed}



def _attn_full_ref(torch, qd, k, v, idx=None):
    """fp32 single-query attention over bf16 K/V (all tokens, or the selection idx): the
    error reference for the policy comparison (16-bit storage has no kernel here)."""
    B, Hq, D = qd.shape
    r = Hq // k.shape[1]
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=qd.device)
    for b in range(B):
        kb, vb = k[b].float(), v[b].float()
        if idx is not None:
            ib = idx[b].long()[..., None].expand(-1, -1, D)
            kb, vb = kb.gather(1, ib), vb.gather(1, ib)
        kb, vb = kb.repeat_interleave(r, 0), vb.repeat_interleave(r, 0)
        logits = (qd[b].float()[:, None, :] * kb).sum(-1) * D ** -0.5
        p = torch.softmax(logits, -1)
        out[b] = (p[..., None] * vb).sum(1)
    return out


def _rel_l2(torch, got, ref):
    e = (got.float() - ref).norm(dim=-1) / ref.norm(dim=-1).clamp_min(1e-30)
    return {"mean": float(e.mean()), "max": float(e.max())}


def variants_compare(torch, mk, q, k, v, qd, n_layers, label, reps=3):
    """The comparison-table policies on one prompt (q, k, v) and one decode query qd.

    Per policy, averaged over the per-layer plans of an n_layers model (the same
    synthetic layer stands in for every layer): kept tokens, packed bytes over
    the 16-bit K/V bytes, time of compress() (pass 1, pass 2 with the policy's
    window, selection, pack) and of decode, and the decode output's relative L2
    error per (sequence, head) against exact attention over the full 16-bit
    cache.  Evicting policies also report the same selection held at 16 bits
    (eviction alone, as H2O / SnapKV store it), computed in fp32 torch.
    """
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    full = _attn_full_ref(torch, qd, k, v)
    bf16_bytes = 2 * B * Hkv * T * D * 2
    res = {}
    for name in mk.POLICIES:
        layers = range(n_layers) if mk.POLICIES[name].schedule == "pyramid" else [0]
        rows = []
        for layer in layers:
            _, n_keep, _, _ = mk.layer_plan(name, T, n_layers, layer)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            mk.compress(q, k, v, name, n_layers, layer)
            ev[0].record()
            for _ in range(reps):
                _, idx, cache = mk.compress(q, k, v, name, n_layers, layer)
            ev[1].record()
            for _ in range(reps):
                out = mk.decode_attn(qd, cache)
            ev[2].record()
            torch.cuda.synchronize()
            row = {"n_keep": n_keep, "packed_share": cache.nbytes() / bf16_bytes,
                   "compress_ms": ev[0].elapsed_time(ev[1]) / reps,
                   "decode_ms": ev[1].elapsed_time(ev[2]) / reps,
                   "err_2bit": _rel_l2(torch, out, full)}
            if idx is not None:
                row["err_16bit_same_selection"] = _rel_l2(torch, _attn_full_ref(torch, qd, k, v, idx), full)
            rows.append(row)
            del cache, idx, out
        n = len(rows)
        agg = {"layers_averaged": n,
               "n_keep_mean": sum(r_["n_keep"] for r_ in rows) / n,
               "compression": 1.0 - sum(r_["packed_share"] for r_ in rows) / n,
               "compress_ms": sum(r_["compress_ms"] for r_ in rows) / n,
               "decode_ms": sum(r_["decode_ms"] for r_ in rows) / n,
               "err_2bit_mean": sum(r_["err_2bit"]["mean"] for r_ in rows) / n,
               "err_2bit_max": max(r_["err_2bit"]["max"] for r_ in rows)}
        if "err_16bit_same_selection" in rows[0]:
            agg["err_16bit_same_selection_mean"] = sum(r_["err_16bit_same_selection"]["mean"] for r_ in rows) / n
        res[name] = agg
    torch.cuda.empty_cache()
    return {"workload": label, "batch": B, "q_heads": Hq,
            "kv_heads": Hkv, "context": T, "head_dim": D, "layers_in_plan": n_layers,
            "error": "relative L2 of the decode output per (sequence, head) vs exact attention over all T "
                     "16-bit tokens", "policies": res}

class StageTimer:
    """HIP events around each call on the current stream; per-stage totals in ms."""

    def __init__(self, torch, names):
        self.torch = torch
        self.names = names
        self.events = []

    def mark(self):
        ev = self.torch.cuda.Event(enable_timing=True)
        ev.record()
        self.events.append(ev)

    def totals(self, steps):
        n = len(self.names)
        tot = {k: 0.0 for k in self.names}
        for s in range(steps):
            evs = self.events[s * (n + 1):(s + 1) * (n + 1)]
            for i, k in enumerate(self.names):
                tot[k] += evs[i].elapsed_time(evs[i + 1])
        return {k: v / steps for k, v in tot.items()}


def cpu_baseline_pyramid(sample):
    """Time the oracle's decode (dequantise, softmax attention in fp64) of the
    sampled sequences' packed caches through all 40 layers; tokens/s."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    half = lambda w: (w & 0xFFFF).astype(np.uint16).view(np.float16)  # noqa: E731
    packed = [{"k_codes": ly["k_codes"], "k_scale": half(ly["k_sz"]), "k_zero": half(ly["k_sz"] >> 16),
               "v_codes": ly["v_codes"], "v_scale": half(ly["v_sz"]), "v_zero": half(ly["v_sz"] >> 16)}
              for ly in sample["layers"]]
    t0 = time.perf_counter()
    for p_ in packed:
        oracle.decode_ref(sample["q"], p_)
    dt = time.perf_counter() - t0
    n = sample["seqs"]
    return {"value": n / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} of the batch's sequences (all 40 heads, all 40 layers) of the same packed cache and "
                      f"queries: the oracle's decode_ref per layer; {dt:.1f} s; BLAS threads = cores"}


def cpu_baseline(wl, n_seq=2):
    """Time the oracle on n_seq sequences (all heads) of the same chain; report tokens/s."""
    import torch

    import oracle
    import synth

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    q, k, v, _ = synth.make_qkv(wl, "cpu")
    qd = synth.make_decode_q(wl, "cpu")
    qs, ks, vs = (x[:n_seq].float().numpy() for x in (q, k, v))
    qds = qd[:n_seq].float().numpy()
    del q, k, v
    n_keep = oracle.keep_count(wl.T, wl.budget_pct)
    nh, nr = oracle.split_heavy_recent(n_keep)
    t0 = time.perf_counter()
    oracle.prefill_ref(qs, ks, vs)
    sc = oracle.window_scores_ref(qs, ks, wl.window)
    idx = oracle.select_ref(sc, nh, nr)
    packed = oracle.quant_pack_ref(ks, vs, idx)
    oracle.decode_ref(qds, packed)
    dt = time.perf_counter() - t0
    return {"value": n_seq * (wl.T + 1) / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n_seq} of {wl.B} sequences (all {wl.Hq} heads) of the same chain: prefill o/lse, "
                      f"window scores, selection, quantise-pack, decode; {dt:.1f} s; BLAS threads = cores"}


def load_traffic(path, kernel_src):
    """HBM bytes per launch of the dominant kernel from a committed counter summary.

    The summary records a hash of the kernel source it was measured on; a
    different source means the figure is stale and None is returned.
    """
    import hashlib

    try:
        text = open(path).read()
    except OSError:
        return None
    want = hashlib.sha256(open(kernel_src, "rb").read()).hexdigest()[:16]
    vals = {}
    for line in text.splitlines():
        if line.startswith("- ") and ":" in line:
            key, val = line[2:].split(":", 1)
            vals[key.strip()] = val.strip().strip("`")
    if vals.get("kernel_source_sha256_16") != want:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def calibration_copy(torch, mb):
    """One device-to-device copy of a known size, for scaling HBM counters."""
    src = torch.empty(mb * (1 << 20), dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(f"# calibration copy: {src.numel()} bytes read, {dst.numel()} written", file=sys.stderr, flush=True)
    del src, dst
    torch.cuda.empty_cache()


def measured_peaks(torch, mk, read_gib=8, gemm_sizes=(8192, 16384), reps=10):
    """Reference rates of this GPU, the denominators beside the vendor peaks: a
    streaming read (the library's read probe: every 16-byte piece of a buffer
    once, non-temporal), a device copy (bytes read + written), and a large bf16
    GEMM (torch.matmul, which hipBLASLt serves; contiguous 2-D operands)."""
    dev = torch.device("cuda:0")

    def timed(fn):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    n = read_gib * (1 << 30) // 2
    x = torch.empty(n, dtype=torch.bfloat16, device=dev).fill_(1.0)
    sink = torch.zeros(mk.api.READ_PROBE_SINK_WORDS, dtype=torch.int32, device=dev)
    read_s = timed(lambda: mk.read_probe(x, sink))
    y = torch.empty_like(x)
    copy_s = timed(lambda: y.copy_(x))
    del x, y, sink
    g = torch.Generator(device=dev).manual_seed(11)
    gemm = {}
    for m in gemm_sizes:
        a = torch.randn((m, m), generator=g, device=dev).to(torch.bfloat16)
        b = torch.randn((m, m), generator=g, device=dev).to(torch.bfloat16)
        gemm[m] = 2.0 * m ** 3 / timed(lambda: torch.matmul(a, b)) / 1e12
        del a, b
    torch.cuda.empty_cache()
    best = max(gemm, key=gemm.get)
    nbytes = n * 2
    # the same probe over a small-batch decode layer's bytes, cold: buffers of that
    # size rotated over >= 1.2 GB, one launch each, replayed as a HIP graph
    small = {}
    for name, size in (("llama7b_decode_layer", mk.packed_bytes(8, 32, 614, 128)),
                       ("mistral_decode_layer", mk.packed_bytes(4, 8, 6600, 128))):
        size = (size + 15) // 16 * 16
        nbuf = max(2, -(-int(1.2e9) // size))
        bufs = [torch.empty(size // 2, dtype=torch.bfloat16, device=dev).fill_(1.0) for _ in range(nbuf)]
        sink = torch.zeros(mk.api.READ_PROBE_SINK_WORDS, dtype=torch.int32, device=dev)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for x in bufs:
                mk.read_probe(x, sink)
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for x in bufs:
                mk.read_probe(x, sink)
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (3 * nbuf)
        small[name] = {"bytes": size, "us": us, "GBs": size / us / 1e3}
        del bufs, sink, graph
        torch.cuda.empty_cache()
    return {"hbm_read_GBs": nbytes / read_s / 1e9,
            "read_kind": f"minikv_read_probe over {read_gib} GiB (16-byte non-temporal loads, grid-stride)",
            "hbm_copy_GBs": 2 * nbytes / copy_s / 1e9,
            "copy_kind": f"device copy of {read_gib} GiB (bytes read + written)",
            "bf16_gemm_TFLOPs": gemm[best],
            "gemm_kind": f"torch.matmul {best} x {best} x {best} bf16 (hipBLASLt), the best of "
                         + ", ".join(f"{m}^3: {t:.0f}" for m, t in gemm.items()),
            "small_reads": small,
            "small_read_kind": "minikv_read_probe over one small-batch decode layer's packed bytes, cold "
                               "(buffers rotated over >= 1.2 GB), per launch in a replayed HIP graph"}


def chain(torch, mk, synth, args):
    """The whole path on the LLaMA2-7B-shaped workload; returns (chain, prefill
    roofline, single-layer decode) objects."""
    dev = torch.device("cuda:0")
    wl = synth.WORKLOADS["llama7b_decode"]
    B, Hq, Hkv, T, D, W = wl.B, wl.Hq, wl.Hkv, wl.T, wl.D, wl.window
    n_keep = mk.keep_count(T, wl.budget_pct)
    n_heavy, n_recent = mk.split_heavy_recent(n_keep)

    q, k, v, _ = synth.make_qkv(wl, dev)
    qdec = synth.make_decode_q(wl, dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
    scores = torch.empty((B, Hkv, T), dtype=torch.float32, device=dev)
    idx = torch.empty((B, Hkv, n_keep), dtype=torch.int32, device=dev)
    cache = mk.PackedCache.alloc(B, Hkv, n_keep, D, dev)
    out = torch.empty_like(qdec)
    ws = torch.zeros(mk.decode_ws_bytes(B, Hq, Hkv, n_keep, D), dtype=torch.uint8, device=dev)

    # single pass: the window scores come out of the pass-1 kernel (one launch)
    fused = mk.prefill_fuses_scores(B, T, Hq, Hkv, W)

    def stage_names(single):
        return (["prefill_attn_scores"] if single else ["prefill_attn", "window_scores"]) + \
            ["select_topk", "quant_pack", "decode_attn"]

    timer = StageTimer(torch, stage_names(fused))

    def step(t=None, single=fused):
        if t:
            t.mark()
        if single:
            mk.prefill_attn_scores(q, k, v, W, o=o, lse=lse, scores=scores)
        else:
            mk.prefill_attn(q, k, v, o=o, lse=lse)
            if t:
                t.mark()
            mk.window_scores(q, k, lse, W, scores=scores)
        if t:
            t.mark()
        mk.select_topk(scores, n_heavy, n_recent, idx=idx)
        if t:
            t.mark()
        mk.quant_pack(k, v, idx, out=cache)
        if t:
            t.mark()
        mk.decode_attn(qdec, cache, out=out, ws=ws)
        if t:
            t.mark()

    for _ in range(args.chain_warmup):
        step()
    torch.cuda.synchronize()
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    t_all0.record()
    for _ in range(args.steps):
        step(timer)
    t_all1.record()
    torch.cuda.synchronize()
    ms_per_step = t_all0.elapsed_time(t_all1) / args.steps
    per_stage = timer.totals(args.steps)

    # the same chain with the two passes as separate launches, for comparison
    two_pass = None
    if fused:
        timer2 = StageTimer(torch, stage_names(False))
        for _ in range(args.chain_warmup):
            step(single=False)
        torch.cuda.synchronize()
        e2 = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e2[0].record()
        for _ in range(args.steps):
            step(timer2, single=False)
        e2[1].record()
        torch.cuda.synchronize()
        two_pass = {"ms_per_step": e2[0].elapsed_time(e2[1]) / args.steps, "stages_ms": timer2.totals(args.steps)}
        step()
        torch.cuda.synchronize()

    # decode alone, rotating over >= 1 GB of distinct packed caches
    cache_bytes = cache.nbytes()
    dec = None
    if args.decode_rotation_gb > 0:
        n_rot = max(2, int(args.decode_rotation_gb * 1e9 / cache_bytes) + 1)
        g = torch.Generator(device=dev).manual_seed(77)
        rot = []
        for i in range(n_rot):
            perm = torch.rand((B, Hkv, T), generator=g, device=dev).argsort(-1)[..., :n_keep]
            ridx = torch.sort(perm, -1).values.to(torch.int32).contiguous()
            rot.append(mk.quant_pack(k, v, ridx))
        torch.cuda.synchronize()
        dec_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for c in rot[:2]:
            mk.decode_attn(qdec, c, out=out, ws=ws)
        reps = 3
        dec_ev[0].record()
        for _ in range(reps):
            for c in rot:
                mk.decode_attn(qdec, c, out=out, ws=ws)
        dec_ev[1].record()
        torch.cuda.synchronize()
        dec_ms = dec_ev[0].elapsed_time(dec_ev[1]) / (reps * n_rot)
        # the same calls replayed as one HIP graph: no host work between the launches,
        # so the figure is the GPU's (the eager loop above is bound by the host's calls)
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for c in rot:
                mk.decode_attn(qdec, c, out=out, ws=ws)
        torch.cuda.current_stream().wait_stream(side)
        with torch.cuda.graph(graph):
            for c in rot:
                mk.decode_attn(qdec, c, out=out, ws=ws)
        graph.replay()
        torch.cuda.synchronize()
        dec_ev[0].record()
        for _ in range(reps):
            graph.replay()
        dec_ev[1].record()
        torch.cuda.synchronize()
        dec_gms = dec_ev[0].elapsed_time(dec_ev[1]) / (reps * n_rot)
        del graph
        dec_bytes = cache_bytes + 2 * B * Hq * D * 2
        dec_gbs = dec_bytes / (dec_ms * 1e-3) / 1e9
        dec_ggbs = dec_bytes / (dec_gms * 1e-3) / 1e9
        dec = {"workload": "llama7b_decode", "tokens_per_s": B / (dec_ms * 1e-3), "ms": dec_ms, "bytes": dec_bytes,
               "achieved_GBs": dec_gbs, "hbm_frac": dec_gbs / PEAK_HBM_GBS,
               "graph_ms": dec_gms, "graph_tokens_per_s": B / (dec_gms * 1e-3), "graph_achieved_GBs": dec_ggbs,
               "graph_hbm_frac": dec_ggbs / PEAK_HBM_GBS, "rotated_caches": n_rot,
               "rotation_bytes": n_rot * cache_bytes}
        del rot

    if args.calibrate_copy_mb and not args.headline_only:
        calibration_copy(torch, args.calibrate_copy_mb)

    # roofline of the prefill kernel (bf16 / fp16 MFMA-bound)
    flops = 2.0 * D * T * (T + 1) * Hq * B   # causal pairs only: QK^T and PV
    if fused:  # plus the window rows' QK^T of the score pass (causal pairs)
        flops += 2.0 * D * (W * T - W * (W - 1) / 2) * Hq * B
    k1_ms = per_stage["prefill_attn_scores" if fused else "prefill_attn"]
    tflops = flops / (k1_ms * 1e-3) / 1e12
    prefill_roof = {"bound": "mfma", "kernel": "fa_fwd_kernel (pass 1" + (" with the window scores)" if fused else ")"),
                    "achieved": tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": tflops / PEAK_BF16_TFLOPS,
                    "traffic": load_traffic(os.path.join(ROOT, "profiles", "fa_fwd_llama7b_hbm_traffic.md"),
                                            os.path.join(ROOT, "bit_quantized_kv_quant_amd", "csrc", "prefill.hip")),
                    "flops_per_launch": flops, "launch_ms": k1_ms}
    res = {"workload": "llama7b_decode chain: prefill + window scores + select + 2-bit pack + decode",
           "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D, "context": T, "window": W,
           "n_keep": n_keep, "n_heavy": n_heavy, "n_recent": n_recent, "steps": args.steps,
           "warmup": args.chain_warmup, "ms_per_step": ms_per_step,
           "prompt_tokens_per_s": B * (T + 1) / (ms_per_step * 1e-3),
           "output_tokens_per_s": B / (ms_per_step * 1e-3), "stages_ms": per_stage,
           "single_pass_scores": fused, "two_pass_chain": two_pass}
    del q, k, v, qdec, o, lse, scores, idx, cache, out, ws
    torch.cuda.empty_cache()
    return res, prefill_roof, dec


def variants(torch, mk, synth):
    """The comparison tables' cache policies on the chain's prompt and on a
    heavy-hitter prompt of the same shape (32-layer plans)."""
    dev = torch.device("cuda:0")
    wl = synth.WORKLOADS["llama7b_decode"]
    q, k, v, _ = synth.make_qkv(wl, dev)
    qdec = synth.make_decode_q(wl, dev)
    res = {"iid": variants_compare(
        torch, mk, q, k, v, qdec, 32, "llama7b_decode prompt (iid Gaussian, outlier key channels), "
        "one decode query per sequence")}
    del q, k, v, qdec
    qh, kh, vh, qdh = synth.make_heavy_qkv(wl, dev)
    res["heavy_hitters"] = variants_compare(
        torch, mk, qh, kh, vh, qdh, 32, "llama7b_decode shape, 5 % of keys and every query share a "
        "direction (strength 7): attention concentrated on heavy hitters")
    del qh, kh, vh, qdh
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path shards per "
              "(sequence, KV head) with no exchange between GPUs, and only the single-GPU case is timed here.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from bit_quantized_kv_quant_amd import build as _build

    _build.ensure_built()  # only when nothing is built
    import bit_quantized_kv_quant_amd as mk
    import synth

    print(f"# libminikv build {mk.build_id()} ({mk.lib_path()})", file=sys.stderr, flush=True)
    if args.only == "prefill_16k":
        print(json.dumps({"prefill_16k": prefill_layer(torch, mk, synth, synth.WORKLOADS["prefill_16k"],
                                                       reps=args.steps)}), flush=True)
        return
    if args.only == "chain":
        ch, roof, dec = chain(torch, mk, synth, args)
        print(json.dumps({"chain": ch, "prefill_roofline": roof, "decode": dec}), flush=True)
        return
    if args.only == "decode_gqa":
        gw = synth.WORKLOADS["mistral_44k"]
        budgets = [mk.keep_count(gw.T, gw.budget_pct)] * gw.layers
        print(json.dumps({"decode_gqa": decode_layers(torch, mk, synth, gw, gw.B, budgets, reps=args.steps,
                                                      n_queries=args.steps)}), flush=True)
        return
    if args.only == "decode_stream":
        gw = synth.WORKLOADS["mistral_44k"]
        print(json.dumps({"decode_stream": decode_stream(torch, mk, synth, gw, args.steps)}), flush=True)
        return

    # reference rates of this GPU (before anything else holds device memory)
    peaks = None if args.headline_only else measured_peaks(torch, mk)
    if peaks:
        print(f"# measured peaks: {json.dumps(peaks)}", file=sys.stderr, flush=True)

    # ---- headline: 40-layer pyramid decode at the ~250 GB batch ----
    head, sample = pyramid_headline(torch, mk, synth, args.pyramid_batch, args.steps, args.warmup,
                                    sample_seqs=0 if args.no_cpu_baseline else 4)
    print(f"# headline: {json.dumps(head)}", file=sys.stderr, flush=True)
    traffic = load_traffic(os.path.join(ROOT, "profiles", "decode_pyramid_hbm_traffic.md"),
                           os.path.join(ROOT, "bit_quantized_kv_quant_amd", "csrc", "decode.hip"))
    achieved = head["bytes_per_launch_avg"] / (head["launch_ms_avg"] * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e2m1 x e4m3 MFMA on 2-bit codes, fp32 softmax; bf16 q / out",
        "data": "synthetic",
        "config": {"workload": "llama13b_pyramid decode: 40 layers x 40 heads, head dim 128, context 8192, "
                               "budget 30 % -> 5 % (2457 -> 409 kept tokens), one query per sequence per step",
                   "batch": head["batch"], "packed_GB": head["packed_GB"], "layers": head["layers"],
                   "q_heads": head["q_heads"], "kv_heads": head["kv_heads"], "head_dim": head["head_dim"],
                   "context": head["context"], "parallelism": "single GPU"},
        "achieved_GBs": head["achieved_GBs"],
        "hbm_frac": head["hbm_frac"],
        "roofline": {"bound": "hbm", "kernel": "decode_partial_kernel<128, 1> (one launch per layer)",
                     "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": traffic, "bytes_per_launch": head["bytes_per_launch_avg"],
                     "launch_ms": head["launch_ms_avg"]},
        "decode_pyramid": head,
    }
    if args.headline_only:
        if args.calibrate_copy_mb:
            calibration_copy(torch, args.calibrate_copy_mb)
        if sample is not None:
            res["cpu_baseline"] = cpu_baseline_pyramid(sample)
        print(json.dumps(res), flush=True)
        return
    res["chain"], res["prefill_roofline"], res["decode"] = chain(torch, mk, synth, args)
    print(f"# chain: {json.dumps(res['chain'])}", file=sys.stderr, flush=True)
    if args.pyramid_sweep:
        pw = synth.WORKLOADS["llama13b_pyramid"]
        budgets = [mk.pyramid_keep(pw.T, pw.layers, l, *pw.pyramid) for l in range(pw.layers)]
        sweep = []
        for bs in (int(x) for x in args.pyramid_sweep.split(",") if x.strip()):
            r = decode_layers(torch, mk, synth, pw, bs, budgets, reps=20 if bs <= 256 else 3)
            sweep.append(r)
            print(f"# pyramid sweep B={bs}: {json.dumps(r)}", file=sys.stderr, flush=True)
        best = max(sweep, key=lambda r: r["tokens_per_s"])
        res["decode_pyramid_sweep"] = {"points": sweep, "max_tokens_per_s": best["tokens_per_s"],
                                       "at_batch": best["batch"]}
    if not args.no_gqa_sweep:
        gw = synth.WORKLOADS["mistral_44k"]
        budgets = [mk.keep_count(gw.T, gw.budget_pct)] * gw.layers
        res["decode_gqa"] = decode_layers(torch, mk, synth, gw, gw.B, budgets, reps=gw.decode_steps,
                                          n_queries=gw.decode_steps)
        print(f"# gqa decode: {json.dumps(res['decode_gqa'])}", file=sys.stderr, flush=True)
        res["decode_stream"] = decode_stream(torch, mk, synth, gw, gw.decode_steps)
        print(f"# streaming decode: {json.dumps(res['decode_stream'])}", file=sys.stderr, flush=True)
    if not args.no_prefill_sweep:
        res["prefill_16k"] = prefill_layer(torch, mk, synth, synth.WORKLOADS["prefill_16k"], reps=10)
        print(f"# prefill 16k: {json.dumps(res['prefill_16k'])}", file=sys.stderr, flush=True)
        res["prefill_gqa_44k"] = prefill_layer(torch, mk, synth, synth.WORKLOADS["mistral_44k"], reps=3, warm=2)
        print(f"# prefill gqa 44k (one layer): {json.dumps(res['prefill_gqa_44k'])}", file=sys.stderr, flush=True)
    if not args.no_variants:
        res["variants"] = variants(torch, mk, synth)
        print(f"# variants: {json.dumps(res['variants'])}", file=sys.stderr, flush=True)
    if peaks:
        # the headline decode and the chain's prefill against the measured rates
        peaks["decode_frac_of_read"] = achieved / peaks["hbm_read_GBs"]
        peaks["prefill_frac_of_gemm"] = res["prefill_roofline"]["achieved"] / peaks["bf16_gemm_TFLOPs"]
        res["measured_peaks"] = peaks
    if sample is not None:
        res["cpu_baseline"] = cpu_baseline_pyramid(sample)
        res["chain"]["cpu_baseline"] = cpu_baseline(synth.WORKLOADS["llama7b_decode"])
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
