"""Plain, slow CPU oracle for the MiniKV 2-bit layer-discriminative KV-cache hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(the HIP library and its Python binding) never imports, links or calls it, and
this package imports nothing from the product path.

Every function is numpy: fp64 for attention and score arithmetic, IEEE fp32
(correctly rounded, round-half-even) where the packed cache must come out
bit-exact, and numpy's IEEE fp16 cast (round-half-even, subnormals kept) for the
stored scale / zero.

Pages the functions follow (cited by page and section):

* "MiniKV: Pushing the Limits of LLM Inference via 2-Bit Layer-Discriminative KV
  Cache", paper-listing page, abstract: 2-bit layer-discriminative KV cache,
  kernels that keep the cache usable by FlashAttention.
* gptget.net summary of arXiv 2411.18077, sections 方法论 (methodology) and
  方法详解 (method details): 2-bit quantisation with an adaptive KV policy,
  per-channel ("sub-channel") key quantisation, per-token value quantisation,
  a compact cache layout, selective flash attention built from a second kernel.
* same summary, 术语表 (glossary), "adaptive KV": keep the KV states chosen by
  importance.
* notesum.ai page for arXiv 2411.18077v1, LongBench table: the "MiniKV Pyramid"
  rows (a per-layer budget).

Where the pages leave a step open, the reading taken is stated in the function's
docstring.  Parity status: every function here is pinned by a CPU test against a
closed form, an invariant, a special case or brute force; the pages' headline
figures (86 % compression, 98.5 % accuracy, +48 % throughput) are context and
parity unpinned.
"""

from .minikv_ref import (  # noqa: F401
    GROUP,
    keep_count,
    pyramid_keep,
    split_heavy_recent,
    prefill_ref,
    window_scores_ref,
    select_ref,
    index_near_ties,
    group_min_max,
    quant_group_ref,
    quant_pack_ref,
    code_near_ties,
    code_parity,
    pack_codes_ref,
    unpack_codes_ref,
    pack_value_codes_ref,
    unpack_value_codes_ref,
    sz_words_ref,
    dequant_ref,
    decode_ref,
    attn_tolerance,
    stream_split_ref,
    concat_packed_ref,
    stream_init_ref,
    stream_append_ref,
    stream_decode_ref,
    packed_bytes_ref,
    compression_ratio_ref,
)
