"""MI355X (gfx950) library for attention over a 2-bit, layer-discriminative KV cache.

The hot path - selective flash attention with per-key window scores,
heavy-hitter + recent selection, 2-bit quantise-and-pack, and decode attention
over the packed cache - runs in the HIP kernels of libminikv.so (C ABI in
include/minikv.h).  This package is the thin Python binding.
"""

from ._lib import MinikvError, build_id, lib, lib_path, status_string  # noqa: F401
from .api import (  # noqa: F401
    PackedCache,
    StreamCache,
    decode_attn,
    decode_ws_bytes,
    keep_count,
    packed_bytes,
    prefill_attn,
    prefill_attn_scores,
    prefill_fuses_scores,
    window_scores,
    pyramid_keep,
    quant_pack,
    read_probe,
    select_topk,
    select_ws_bytes,
    split_heavy_recent,
)
from .variants import POLICIES, Policy, compress, layer_plan  # noqa: F401
