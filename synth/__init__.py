"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and bench.py.

This module holds workload shapes and random draws only: none of the method's
arithmetic (no attention, selection, budgets or quantisation) lives here, so the
oracle and the HIP path stay independent of each other.

The pages measure on LongBench (notesum.ai page for arXiv 2411.18077v1, LongBench
table; gptget.net summary, 关键结果: prompts up to 44K tokens).  Those items are
not used; seeded Gaussian K/V with outlier key channels, at the attention shapes
of LLaMA2-7B, LLaMA2-13B and Mistral-7B, stand in for them.
"""

from .workloads import (  # noqa: F401
    Workload,
    WORKLOADS,
    tiny_inputs,
    torch_generator,
    make_qkv,
    make_heavy_qkv,
    make_decode_q,
    make_kept_kv,
    outlier_channels,
    bf16_round,
)
