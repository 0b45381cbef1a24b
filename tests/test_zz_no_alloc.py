"""The allocation-free decode entry point (library-owned scratch array) against
minikv_decode_attn with a caller workspace: two calls in a row, the second on
a smaller input, each bit-identical to the existing entry point's output (the
same kernels) and within max(2e-3, 1 bf16 ulp) of the fp64 oracle."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
import bit_quantized_kv_quant_amd as mk
from bit_quantized_kv_quant_amd import _lib
from gpu_util import assert_attn_close, packed_to_np, require_gpu, to_np

pytestmark = pytest.mark.gpu


def _case(dev, B, Hq, Hkv, n, D, seed):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, Hkv, n, D)).astype(np.float32) * 3
    k[..., :4] *= 8
    v = rng.standard_normal((B, Hkv, n, D)).astype(np.float32)
    q = synth.bf16_round(rng.standard_normal((B, Hq, D)).astype(np.float32))
    cache = mk.quant_pack(torch.from_numpy(k).to(dev).to(torch.bfloat16),
                          torch.from_numpy(v).to(dev).to(torch.bfloat16))
    return torch.from_numpy(q).to(dev).to(torch.bfloat16), cache


def _noalloc(q, cache):
    out = torch.full_like(q, float("nan"))
    s = cache.struct()
    st = _lib.lib().minikv_decode_attn_noalloc(ctypes.c_void_p(q.data_ptr()), ctypes.byref(s), q.shape[1],
                                               0.0, ctypes.c_void_p(out.data_ptr()),
                                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    _lib.check("minikv_decode_attn_noalloc", st)
    return out


def test_noalloc_decode_matches_workspace_entry_point():
    dev = require_gpu()
    # a split plan (52 token ranges per KV head, merged by the merge kernel)
    # and a smaller one right after it (16 ranges: two 8-wave workgroups per
    # head, handed over by a ticket), then 24 ranges (three workgroups, which
    # take the tickets the previous call left zero again), one workgroup per
    # head, and a plan with one range per KV head, which uses no scratch
    cases = [(4, 32, 8, 6600, 128, 1), (2, 8, 2, 1300, 64, 2), (1, 4, 4, 2900, 128, 5), (2, 4, 4, 301, 128, 3),
             (64, 64, 64, 200, 128, 4)]
    for B, Hq, Hkv, n, D, seed in cases:
        print("noalloc decode B", B, "Hq", Hq, "Hkv", Hkv, "n", n, "D", D, flush=True)
        q, cache = _case(dev, B, Hq, Hkv, n, D, seed)
        a = _noalloc(q, cache)
        b = mk.decode_attn(q, cache)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "differs from minikv_decode_attn"
        assert_attn_close(to_np(a), oracle.decode_ref(to_np(q), packed_to_np(cache)), "noalloc decode")
