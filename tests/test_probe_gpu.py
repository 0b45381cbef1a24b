"""GPU check of the streaming-read probe (a measurement aid, not a step of the method):
every 32-bit word of the buffer is read, so the XOR of the sink equals the XOR of the buffer's
words, for sizes below, at and past the probe's unrolled grid-stride round (64 MiB)."""

import numpy as np
import pytest
import torch

import bit_quantized_kv_quant_amd as mk
from gpu_util import require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, (8 << 20) - 16, (64 << 20) + 48, (160 << 20) + 4080])
def test_read_probe_reads_every_word(nbytes):
    dev = require_gpu()
    print("read probe bytes", nbytes, flush=True)
    rng = np.random.default_rng(nbytes % 1000003)
    words = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    x = torch.from_numpy(words.view(np.int32)).to(dev)
    sink = mk.read_probe(x)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)
