"""Write tests/golden/tiny_oracle.npz: the oracle's outputs on the tiny workload.

Calls only oracle/ and the seeded generator in synth/; a regression anchor for
the oracle itself (test_oracle_golden.py recomputes and compares).

    python tests/golden/make_tiny_golden.py
"""

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402


def compute():
    wl = synth.WORKLOADS["tiny"]
    d = synth.tiny_inputs(wl.seed)
    qb, kb, vb = (synth.bf16_round(d[n]) for n in ("q", "k", "v"))
    qdec = synth.bf16_round(d["q_dec"])
    scores = oracle.window_scores_ref(qb, kb, wl.window)
    idx = oracle.select_ref(scores, wl.n_heavy, wl.n_recent)
    packed = oracle.quant_pack_ref(d["k"], d["v"], idx)
    out = oracle.decode_ref(qdec, packed)
    rows = np.array([0, 1, 31, 32, 100, 239, 240, 255])
    o, lse = oracle.prefill_ref(qb, kb, vb, rows=rows)
    res = {"scores": scores, "idx": idx, "decode_out": out, "prefill_rows": rows,
           "prefill_o": o, "prefill_lse": lse}
    res.update({k: v for k, v in packed.items()})
    return res


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.npz")
    np.savez_compressed(path, **compute())
    print("wrote", path)
