"""Host-side parts of bench.py (no GPU): the one-GPU rule and the committed
traffic figure's staleness check."""

import hashlib
import os
import shutil
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_figure_follows_the_kernel_source(tmp_path):
    profile = os.path.join(ROOT, "profiles", "fa_fwd_llama7b_hbm_traffic.md")
    src = os.path.join(ROOT, "bit_quantized_kv_quant_amd", "csrc", "prefill.hip")
    got = bench.load_traffic(profile, src)
    # a figure is returned exactly when the summary records this source's hash
    recorded = [ln.split("`")[1] for ln in open(profile) if ln.startswith("- kernel_source_sha256_16:")]
    want = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    assert recorded and (got is not None) == (recorded[0] == want)
    if got is not None:
        assert got > 0
    # any edit of the source makes the figure stale
    edited = tmp_path / "prefill.hip"
    shutil.copy(src, edited)
    with open(edited, "a") as f:
        f.write("\n// edited\n")
    assert bench.load_traffic(profile, str(edited)) is None
    assert bench.load_traffic(str(tmp_path / "missing.md"), src) is None
