"""The quantiser's divide-free fl32(r / 3) (quant_pack.hip, div3) equals the IEEE
quotient for every finite fp32 r >= 0.

The kernel computes q0 = fl(r * c) with c = fl32(1/3), then one fma correction
q1 = fma(fma(-3, q0, r), c, q0).  Both steps are plain IEEE single-precision
operations (round to nearest even, correctly rounded fma), so the identity is a
property of the arithmetic, checked here over all 2^31 - 2^23 inputs with the
host's fused multiply-add.  The range of a quantisation group is a difference
mx - mn >= +0 of finite values, so this covers every input the kernel sees
(+inf, reachable only from a range above the largest float, is special-cased
there).
"""
import os
import shutil
import subprocess
import tempfile

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
int main(void) {
    const float c = 1.0f / 3.0f;
    unsigned long long bad = 0;
    for (uint32_t u = 0; u < 0x7f800000u; ++u) {
        float r; memcpy(&r, &u, 4);
        volatile float vr = r;
        float want = vr / 3.0f;
        float q0 = vr * c;
        float q1 = fmaf(fmaf(-3.0f, q0, vr), c, q0);
        uint32_t a, b; memcpy(&a, &want, 4); memcpy(&b, &q1, 4);
        bad += a != b;
    }
    printf("%llu\n", bad);
    return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_div3_matches_ieee_quotient_for_every_nonnegative_float():
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "div3.c")
        exe = os.path.join(d, "div3")
        open(c, "w").write(SRC)
        # -mfma: fmaf is the correctly rounded hardware fma; no contraction elsewhere
        subprocess.run(["gcc", "-O2", "-mfma", "-ffp-contract=off", c, "-o", exe, "-lm"], check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout.strip()
    assert out == "0", f"{out} mismatches"
