"""The quantiser's code decision (quant_pack.hip, code_of) equals the rule's IEEE
evaluation for every positive fp16 scale.

With d = fl32(x - z) and an fp16 scale s > 0 the rule is
code = clamp(rint(fl32(d / s)), 0, 3), round-half-even throughout.  The kernel
decides it without dividing, as (d > s/2) + (d >= 3s/2) + (d > 5s/2), where the
three products are exact in fp32.  Why it holds: rint(u) >= 1 exactly when
fl32(d / s) > 1/2, that is when d / s lies above the rounding midpoint
1/2 + 2^-25; that bound sits less than one fp32 ulp above s/2 (s has 11
significant bits), so the first fp32 value past it is the one right after s/2.
The other two thresholds work the same way: the midpoint below 3/2 (ties go to
3/2) and the one above 5/2 (ties go to 5/2) each lie less than an ulp from 3s/2
and 5s/2.  Checked here for every positive fp16 s (subnormals included), at
every fp32 d within 16 ulps of each threshold and at a spread of d from -s to
6s, against correctly rounded host division and nearbyintf.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

SRC = r"""
#include <fenv.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float half_to_float(uint16_t h) {   /* exact: fp16 -> fp32 */
    int e = (h >> 10) & 31, m = h & 1023;
    float v = e ? ldexpf((float)(1024 + m), e - 25) : ldexpf((float)m, -24);
    return (h & 0x8000) ? -v : v;
}
static unsigned ref_code(float d, float s) {  /* the rule, evaluated as written */
    volatile float q = d / s;
    float r = nearbyintf(q);
    return r <= 0.0f ? 0u : (r >= 3.0f ? 3u : (unsigned)r);
}
static unsigned fast_code(float d, float s) {  /* the kernel's divide-free decision */
    volatile float h1 = 0.5f * s, h2 = 1.5f * s, h3 = 2.5f * s;
    return (unsigned)(d > h1) + (unsigned)(d >= h2) + (unsigned)(d > h3);
}
int main(void) {
    fesetround(FE_TONEAREST);
    unsigned long long bad = 0, n = 0;
    for (uint32_t h = 1; h < 0x7C00u; ++h) {     /* every positive finite fp16 */
        const float s = half_to_float((uint16_t)h);
        const float th[3] = {0.5f * s, 1.5f * s, 2.5f * s};
        for (int m = 0; m < 3; ++m) {
            float d = th[m];
            for (int k = 0; k < 16; ++k) d = nextafterf(d, -INFINITY);
            for (int k = 0; k < 33; ++k, d = nextafterf(d, INFINITY)) {
                bad += ref_code(d, s) != fast_code(d, s);
                ++n;
            }
        }
        for (int k = -64; k <= 384; ++k) {       /* a spread of d over [-s, 6s] */
            const float d = (float)k / 64.0f * s;
            bad += ref_code(d, s) != fast_code(d, s);
            ++n;
        }
    }
    printf("%llu %llu\n", bad, n);
    return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_code_thresholds_match_ieee_rule_for_every_fp16_scale():
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "codes.c")
        exe = os.path.join(d, "codes")
        open(c, "w").write(SRC)
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-frounding-math", c, "-o", exe, "-lm"], check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout.split()
    bad, n = int(out[0]), int(out[1])
    assert n > 3_000_000
    assert bad == 0, f"{bad} of {n} decisions differ"
