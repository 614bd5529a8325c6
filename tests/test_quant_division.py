"""The divisions the in-kernel activation quantiser replaces, checked on the
CPU for every input they can see.  CPU only (gcc).

For a group with amax >= 2^-55 the kernel issues no division:

    s  = fma(fma(-s0, 448, amax), C, s0)   with s0 = RN(amax * C), C = RN(1/448)
    y  = fma(fma(-s, y0, 1), y0, y0)       y0 = the hardware reciprocal of s
    q  = fma(fma(-q0, s, x), y, q0)        with q0 = RN(x * y)

(the last is the correction step of Markstein's division for a correctly
rounded reciprocal).  The codes are decided by the float32 quotient, so q must
be the correctly rounded x / s wherever that can move an e4m3fn code: every
e4m3fn rounding boundary is at least 2^-10.  x and amax are bf16, so the whole
input space is small: every positive finite bf16 amax (s must equal
RN(amax / 448)), both float neighbours of 1 / s as y0 (the hardware
reciprocal is within one ulp; y must equal RN(1 / s)), and every positive
finite bf16 x <= amax, about 4.9e8 pairs (negative values mirror positive
ones under round to nearest even).  The quotient step is also checked with y
one ulp off either way, so it does not lean on the Newton step alone.
"""
import os
import shutil
import subprocess

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static float bf(uint32_t h) { uint32_t b = h << 16; float v; memcpy(&v, &b, 4); return v; }
static uint32_t bits(float v) { uint32_t b; memcpy(&b, &v, 4); return b; }
int main(void) {
  long long pairs = 0, differ = 0, differ_visible = 0, s_bad = 0, y_bad = 0, off_visible = 0;
  float worst = 0.0f;
  const float C = 1.0f / 448.0f;
  for (int ab = 1; ab < 0x7F80; ++ab) {
    const float amax = bf(ab), want = amax / 448.0f;
    if (amax < 0x1p-55f) continue;
    const float s0 = amax * C, s = fmaf(fmaf(-s0, 448.0f, amax), C, s0);
    if (bits(s) != bits(want)) ++s_bad;
    const float rn = 1.0f / want, y0s[2] = {nextafterf(rn, 0.0f), nextafterf(rn, INFINITY)};
    for (int i = 0; i < 2; ++i) {
      const float y0 = y0s[i], y = fmaf(fmaf(-want, y0, 1.0f), y0, y0);
      if (bits(y) != bits(rn)) ++y_bad;
    }
  }
#pragma omp parallel for schedule(dynamic, 64) reduction(+:off_visible)
  for (int ab = 1; ab < 0x7F80; ++ab) {
    const float amax = bf(ab), s = amax / 448.0f;
    if (amax < 0x1p-55f) continue;
    const float rn = 1.0f / s, ys[2] = {nextafterf(rn, 0.0f), nextafterf(rn, INFINITY)};
    for (int i = 0; i < 2; ++i)
      for (int xb = 1; xb <= ab; ++xb) {
        const float x = bf(xb), want = x / s, q0 = x * ys[i], q = fmaf(fmaf(-q0, s, x), ys[i], q0);
        if (bits(q) != bits(want) && (want >= 0x1p-11f || q >= 0x1p-11f)) ++off_visible;
      }
  }
#pragma omp parallel for schedule(dynamic, 64) reduction(+:pairs, differ, differ_visible) reduction(max:worst)
  for (int ab = 1; ab < 0x7F80; ++ab) {
    const float amax = bf(ab), s = amax / 448.0f;
    if (amax < 0x1p-55f) continue;
    const float y = 1.0f / s;
    for (int xb = 1; xb <= ab; ++xb) {
      const float x = bf(xb), want = x / s;
      const float q0 = x * y, q = fmaf(fmaf(-q0, s, x), y, q0);
      ++pairs;
      if (bits(q) != bits(want)) {
        ++differ;
        if (want > worst) worst = want;
        if (want >= 0x1p-11f || q >= 0x1p-11f) ++differ_visible;
      }
    }
  }
  printf("%lld %lld %lld %a %lld %lld %lld\n", pairs, differ, differ_visible, worst, s_bad, y_bad, off_visible);
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_reciprocal_division_matches_ieee_on_every_bf16_pair(tmp_path):
    c = tmp_path / "div.c"
    c.write_text(SRC)
    exe = tmp_path / "div"
    # -ffp-contract=off: the C must do exactly the roundings written above
    subprocess.run(["gcc", "-O2", "-mfma", "-ffp-contract=off", "-fopenmp", str(c), "-o", str(exe), "-lm"],
                   check=True)
    env = dict(os.environ, OMP_NUM_THREADS=str(min(8, os.cpu_count() or 1)))
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True, env=env, timeout=600).stdout
    pairs, differ, visible, worst, s_bad, y_bad, off_visible = out.split()
    assert int(pairs) > 4.8e8
    assert int(s_bad) == 0 and int(y_bad) == 0 and int(off_visible) == 0
    # no difference where a code could see it; the rest are far below the
    # smallest e4m3fn boundary (underflowing remainders of tiny quotients)
    assert int(visible) == 0
    assert float.fromhex(worst) < 2.0 ** -40
