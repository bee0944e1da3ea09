"""Exhaustive CPU checks of the library's short forms of the row-scale
arithmetic (value-axis scale grouping, abstract of "Quantizing Recurrent
Language Models Is Easier Than You Think": one scale per row, max / Q).

The step kernels do not divide by Q.  They use three instructions instead:
    q0 = m * fl(1/Q);  r = fma(-q0, Q, m);  scale = fma(r, fl(1/Q), q0)
and claim the result equals the IEEE quotient fl(m / Q) for every
non-negative float m, for Q = 127 and Q = 7.  For the rounding inverse they
take the nearest fl(Q / m) and step it down once when the exact residual
fma(-i, m, Q) is negative, claiming the result is the largest float f with
f * m <= Q.

The inverse is not formed from the IEEE quotient any more: the kernels take
v_rcp_f32 (within one ulp of 1/m), one Newton correction q0 = Q r,
qf = fma(fma(-q0, m, Q), r, q0), and step qf down once when its residual is
negative; they claim the result is that same largest float for every m in
[Q 2^-126, 2^126] whatever the reciprocal's rounding, so the check takes r as
each of the three floats nearest 1/m.  The overflow test becomes one compare,
m > Q 2^(SRB-128), claimed equal to "the nearest Q / m times 2^SRB is
finite" for every non-negative float and SRB in {0, 8, 16}.

All claims are checked here for every non-negative finite float (2^31 bit
patterns per Q), in C built with gcc: fmaf and the basic operations are
IEEE on both the host and gfx950 (the kernels are compiled without
fast-math, with denormals kept), so the host computes exactly what the
kernel does.  Maximality of the inverse is checked with exact products in
double (a 24 x 24-bit product fits in 53 bits).
"""
import os
import shutil
import subprocess
import tempfile

import pytest

PROG = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* the kernels' short forms, restated */
static float div_short(float m, float Q) {
  const float RQ = 1.0f / Q;
  const float q0 = m * RQ;
  const float r = fmaf(-q0, Q, m);
  return fmaf(r, RQ, q0);
}
static float inv_short(float Q, float m) {
  const float i = Q / m;
  return fmaf(-i, m, Q) < 0.0f ? nextafterf(i, 0.0f) : i;
}

/* the estimate path: reciprocal r, one Newton correction, one step down */
static float inv_rcp(float Q, float m, float r) {
  const float q0 = Q * r;
  const float qf = fmaf(fmaf(-q0, m, Q), r, q0);
  return fmaf(-qf, m, Q) < 0.0f ? nextafterf(qf, 0.0f) : qf;
}
/* f is the largest float with f m <= Q: f m <= Q < next(f) m, exact in double */
static int is_rtz_inverse(float f, float m, float Q) {
  const float up = nextafterf(f, INFINITY);
  return (double)f * (double)m <= (double)Q && (double)up * (double)m > (double)Q;
}

int main(void) {
  const float Qs[2] = {127.0f, 7.0f};
  const uint32_t Qbits[2] = {0x42FE0000u, 0x40E00000u};
  const int srbs[3] = {0, 8, 16};
  long long bad_div = 0, bad_inv = 0, checked_inv = 0, bad_rcp = 0, checked_rcp = 0, bad_lim = 0;
  for (int qi = 0; qi < 2; ++qi) {
    const float Q = Qs[qi];
    const float lo = Q * 0x1p-126f, hi = 0x1p126f;
    float lim[3];
    for (int s = 0; s < 3; ++s) lim[s] = f_of(Qbits[qi] - ((uint32_t)(128 - srbs[s]) << 23));
#pragma omp parallel for reduction(+ : bad_div, bad_inv, checked_inv, bad_rcp, checked_rcp, bad_lim) schedule(static, 1 << 16)
    for (long long b = 0; b < 0x7F800000LL; ++b) {
      const float m = f_of((uint32_t)b);
      float want = m / Q, got = div_short(m, Q);
      if (memcmp(&want, &got, 4) != 0) ++bad_div;
      if (m > 0.0f && isfinite(Q / m)) {
        ++checked_inv;
        if (!is_rtz_inverse(inv_short(Q, m), m, Q)) ++bad_inv;
      }
      for (int s = 0; s < 3; ++s) {
        const float i = Q / m;
        const int fin = m > 0.0f && isfinite(i) && isfinite(i * ldexpf(1.0f, srbs[s]));
        if (fin != (m > lim[s])) ++bad_lim;
      }
      if (m >= lo && m <= hi) {
        const float rn = 1.0f / m;
        const float rs[3] = {nextafterf(rn, 0.0f), rn, nextafterf(rn, INFINITY)};
        for (int c = 0; c < 3; ++c) {
          ++checked_rcp;
          if (!is_rtz_inverse(inv_rcp(Q, m, rs[c]), m, Q)) ++bad_rcp;
        }
      }
    }
  }
  printf("%lld %lld %lld %lld %lld %lld\n", bad_div, bad_inv, checked_inv, bad_rcp, checked_rcp, bad_lim);
  return 0;
}
"""


@pytest.fixture(scope="module")
def results():
    gcc = shutil.which("gcc")
    if not gcc:
        pytest.skip("gcc not available")
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "scale.c"), os.path.join(d, "scale")
        with open(src, "w") as f:
            f.write(PROG)
        flags = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp"]
        cpu = open("/proc/cpuinfo").read() if os.path.exists("/proc/cpuinfo") else ""
        if " fma " in cpu:
            flags.append("-mfma")   # hardware fused multiply-add (fmaf is exact either way)
        subprocess.run([gcc, *flags, src, "-o", exe, "-lm"], check=True, capture_output=True)
        env = dict(os.environ, OMP_NUM_THREADS=str(min(16, os.cpu_count() or 1)))
        out = subprocess.run([exe], check=True, capture_output=True, text=True, env=env, timeout=900).stdout
    return [int(x) for x in out.split()]


def test_scale_short_form_equals_ieee_quotient_for_every_float(results):
    assert results[0] == 0


def test_inverse_is_largest_float_not_above_quotient_for_every_float(results):
    assert results[1] == 0
    assert results[2] > 2 * 2_000_000_000   # every positive float with a finite Q / m, both Q


def test_inverse_from_reciprocal_estimate_is_exact_for_every_float_in_range(results):
    assert results[3] == 0
    assert results[4] > 3 * 2 * 2_000_000_000   # three reciprocals, both Q, every m in [Q 2^-126, 2^126]


def test_overflow_limit_compare_equals_finite_inverse_for_every_float(results):
    assert results[5] == 0
