"""Host checks of arithmetic shortcuts the GPU kernels take, each
claimed to give exactly the result of the plain formula:

* the QSGD decoder's step size d = fl(norm / 7) computed without a
  division, as one multiplication by fl(1/7) and one correction with the
  exact remainder (checked here over every fp32 bit pattern);
* the rowwise FP8 encoder's row scale fl(amax / 448), computed the same
  way for amax >= 2^-120 (checked over every such fp32 value);
* the QSGD encoder's ratio fl(|v| / d), d shared by the bucket, computed
  from r = fl(1/d) the same way inside the guard it states (checked over
  billions of pairs, densest where the ratio decides a level);
* the rowwise FP8 encoder's E4M3 code of fl(x / scale), computed from
  fl(x * r) with r within an ulp of 1/scale, except where that product lies
  within 8 ulps of an E4M3 rounding point or below 2^-6 (checked here on
  crafted quotients that straddle every rounding point, with r one ulp off
  either way, against the code of the true quotient), and with r computed
  exactly as the kernel computes it: one Newton step
  fma(fma(-sc, r0, 1), r0, r0) on a hardware reciprocal r0 that is fl(1/sc)
  or one of its neighbours (its documented accuracy), the two fmas
  evaluated in exact rational arithmetic and rounded once each.

Both are the formulas as the kernels write them, evaluated with IEEE fp32
arithmetic on the host (numpy float32; C fmaf)."""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

DIV7_C = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static float f(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }
static uint32_t b(float x) { uint32_t v; memcpy(&v, &x, 4); return v; }
int main(void) {
    const float r7 = 0x1.24924ap-3f;
    unsigned long long bad = 0;
    #pragma omp parallel for reduction(+:bad) schedule(static)
    for (long long i = 0; i < (1LL << 32); ++i) {
        const float a = f((uint32_t)i);
        const float want = a / 7.0f;
        const float q0 = a * r7;
        const float q1 = fmaf(fmaf(-7.0f, q0, a), r7, q0);
        const float got = (q0 == 0.0f || !isfinite(q0)) ? q0 : q1;
        if (isnan(want) ? !isnan(got) : b(got) != b(want)) ++bad;
    }
    printf("%llu\n", bad);
    return 0;
}
"""


DIV448_C = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static float f(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }
static uint32_t b(float x) { uint32_t v; memcpy(&v, &x, 4); return v; }
int main(void) {
    const float r448 = 0x1.24924ap-9f;
    unsigned long long bad = 0;
    #pragma omp parallel for reduction(+:bad) schedule(static)
    for (long long i = 0; i < (1LL << 32); ++i) {
        const float a = f((uint32_t)i);
        const float want = a / 448.0f;
        float got;
        if (!(a >= 0x1p-120f && a <= 0x1.fffffep127f)) {
            got = a / 448.0f;
        } else {
            const float q0 = a * r448;
            got = fmaf(fmaf(-448.0f, q0, a), r448, q0);
        }
        if (isnan(want) ? !isnan(got) : b(got) != b(want)) ++bad;
    }
    printf("%llu\n", bad);
    return 0;
}
"""


# fl(x / d) for x >= +0 and a divisor shared by a bucket (quot_fast in the
# kernels' device header): q0 = fl(x r), r = fl(1/d), then
# fl(q0 + fl(x - q0 d) r) with fmas, taken only when d and 1/d are normal,
# x is +0 or finite and at least 2^-102, and 2^-100 <= |q0| <= 2^126; else
# the kernel divides.  Checked
# here against x / d over a spread of divisors (significands at both ends
# of the binade, random ones, exponents at both limits of the guard) and,
# per divisor of either sign, every float x whose quotient is about 1 to 8
# (where QSGD's |v|/d decides a level above 0), every 16th one down to
# quotients of 2^-4, every 256th down to 2^-40, and every 4093rd over the
# rest of the range, x below 2^-102 included.
QUOT_C = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static float f(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }
static uint32_t b(float x) { uint32_t v; memcpy(&v, &x, 4); return v; }
static int dok(float d) { const float a = fabsf(d); return a >= 0x1p-126f && a <= 0x1p126f; }
static float quot(float x, float d, float r, int ok, int* fast) {
    const float q0 = x * r;
    const float rem = fmaf(-q0, d, x);
    const float aq = fabsf(q0);
    *fast = ok && (x == 0.0f || (x >= 0x1p-102f && x <= 0x1.fffffep127f && aq >= 0x1p-100f && aq <= 0x1p126f));
    return fmaf(rem, r, q0);
}
int main(void) {
    uint32_t ds[200];
    int nd = 0;
    uint64_t st = 0x9E3779B97F4A7C15ull;
    for (uint32_t m = 0; m < 24; ++m) ds[nd++] = 0x3F800000u + m;             /* 1 + small */
    for (uint32_t m = 0; m < 24; ++m) ds[nd++] = 0x3FFFFFFFu - m;             /* 2 - small */
    ds[nd++] = 0x00800000u; ds[nd++] = 0x00800001u; ds[nd++] = 0x00FFFFFFu;   /* 2^-126 .. */
    ds[nd++] = 0x7E800000u; ds[nd++] = 0x7E7FFFFFu; ds[nd++] = 0x7E800001u;   /* 2^126 .. */
    ds[nd++] = 0x3EDB6DB7u;                                                   /* ~ 3/7 */
    while (nd < 200) {
        st ^= st << 13; st ^= st >> 7; st ^= st << 17;
        ds[nd++] = 0x00800000u + (uint32_t)(st % (0x7F000000u - 0x00800000u));
    }
    unsigned long long bad = 0, fastn = 0;
    for (int t = 0; t < nd; ++t) {
        const float d = f(ds[t]);
        const int ok = dok(d);
        const float r = ok ? 1.0f / d : 0.0f;
        const long long ed = (ds[t] >> 23) & 0xFF;
        #pragma omp parallel for reduction(+:bad,fastn) schedule(dynamic)
        for (long long e = 0; e < 255; ++e) {
            const long long rel = e - ed;  /* quotient's binade, about */
            uint32_t step = 4093u;
            if (rel >= 0 && rel <= 3) step = 1u;
            else if (rel >= -4 && rel <= 3) step = 16u;
            else if (rel >= -40 && rel <= 3) step = 256u;
            for (uint32_t m = 0; m < (1u << 23); m += step) {
                for (int sg = 0; sg < 2; ++sg) {  /* d of either sign; x >= +0 */
                    const float x = f(((uint32_t)e << 23) | m);
                    const float dd = sg ? -d : d, rr = sg ? -r : r;
                    int fast;
                    const float got = quot(x, dd, rr, ok, &fast);
                    if (!fast) continue;
                    ++fastn;
                    const float want = x / dd;
                    if (b(got) != b(want)) ++bad;
                }
            }
        }
    }
    printf("%llu\n", bad);
    fprintf(stderr, "%llu\n", fastn);
    return 0;
}
"""


def run_c(src_text):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    d = tempfile.mkdtemp()
    try:
        src, exe = os.path.join(d, "t.c"), os.path.join(d, "t")
        with open(src, "w") as fh:
            fh.write(src_text)
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", src, "-o", exe, "-lm"], check=True,
                       capture_output=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True,
                             env={**os.environ, "OMP_NUM_THREADS": str(min(8, os.cpu_count() or 1))})
        return int(out.stdout.strip())
    finally:
        shutil.rmtree(d)


@pytest.mark.slow
def test_div448_every_float():
    """fl(1/448) is 0x1.24924ap-9; the corrected product is the correctly
    rounded amax/448 wherever the kernel uses it (amax in [2^-120, max])."""
    assert np.float32(1.0) / np.float32(448.0) == np.float32(float.fromhex("0x1.24924ap-9"))
    assert run_c(DIV448_C) == 0


@pytest.mark.slow
def test_shared_divisor_quotient_matches_division():
    """The corrected reciprocal product equals x / d bit for bit wherever
    the kernels' guard takes it."""
    assert run_c(QUOT_C) == 0


@pytest.mark.slow
def test_div7_every_float():
    """fl(1/7) is 0x1.24924ap-3 and the corrected product equals the
    correctly rounded a/7 for all 2^32 inputs (zeros, subnormals,
    infinities and NaN included)."""
    assert np.float32(1.0) / np.float32(7.0) == np.float32(float.fromhex("0x1.24924ap-3"))
    assert run_c(DIV7_C) == 0


def e4m3_midpoints():
    """Every point where round-to-nearest-even to E4M3 changes its result,
    for magnitudes in (0, 448): halfway between neighbouring codes."""
    vals = [m * 2.0 ** -9 for m in range(8)]  # subnormals
    for e in range(-6, 9):
        for m in range(8):
            v = (1 + m / 8) * 2.0 ** e
            if v <= 448:
                vals.append(v)
    vals = np.array(sorted(set(vals)))
    return (vals[:-1] + vals[1:]) / 2


def fast_code(ora, x, sc, r=None, window=8):
    """The kernel's path: q = fl(x * r), r ~ 1/sc; the division when q is
    below 2^-6 or its discarded bits are within `window` of the rounding
    point (or sc is subnormal)."""
    if r is None:
        r = np.float32(1.0) / sc
    q = (x * r).astype(np.float32)
    near = (q.view(np.uint32) - np.uint32(0x80000 - window)) & np.uint32(0xFFFFF)
    exact = (np.abs(q) < np.float32(2.0 ** -6)) | (near <= 2 * window) | (sc < np.float32(2.0 ** -126))
    y = np.where(exact, (x / sc).astype(np.float32), q).astype(np.float32)
    y = np.clip(y, np.float32(-448), np.float32(448))
    return ora.e4m3_from_f32_n(y), exact


def reciprocals(sc):
    """fl(1/sc) and its two neighbours: the kernel's reciprocal is within
    one ulp of the true 1/sc."""
    r = np.float32(1.0) / sc
    return [r, np.nextafter(r, np.float32(np.inf)), np.nextafter(r, np.float32(0))]


def test_fp8_reciprocal_path_matches_division(ora):
    rng = np.random.default_rng(11)
    mids = e4m3_midpoints()
    checked = fast_hits = 0
    for trial in range(200):
        # a row scale of any magnitude: amax / 448 for a random amax
        amax = np.float32(np.ldexp(rng.uniform(1, 2), int(rng.integers(-100, 100))))
        sc = np.float32(amax / np.float32(448))
        # values whose quotient is within +-24 ulps of each rounding point,
        # both signs, plus uniform values over the row's range
        t = (mids.astype(np.float64) * np.float64(sc)).astype(np.float32)
        k = rng.integers(-24, 25, t.size)
        x = np.nextafter(t, np.where(k >= 0, np.inf, -np.inf).astype(np.float32))
        for _ in range(3):
            step = np.abs(k) > _
            x = np.where(step, np.nextafter(x, np.where(k >= 0, np.inf, -np.inf).astype(np.float32)), x)
        x = np.concatenate([x, -x, rng.uniform(-1, 1, 4096).astype(np.float32) * amax, [amax, -amax]])
        x = x.astype(np.float32)
        want = ora.e4m3_from_f32_n(np.clip((x / sc).astype(np.float32), np.float32(-448), np.float32(448)))
        for r in reciprocals(sc):
            got, exact = fast_code(ora, x, sc, r)
            assert np.array_equal(got, want), trial
            checked += x.size
            fast_hits += int((~exact).sum())
    assert fast_hits > 0.8 * checked  # the shortcut is the common path


def test_fp8_reciprocal_path_differs_from_division_in_the_quotient(ora):
    """The shortcut is not an identity on fp32: the product and the
    quotient differ for many elements, only their codes agree."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal(1 << 16).astype(np.float32)
    sc = np.float32(np.float32(np.abs(x).max()) / np.float32(448))
    q = (x * (np.float32(1) / sc)).astype(np.float32)
    y = (x / sc).astype(np.float32)
    assert (q != y).sum() > 1000
    got, _ = fast_code(ora, x, sc)
    assert np.array_equal(got, ora.e4m3_from_f32_n(np.clip(y, np.float32(-448), np.float32(448))))


def f32_rne(q):
    """A rational rounded to the nearest fp32 (ties to even); normal range."""
    from fractions import Fraction

    q = Fraction(q)
    if q == 0:
        return np.float32(0.0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    assert -126 <= e <= 127
    scaled = a / Fraction(2) ** (e - 23)  # in [2^23, 2^24)
    m = scaled.numerator // scaled.denominator
    rem = scaled - m
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m % 2 == 1):
        m += 1
    return np.float32(sign * float(Fraction(m) * Fraction(2) ** (e - 23)))


def kernel_reciprocal(sc, r0):
    """The encoder's r: one Newton step on a hardware reciprocal r0,
    fma(fma(-sc, r0, 1), r0, r0), each fma rounded once."""
    from fractions import Fraction

    s, q = Fraction(float(sc)), Fraction(float(r0))
    e = f32_rne(1 - s * q)
    return f32_rne(Fraction(float(e)) * q + q)


def test_fp8_kernel_reciprocal_is_inside_the_tested_window(ora):
    """The r the kernel really uses: the hardware reciprocal is accurate to
    1 ulp, so r0 is fl(1/sc) or a neighbour; after the Newton step r must
    lie within one ulp of fl(1/sc) (the window the tests above cover), and
    the codes it gives must equal those of the division, on quotients
    placed around every E4M3 rounding point."""
    rng = np.random.default_rng(23)
    mids = e4m3_midpoints()
    for trial in range(300):
        amax = np.float32(np.ldexp(rng.uniform(1, 2), int(rng.integers(-100, 100))))
        sc = np.float32(amax / np.float32(448))
        ref = np.float32(1.0) / sc
        ulp_window = {ref, np.nextafter(ref, np.float32(np.inf)), np.nextafter(ref, np.float32(0))}
        t = (mids.astype(np.float64) * np.float64(sc)).astype(np.float32)
        k = rng.integers(-12, 13, t.size)
        x = t.copy()
        for _ in range(12):
            step = np.abs(k) > _
            x = np.where(step, np.nextafter(x, np.where(k >= 0, np.inf, -np.inf).astype(np.float32)), x)
        x = np.concatenate([x, -x, rng.uniform(-1, 1, 2048).astype(np.float32) * amax]).astype(np.float32)
        want = ora.e4m3_from_f32_n(np.clip((x / sc).astype(np.float32), np.float32(-448), np.float32(448)))
        for r0 in (ref, np.nextafter(ref, np.float32(np.inf)), np.nextafter(ref, np.float32(0))):
            r = kernel_reciprocal(sc, r0)
            assert r in ulp_window, (trial, float(sc), float(r0), float(r))
            got, _ = fast_code(ora, x, sc, r)
            assert np.array_equal(got, want), trial


def test_f32_rne_rounds_ties_to_even():
    from fractions import Fraction

    one = Fraction(1)
    ulp = Fraction(1, 2 ** 23)
    assert f32_rne(one + ulp / 2) == np.float32(1.0)          # tie, even stays
    assert f32_rne(one + ulp + ulp / 2) == np.float32(1.0) + np.float32(2.0 ** -22)  # tie, odd rounds up
    assert f32_rne(one + ulp / 2 + Fraction(1, 2 ** 60)) == np.nextafter(np.float32(1), np.float32(2))
    assert f32_rne(Fraction(1, 3)) == np.float32(1) / np.float32(3)
