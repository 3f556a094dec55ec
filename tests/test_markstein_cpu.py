"""CPU check of the division method the quantizer's element encoder uses.

The encoder needs the correctly rounded FP32 quotient |w| / d (the E2M1 code
that follows depends on every bit of it, and the oracle divides in IEEE
binary32).  For d in [2^-98, 2^100] it takes the correctly rounded reciprocal
r = RN(1/d) and one Markstein correction: q0 = RN(x r), e = fma(-q0, d, x),
q = fma(e, r, q0).  This test restates that sequence in C (fmaf is the
correctly rounded fused multiply-add) and compares it, bit for bit, with IEEE
division on 2^24 random operand pairs over every binade of that range, plus
exact multiples, results near the subnormal boundary and the range ends
(every pair with a dividend of at least 2^-100 and a normal IEEE quotient
must agree; the encoder's quotients never exceed ~12, and a smaller dividend
only has to give a quotient below 0.25, the first E2M1 rounding threshold).  The
device code itself is compared with IEEE division on the GPU
(tests/test_gpu_conversions.py)."""
import ctypes
import os
import subprocess
import tempfile

import numpy as np
import pytest

C_SRC = r"""
#include <math.h>
#include <stdint.h>
void markstein(const float* x, const float* d, float* q, int64_t n) {
  for (int64_t i = 0; i < n; ++i) {
    float r = 1.0f / d[i];
    float q0 = x[i] * r;
    float e = fmaf(-q0, d[i], x[i]);
    q[i] = fmaf(e, r, q0);
  }
}
"""


@pytest.fixture(scope="module")
def markstein_lib():
    tmp = tempfile.mkdtemp(prefix="markstein_")
    src = os.path.join(tmp, "m.c")
    lib = os.path.join(tmp, "libm_check.so")
    with open(src, "w") as f:
        f.write(C_SRC)
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-shared",
                    "-fPIC", src, "-o", lib, "-lm"], check=True)
    L = ctypes.CDLL(lib)
    L.markstein.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64]
    return L


def _run(L, x, d):
    q = np.empty_like(x)
    L.markstein(x.ctypes.data, d.ctypes.data, q.ctypes.data, x.size)
    return q


def test_markstein_equals_ieee_division(markstein_lib):
    rng = np.random.default_rng(np.random.SeedSequence([5150, 3]))
    n = 1 << 24
    d = ((rng.random(n) + 0.5) * np.exp2(rng.integers(-98, 100, n).astype(np.float64)))
    d = np.clip(d, 2.0**-98, 2.0**100).astype(np.float32)
    x = ((rng.random(n) + 0.5) * np.exp2(rng.integers(-126, 128, n).astype(np.float64)))
    x = x.astype(np.float32)
    with np.errstate(over="ignore", under="ignore"):
        # exact multiples (quotient exactly representable) and quotients that
        # land near the subnormal boundary
        exact = (d * np.float32(5.0)).astype(np.float32)
        tiny = (d * np.float32(2.0**-126)).astype(np.float32)
    xs = np.concatenate([x, exact, tiny, np.float32([0.0, 2.0**-126, 3.0e38])])
    ds = np.concatenate([d, d, d, np.float32([1.0, 2.0**-98, 2.0**100])])
    keep = np.isfinite(xs) & (xs >= 2.0**-126)  # normal dividends (x == 0 handled below)
    keep[-3] = True
    xs, ds = xs[keep], ds[keep]
    got = _run(markstein_lib, xs, ds)
    with np.errstate(over="ignore", under="ignore"):
        want = (xs / ds).astype(np.float32)
    # Where the method applies -- a dividend of at least 2^-100, so that the
    # residual x - q0 d does not lose bits to underflow -- every normal
    # quotient must be correctly rounded.  The encoder's quotients are at most
    # ~12 (|w| <= 6.4 d by construction of the block scale), so overflowing
    # ones never occur.  A smaller dividend (or a quotient below the normal
    # range) only has to give a quotient below the first E2M1 rounding
    # threshold, 0.25, which x < 2^-100 <= d / 4 guarantees.
    exact_region = np.isfinite(want) & (want >= 2.0**-126) & (xs >= 2.0**-100)
    assert exact_region.sum() > 3 * n // 2
    assert (got[~exact_region & (want < 0.125)] < 0.25).all()
    got, want, xs, ds = got[exact_region], want[exact_region], xs[exact_region], ds[exact_region]
    bad = np.nonzero(got.view(np.uint32) != want.view(np.uint32))[0]
    assert bad.size == 0, "x=%r d=%r: %r != %r" % (xs[bad[0]], ds[bad[0]], got[bad[0]],
                                                  want[bad[0]])


def test_markstein_catches_a_wrong_reciprocal(markstein_lib):
    # the comparison has teeth: dropping the correction step (q = q0) is not
    # correctly rounded on many of the same operands
    rng = np.random.default_rng(np.random.SeedSequence([5150, 4]))
    d = (rng.random(1 << 16) + 0.5).astype(np.float32)
    x = (rng.random(1 << 16) + 0.5).astype(np.float32)
    q0 = (x * (np.float32(1.0) / d)).astype(np.float32)
    assert (q0.view(np.uint32) != (x / d).astype(np.float32).view(np.uint32)).sum() > 100
    got = _run(markstein_lib, x, d)
    assert np.array_equal(got.view(np.uint32), (x / d).astype(np.float32).view(np.uint32))
