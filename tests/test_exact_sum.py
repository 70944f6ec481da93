"""Host build of the hash's exact-summation helpers (csrc/exact_sum.h), checked
against Python's exact rationals: the sign of |A| - |B| for two sums of
float64 terms, and the signs of A and B, must be those of the exact sums.

The cases are built where float64 summation goes wrong: terms spread over
hundreds of binary orders, sums that cancel to a tiny remainder or to exactly
zero, and pairs of sums whose difference lies far below float64's resolution
of either sum (the near-ties the hash's last resort exists for)."""
import ctypes
import shutil
import subprocess
from fractions import Fraction
from pathlib import Path

import numpy as np
import pytest

HDR = Path(__file__).resolve().parents[1] / "lsh_attention_amd" / "csrc" / "exact_sum.h"

WRAP = r"""
#include "exact_sum.h"
extern "C" int cmp_abs(const double* a, const double* b, int n, int* sa, int* sb) {
  double ea[64], eb[64], d[128];
  return lsh::exact_abs_compare(a, b, n, ea, eb, d, *sa, *sb);
}
"""


@pytest.fixture(scope="module")
def lib(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("no host C++ compiler")
    d = tmp_path_factory.mktemp("exact_sum")
    (d / "w.cpp").write_text(WRAP)
    so = d / "w.so"
    # -ffp-contract=off and no fast-math: the same IEEE double semantics the
    # device build gets (TwoSum has no products to contract anyway)
    subprocess.run(["g++", "-O2", "-ffp-contract=off", "-shared", "-fPIC", f"-I{HDR.parent}", str(d / "w.cpp"),
                    "-o", str(so)], check=True)
    f = ctypes.CDLL(str(so)).cmp_abs
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.POINTER(ctypes.c_double)] * 2 + [ctypes.c_int] + [ctypes.POINTER(ctypes.c_int)] * 2
    return f


def _call(f, a, b):
    a = np.ascontiguousarray(a, dtype=np.float64)
    b = np.ascontiguousarray(b, dtype=np.float64)
    assert a.shape == b.shape and a.size <= 64
    sa, sb = ctypes.c_int(), ctypes.c_int()
    dp = ctypes.POINTER(ctypes.c_double)
    c = f(a.ctypes.data_as(dp), b.ctypes.data_as(dp), a.size, ctypes.byref(sa), ctypes.byref(sb))
    return c, sa.value, sb.value


def _sign(q):
    return (q > 0) - (q < 0)


def _exact(a, b):
    A = sum((Fraction(float(t)) for t in a), Fraction(0))
    B = sum((Fraction(float(t)) for t in b), Fraction(0))
    return _sign(abs(A) - abs(B)), _sign(A), _sign(B)


def _check(f, a, b):
    got = _call(f, a, b)
    want = _exact(a, b)
    assert got == want, (got, want, list(a), list(b))
    return got


def test_hand_cases(lib):
    z = np.zeros(64)
    assert _check(lib, z, z) == (0, 0, 0)
    a = z.copy()
    a[:3] = [1.0, 2.0**-70, -1.0]             # cancels to 2^-70 (float64 sum: 0)
    b = z.copy()
    b[:2] = [2.0**-71, 2.0**-71]              # exactly 2^-70
    assert _check(lib, a, b) == (0, 1, 1)
    b[1] = 2.0**-72                           # 3 * 2^-72 < 2^-70
    assert _check(lib, a, b) == (1, 1, 1)
    b[:2] = [-(2.0**-71), -(2.0**-70)]        # |B| = 3 * 2^-71 > 2^-70, B negative
    assert _check(lib, a, b) == (-1, 1, -1)
    c = z.copy()
    c[:4] = [2.0**300, 1.0, -(2.0**300), -1.0]  # exact zero through a huge cancellation
    assert _check(lib, c, b) == (-1, 0, -1)


def test_products_of_bf16_and_fp32_values(lib):
    """Sums of 64 exact products of fp32 values (48-bit significands) with
    exponents spread over +-60 binary orders, and a second sum equal to the
    first up to one tiny term placed at a random depth below it."""
    rng = np.random.default_rng(5)
    for trial in range(300):
        x = (rng.standard_normal(64) * 2.0 ** rng.integers(-60, 61, 64)).astype(np.float32).astype(np.float64)
        r = (rng.standard_normal(64) * 2.0 ** rng.integers(-20, 21, 64)).astype(np.float32).astype(np.float64)
        if trial % 2:
            # bf16-valued factors
            x = (x.astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32).astype(np.float64)
            r = (r.astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32).astype(np.float64)
        pa = x * r                                 # exact in float64
        assert all(Fraction(float(p)) == Fraction(float(u)) * Fraction(float(v)) for p, u, v in zip(pa, x, r))
        pb = pa.copy()
        k = int(rng.integers(0, 64))
        big = float(np.max(np.abs(pa)))
        pb[k] = pa[k] + (big * 2.0 ** -float(rng.integers(54, 200))) * (1 if trial % 3 else -1)
        if trial % 5 == 0:
            pb = -pb                               # equal magnitudes of opposite sign
        _check(lib, pa, pb)
        _check(lib, pb, pa)
        _check(lib, pa, pa[rng.permutation(64)])   # equal sums in another order: |A| == |B|


def test_cancellation_to_below_float64(lib):
    """A sum whose float64 evaluation (in any order) is far from its value: big
    terms that cancel exactly around small ones."""
    rng = np.random.default_rng(11)
    for _ in range(200):
        big = rng.standard_normal(20) * 2.0 ** rng.integers(0, 80, 20)
        small = rng.standard_normal(24) * 2.0 ** rng.integers(-120, -60, 24)
        a = np.concatenate([big, -big, small])
        rng.shuffle(a)
        small2 = small.copy()
        small2[0] = np.nextafter(small2[0], np.inf)
        b = np.concatenate([big, small2, -big])
        _check(lib, a, b)
        assert _call(lib, a, a)[0] == 0
