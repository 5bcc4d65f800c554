"""The float64 exp2 of the streaming and nucleus kernels takes the argument's
integer part from a sum with 1.5 * 2^32 after an fma whose clamp bit bounds
the argument, instead of max / rint / convert.  The kernels rely on that
giving the same bits as the plain form; this checks the identity in exact
arithmetic on the host (IEEE float64 with round-to-nearest-even, fma emulated
exactly with fractions), over random arguments of the row-sum range:

  plain    y = fma(l, cs, n);  j = rint(max(y, -280000));  f = y - j
  clamped  y' = clamp(fma(l, -cs 2^-20, -n 2^-20), 0, 1);  t = M - y';
           j = low word of t (two's complement);  f = -(y' - (M - t)) 2^20

and the degree-3 tail with the coefficients scaled by (-2^20)^i gives the
same value to the bit.  No GPU."""
import math
import struct
from fractions import Fraction

import numpy as np

E1, E2, E3 = 0.0027076061740622863, 3.6655655969101062e-06, 3.3083026805413713e-09   # (ln2/256)^i / i!
MAGIC = 1.5 * 2.0 ** 32
S = 2.0 ** -20
F1, F2, F3 = -E1 * 2.0 ** 20, E2 * 2.0 ** 40, -E3 * 2.0 ** 60


def fma(a, b, c):
    if not (math.isfinite(a) and math.isfinite(b) and math.isfinite(c)):
        return a * b + c                      # infinities: no rounding to emulate
    return float(Fraction(a) * Fraction(b) + Fraction(c))


def low_word(x):
    lo = struct.unpack("<Q", struct.pack("<d", x))[0] & 0xFFFFFFFF
    return lo - (1 << 32) if lo >= (1 << 31) else lo


def plain(l, cs, n):
    y = max(fma(l, cs, n), -280000.0)
    j = float(np.rint(y))
    f = y - j
    q = fma(fma(fma(f, E3, E2), f, E1), f, 1.0)
    return int(j), q


def clamped(l, cs, n):
    yp = min(max(fma(l, -cs * S, -n * S), 0.0), 1.0)
    t = MAGIC - yp
    fp = yp - (MAGIC - t)
    q = fma(fma(fma(fp, F3, F2), fp, F1), fp, 1.0)
    return low_word(t), q


def term(j, q):
    return math.ldexp(2.0 ** ((j & 255) / 256) * q, j >> 8)


def test_clamped_split_gives_the_plain_terms_bit_for_bit():
    rng = np.random.default_rng(11)
    for _ in range(6000):
        T = float(rng.choice([0.05, 0.7, 0.8, 1.0, 4.0]))
        cs = 256 * 1.4426950408889634 / T
        m = float(np.float32(rng.normal() * 3))
        l = float(np.float32(m - abs(rng.normal()) * rng.choice([1, 5, 30, 300, 3000])))
        n = -m * cs
        ja, qa = plain(l, cs, n)
        jb, qb = clamped(l, cs, n)
        assert term(ja, qa) == term(jb, qb), (l, m, T)
        if ja > -280000:                      # where the plain form does not clamp, even j and f agree
            assert ja == jb and qa == qb, (l, m, T)


def test_clamped_split_handles_the_edges():
    cs, n = 256 * 1.4426950408889634, 0.0
    # the maximum itself (y = 0), -inf (every term 0), and arguments past both lower bounds
    assert clamped(0.0, cs, n) == plain(0.0, cs, n) == (0, 1.0)
    assert term(*clamped(-math.inf, cs, n)) == 0.0 == term(*plain(-math.inf, cs, n))
    for l in (-800.0, -3000.0, -1e30):
        assert term(*clamped(l, cs, n)) == 0.0 == term(*plain(l, cs, n))
