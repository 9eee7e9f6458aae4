"""Test helper (not a test module): NVFP4-linear quantizer inputs whose scaled
value x' = RN32(x / g) decides a code or a scale by one float32 ulp.

For a decision threshold tau of the block quantizer (an E2M1 midpoint times
the block scale s, or six times the midpoint of two neighbouring E4M3 scales;
all have at most 7 significant bits, so they are exact float32 values) the
decision changes between two adjacent float32 values, tau and its neighbour.
A case puts the exact quotient x / g within a tenth of half an ulp of the
midpoint between those two, on a seeded side: a quotient rounded the wrong
way by even a fraction of an ulp there moves x' across tau.  x is a BF16
value near tau * c for a seeded c, and the global scale g is the float32
nearest to x / m (m the midpoint); the exact distance of x / g from m is then
checked with rationals and the case is kept only when it is small.

Each case is one 16-value block (with its own g): for an E2M1 threshold a
second element sets the block scale to s (its quotient is within 2^-8 of
6 s, far from any scale boundary) and x sits below it; for a scale
threshold x is the block maximum.  The remaining values are small seeded
fillers.  Only exact rational arithmetic and the oracle's published tables
are used here.
"""

from fractions import Fraction

import numpy as np

E2M1_MIDS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def _e4m3_positive():
    """Values of the E4M3 codes 1..126 from their bit fields (bias 7,
    3 mantissa bits, subnormals m 2^-9)."""
    out = []
    for j in range(1, 127):
        e, m = j >> 3, j & 7
        out.append(Fraction(8 + m, 8) * Fraction(2) ** (e - 7) if e else Fraction(m, 512))
    return out


def _ulp_f32(v):
    """ulp of the float32 interval [2^e, 2^(e+1)) holding the positive
    rational v (normal range)."""
    e = v.numerator.bit_length() - v.denominator.bit_length()
    if Fraction(2) ** e > v:
        e -= 1
    return Fraction(2) ** (e - 23), e


def _bf16_nearest(v):
    """The BF16 value nearest to the positive rational v (normal range),
    ties to even, as a Fraction."""
    e = v.numerator.bit_length() - v.denominator.bit_length()
    if Fraction(2) ** e > v:
        e -= 1
    q = Fraction(2) ** (e - 7)
    n, r = divmod(v, q)
    n = int(n)
    if r > q / 2 or (r == q / 2 and n % 2):
        n += 1
    return n * q


def _f32_nearest(v):
    e = v.numerator.bit_length() - v.denominator.bit_length()
    if Fraction(2) ** e > v:
        e -= 1
    q = Fraction(2) ** (e - 23)
    n, r = divmod(v, q)
    n = int(n)
    if r > q / 2 or (r == q / 2 and n % 2):
        n += 1
    return n * q


def _to_bits(frac):
    """BF16 bit pattern of an exactly representable positive rational."""
    f = np.float32(float(frac))
    assert Fraction(float(f)) == frac
    return int(f.view(np.uint32) >> 16)


def thresholds():
    """(tau, s, kind): every E2M1 decision threshold at every scale, and
    every scale decision threshold (6 x the midpoint of E4M3 neighbours)."""
    vs = _e4m3_positive()
    out = [(t * v, v, "code") for v in vs for t in map(Fraction, E2M1_MIDS)]
    prev = Fraction(0)
    for v in vs:
        out.append((3 * (prev + v), None, "scale"))
        prev = v
    return out


def quotient_cases(n_cases, seed=3):
    """Returns a list of (bits [16] uint16, g float32, kind, tau)."""
    rng = np.random.default_rng(seed)
    ths = thresholds()
    cases = []
    while len(cases) < n_cases:
        tau, s, kind = ths[int(rng.integers(len(ths)))]
        if tau < Fraction(2) ** -100:
            continue
        c = Fraction(float(np.float32(rng.uniform(0.5, 2.0) * 2.0 ** int(rng.integers(-6, 7)))))
        x = _bf16_nearest(tau * c)
        ulp, e = _ulp_f32(tau)
        below = ulp / 2 if tau == Fraction(2) ** e else ulp   # the float32 below a power of two is ulp / 2 away
        m = tau + ulp / 2 if rng.random() < 0.5 else tau - below / 2
        g = _f32_nearest(x / m)
        half = (ulp if m > tau else below) / 2
        if abs(x / g - m) >= half / 10 or x / g == m:
            continue
        vals = [0] * 16
        pos = rng.permutation(16)
        vals[pos[0]] = _to_bits(x)
        if kind == "code":
            vals[pos[1]] = _to_bits(_bf16_nearest(6 * s * g))
            fill_top = s * g
        else:
            fill_top = x / 4
        for p in pos[2 if kind == "code" else 1:]:
            vals[p] = _to_bits(_bf16_nearest(fill_top * Fraction(float(rng.uniform(0.01, 1.0)))))
        bits = np.array(vals, dtype=np.uint16) | (rng.integers(0, 2, 16).astype(np.uint16) << 15)
        cases.append((bits, np.float32(float(g)), kind, tau))
    return cases
