"""Pins for the NVFP4 linear-layer oracle (CPU only).

Method: "Pika H3 Flex in FastVideo: 7x Faster, and Near Real Time in 4-bit",
section "NVFP4 QAD" (4-bit weights and activations, one 8-bit scale per 16
values, static activation scales) and section "FP4 attention" (E2M1 values,
E4M3 block scales).
"""

import numpy as np

from oracle import nvfp4
from oracle import nvfp4_linear as lin


def bf16_values(rng, shape, scale=1.0):
    x = (rng.standard_t(3, shape) * scale).astype(np.float32)
    return (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)


def test_unit_global_scale_is_the_qk_quantizer_without_transforms():
    rng = np.random.default_rng(50)
    x = bf16_values(rng, (6, 128), 3.0)
    bits = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    c, s = lin.quantize(x, 1.0)
    ref = nvfp4.qk_prep_fp4(bits[None], bits[None], smooth=False, rotate=False)
    assert np.array_equal(c, ref["q_codes"][0]) and np.array_equal(s, ref["q_scales"][0])


def test_power_of_two_global_scale_moves_only_the_scales():
    # x / 2^e is exact, so the codes are unchanged and every block scale is the
    # one of x divided by 2^e (as long as it stays a normal E4M3 value).
    rng = np.random.default_rng(51)
    x = bf16_values(rng, (5, 64), 40.0)
    c1, s1 = lin.quantize(x, 1.0)
    c4, s4 = lin.quantize(x, 4.0)
    e4 = nvfp4.e4m3_decode_table()
    assert np.array_equal(c1, c4)
    ok = e4[s1] >= 4 * 2.0 ** -6                     # both scales normal
    assert np.all(e4[s4][ok] * 4 == e4[s1][ok])
    assert np.allclose(lin.dequantize(c4, s4, 4.0)[np.repeat(ok, 16, axis=1)],
                       lin.dequantize(c1, s1, 1.0)[np.repeat(ok, 16, axis=1)])


def test_clipping_at_6_times_448_times_g():
    x = np.zeros((1, 16))
    x[0, 0] = 1.0e6
    x[0, 1] = -50.0
    c, s = lin.quantize(x, 2.0)
    v = lin.dequantize(c, s, 2.0)
    assert v[0, 0] == 6 * 448 * 2.0 and s[0, 0] == 0x7E
    assert v[0, 1] == 0.0 and c[0, 0] >> 4 == 8        # -25 / 448 rounds to the signed zero code


def test_product_equals_a_loop():
    rng = np.random.default_rng(52)
    x = bf16_values(rng, (3, 32))
    w = bf16_values(rng, (4, 32), 0.1)
    xc, xs = lin.quantize(x, 0.5)
    wc, ws = lin.quantize(w, 0.01)
    y = lin.linear(xc, xs, 0.5, wc, ws, 0.01)
    xh = lin.dequantize(xc, xs, 0.5)
    wh = lin.dequantize(wc, ws, 0.01)
    for m in range(3):
        for n in range(4):
            assert abs(y[m, n] - sum(xh[m, k] * wh[n, k] for k in range(32))) <= 1e-12 * (1 + abs(y[m, n]))


def test_quantization_error_is_bounded_by_half_a_step():
    # with the usual global scale amax / (6 * 448) nothing clips, and every
    # dequantized value is within half of the widest E2M1 step (2) times its
    # scale and g of the input
    rng = np.random.default_rng(53)
    x = bf16_values(rng, (20, 64), 5.0)
    g = float(np.float32(np.abs(x).max() / (6 * 448)))
    c, s = lin.quantize(x, g)
    v = lin.dequantize(c, s, g)
    step = nvfp4.e4m3_decode_table()[s] * g              # E2M1 steps are at most 2 (between 4 and 6)
    assert np.all(np.abs(v - x) <= np.repeat(step, 16, axis=1) * 1.0 + 1e-9 * np.abs(x))


# ---- RN32(x / g) against exact rational rounding ------------------------------

from fractions import Fraction  # noqa: E402

F32_MAX_EXP = 128


def rn32_exact(fr):
    """Nearest float32 to the rational ``fr`` (ties to the even significand),
    with float32's subnormals (quantum 2^-149) and overflow to infinity."""
    if fr == 0:
        return 0.0
    neg = fr < 0
    a = -fr if neg else fr
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    quantum = max(e, -126) - 23
    scaled = a / Fraction(2) ** quantum
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = Fraction(n) * Fraction(2) ** quantum
    out = float("inf") if val >= Fraction(2) ** F32_MAX_EXP else float(val)
    return -out if neg else out


def f32_from_bits(b):
    return np.array(b, dtype=np.uint32).view(np.float32)


def random_bf16(rng, n, emin=-133, emax=127):
    """BF16 values with exponents spread over [emin, emax] (subnormals when
    emin < -126) and random signs."""
    sig = rng.integers(128, 256, n).astype(np.float64)
    e = rng.integers(emin, emax + 1, n)
    x = np.ldexp(sig / 128.0, e)
    x = np.where(e < -126, np.ldexp(np.floor(np.ldexp(x, 133)), -133), x)   # BF16 subnormal grid
    return np.where(rng.random(n) < 0.5, -x, x)


def random_f32(rng, n, emin=-30, emax=30):
    sig = (rng.integers(1 << 23, 1 << 24, n) | 1).astype(np.float64)      # odd: never a power of two
    return np.ldexp(sig / 2.0 ** 23, rng.integers(emin, emax + 1, n)).astype(np.float32)


def check_quotients(x, g):
    got = lin.scaled_input(x, g)
    for xi, gi in zip(np.atleast_1d(x), np.atleast_1d(got)):
        want = rn32_exact(Fraction(float(xi)) / Fraction(float(np.float32(g))))
        if xi == 0:
            want = np.copysign(0.0, xi)                 # g > 0: a zero keeps its sign
        assert np.float32(want).view(np.uint32) == np.float32(gi).view(np.uint32), (xi, g, gi, want)
    return got


def test_quotient_random_against_fraction():
    rng = np.random.default_rng(60)
    for g in random_f32(rng, 40):
        x = random_bf16(rng, 60, -40, 40)
        check_quotients(x, g)


def near_midpoint_pairs(rng, want, max_frac=2.0 ** -12):
    """(x, g) pairs whose exact quotient x / g lies within max_frac half-ulps
    of a float32 rounding boundary (a midpoint between two float32 values),
    found with exact integers: for significands X (BF16, 8 bits) and G
    (float32, 24 bits, odd), t = X 2^k / G scaled into [2^24, 2^25) is the
    quotient in half-ulps, and the midpoints are the odd integers.  With
    N = floor(t) and R = X 2^k mod G, the nearest midpoint is R / G away
    when N is odd and (G - R) / G away when N is even."""
    out = []
    while len(out) < want:
        G = int(rng.integers(1 << 23, 1 << 24)) | 1
        for X in range(129, 256, 2):
            k = (G << 24).bit_length() - X.bit_length()
            while (X << k) < (G << 24):
                k += 1
            while (X << k) >= (G << 25):
                k -= 1
            N, R = divmod(X << k, G)
            dist = Fraction(R, G) if N % 2 == 1 else Fraction(G - R, G)
            if dist < max_frac:
                g = np.float32(np.ldexp(G / 2.0 ** 23, int(rng.integers(-3, 4))))
                x = float(np.ldexp(X / 128.0, int(rng.integers(-8, 9))))
                out.append((x, g))
    return out


def test_quotient_next_to_rounding_boundaries():
    # The correctly rounded quotient against RN32(x * RN32(1/g)): on quotients
    # this close to a rounding boundary the multiply by the rounded reciprocal
    # lands on the wrong side for some pairs, the division never does.
    rng = np.random.default_rng(61)
    pairs = near_midpoint_pairs(rng, 40)
    differ = 0
    for x, g in pairs:
        got = check_quotients(np.array([x]), g)[0]
        r = np.float32(1.0 / np.float64(g))
        differ += np.float32(np.float64(x) * np.float64(r)) != got
    assert differ > 0


def test_quotient_subnormal_and_overflow():
    rng = np.random.default_rng(62)
    # results in float32's subnormal range (and below its smallest subnormal)
    check_quotients(random_bf16(rng, 80, -133, -100), np.float32(3.0e12))
    check_quotients(random_bf16(rng, 80, -133, -110), np.float32(1.7e5))
    # quotients on both sides of the overflow threshold 2^128 - 2^103
    big = np.array([3.3895314e38, -3.3895314e38, 2.0 ** 127, 1.5 * 2.0 ** 127, 0.0, -0.0])
    got = check_quotients(big, np.float32(0.75))
    assert np.isinf(got[0]) and np.isinf(got[1]) and got[1] < 0
    g_edge = np.float32(2.0 ** 127 / (2.0 ** 128 - 2.0 ** 103))        # x / g at the threshold itself
    check_quotients(np.array([2.0 ** 127, 1.9921875 * 2.0 ** 126]), g_edge)
    # signed zeros keep their sign
    z = lin.scaled_input(np.array([0.0, -0.0]), np.float32(0.3))
    assert not np.signbit(z[0]) and np.signbit(z[1])


def test_overflowed_quotient_saturates_like_clipping():
    # an infinite x' takes scale 448 (code 0x7E) and code +-6 (index 7), the
    # same as a finite x' beyond 6 * 448
    x = np.zeros((1, 16))
    x[0, 0], x[0, 1], x[0, 2] = 3.3895314e38, -3.3895314e38, 1.0e30
    c, s = lin.quantize(x, np.float32(0.5))
    assert s[0, 0] == 0x7E
    assert c[0, 0] == (0x7 | (0xF << 4)) and c[0, 1] & 0xF == 0x7


def test_quotient_cases_decide_codes_by_one_ulp():
    # The constructed blocks (tests/quotient_cases.py) put x / g next to the
    # midpoint beside a code or scale threshold: the oracle's correctly
    # rounded quotient and the multiply by a rounded reciprocal give different
    # codes or scales on many of them, so bit-exact agreement on these blocks
    # pins the quotient's rounding.
    from quotient_cases import quotient_cases
    from long_sequence_dense_amd import inputs
    cases = quotient_cases(60)
    differ = 0
    for bits, g, kind, tau in cases:
        x = inputs.bf16_bits_to_f32(bits).astype(np.float64)[None]
        c, s = lin.quantize(x, g)
        r = np.float32(1.0 / np.float64(g))
        alt = (x * np.float64(r)).astype(np.float32)
        ca, sa = nvfp4._quantize_rows(alt, rotate=False)
        differ += (not np.array_equal(c, ca)) or (not np.array_equal(s, sa))
        # the deciding element's x' is the threshold or its float32 neighbour
        xs = lin.scaled_input(x, g)[0]
        d = np.abs(np.abs(xs.astype(np.float64)) - float(tau))
        assert d.min() <= float(np.spacing(np.float32(float(tau)))), (kind, float(tau))
    assert differ >= len(cases) // 10, differ
