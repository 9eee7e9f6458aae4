"""Pins for the NVFP4 Q/K preparation oracle (CPU only).

Method: "Pika H3 Flex in FastVideo: 7x Faster, and Near Real Time in 4-bit",
section "FP4 attention" (mean-key subtraction, a shared orthonormal Hadamard
rotation of Q and K, E2M1 values with one E4M3 scale per 16 channels and a unit
global scale); the 16-value block with a small entry rounding to zero is of the
kind the figure on the yuxiaoba review "Decoding can cost more than denoising"
shows (its caption gives no values, so the block is constructed here).

Everything the oracle computes is compared with something other than itself:
bit-field definitions and torch's float8 decoder for the codecs, Fraction
brute-force argmin for every rounding decision, the integer Sylvester matrix
for the butterfly, a Fraction exact sum for the mean, float32-scalar loops for a
whole row, and the exact invariances of the transforms.
"""

import math
import struct
from fractions import Fraction

import numpy as np
import pytest

from oracle import nvfp4
from oracle.attention import attention_fp64

E2M1_MAGS = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2),
             Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def f32(x):
    return np.float32(x)


def f32_from_bits(b):
    return struct.unpack("<f", struct.pack("<I", b & 0xFFFFFFFF))[0]


def f32_bits(x):
    return struct.unpack("<I", struct.pack("<f", float(x)))[0]


def next_up(x):
    return np.nextafter(np.float32(x), np.float32(np.inf), dtype=np.float32)


def next_down(x):
    return np.nextafter(np.float32(x), np.float32(-np.inf), dtype=np.float32)


def e4m3_value_fraction(code):
    """E4M3 value from its bit fields, exact (no float arithmetic)."""
    e = (code >> 3) & 0xF
    m = code & 7
    sign = -1 if code & 0x80 else 1
    if e == 0:
        return sign * Fraction(m, 8) * Fraction(1, 64)
    return sign * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


E4M3_POS = [e4m3_value_fraction(c) for c in range(0x7F)]


def brute_scale_code(a):
    """Nearest E4M3 code (0..0x7E) to a/6, ties to the even code."""
    t = Fraction(float(a)) / 6
    return min(range(0x7F), key=lambda c: (abs(E4M3_POS[c] - t), c & 1))


def brute_e2m1_code(y, s):
    sign = 8 if math.copysign(1.0, float(y)) < 0 else 0
    if s == 0:
        return sign
    t = abs(Fraction(float(y))) / Fraction(s)
    e = min(range(8), key=lambda i: (abs(E2M1_MAGS[i] - t), i & 1))
    return sign | e


# ---- codecs ---------------------------------------------------------------------

def test_e4m3_table_bitfields_and_torch():
    tab = nvfp4.e4m3_decode_table()
    for c in range(256):
        if c & 0x7F == 0x7F:
            assert np.isnan(tab[c])
        else:
            assert Fraction(tab[c]) == e4m3_value_fraction(c)
    assert tab[0x7E] == 448.0 and tab[0x01] == 2.0 ** -9 and tab[0x38] == 1.0
    torch = pytest.importorskip("torch")
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("torch without float8_e4m3fn")
    tt = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    fin = ~np.isnan(tab)
    assert np.array_equal(np.isnan(tt), np.isnan(tab))
    assert np.array_equal(tt[fin], tab[fin])


def test_e2m1_table():
    tab = nvfp4.e2m1_decode_table()
    expect = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(tab[:8]) == expect
    assert list(-tab[8:]) == expect
    assert math.copysign(1.0, tab[8]) < 0          # code 8 is -0


def test_scale_code_roundtrip_all_codes():
    vals = np.array([float(v) for v in E4M3_POS])
    a = (vals * 6.0).astype(np.float32)            # exact: <= 6 significant bits
    assert np.array_equal(a.astype(np.float64), vals * 6.0)
    assert np.array_equal(nvfp4.e4m3_scale_code(a), np.arange(0x7F, dtype=np.uint8))


def test_e2m1_roundtrip_all_codes():
    tab = nvfp4.e2m1_decode_table()
    y = tab.astype(np.float32).reshape(1, 16)
    got = nvfp4.e2m1_codes(y, np.array([1.0]))
    assert list(got[0]) == list(range(16))


# ---- rounding decisions vs Fraction brute force ---------------------------------

def _adversarial_amax():
    out = [0.0, 2.0 ** -149, 1e-20, 6 * 2.0 ** -10, 6 * 2.0 ** -9, 2688.0, 2688.0 * 1.01, 3e38]
    for j in range(126):
        mid6 = float((E4M3_POS[j] + E4M3_POS[j + 1]) / 2 * 6)
        x = f32(mid6)
        assert float(x) == mid6                     # the threshold is exact in fp32
        out += [x, next_up(x), next_down(x), next_up(next_up(x)), next_down(next_down(x))]
    return np.array(out, dtype=np.float32)


def test_scale_rounding_adversarial_vs_brute_force():
    a = _adversarial_amax()
    got = nvfp4.e4m3_scale_code(a)
    for ai, g in zip(a, got):
        assert g == brute_scale_code(ai), (float(ai), g)


def test_scale_rounding_random_vs_brute_force():
    rng = np.random.default_rng(20)
    # log-uniform over the whole useful range, plus raw random fp32 bit patterns
    a = np.exp(rng.uniform(np.log(1e-5), np.log(5000.0), 15000)).astype(np.float32)
    bits = rng.integers(0, 0x7F800000, 5000, dtype=np.uint32)
    a = np.concatenate([a, bits.view(np.float32)])
    got = nvfp4.e4m3_scale_code(a)
    bad = [(float(x), int(g)) for x, g in zip(a, got) if g != brute_scale_code(x)]
    assert not bad, bad[:5]


def test_e2m1_ties_and_neighbours_every_scale():
    s_vals = np.array([float(v) for v in E4M3_POS], dtype=np.float64)
    ys, ss = [], []
    for s in s_vals:
        for k, t in enumerate([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 6.5]):
            x = f32(t * s)
            assert s == 0 or float(x) == t * s
            for v in (x, next_up(x), next_down(x)):
                ys += [v, -v]
                ss += [s, s]
    y = np.array(ys, dtype=np.float32).reshape(-1, 1)
    s = np.array(ss)
    got = nvfp4.e2m1_codes(np.repeat(y, 16, axis=1), s)[:, 0]
    for yi, si, g in zip(y[:, 0], s, got):
        assert g == brute_e2m1_code(yi, si), (float(yi), si, g)


def test_e2m1_random_vs_brute_force():
    rng = np.random.default_rng(21)
    n = 20000
    sc = rng.integers(0, 0x7F, n)
    s = np.array([float(E4M3_POS[c]) for c in sc])
    y = (rng.uniform(-7.0, 7.0, n) * s).astype(np.float32)
    y[::7] = (rng.standard_normal(n)[::7] * 1e-3).astype(np.float32)
    got = nvfp4.e2m1_codes(y.reshape(-1, 1).repeat(16, axis=1), s)[:, 0]
    bad = [(float(a), b, int(g)) for a, b, g in zip(y, s, got) if g != brute_e2m1_code(a, b)]
    assert not bad, bad[:5]


def test_signed_zero_codes():
    y = np.array([[0.0, -0.0] + [1.0] * 14], dtype=np.float32)
    got = nvfp4.e2m1_codes(y, np.array([1.0]))[0]
    assert got[0] == 0 and got[1] == 8
    z = np.array([[-0.0, 0.0, -1e-30] + [0.0] * 13], dtype=np.float32)
    got0 = nvfp4.e2m1_codes(z, np.array([0.0]))[0]
    assert list(got0[:3]) == [8, 0, 8]


def test_small_value_in_block_rounds_to_zero():
    # a 16-value block {100, 1, 0, ...}: the shared scale is the E4M3 value
    # nearest 100/6 = 16.67, i.e. 16; 1/16 is below 0.25 so that entry is 0,
    # and 100/16 = 6.25 saturates to 6.
    y = np.zeros((1, 16), dtype=np.float32)
    y[0, 0], y[0, 1] = 100.0, 1.0
    sc = nvfp4.e4m3_scale_code(np.array([100.0], dtype=np.float32))
    s = nvfp4.e4m3_decode_table()[sc]
    assert s[0] == 16.0
    codes = nvfp4.e2m1_codes(y, s)[0]
    assert codes[0] == 7 and codes[1] == 0


# ---- Hadamard -------------------------------------------------------------------

def sylvester(n):
    h = np.array([[1]], dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def test_sylvester_orthogonality_and_popcount_form():
    h = sylvester(128)
    assert np.array_equal(h @ h.T, 128 * np.eye(128, dtype=np.int64))
    for i in range(0, 128, 13):
        for j in range(128):
            assert h[i, j] == (-1) ** bin(i & j).count("1")


def test_butterfly_equals_integer_matrix_on_exact_inputs():
    rng = np.random.default_rng(22)
    x = rng.integers(-1024, 1025, (64, 128))
    got = nvfp4.hadamard_butterfly_fp32(x.astype(np.float32))
    assert np.array_equal(got.astype(np.int64), x @ sylvester(128))


def test_butterfly_fp32_scalar_loop():
    # The same fixed-order transform with numpy float32 scalar arithmetic
    # (one IEEE single operation per step, no float64 anywhere).
    rng = np.random.default_rng(23)
    x = (rng.standard_t(3, (3, 128)) * 7).astype(np.float32)
    got = nvfp4.hadamard_butterfly_fp32(x)
    for r in range(3):
        v = [np.float32(t) for t in x[r]]
        for s in range(7):
            h = 1 << s
            for i in range(128):
                if i & h == 0:
                    a, b = v[i], v[i + h]
                    v[i], v[i + h] = np.float32(a + b), np.float32(a - b)
        assert np.array_equal(np.array(v, dtype=np.float32).view(np.uint32), got[r].view(np.uint32))


def test_hadamard_scale_is_nearest_float32():
    c = Fraction(float(nvfp4.HADAMARD_SCALE_F32))
    assert f32_bits(nvfp4.HADAMARD_SCALE_F32) == 0x3DB504F3
    ulp = Fraction(2) ** -27                       # c in [2^-4, 2^-3)
    lo, hi = c - ulp / 2, c + ulp / 2
    assert lo * lo < Fraction(1, 128) < hi * hi


def test_hadamard_scale_other_lengths():
    assert nvfp4.hadamard_scale_f32(128) == nvfp4.HADAMARD_SCALE_F32
    assert nvfp4.hadamard_scale_f32(64) == np.float32(0.125)
    for n in (2, 4, 16, 32, 64, 128, 256, 1024):
        assert nvfp4.hadamard_scale_f32(n) == nearest_f32_to_inv_sqrt(n), n
    with pytest.raises(ValueError):
        nvfp4.hadamard_scale_f32(96)


def test_butterfly_length_64_equals_integer_matrix():
    rng = np.random.default_rng(37)
    x = rng.integers(-1024, 1025, (16, 64))
    got = nvfp4.hadamard_butterfly_fp32(x.astype(np.float32))
    assert np.array_equal(got.astype(np.int64), x @ sylvester(64))


# ---- mean -----------------------------------------------------------------------

def test_mean_exact_against_fraction():
    rng = np.random.default_rng(24)
    L, d = 37, 128
    bits = rng.integers(0, 0x10000, (L, d), dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    bits[exp == 0xFF] &= 0x807F                    # no Inf/NaN
    k = nvfp4.bf16_bits_to_f64(bits)
    got = nvfp4.kmean_exact(k)
    for c in range(d):
        s = sum(Fraction(float(t)) for t in k[:, c])
        want = np.float32(float(s) / L)            # float(Fraction) is RN64
        assert f32_bits(got[c]) == f32_bits(want)


def test_mean_cancellation_case():
    k = np.zeros((4, 128))
    k[:, 0] = [2.0 ** 100, 1.0, -(2.0 ** 100), 2.0 ** -100]
    got = nvfp4.kmean_exact(k)
    assert got[0] == np.float32((1.0 + 2.0 ** -100) / 4)
    assert np.all(got[1:] == 0)


# ---- one whole row by brute force ------------------------------------------------

def nearest_f32_to_inv_sqrt(n):
    """RN32(1/sqrt(n)) by exact search: the float32 c with (c - ulp/2)^2 <
    1/n < (c + ulp/2)^2 (no float arithmetic on the constant)."""
    target = Fraction(1, n)
    c = Fraction(float(np.float32(1.0 / math.sqrt(n))))
    for cand in (c, Fraction(float(next_up(np.float32(c)))), Fraction(float(next_down(np.float32(c))))):
        e = math.floor(math.log2(float(cand)))
        ulp = Fraction(2) ** (e - 23)
        if (cand - ulp / 2) ** 2 <= target <= (cand + ulp / 2) ** 2:
            return np.float32(cand)
    raise AssertionError(n)


def brute_prep_rows(xrows, rotate=True):
    """float32 rows [n, d] (already mean-subtracted) -> (packed codes, scales)
    with float32 scalar butterfly and Fraction-argmin rounding, plain loops."""
    d = len(xrows[0])
    c = nearest_f32_to_inv_sqrt(d)
    codes_out, scales_out = [], []
    for row in xrows:
        v = [np.float32(t) for t in row]
        if rotate:
            for s in range(d.bit_length() - 1):
                h = 1 << s
                for i in range(d):
                    if i & h == 0:
                        a, b = v[i], v[i + h]
                        v[i], v[i + h] = np.float32(a + b), np.float32(a - b)
            y = [np.float32(t * c) for t in v]
        else:
            y = v
        codes, scales = [], []
        for b in range(d // 16):
            blk = y[16 * b:16 * b + 16]
            sc = brute_scale_code(max(abs(t) for t in blk))
            scales.append(sc)
            codes += [brute_e2m1_code(t, E4M3_POS[sc]) for t in blk]
        codes_out.append([codes[2 * j] | (codes[2 * j + 1] << 4) for j in range(d // 2)])
        scales_out.append(scales)
    return np.array(codes_out, dtype=np.uint8), np.array(scales_out, dtype=np.uint8)


def fraction_mean_f32(kh):
    L = kh.shape[0]
    return np.array([np.float32(float(sum(Fraction(float(t)) for t in kh[:, c])) / L)
                     for c in range(kh.shape[1])], dtype=np.float32)


def test_prep_matches_brute_force_rows():
    rng = np.random.default_rng(25)
    H, L = 2, 24
    q = rng.standard_t(3, (H, L, 128)).astype(np.float32)
    k = (rng.standard_t(3, (H, L, 128)) + rng.normal(0, 2, (H, 1, 128))).astype(np.float32)
    q[:, :, 5] *= 20
    k[:, :, 5] *= 20
    q[0, 3] = 0.0                                   # an all-zero row: scales 0
    q[0, 4, :] = 0.0
    q[0, 4, 9] = 1e-3                               # tiny row
    qb = (q.view(np.uint32) >> 16).astype(np.uint16)   # truncation is fine: any BF16 input
    kb = (k.view(np.uint32) >> 16).astype(np.uint16)
    out = nvfp4.qk_prep_fp4(qb, kb)
    for h in range(H):
        kh = nvfp4.bf16_bits_to_f64(kb[h])
        kbar = np.array([np.float32(float(sum(Fraction(float(t)) for t in kh[:, c])) / L)
                         for c in range(128)], dtype=np.float32)
        assert np.array_equal(out["k_mean"][h].view(np.uint32), kbar.view(np.uint32))
        xk = np.array([[np.float32(np.float32(kh[l, c]) - kbar[c]) for c in range(128)]
                       for l in range(L)], dtype=np.float32)
        xq = nvfp4.bf16_bits_to_f64(qb[h]).astype(np.float32)
        for name, x in (("q", xq), ("k", xk)):
            bc, bs = brute_prep_rows(x)
            assert np.array_equal(out[name + "_codes"][h], bc), name
            assert np.array_equal(out[name + "_scales"][h], bs), name


@pytest.mark.parametrize("smooth,rotate", [(False, False), (True, False), (False, True)])
def test_prep_variants_match_brute_force_rows(smooth, rotate):
    # The ablation variants: without smoothing K is quantized as given and the
    # reported mean is zero; without the rotation the blocks are consecutive
    # original channels with no 1/sqrt(d) factor.
    rng = np.random.default_rng(30 + 2 * smooth + rotate)
    H, L = 2, 12
    q = rng.standard_t(3, (H, L, 128)).astype(np.float32)
    k = (rng.standard_t(3, (H, L, 128)) + rng.normal(0, 2, (H, 1, 128))).astype(np.float32)
    q[:, :, 7] *= 20
    k[:, :, 7] *= 20
    q[1, 2] = 0.0
    qb = (q.view(np.uint32) >> 16).astype(np.uint16)
    kb = (k.view(np.uint32) >> 16).astype(np.uint16)
    out = nvfp4.qk_prep_fp4(qb, kb, smooth=smooth, rotate=rotate)
    for h in range(H):
        kh = nvfp4.bf16_bits_to_f64(kb[h])
        if smooth:
            kbar = fraction_mean_f32(kh)
            xk = np.array([[np.float32(np.float32(kh[l, c]) - kbar[c]) for c in range(128)]
                           for l in range(L)], dtype=np.float32)
        else:
            kbar = np.zeros(128, np.float32)
            xk = kh.astype(np.float32)
        assert np.array_equal(out["k_mean"][h].view(np.uint32), kbar.view(np.uint32))
        xq = nvfp4.bf16_bits_to_f64(qb[h]).astype(np.float32)
        for name, x in (("q", xq), ("k", xk)):
            bc, bs = brute_prep_rows(x, rotate=rotate)
            assert np.array_equal(out[name + "_codes"][h], bc), name
            assert np.array_equal(out[name + "_scales"][h], bs), name


@pytest.mark.parametrize("smooth,rotate", [(False, False), (True, True)])
def test_prep_toy_width_matches_brute_force_rows(smooth, rotate):
    # 64-channel rows (the pages' toy heads): 6-stage butterfly, RN32(1/8).
    rng = np.random.default_rng(36 + smooth)
    L = 10
    q = (rng.standard_normal((1, L, 64)) * 3).astype(np.float32)
    k = (rng.standard_normal((1, L, 64)) + rng.normal(0, 2, (1, 1, 64))).astype(np.float32)
    qb = (q.view(np.uint32) >> 16).astype(np.uint16)
    kb = (k.view(np.uint32) >> 16).astype(np.uint16)
    out = nvfp4.qk_prep_fp4(qb, kb, smooth=smooth, rotate=rotate)
    assert out["q_codes"].shape == (1, L, 32) and out["q_scales"].shape == (1, L, 4)
    kh = nvfp4.bf16_bits_to_f64(kb[0])
    kbar = fraction_mean_f32(kh) if smooth else np.zeros(64, np.float32)
    xk = np.array([[np.float32(np.float32(kh[l, c]) - kbar[c]) for c in range(64)] for l in range(L)],
                  dtype=np.float32)
    for name, x in (("q", nvfp4.bf16_bits_to_f64(qb[0]).astype(np.float32)), ("k", xk)):
        bc, bs = brute_prep_rows(x, rotate=rotate)
        assert np.array_equal(out[name + "_codes"][0], bc), name
        assert np.array_equal(out[name + "_scales"][0], bs), name


def test_smoothing_is_identity_on_zero_mean_keys():
    # Keys in +- pairs have an exactly zero column mean: smoothing changes
    # nothing, with or without the rotation; Q never depends on smoothing.
    rng = np.random.default_rng(38)
    half = (rng.standard_t(3, (2, 20, 128)) * 4).astype(np.float32)
    kb = (np.concatenate([half, -half], axis=1).view(np.uint32) >> 16).astype(np.uint16)
    qb = (rng.standard_t(3, (2, 40, 128)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    for rotate in (False, True):
        a = nvfp4.qk_prep_fp4(qb, kb, smooth=True, rotate=rotate)
        b = nvfp4.qk_prep_fp4(qb, kb, smooth=False, rotate=rotate)
        assert np.all(a["k_mean"] == 0)
        for key in ("q_codes", "q_scales", "k_codes", "k_scales"):
            assert np.array_equal(a[key], b[key]), (rotate, key)


def test_plain_quantization_is_lossless_on_the_grid():
    # Blocks made of E2M1 values times one E4M3 scale s, each with an entry
    # +-6s: the nearest scale to max/6 is s itself and every value is a grid
    # point, so the plain variant (no smoothing, no rotation) loses nothing.
    rng = np.random.default_rng(39)
    e2 = nvfp4.e2m1_decode_table()
    e4 = nvfp4.e4m3_decode_table()
    n = 50
    sc = rng.integers(0x08, 0x76, (n, 8))           # normal scales with headroom
    cd = rng.integers(0, 16, (n, 128))
    cd[:, ::16] = rng.choice([7, 15], (n, 8))       # one +-6 per block
    x = e2[cd] * np.repeat(e4[sc], 16, axis=1)
    xb = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(nvfp4.bf16_bits_to_f64(xb), x)
    out = nvfp4.qk_prep_fp4(xb[None], xb[None], smooth=False, rotate=False)
    for name in ("q", "k"):
        back = nvfp4.dequant_nvfp4(out[name + "_codes"][0], out[name + "_scales"][0])
        assert np.array_equal(back, x)


def test_rows_and_heads_selection():
    rng = np.random.default_rng(26)
    q = (rng.integers(0, 0x6000, (3, 40, 128))).astype(np.uint16)
    k = (rng.integers(0, 0x6000, (3, 40, 128))).astype(np.uint16)
    full = nvfp4.qk_prep_fp4(q, k)
    part = nvfp4.qk_prep_fp4(q, k, heads=[2], rows=[0, 39])
    for key in ("q_codes", "q_scales", "k_codes", "k_scales"):
        assert np.array_equal(part[key][0], full[key][2][[0, 39]])
    assert np.array_equal(part["k_mean"][0], full["k_mean"][2])


# ---- dequantization and the end-to-end effect -----------------------------------

def test_dequant_products_exact_in_bf16():
    e2 = nvfp4.e2m1_decode_table()
    e4 = nvfp4.e4m3_decode_table()
    for s in e4[:0x7F]:
        for v in e2:
            p = v * s
            b = np.array([p], dtype=np.float32)
            assert float(b[0]) == p
            bf = (b.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
            assert float(bf[0]) == p                # truncating to BF16 loses nothing
            assert p == 0 or abs(p) >= 2.0 ** -10


def test_dequant_layout():
    codes = np.array([[0x21] + [0] * 63], dtype=np.uint8)     # channel0 code1, channel1 code2
    scales = np.array([[0x38] + [0x40] * 7], dtype=np.uint8)  # 1.0, then 2.0
    v = nvfp4.dequant_nvfp4(codes, scales)
    assert v[0, 0] == 0.5 and v[0, 1] == 1.0 and np.all(v[0, 2:] == 0)


def test_transforms_exact_before_quantization():
    # Smoothing and the shared rotation leave softmax(QK^T) and the output
    # unchanged when nothing is quantized.
    rng = np.random.default_rng(27)
    q = rng.standard_t(3, (2, 200, 128))
    k = rng.standard_t(3, (2, 200, 128)) + rng.normal(0, 2, (2, 1, 128))
    v = rng.standard_normal((2, 200, 128))
    hm = sylvester(128) / math.sqrt(128)
    kbar = k.mean(axis=1, keepdims=True)
    o1, _ = attention_fp64(q, k, v, 1 / math.sqrt(128))
    o2, _ = attention_fp64(q @ hm, (k - kbar) @ hm, v, 1 / math.sqrt(128))
    assert np.max(np.abs(o1 - o2)) <= 1e-12


def test_quantized_scores_track_exact_scores():
    # The dequantized, rotated, smoothed Q/K reproduce q.(k - kbar) up to the
    # E2M1 step: each element error is at most half a grid step of its block.
    rng = np.random.default_rng(28)
    H, L = 1, 64
    q = rng.standard_normal((H, L, 128)).astype(np.float32)
    k = (rng.standard_normal((H, L, 128)) + 3.0).astype(np.float32)
    qb = (q.view(np.uint32) >> 16).astype(np.uint16)
    kb = (k.view(np.uint32) >> 16).astype(np.uint16)
    out = nvfp4.qk_prep_fp4(qb, kb)
    qh = nvfp4.dequant_nvfp4(out["q_codes"][0], out["q_scales"][0])
    kh = nvfp4.dequant_nvfp4(out["k_codes"][0], out["k_scales"][0])
    qf = nvfp4.bf16_bits_to_f64(qb[0])
    kf = nvfp4.bf16_bits_to_f64(kb[0]) - out["k_mean"][0].astype(np.float64)
    exact = qf @ kf.T
    approx = qh @ kh.T
    rel = np.linalg.norm(approx - exact) / np.linalg.norm(exact)
    assert rel < 0.2
    hm = sylvester(128) / math.sqrt(128)
    yq = qf @ hm
    sv = nvfp4.e4m3_decode_table()[out["q_scales"][0]]
    err = np.abs(qh - yq).reshape(L, 8, 16)
    assert np.all(err <= sv[..., None] * 1.0 + 1e-6 * np.abs(yq).reshape(L, 8, 16).max())


# ---- planted mistakes -----------------------------------------------------------

def test_planted_tie_mistake_fails():
    bad_mid = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]

    def wrong_codes(y, s):                           # ties always up
        mag = np.abs(np.asarray(y, np.float64))
        s = np.asarray(s, np.float64)[..., None]
        e = sum((mag >= t * s).astype(np.int64) for t in bad_mid)
        return ((np.signbit(y).astype(np.int64) << 3) | e).astype(np.uint8)

    y = np.full((1, 16), 2.5, dtype=np.float32)
    assert wrong_codes(y, np.array([1.0]))[0, 0] != brute_e2m1_code(np.float32(2.5), 1)
    assert nvfp4.e2m1_codes(y, np.array([1.0]))[0, 0] == brute_e2m1_code(np.float32(2.5), 1)


def test_planted_nibble_swap_fails():
    rng = np.random.default_rng(29)
    x = rng.standard_normal((2, 128)).astype(np.float32)
    bc, _ = brute_prep_rows(x)
    swapped = ((bc >> 4) | (bc << 4)).astype(np.uint8)
    assert not np.array_equal(swapped, bc)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    out = nvfp4.qk_prep_fp4(xb[None], xb[None])
    bq, _ = brute_prep_rows(nvfp4.bf16_bits_to_f64(xb).astype(np.float32))
    assert np.array_equal(out["q_codes"][0], bq)
