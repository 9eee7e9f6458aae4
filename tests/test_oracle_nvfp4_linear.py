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
