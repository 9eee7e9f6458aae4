"""Reference NVFP4 W4A4 linear layer.  TEST INFRASTRUCTURE ONLY.

Source: "Pika H3 Flex in FastVideo: 7x Faster, and Near Real Time in 4-bit",
section "NVFP4 QAD": every attention and feed-forward linear runs with 4-bit
weights and activations, one 8-bit scale per 16 values; activation scales are
static, set per layer from calibration (a clipping level).  The block format is
the one of section "FP4 attention" (E2M1 values, E4M3 scale per 16).

Readings (the pages give no numerics for these steps):
  * a tensor has one float32 global scale g > 0 besides its block scales: the
    quantizer sees x' = RN32(x / g), the correctly rounded float32 quotient
    (one IEEE division; a quotient beyond the float32 range becomes +-inf),
    quantizes x' by P5-P7 of oracle.nvfp4 (blocks of 16 consecutive values
    along each row), and a code e with block scale s stands for e * s * g.
    With g = 1 this is exactly the Q/K quantizer without rotation.  Values
    beyond 6 * 448 * g saturate (an infinite x' takes scale 448 and code +-6):
    g sets the clipping level.
  * Y = X^ W^T computed from the exact dequantized values, in fp64 here;
    the GPU rounds Y to BF16.

Pins (tests/test_oracle_nvfp4_linear.py): RN32(x / g) against an exact
rational (Fraction) rounding to float32 with ties to even, on random inputs,
on quotients placed next to float32 rounding boundaries, in the subnormal
range and past the overflow threshold; g = 1 equals the Q/K quantizer without
transforms; g = a power of two shifts only the scales; clipping saturates at
6 * 448 * g; the product equals a plain loop on tiny shapes.
"""

import numpy as np

from .nvfp4 import _quantize_rows, dequant_nvfp4


def scaled_input(x, global_scale=1.0):
    """x' = RN32(x / g) for float values x (exact in BF16, hence in float32)
    and the float32 global scale g: the IEEE fp64 quotient of the two, rounded
    to float32.  For / on float32 operands that double rounding equals the one
    IEEE float32 division (Figueroa, 53 >= 2*24+2), subnormal and overflowing
    (+-inf) results included."""
    x = np.asarray(x, dtype=np.float64)
    g = np.float64(np.float32(global_scale))
    with np.errstate(over="ignore"):
        return (x / g).astype(np.float32)


def quantize(x, global_scale=1.0):
    """x: float values exactly representable in BF16, [rows, K] with K a
    multiple of 16.  Returns (codes [rows, K/2] u8, scales [rows, K/16] u8)."""
    return _quantize_rows(scaled_input(x, global_scale), rotate=False)


def dequantize(codes, scales, global_scale=1.0):
    return dequant_nvfp4(codes, scales) * np.float64(np.float32(global_scale))


def linear(x_codes, x_scales, x_global, w_codes, w_scales, w_global):
    """Y = X^ W^T in fp64 from the exact dequantized operands: [M, N]."""
    xh = dequantize(x_codes, x_scales, x_global)
    wh = dequantize(w_codes, w_scales, w_global)
    return xh @ wh.T


def linear_bound(x_codes, x_scales, x_global, w_codes, w_scales, w_global, u=2.0 ** -8):
    """Elementwise error bound of a BF16-MFMA computation of ``linear`` (test
    tolerance): products of the exact BF16 operands are exact, their fp32 sum
    over K adds sqrt(K) 2^-24 sum |terms|, the product of the two global
    scales and its application to the sum are fp32 roundings (2^-24 each), the
    output is rounded to BF16 (u)."""
    xh = dequantize(x_codes, x_scales, x_global)
    wh = dequantize(w_codes, w_scales, w_global)
    K = xh.shape[1]
    y = xh @ wh.T
    return np.sqrt(K) * 2.0 ** -24 * (np.abs(xh) @ np.abs(wh).T) + (u + 2.0 ** -23) * np.abs(y)
