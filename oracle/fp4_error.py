"""Attention error of the FP4-QK variants.  TEST INFRASTRUCTURE ONLY.

Source: "Pika H3 Flex in FastVideo: 7x Faster, and Near Real Time in 4-bit",
section "FP4 attention": quantizing Q and K naively loses accuracy; smoothing K
and the shared Hadamard rotation recover part of it (its table of per-layer
FP4 attention errors on real activations lists plain FP4 above FP4 with both
transforms); its toy heads have 64 channels, 32 keys, Gaussian values, one bias
per channel shared by every key and two channels scaled up.

The pages do not define the error.  Reading used here: the relative Frobenius
norm ||O_fp4 - O_ref||_F / ||O_ref||_F over every head and query row, where
O_ref is the exact attention of the BF16 inputs and O_fp4 the exact attention
of the dequantized NVFP4 Q and K (in the rotated basis when the rotation is on,
which leaves every score unchanged before quantization) with the same V.  Both
are computed in fp64 with ``oracle.attention``; P and V are not rounded here.

Pins (tests/test_oracle_fp4_error.py): zero error on inputs that NVFP4 holds
exactly, and equality with a direct evaluation from the pinned quantizer and
attention on a small case; the ordering the pages report is then checked on the
toy heads and on the long-clip input structure.
"""

import numpy as np

from .attention import attention_fp64
from .nvfp4 import bf16_bits_to_f64, dequant_nvfp4, qk_prep_fp4


def fp4_outputs(q_bits, k_bits, v_bits, scale, smooth=True, rotate=True, rows=None):
    """(O_ref, O_fp4) in fp64 for BF16 bit arrays [H, L, d]; ``rows``: query
    rows to evaluate (default all)."""
    prep = qk_prep_fp4(q_bits, k_bits, smooth=smooth, rotate=rotate)
    q = bf16_bits_to_f64(q_bits)
    k = bf16_bits_to_f64(k_bits)
    v = bf16_bits_to_f64(v_bits)
    qh = dequant_nvfp4(prep["q_codes"], prep["q_scales"])
    kh = dequant_nvfp4(prep["k_codes"], prep["k_scales"])
    o_ref, _ = attention_fp64(q, k, v, scale, rows=rows)
    o_fp4, _ = attention_fp64(qh, kh, v, scale, rows=rows)
    return o_ref, o_fp4


def relative_error(o_approx, o_ref):
    """||o_approx - o_ref||_F / ||o_ref||_F (fp64)."""
    d = np.asarray(o_approx, np.float64) - np.asarray(o_ref, np.float64)
    return float(np.linalg.norm(d.ravel()) / np.linalg.norm(np.asarray(o_ref, np.float64).ravel()))


def fp4_attention_error(q_bits, k_bits, v_bits, scale, smooth=True, rotate=True, rows=None):
    """Relative Frobenius error of FP4-QK attention against exact attention."""
    o_ref, o_fp4 = fp4_outputs(q_bits, k_bits, v_bits, scale, smooth, rotate, rows)
    return relative_error(o_fp4, o_ref)
