"""Pins for the FP4-QK error harness and the ordering the pages report (CPU only).

Method: "Pika H3 Flex in FastVideo: 7x Faster, and Near Real Time in 4-bit",
section "FP4 attention": naive NVFP4 Q/K loses accuracy, smoothing K and the
shared Hadamard rotation recover part of it (its per-layer error table: plain
FP4 above FP4 with both transforms); its toy heads (64 channels, 32 keys,
Gaussian values, a per-channel key bias, two channels scaled up).
"""

import math

import numpy as np

from long_sequence_dense_amd.inputs import f32_to_bf16_bits, make_inputs, toy_heads
from oracle import nvfp4
from oracle.fp4_error import fp4_attention_error, fp4_outputs, relative_error

VARIANTS = [(False, False), (True, False), (False, True), (True, True)]


def grid_inputs(rng, H, L, d):
    """BF16 bits of values NVFP4 holds exactly (E2M1 x E4M3, one +-6 per block)."""
    e2 = nvfp4.e2m1_decode_table()
    e4 = nvfp4.e4m3_decode_table()
    sc = rng.integers(0x28, 0x40, (H, L, d // 16))
    cd = rng.integers(0, 16, (H, L, d))
    cd[..., ::16] = rng.choice([7, 15], (H, L, d // 16))
    x = e2[cd] * np.repeat(e4[sc], 16, axis=-1)
    return f32_to_bf16_bits(x.astype(np.float32))


def test_zero_error_when_nvfp4_is_exact():
    rng = np.random.default_rng(40)
    q = grid_inputs(rng, 2, 48, 128)
    k = grid_inputs(rng, 2, 48, 128)
    v = f32_to_bf16_bits(rng.standard_normal((2, 48, 128)).astype(np.float32))
    assert fp4_attention_error(q, k, v, 0.05, smooth=False, rotate=False) == 0.0
    # the transforms move the values off the grid: some error appears
    assert fp4_attention_error(q, k, v, 0.05, smooth=True, rotate=True) > 0.0


def test_outputs_match_a_direct_loop():
    # Softmax of the dequantized scores, written out with Python loops.
    rng = np.random.default_rng(41)
    H, L, d = 1, 6, 64
    q = f32_to_bf16_bits(rng.standard_normal((H, L, d)).astype(np.float32) * 2)
    k = f32_to_bf16_bits((rng.standard_normal((H, L, d)) + 1.5).astype(np.float32))
    v = f32_to_bf16_bits(rng.standard_normal((H, L, d)).astype(np.float32))
    for smooth, rotate in VARIANTS:
        prep = nvfp4.qk_prep_fp4(q, k, smooth=smooth, rotate=rotate)
        qh = nvfp4.dequant_nvfp4(prep["q_codes"][0], prep["q_scales"][0])
        kh = nvfp4.dequant_nvfp4(prep["k_codes"][0], prep["k_scales"][0])
        vf = nvfp4.bf16_bits_to_f64(v[0])
        _, o_fp4 = fp4_outputs(q, k, v, 0.125, smooth, rotate)
        for i in range(L):
            s = [0.125 * sum(qh[i, c] * kh[j, c] for c in range(d)) for j in range(L)]
            w = [math.exp(t - max(s)) for t in s]
            for c in range(d):
                want = sum(w[j] * vf[j, c] for j in range(L)) / sum(w)
                assert abs(o_fp4[0, i, c] - want) <= 1e-12 * (1 + abs(want))


def test_relative_error_definition():
    a = np.array([[3.0, 4.0]])
    assert relative_error(a, a) == 0.0
    assert relative_error(a + np.array([[4.0, -3.0]]), a) == 1.0     # |(4,-3)| / |(3,4)|
    assert abs(relative_error(a * 1.25, a) - 0.25) < 1e-15


def _errors(d):
    return {fv: fp4_attention_error(d["q"], d["k"], d["v"], d["scale"], *fv) for fv in VARIANTS}


def test_toy_heads_plain_worse_than_smooth_and_rotate():
    t = toy_heads(64)
    t["scale"] = 1.0 / 8.0
    e = _errors(t)
    assert e[(True, True)] < 0.8 * e[(False, False)], e


def test_long_clip_structure_plain_worse_than_smooth_and_rotate():
    # Student-t(3) Q/K with three x20 channels, at a small length.
    d = make_inputs("fp4", H=2, L=512)
    e = _errors(d)
    assert e[(True, True)] < 0.8 * e[(False, False)], e


def test_shared_key_bias_is_what_smoothing_removes():
    # With a per-channel key bias and no outliers, smoothing alone recovers
    # most of the loss; the rotation alone does not.
    d = make_inputs("tiny", H=2, L=512)
    e = _errors(d)
    assert e[(True, False)] < 0.8 * e[(False, False)], e
    assert e[(False, True)] > 0.9 * e[(False, False)], e
