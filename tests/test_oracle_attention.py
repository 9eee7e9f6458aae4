"""Pins for the fp64 attention oracle (CPU only).

The oracle is checked against things other than itself: a pure-Python triple
loop, softmax normalisation, closed forms, and the two exact invariances the
FP4 method relies on ("Pika H3 Flex in FastVideo: 7x Faster, and Near Real
Time in 4-bit", section "FP4 attention": mean-key subtraction and a shared
orthonormal rotation leave the attention unchanged).  A few planted mistakes in
a copy of the oracle must fail these pins.
"""

import math

import numpy as np
import pytest

from oracle.attention import attention_fp64, attention_rows_fp64


def brute_attention(q, k, v, scale):
    """Triple loop straight from the definition, Python floats only."""
    H, L, d = q.shape
    out = np.zeros((H, L, d))
    lse = np.zeros((H, L))
    for h in range(H):
        for i in range(L):
            s = [scale * sum(q[h, i, c] * k[h, j, c] for c in range(d)) for j in range(L)]
            m = max(s)
            p = [math.exp(x - m) for x in s]
            den = sum(p)
            for c in range(d):
                out[h, i, c] = sum(p[j] * v[h, j, c] for j in range(L)) / den
            lse[h, i] = m + math.log(den)
    return out, lse


def sylvester(n):
    h = np.array([[1]], dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


@pytest.mark.parametrize("L,d", [(5, 16), (9, 64), (4, 128)])
def test_brute_force_tiny(L, d):
    rng = np.random.default_rng(L * 1000 + d)
    q, k, v = (rng.standard_normal((2, L, d)) for _ in range(3))
    scale = 1.0 / math.sqrt(d)
    o, lse = attention_fp64(q, k, v, scale)
    ob, lseb = brute_attention(q, k, v, scale)
    assert np.max(np.abs(o - ob)) <= 1e-12
    assert np.max(np.abs(lse - lseb)) <= 1e-12


def test_rows_subset_matches_full():
    rng = np.random.default_rng(7)
    q, k, v = (rng.standard_normal((2, 300, 32)) for _ in range(3))
    rows = np.array([0, 5, 128, 299])
    o, lse = attention_fp64(q, k, v, 0.3)
    os_, lses = attention_fp64(q, k, v, 0.3, rows=rows, block=3)
    # BLAS may block a 3-row product differently from a 300-row one
    assert np.max(np.abs(o[:, rows] - os_)) <= 1e-14
    assert np.max(np.abs(lse[:, rows] - lses)) <= 1e-13


def test_softmax_rows_sum_to_one():
    # With V = identity, row i of O is the softmax row p_i / l_i itself.
    rng = np.random.default_rng(3)
    L = 48
    q = rng.standard_normal((1, L, L)) * 3
    k = rng.standard_normal((1, L, L)) * 3
    v = np.eye(L)[None]
    o, _ = attention_fp64(q, k, v, 0.5)
    assert np.all(o >= 0)
    assert np.max(np.abs(o.sum(axis=-1) - 1.0)) <= 1e-14


def test_single_key_returns_its_value():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((3, 1, 128))
    k = rng.standard_normal((3, 1, 128))
    v = rng.standard_normal((3, 1, 128))
    o, lse = attention_fp64(q, k, v, 1.0 / math.sqrt(128))
    assert np.array_equal(o, v)
    s = np.einsum("hld,hld->hl", q, k) / math.sqrt(128)
    assert np.max(np.abs(lse - s)) <= 1e-14


def test_zero_query_and_identical_keys_average_v():
    rng = np.random.default_rng(5)
    L = 257
    v = rng.standard_normal((1, L, 64))
    k = rng.standard_normal((1, L, 64))
    q0 = np.zeros((1, 4, 64))
    o, lse = attention_fp64(q0, k, v, 1.0)
    assert np.max(np.abs(o - v.mean(axis=1, keepdims=True))) <= 1e-14
    assert np.max(np.abs(lse - math.log(L))) <= 1e-13
    q = rng.standard_normal((1, 4, 64))
    kc = np.repeat(rng.standard_normal((1, 1, 64)), L, axis=1)
    o2, _ = attention_fp64(q, kc, v, 1.0)
    assert np.max(np.abs(o2 - v.mean(axis=1, keepdims=True))) <= 1e-14


def test_dominant_logit_selects_value_exactly():
    rng = np.random.default_rng(6)
    L, d = 64, 16
    k = rng.standard_normal((1, L, d))
    k[0, 17] = 0.0
    k[0, 17, 0] = 1000.0
    q = np.zeros((1, 1, d))
    q[0, 0, 0] = 1.0
    v = rng.standard_normal((1, L, d))
    o, _ = attention_fp64(q, k, v, 1.0)          # gap > 800: other weights underflow
    assert np.array_equal(o[0, 0], v[0, 17])


def test_mean_key_shift_invariance():
    rng = np.random.default_rng(8)
    q, k, v = (rng.standard_normal((2, 200, 128)) for _ in range(3))
    k = k + rng.normal(0, math.sqrt(2), (2, 1, 128))
    kbar = k.mean(axis=1, keepdims=True)
    o1, _ = attention_fp64(q, k, v, 1 / math.sqrt(128))
    o2, _ = attention_fp64(q, k - kbar, v, 1 / math.sqrt(128))
    o3, _ = attention_fp64(q, k + 5.0 * rng.standard_normal((2, 1, 128)), v, 1 / math.sqrt(128))
    assert np.max(np.abs(o1 - o2)) <= 1e-12
    assert np.max(np.abs(o1 - o3)) <= 1e-12


def test_shared_orthonormal_rotation_invariance():
    rng = np.random.default_rng(9)
    q, k, v = (rng.standard_normal((2, 150, 128)) for _ in range(3))
    hm = sylvester(128).astype(np.float64) / math.sqrt(128)
    assert np.max(np.abs(hm @ hm.T - np.eye(128))) <= 1e-15
    o1, l1 = attention_fp64(q, k, v, 1 / math.sqrt(128))
    o2, l2 = attention_fp64(q @ hm, k @ hm, v, 1 / math.sqrt(128))
    assert np.max(np.abs(o1 - o2)) <= 1e-12
    assert np.max(np.abs(l1 - l2)) <= 1e-12
    dots = np.einsum("ld,ld->l", q[0], k[0])
    dots_r = np.einsum("ld,ld->l", q[0] @ hm, k[0] @ hm)
    assert np.max(np.abs(dots - dots_r) / np.maximum(1.0, np.abs(dots))) <= 1e-13


def test_lse_matches_library_logsumexp():
    from scipy.special import logsumexp
    rng = np.random.default_rng(10)
    q, k, v = (rng.standard_normal((1, 90, 32)) for _ in range(3))
    _, lse = attention_fp64(q, k, v, 0.7)
    s = 0.7 * (q[0] @ k[0].T)
    assert np.max(np.abs(lse[0] - logsumexp(s, axis=1))) <= 1e-13


# ---- planted mistakes: each mutant of the row kernel must fail a pin ------------

def _mutant_no_scale(q_rows, k, v, scale):
    return attention_rows_fp64(q_rows, k, v, 1.0)


def _mutant_k_as_v(q_rows, k, v, scale):
    return attention_rows_fp64(q_rows, k, k, scale)


def _mutant_no_normalise(q_rows, k, v, scale):
    s = (q_rows @ k.T) * scale
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    return p @ v, m[:, 0]


def _mutant_transposed_q(q_rows, k, v, scale):
    s = (q_rows[:, ::-1] @ k.T) * scale
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    return (p @ v) / l, m[:, 0] + np.log(l[:, 0])


@pytest.mark.parametrize("mutant", [_mutant_no_scale, _mutant_k_as_v,
                                    _mutant_no_normalise, _mutant_transposed_q])
def test_planted_mistakes_fail_brute_force(mutant, monkeypatch):
    import oracle.attention as att
    monkeypatch.setattr(att, "attention_rows_fp64", mutant)
    rng = np.random.default_rng(11)
    q, k, v = (rng.standard_normal((1, 6, 16)) for _ in range(3))
    o, _ = att.attention_fp64(q, k, v, 0.25)
    ob, _ = brute_attention(q, k, v, 0.25)
    assert np.max(np.abs(o - ob)) > 1e-6
