"""Pins for the fp64 attention-gradient oracle (CPU only).

The gradients are checked against central finite differences of the forward
oracle's <dO, O> (itself pinned by brute force), against closed forms and
exact sums that follow from softmax rows summing to one, and against the
covariance of dQ, dK under a shared orthonormal rotation of Q and K (the
rotation of "Pika H3 Flex in FastVideo: 7x Faster, and Near Real Time in
4-bit", section "FP4 attention").  Planted mistakes in a copy of the gradient
formulas fail the finite differences.
"""

import math

import numpy as np
import pytest

from oracle.attention import attention_fp64
from oracle.attention_bwd import attention_bwd_dq_rows_fp64, attention_bwd_fp64


def loss(q, k, v, do, scale):
    o, _ = attention_fp64(q, k, v, scale)
    return float((o * do).sum())


def finite_diff(q, k, v, do, scale, which, h=1e-6):
    args = {"q": q, "k": k, "v": v}
    x = args[which]
    g = np.zeros_like(x)
    for idx in np.ndindex(*x.shape):
        xp = x.copy()
        xm = x.copy()
        xp[idx] += h
        xm[idx] -= h
        ap = dict(args, **{which: xp})
        am = dict(args, **{which: xm})
        g[idx] = (loss(ap["q"], ap["k"], ap["v"], do, scale) - loss(am["q"], am["k"], am["v"], do, scale)) / (2 * h)
    return g


def sylvester(n):
    h = np.array([[1]], dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def tiny(seed, H=1, L=5, d=8):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((H, L, d)) for _ in range(4)]


@pytest.mark.parametrize("seed,L,d", [(0, 5, 8), (1, 3, 16), (2, 7, 4)])
def test_gradients_match_finite_differences(seed, L, d):
    q, k, v, do = tiny(seed, 1, L, d)
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = attention_bwd_fp64(q, k, v, do, scale)
    for name, g in (("q", dq), ("k", dk), ("v", dv)):
        fd = finite_diff(q, k, v, do, scale, name)
        assert np.max(np.abs(g - fd)) <= 1e-7 * (1 + np.max(np.abs(fd))), name


def test_single_key_closed_form():
    q, k, v, do = tiny(3, 2, 1, 16)
    dq, dk, dv = attention_bwd_fp64(q, k, v, do, 0.3)
    assert np.array_equal(dv, do)
    assert np.all(dq == 0) and np.all(dk == 0)


def test_identical_keys_give_zero_dq():
    q, k, v, do = tiny(4, 1, 6, 8)
    k[:] = k[:, :1]
    dq, _, _ = attention_bwd_fp64(q, k, v, do, 0.5)
    assert np.max(np.abs(dq)) <= 1e-15


def test_softmax_sums():
    # every softmax row sums to one: sum_j dS_ij = 0, so the key-side gradient
    # dK sums to zero over keys, and dV sums over keys to the sum of dO.
    rng = np.random.default_rng(5)
    q, k, v, do = (rng.standard_normal((2, 300, 32)) for _ in range(4))
    dq, dk, dv = attention_bwd_fp64(q, k, v, do, 0.2, block=77)
    assert np.max(np.abs(dk.sum(axis=1))) <= 1e-11 * np.max(np.abs(dk)) * 300
    assert np.max(np.abs(dv.sum(axis=1) - do.sum(axis=1))) <= 1e-11 * 300


def test_rotation_covariance():
    rng = np.random.default_rng(6)
    q, k, v, do = (rng.standard_normal((1, 40, 16)) for _ in range(4))
    hm, _ = np.linalg.qr(rng.standard_normal((16, 16)))
    dq, dk, dv = attention_bwd_fp64(q, k, v, do, 0.25)
    dq2, dk2, dv2 = attention_bwd_fp64(q @ hm, k @ hm, v, do, 0.25)
    assert np.max(np.abs(dq2 - dq @ hm)) <= 1e-12
    assert np.max(np.abs(dk2 - dk @ hm)) <= 1e-12
    assert np.max(np.abs(dv2 - dv)) <= 1e-12


def test_blocking_and_rows_agree():
    rng = np.random.default_rng(7)
    q, k, v, do = (rng.standard_normal((2, 130, 16)) for _ in range(4))
    a = attention_bwd_fp64(q, k, v, do, 0.3)
    b = attention_bwd_fp64(q, k, v, do, 0.3, block=17)
    for x, y in zip(a, b):
        assert np.max(np.abs(x - y)) <= 1e-12
    rows = np.array([0, 64, 129])
    dqr = attention_bwd_dq_rows_fp64(q[1, rows], k[1], v[1], do[1, rows], 0.3)
    assert np.max(np.abs(dqr - a[0][1, rows])) <= 1e-12


def test_planted_mistakes_fail():
    q, k, v, do = tiny(8, 1, 5, 8)
    scale = 1.0 / math.sqrt(8)
    fdq = finite_diff(q, k, v, do, scale, "q")
    fdk = finite_diff(q, k, v, do, scale, "k")
    s = scale * q[0] @ k[0].T
    p = np.exp(s - s.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    dp = do[0] @ v[0].T
    good = p * (dp - (p * dp).sum(1, keepdims=True))
    no_d = p * dp                                          # D term dropped
    wrong = [scale * no_d @ k[0], good @ k[0], scale * good.T @ k[0]]   # no D; no scale; dS transposed
    for w in wrong:
        assert np.max(np.abs(w - fdq[0])) > 1e-3
    assert np.max(np.abs(scale * good @ q[0] - fdk[0])) > 1e-3   # dS instead of dS^T for dK


# ---- training-time FP4-QK gradients (straight-through quantizer) -------------

def test_fp4_ste_equals_plain_gradient_when_quantization_is_exact():
    # Values NVFP4 holds exactly (E2M1 x E4M3, a +-6 in every block), no
    # transforms: the straight-through gradient is the plain gradient.
    from oracle import nvfp4
    from oracle.attention_bwd import fp4qk_bwd_ste_fp64
    rng = np.random.default_rng(9)
    e2 = nvfp4.e2m1_decode_table()
    e4 = nvfp4.e4m3_decode_table()

    def grid(n):
        sc = rng.integers(0x28, 0x38, (1, n, 8))
        cd = rng.integers(0, 16, (1, n, 128))
        cd[..., ::16] = rng.choice([7, 15], (1, n, 8))
        return e2[cd] * np.repeat(e4[sc], 16, axis=-1)

    q, k = grid(24), grid(24)
    v, do = rng.standard_normal((1, 24, 128)), rng.standard_normal((1, 24, 128))
    bits = lambda x: (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    prep = nvfp4.qk_prep_fp4(bits(q), bits(k), smooth=False, rotate=False)
    got = fp4qk_bwd_ste_fp64(prep["q_codes"], prep["q_scales"], prep["k_codes"], prep["k_scales"], v, do, 0.05,
                             rotate=False, smooth=False)
    want = attention_bwd_fp64(q, k, v, do, 0.05)
    for g, w in zip(got, want):
        assert np.max(np.abs(g - w)) <= 1e-12 * (1 + np.max(np.abs(w)))


def test_fp4_ste_rotation_and_mean_terms():
    # The rotation is undone by the same orthonormal matrix (it is symmetric),
    # and the mean subtraction's Jacobian is I - 11^T / L, checked here by
    # finite differences of the linear map K -> K - mean(K) composed with the
    # rotation; the attention gradient itself sums to zero over keys, so the
    # mean term only removes rounding.
    from oracle import nvfp4
    from oracle.attention_bwd import fp4qk_bwd_ste_fp64
    rng = np.random.default_rng(10)
    q = rng.standard_normal((1, 20, 128)).astype(np.float32)
    k = (rng.standard_normal((1, 20, 128)) + 2.0).astype(np.float32)
    bits = lambda x: (x.view(np.uint32) >> 16).astype(np.uint16)
    prep = nvfp4.qk_prep_fp4(bits(q), bits(k))
    v, do = rng.standard_normal((1, 20, 128)), rng.standard_normal((1, 20, 128))
    dq, dk, dv = fp4qk_bwd_ste_fp64(prep["q_codes"], prep["q_scales"], prep["k_codes"], prep["k_scales"], v, do, 0.1)
    qh = nvfp4.dequant_nvfp4(prep["q_codes"], prep["q_scales"])
    kh = nvfp4.dequant_nvfp4(prep["k_codes"], prep["k_scales"])
    dqh, dkh, dv2 = attention_bwd_fp64(qh, kh, v, do, 0.1)
    hm = sylvester(128) / math.sqrt(128)
    assert np.max(np.abs(hm @ hm - np.eye(128))) <= 1e-12
    assert np.max(np.abs(dq @ hm - dqh)) <= 1e-12 * np.max(np.abs(dqh))     # rotating back recovers dQh
    assert np.array_equal(dv, dv2)
    # chain rule through f(K) = (K - mean(K)) R by finite differences of a
    # linear functional <G, f(K)> with G = dKh
    g = dkh[0]
    f = lambda kk: float((g * ((kk - kk.mean(axis=0, keepdims=True)) @ hm)).sum())
    k0 = rng.standard_normal((20, 128))
    fd = np.zeros_like(k0)
    for idx in [(0, 0), (3, 17), (19, 127), (7, 64)]:
        e = np.zeros_like(k0)
        e[idx] = 1e-3
        fd[idx] = (f(k0 + e) - f(k0 - e)) / 2e-3
        assert abs(fd[idx] - dk[0][idx]) <= 1e-9 * (1 + abs(dk[0][idx]))
    assert np.max(np.abs(dkh.sum(axis=1))) <= 1e-12 * np.abs(dkh).sum()


def test_row_stats_and_key_subset_equal_the_full_gradient():
    # the forms used for sampled checks at full size: per-query LSE and D over
    # all keys, then dK, dV of a subset of keys from every query
    from oracle.attention_bwd import attention_bwd_keys_fp64, attention_row_stats_fp64
    rng = np.random.default_rng(40)
    L, d = 300, 16
    q, k, v, do = (rng.standard_normal((1, L, d)) * s for s in (2.0, 2.0, 1.0, 1.0))
    scale = 0.7
    dq, dk, dv = attention_bwd_fp64(q, k, v, do, scale)
    lse, dsum = attention_row_stats_fp64(q[0], k[0], v[0], do[0], scale)
    o, lse_ref = attention_fp64(q, k, v, scale)
    assert np.allclose(lse, lse_ref[0], rtol=0, atol=1e-12)
    assert np.allclose(dsum, (do[0] * o[0]).sum(axis=1), rtol=1e-12, atol=1e-12)
    keys = np.array([0, 1, 77, 150, 299])
    gk, gv = attention_bwd_keys_fp64(q[0], k[0], v[0], do[0], scale, keys, lse, dsum, block=64)
    assert np.allclose(gk, dk[0, keys], rtol=1e-10, atol=1e-12)
    assert np.allclose(gv, dv[0, keys], rtol=1e-10, atol=1e-12)
    # a D taken from another row, or an LSE off by a constant, changes dK
    bad_k, _ = attention_bwd_keys_fp64(q[0], k[0], v[0], do[0], scale, keys, lse, np.roll(dsum, 1))
    assert not np.allclose(bad_k, dk[0, keys], rtol=1e-3, atol=1e-6)
    _, bad_v = attention_bwd_keys_fp64(q[0], k[0], v[0], do[0], scale, keys, lse + 0.01, dsum)
    assert not np.allclose(bad_v, dv[0, keys], rtol=1e-3, atol=1e-6)


def test_hadamard_orthonormal():
    from oracle.attention_bwd import hadamard_orthonormal
    for d in (2, 16, 128):
        r = hadamard_orthonormal(d)
        assert np.allclose(r @ r, np.eye(d), atol=1e-14) and np.array_equal(r, r.T)
        assert np.array_equal(np.rint(r * np.sqrt(d)).astype(np.int64), sylvester(d))
