"""fp64 reference gradients of dense, non-causal softmax attention.  TEST INFRASTRUCTURE ONLY.

What is computed (calculus of the plain definition in ``oracle.attention``).
For one head, with S = sigma Q K^T, P = the row-wise softmax of S, O = P V,
and an upstream gradient dO of O:

    dV   = P^T dO
    dP   = dO V^T
    D_i  = sum_j P_ij dP_ij                (equal to sum_c dO_ic O_ic)
    dS   = P * (dP - D)                    (elementwise, D_i along row i)
    dQ   = sigma dS K
    dK   = sigma dS^T Q

Source: "Pika H3 Flex in FastVideo: 7x Faster, and Near Real Time in 4-bit",
section "NVFP4 QAD" (the model is distilled with the deployed numerics in the
loop) and section "FP4 attention" (the training-time FP4 attention matches the
inference kernel): training through attention needs these gradients.  Softmax
rows are normalised exactly in fp64 (the row max is subtracted only to keep
exp() in range).

Pins (tests/test_oracle_attention_bwd.py): central finite differences of
<dO, O> on tiny inputs; closed forms (one key: dV = dO, dQ = dK = 0; identical
keys: dQ = 0); the exact sums implied by softmax (sum over keys of dK is zero,
sum over keys of dV is the sum over queries of dO); covariance under a shared
orthonormal rotation of Q and K; planted mistakes fail the finite differences.

Inputs are float64 arrays (the exact values of BF16 inputs); numpy's fp64
matmul is the only library primitive used.
"""

import numpy as np


def _softmax_rows(s):
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    return p / p.sum(axis=1, keepdims=True)


def attention_bwd_fp64(q, k, v, do, scale, block=1024):
    """Gradients (dq, dk, dv) of <dO, O> for [H, L, d] float64 tensors.

    Query rows are processed ``block`` at a time only to bound memory; the
    key-side gradients sum the blocks' contributions.
    """
    q, k, v, do = (np.asarray(t, dtype=np.float64) for t in (q, k, v, do))
    if not (q.shape == k.shape == v.shape == do.shape) or q.ndim != 3:
        raise ValueError("q, k, v, do must all be [H, L, d]")
    H, L, d = q.shape
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(H):
        for b0 in range(0, L, block):
            sl = slice(b0, min(L, b0 + block))
            p = _softmax_rows((q[h, sl] @ k[h].T) * float(scale))
            dp = do[h, sl] @ v[h].T
            dsum = (p * dp).sum(axis=1, keepdims=True)
            ds = p * (dp - dsum)
            dv[h] += p.T @ do[h, sl]
            dq[h, sl] = float(scale) * (ds @ k[h])
            dk[h] += float(scale) * (ds.T @ q[h, sl])
    return dq, dk, dv


def attention_bwd_dq_rows_fp64(q_rows, k, v, do_rows, scale):
    """dQ of one head for a set of query rows (row-local: each row needs only
    its own q, dO and all keys).  q_rows, do_rows [n, d]; k, v [L, d]."""
    q_rows, k, v, do_rows = (np.asarray(t, dtype=np.float64) for t in (q_rows, k, v, do_rows))
    p = _softmax_rows((q_rows @ k.T) * float(scale))
    dp = do_rows @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    return float(scale) * (ds @ k)


def fp4qk_bwd_ste_fp64(q_codes, q_scales, k_codes, k_scales, v, do, scale, rotate=True, smooth=True):
    """Training-time gradients of FP4-QK attention with the quantizer passed
    straight through (the gradient of a rounding step taken as the identity).

    The forward is O = attention(Qh, Kh, V) with Qh = dequant(quant(Q R)) and
    Kh = dequant(quant((K - 1 kbar^T) R)), R = H / sqrt(d) (the shared
    orthonormal Hadamard rotation, symmetric, so R^T = R) when ``rotate`` and
    the identity otherwise, kbar the per-channel mean of K over the L tokens
    when ``smooth``.  Then, exactly:
        dV  = the attention gradient at (Qh, Kh, V)
        dQ  = dQh R^T
        dK' = dKh R^T,  dK = dK' - 1 mean_rows(dK')   (the mean's Jacobian)
    Inputs: packed NVFP4 codes/scales [H, L, d/2], [H, L, d/16]; v, do float64
    [H, L, d].  Returns (dq, dk, dv) float64 with respect to the original Q,
    K (before smoothing and rotation) and V.
    """
    from .nvfp4 import dequant_nvfp4

    qh = dequant_nvfp4(q_codes, q_scales)
    kh = dequant_nvfp4(k_codes, k_scales)
    dqh, dkh, dv = attention_bwd_fp64(qh, kh, v, do, scale)
    d = qh.shape[-1]
    if rotate:
        h = np.array([[1.0]])
        while h.shape[0] < d:
            h = np.block([[h, h], [h, -h]])
        r = h / np.sqrt(d)
        dq = dqh @ r.T
        dk = dkh @ r.T
    else:
        dq, dk = dqh, dkh
    if smooth:
        dk = dk - dk.mean(axis=1, keepdims=True)
    return dq, dk, dv


BF16_UNIT = 2.0 ** -8      # unit roundoff of BF16 (8 significant bits, round to nearest)


def attention_bwd_bound_fp64(q, k, v, do, scale, u=BF16_UNIT, block=1024):
    """Elementwise bounds on the error of a BF16 backward (used as test
    tolerances, derived from that arithmetic, not a property of the method).

    Model, with u the BF16 unit roundoff: D is formed from the output O rounded
    to BF16 (|D err| <= u sum_c |dO_ic O_ic|), P and dS enter the products
    rounded to BF16 (u each),
    the products are exact and their fp32 sums add a sqrt(L) 2^-24 relative
    term, and the outputs are rounded to BF16 (u).  With a_i = sum_c |dO_ic
    O_ic| and t = u + sqrt(L) 2^-24:
        B_dQ = sigma (u a_i (P |K|)_ic + t (|dS| |K|)_ic) + u |dQ_ic|
        B_dK = sigma (u (P^T (a |Q|))_jc + t (|dS|^T |Q|)_jc) + u |dK_jc|
        B_dV = t (P^T |dO|)_jc + u |dV_jc|
    Returns (bq, bk, bv) float64 [H, L, d].
    """
    q, k, v, do = (np.asarray(t, dtype=np.float64) for t in (q, k, v, do))
    H, L, d = q.shape
    t = u + np.sqrt(L) * 2.0 ** -24
    bq = np.empty_like(q)
    bk = np.zeros_like(k)
    bv = np.zeros_like(v)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    sc = float(scale)
    for h in range(H):
        ak, aq = np.abs(k[h]), np.abs(q[h])
        for b0 in range(0, L, block):
            sl = slice(b0, min(L, b0 + block))
            p = _softmax_rows((q[h, sl] @ k[h].T) * sc)
            o = p @ v[h]
            dp = do[h, sl] @ v[h].T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            a = np.abs(do[h, sl] * o).sum(axis=1, keepdims=True)
            dq = sc * (ds @ k[h])
            bq[h, sl] = sc * (u * a * (p @ ak) + t * (np.abs(ds) @ ak)) + u * np.abs(dq)
            bk[h] += sc * (u * (p.T @ (a * aq[sl])) + t * (np.abs(ds).T @ aq[sl]))
            bv[h] += t * (p.T @ np.abs(do[h, sl]))
            dk[h] += sc * (ds.T @ q[h, sl])
            dv[h] += p.T @ do[h, sl]
    return bq, bk + u * np.abs(dk), bv + u * np.abs(dv)


def attention_bwd_dq_bound_rows_fp64(q_rows, k, v, do_rows, scale, u=BF16_UNIT):
    """B_dQ of attention_bwd_bound_fp64 for a set of query rows of one head."""
    q_rows, k, v, do_rows = (np.asarray(t, dtype=np.float64) for t in (q_rows, k, v, do_rows))
    L = k.shape[0]
    t = u + np.sqrt(L) * 2.0 ** -24
    sc = float(scale)
    p = _softmax_rows((q_rows @ k.T) * sc)
    o = p @ v
    dp = do_rows @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    a = np.abs(do_rows * o).sum(axis=1, keepdims=True)
    ak = np.abs(k)
    return sc * (u * a * (p @ ak) + t * (np.abs(ds) @ ak)) + u * np.abs(sc * (ds @ k))


def rotate_bound(b, g, u=BF16_UNIT, omitted=None):
    """Bound after rotating back by R = H / sqrt(d): |err(x R)| <= (sum of the
    row's bounds) / sqrt(d) + u |x R| for the result rounded again to BF16.
    ``b``: bounds in the rotated basis, ``g``: the rotated-back gradient;
    ``omitted``: the magnitude of a term the kernel leaves out (the mean-key
    Jacobian's term, zero in exact arithmetic), added to the bound."""
    b = np.asarray(b, dtype=np.float64)
    d = b.shape[-1]
    out = b.sum(axis=-1, keepdims=True) / np.sqrt(d) + u * np.abs(np.asarray(g, dtype=np.float64))
    return out if omitted is None else out + np.abs(omitted)
