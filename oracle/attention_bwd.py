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
