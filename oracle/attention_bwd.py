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
The row-local and key-subset forms (for sampled checks at full size) equal
the full gradient's rows, and the row statistics equal the forward oracle's
LSE and the row sums of dO * O.

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


def attention_row_stats_fp64(q_rows, k, v, do_rows, scale):
    """Per-query statistics of one head for a set of query rows (row-local):
    LSE_i = m_i + ln sum_j exp(s_ij - m_i) and D_i = sum_j P_ij dP_ij, which is
    sum_c dO_ic O_ic.  q_rows, do_rows [n, d]; k, v [L, d].  Returns (lse [n],
    dsum [n])."""
    q_rows, k, v, do_rows = (np.asarray(t, dtype=np.float64) for t in (q_rows, k, v, do_rows))
    s = (q_rows @ k.T) * float(scale)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    p = e / l
    dp = do_rows @ v.T
    return m[:, 0] + np.log(l[:, 0]), (p * dp).sum(axis=1)


def attention_bwd_keys_fp64(q, k, v, do, scale, keys, lse, dsum, block=4096):
    """dK and dV of one head for a set of key rows: every query contributes,
    through P_ij = exp(s_ij - LSE_i) and dS_ij = P_ij (dP_ij - D_i) with the
    per-query LSE and D of ``attention_row_stats_fp64`` over all L queries.
    q, k, v, do [L, d]; keys: index array; lse, dsum [L].  Queries are taken
    ``block`` at a time only to bound memory.  Returns (dk [n, d], dv [n, d])."""
    q, k, v, do = (np.asarray(t, dtype=np.float64) for t in (q, k, v, do))
    keys = np.asarray(keys, dtype=np.int64)
    kj, vj = k[keys], v[keys]
    dk = np.zeros((keys.size, k.shape[1]))
    dv = np.zeros((keys.size, v.shape[1]))
    sc = float(scale)
    for b0 in range(0, q.shape[0], block):
        sl = slice(b0, min(q.shape[0], b0 + block))
        p = np.exp((q[sl] @ kj.T) * sc - np.asarray(lse, dtype=np.float64)[sl, None])
        ds = p * (do[sl] @ vj.T - np.asarray(dsum, dtype=np.float64)[sl, None])
        dv += p.T @ do[sl]
        dk += sc * (ds.T @ q[sl])
    return dk, dv


def hadamard_orthonormal(d):
    """H_d / sqrt(d): Sylvester's Hadamard matrix (natural order), scaled to
    be orthonormal; symmetric and its own inverse."""
    h = np.array([[1.0]])
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h / np.sqrt(d)


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
        r = hadamard_orthonormal(d)
        dq = dqh @ r.T
        dk = dkh @ r.T
    else:
        dq, dk = dqh, dkh
    if smooth:
        dk = dk - dk.mean(axis=1, keepdims=True)
    return dq, dk, dv
