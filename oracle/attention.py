"""fp64 reference for dense, non-causal softmax attention.  TEST INFRASTRUCTURE ONLY.

What is computed (the plain definition, no tiling, no online softmax):
for every head h and query row i,

    s_ij  = sigma * sum_c q_ic k_jc            (all keys j of the same head)
    m_i   = max_j s_ij
    p_ij  = exp(s_ij - m_i)
    l_i   = sum_j p_ij
    O_ic  = (sum_j p_ij v_jc) / l_i
    LSE_i = m_i + ln(l_i)

Source: "Pika H3 Flex in FastVideo: 7x Faster, and Near Real Time in 4-bit",
section "What Pika H3 Flex does" (the model uses dense attention) and section
"Faster at BF16" (a 15-second clip is about 109k tokens of one joint sequence,
attention over all of them); section "FP4 attention" for the FP4-QK variant,
where Q and K are replaced by their dequantized NVFP4 values and P, V stay
higher precision.  Subtracting m_i is exact in real arithmetic (softmax ignores
a shift shared by a row) and only keeps exp() in range.

Pins (tests/test_oracle_attention.py): brute-force triple loop on tiny inputs,
softmax rows summing to one, closed forms (L = 1, constant keys, a dominant
logit), invariance to a per-head key shift and to a shared orthonormal rotation
of Q and K, and the LSE identity against a direct log-sum-exp.

Inputs are float64 arrays (the exact values of the BF16 inputs); numpy's fp64
matmul is the only library primitive used.
"""

import numpy as np


def _check(q, k, v):
    if q.ndim != 3 or k.ndim != 3 or v.ndim != 3:
        raise ValueError("q, k, v must be [H, L, d]")
    if k.shape != v.shape or q.shape[0] != k.shape[0] or q.shape[2] != k.shape[2]:
        raise ValueError("shape mismatch: q %s k %s v %s" % (q.shape, k.shape, v.shape))


def attention_rows_fp64(q_rows, k, v, scale):
    """Attention for one head and a set of query rows.

    q_rows [n, d], k [L, d], v [L, d] float64; ``scale`` is sigma.
    Returns (O [n, d], LSE [n]) in float64.
    """
    s = (q_rows @ k.T) * float(scale)          # [n, L]
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ v) / l
    lse = m[:, 0] + np.log(l[:, 0])
    return o, lse


def attention_fp64(q, k, v, scale, rows=None, block=512):
    """Dense non-causal attention over [H, L, d] float64 tensors.

    ``rows``: optional 1-D index array of query rows to compute (the same rows
    for every head); default all rows.  Query rows are processed ``block`` at a
    time only to bound memory; each row's result does not depend on the others.
    Returns (O [H, n, d], LSE [H, n]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    _check(q, k, v)
    H, L, d = q.shape
    idx = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((H, idx.size, d), dtype=np.float64)
    lse = np.empty((H, idx.size), dtype=np.float64)
    for h in range(H):
        for b0 in range(0, idx.size, block):
            sel = idx[b0:b0 + block]
            o, l_ = attention_rows_fp64(q[h, sel], k[h], v[h], scale)
            out[h, b0:b0 + sel.size] = o
            lse[h, b0:b0 + sel.size] = l_
    return out, lse
