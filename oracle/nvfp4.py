"""Reference Q/K preparation for FP4-QK attention.  TEST INFRASTRUCTURE ONLY.

Source: "Pika H3 Flex in FastVideo: 7x Faster, and Near Real Time in 4-bit",
section "FP4 attention": before quantizing, each head's mean key is subtracted
(exact for softmax because every score of a query moves by the same amount),
Q and K are both multiplied by one shared orthonormal Hadamard matrix (exact
because the rotation preserves dot products), and both are quantized to NVFP4:
4-bit E2M1 values, one E4M3 scale per 16 channels, global scale 1.  Section
"NVFP4 QAD" gives the block size (one 8-bit scale per 16 values).  The figure
caption on the yuxiaoba review ("Decoding can cost more than denoising") shows
a 16-value key block whose small entry rounds to zero.

The pages give no numerics for these steps, so this module fixes one procedure
(one plain reading of each step, stated below).  For head h and token row l,
P1-P2 on K only:

P0  x_c = the BF16 input as a real number (exact).
P1  kbar_c = RN32( RN64(S_c) / L ),  S_c = exact sum over the L tokens of
    K[h, :, c]  (``math.fsum`` returns RN64 of the exact sum; the division is
    one IEEE fp64 division).
P2  x_c <- RN32(x_c - kbar_c).
P3  7-stage butterfly in Sylvester (natural) order: for s = 0..6, for every
    channel i with bit s clear and j = i + 2^s,
    (x_i, x_j) <- (RN32(x_i + x_j), RN32(x_i - x_j)).
    Exactly, this is x H with H[i][j] = (-1)^popcount(i & j).
P4  y_c = RN32(x_c * c),  c = RN32(1/sqrt(128)) = 0x3DB504F3, which makes the
    rotation orthonormal up to that rounding.
P5  per 16-channel block b: a = max_c |y_c|; the scale s is the E4M3 (OCP,
    bias 7, max 448, no infinities) value nearest to the exact a / 6, ties to
    the even code, values above 448 saturate to 448 (code 0x7E).
P6  codes: if s == 0 every code is the signed zero signbit(y)<<3; otherwise the
    E2M1 magnitude index e nearest to the exact |y| / s, ties to the even
    index, quotients above 6 saturate to index 7; code = signbit(y)<<3 | e.
P7  byte j of a row = code[2j] | code[2j+1] << 4; scale byte = E4M3 bits of s.

Ablation variants (same section: quantizing naively costs accuracy, and the
two exact transforms recover most of it; its table of per-layer errors lists
plain FP4 above FP4 with smoothed K and the Hadamard rotation).  ``smooth``
off skips P1-P2 (K is quantized as given and the reported mean is zero);
``rotate`` off skips P3-P4 (y = x, blocks of consecutive original channels).
The defaults (both on) are the method.  For the pages' toy heads the row
length d may also be 64 (four blocks; with the rotation, a 6-stage butterfly
and RN32(1/sqrt(64)) = 1/8).

Arithmetic: values are held in float64.  Each RN32 is a float64 operation
followed by a cast to float32.  For +, -, * and / of float32 operands this
double rounding equals the single IEEE float32 operation because 53 >= 2*24+2
(S. Figueroa, "When is double rounding innocuous?", SIGNUM 1995).  The rounding
decisions of P5 and P6 are exact comparisons: every threshold (a midpoint times
6, or an E2M1 midpoint times s) has at most 7 significant bits, so it is exact.

Pins (tests/test_oracle_nvfp4.py): all 256 E4M3 and 16 E2M1 codes against
their bit-field definitions; the scale and code rounding against a Fraction
brute-force argmin on random and adversarial inputs, including every exact tie;
the butterfly against the integer Sylvester matrix product on small-integer
inputs (where every fp32 operation is exact) and H H^T = 128 I; the mean against
a Fraction exact sum; the zero-rounding block of the figure caption; exact BF16
representability of every dequantized product; end-to-end dot-product and
attention invariance of the transforms before quantization.
"""

import math

import numpy as np

D_HEAD = 128
BLOCK = 16

# RN32(1/sqrt(128)): the float32 nearest to 2**-3.5.
HADAMARD_SCALE_F32 = np.float32(np.frombuffer(np.uint32(0x3DB504F3).tobytes(), dtype=np.float32)[0])

# E2M1 magnitudes by index (exponent 2 bits bias 1, mantissa 1 bit).
_E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
# Midpoints between consecutive E2M1 magnitudes.
_E2M1_MID = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float64)


def bf16_bits_to_f64(bits):
    """Exact value of BF16 bit patterns (uint16 array) as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f32_bits(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)


def e4m3_decode_table():
    """Values of all 256 OCP FP8 E4M3 codes (sign, 4-bit exponent bias 7,
    3-bit mantissa; exponent 0 is subnormal m/8 * 2^-6; S.1111.111 is NaN)."""
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            out[code] = np.nan
        elif e == 0:
            out[code] = sign * (m / 8.0) * 2.0 ** -6
        else:
            out[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


def e2m1_decode_table():
    """Values of all 16 FP4 E2M1 codes (sign bit 3, 2-bit exponent bias 1,
    1-bit mantissa; exponent 0 is subnormal m/2)."""
    out = np.empty(16, dtype=np.float64)
    for code in range(16):
        sign = -1.0 if code & 0x8 else 1.0
        e = (code >> 1) & 0x3
        m = code & 0x1
        out[code] = sign * (m / 2.0 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1))
    return out


_E4M3 = e4m3_decode_table()
_E4M3_POS = _E4M3[:0x7F]                       # codes 0x00..0x7E, increasing
_E4M3_MID6 = 6.0 * 0.5 * (_E4M3_POS[:-1] + _E4M3_POS[1:])   # 126 thresholds, exact
_E2M1 = e2m1_decode_table()


def kmean_exact(k_head):
    """P1: per-channel mean key of one head, k_head [L, d] float64 (exact BF16
    values).  Returns float32 [d] = RN32(RN64(exact column sum) / L)."""
    L, d = k_head.shape
    out = np.empty(d, dtype=np.float32)
    for c in range(d):
        s = math.fsum(k_head[:, c].tolist())
        out[c] = np.float32(s / L)
    return out


def hadamard_scale_f32(n):
    """P4's constant for rows of length n (a power of two): RN32(1/sqrt(n)).
    1/sqrt(n) is irrational or a power of two, so rounding its fp64 value to
    float32 cannot hit a float32 midpoint and equals the direct rounding."""
    if n < 1 or n & (n - 1):
        raise ValueError("rotation length must be a power of two")
    return np.float32(1.0 / math.sqrt(n))


def hadamard_butterfly_fp32(x):
    """P3: in-order Sylvester butterfly over the last axis (length 128, or
    another power of two) with a float32 rounding after every add and
    subtract.  ``x`` holds float32 values (any float dtype); returns float32."""
    x = np.asarray(x, dtype=np.float32).copy()
    n = x.shape[-1]
    if n < 2 or n & (n - 1):
        raise ValueError("butterfly length must be a power of two")
    lead = x.shape[:-1]
    for s in range(n.bit_length() - 1):
        h = 1 << s
        v = x.reshape(lead + (n // (2 * h), 2, h)).astype(np.float64)
        a = v[..., 0, :]
        b = v[..., 1, :]
        new = np.empty_like(v)
        new[..., 0, :] = a + b
        new[..., 1, :] = a - b
        x = new.astype(np.float32).reshape(lead + (n,))
    return x


def e4m3_scale_code(amax):
    """P5: E4M3 code of the value nearest to amax/6 (amax >= 0, float32
    values), ties to the even code, saturating at 448.  Counts the midpoints
    passed: a tie at a midpoint between codes j and j+1 goes up only when j+1
    is even."""
    a = np.asarray(amax, dtype=np.float32).astype(np.float64)
    code = np.zeros(a.shape, dtype=np.int64)
    for j, thr in enumerate(_E4M3_MID6):
        if j % 2 == 0:
            code += (a > thr)
        else:
            code += (a >= thr)
    return code.astype(np.uint8)


def e2m1_codes(y, s):
    """P6: 4-bit codes for y [..., 16] (float32 values) with block scale values
    s [...] (float64, non-negative E4M3 values)."""
    y = np.asarray(y, dtype=np.float32)
    mag = np.abs(y).astype(np.float64)
    s = np.asarray(s, dtype=np.float64)[..., None]
    e = np.zeros(y.shape, dtype=np.int64)
    for k, t in enumerate(_E2M1_MID):
        thr = t * s                      # exact: <= 7 significant bits
        if k % 2 == 0:
            e += (mag > thr)
        else:
            e += (mag >= thr)
    e = np.where(s == 0.0, 0, e)
    sign = np.signbit(y).astype(np.int64) << 3
    return (sign | e).astype(np.uint8)


def _quantize_rows(x_f32, rotate=True):
    """P3-P7 (P5-P7 only when ``rotate`` is off) for rows of d float32
    values; returns (codes [n, d/2] u8, scales [n, d/16] u8)."""
    n, d = x_f32.shape
    if rotate:
        hx = hadamard_butterfly_fp32(x_f32)
        y = (hx.astype(np.float64) * np.float64(hadamard_scale_f32(d))).astype(np.float32)
    else:
        y = np.asarray(x_f32, dtype=np.float32)
    yb = y.reshape(n, d // BLOCK, BLOCK)
    amax = np.abs(yb).max(axis=-1)
    scode = e4m3_scale_code(amax)
    sval = _E4M3[scode]
    codes = e2m1_codes(yb, sval).reshape(n, d)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, scode


def qk_prep_fp4(q_bits, k_bits, heads=None, rows=None, smooth=True, rotate=True):
    """The full preparation P0-P7 for BF16 Q and K given as uint16 bit arrays
    [H, L, d] (d = 128; 64 for the toy heads).

    ``heads``: optional head indices to process (default all); ``rows``:
    optional token-row indices whose codes are returned (the mean always uses
    every row of K).  ``smooth`` / ``rotate``: the ablation switches of the
    module header.  Returns a dict with q_codes [h, n, d/2], q_scales
    [h, n, d/16], k_codes, k_scales (same shapes) and k_mean [h, d] float32.
    """
    q_bits = np.asarray(q_bits)
    k_bits = np.asarray(k_bits)
    if q_bits.shape != k_bits.shape or q_bits.ndim != 3 or q_bits.shape[2] not in (64, D_HEAD):
        raise ValueError("q and k must both be [H, L, 128] (or [H, L, 64])")
    H, L, d = q_bits.shape
    hs = list(range(H)) if heads is None else list(heads)
    ridx = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    n = ridx.size
    out = {
        "q_codes": np.empty((len(hs), n, d // 2), np.uint8),
        "q_scales": np.empty((len(hs), n, d // BLOCK), np.uint8),
        "k_codes": np.empty((len(hs), n, d // 2), np.uint8),
        "k_scales": np.empty((len(hs), n, d // BLOCK), np.uint8),
        "k_mean": np.zeros((len(hs), d), np.float32),
    }
    for i, h in enumerate(hs):
        if smooth:
            kh = bf16_bits_to_f64(k_bits[h])
            kbar = kmean_exact(kh)
            xk = (kh[ridx] - kbar.astype(np.float64)).astype(np.float32)
            out["k_mean"][i] = kbar
        else:
            xk = bf16_bits_to_f64(k_bits[h][ridx]).astype(np.float32)
        xq = bf16_bits_to_f64(q_bits[h][ridx]).astype(np.float32)
        out["q_codes"][i], out["q_scales"][i] = _quantize_rows(xq, rotate)
        out["k_codes"][i], out["k_scales"][i] = _quantize_rows(xk, rotate)
    return out


def dequant_nvfp4(codes, scales):
    """Exact real values of packed NVFP4 rows: codes [..., d/2] u8 (low nibble
    = even channel), scales [..., d/16] E4M3 bytes.  Returns float64 [..., d]."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    lo = codes & 0xF
    hi = codes >> 4
    c = np.stack([lo, hi], axis=-1).reshape(codes.shape[:-1] + (codes.shape[-1] * 2,))
    vals = _E2M1[c]
    sv = _E4M3[scales]
    vals = vals.reshape(vals.shape[:-1] + (scales.shape[-1], BLOCK)) * sv[..., None]
    return vals.reshape(codes.shape[:-1] + (codes.shape[-1] * 2,))
