"""Seeded synthetic inputs for the attention paths (shared by tests, smoke and bench).

This module only draws random numbers and rounds them to BF16; it holds none of
the attention or quantization arithmetic, and it imports neither the GPU
binding nor the CPU oracle.

The workloads stand in for the real activations of a video+audio diffusion
transformer whose 15-second clips are about 109k tokens of one joint sequence
("Pika H3 Flex in FastVideo: 7x Faster, and Near Real Time in 4-bit", section
"Faster at BF16"); the toy heads of its section "FP4 attention" motivate the
shared key bias and the scaled-up outlier channels.  Head count and head size
(40 x 128) are the configuration choice of this library, not the pages'.

Recipe, per tensor and head (every head regenerates independently):
  rng = numpy Generator(PCG64(SeedSequence([seed, tensor_id, head])))
  tensor_id: Q = 0, K = 1, V = 2, key offset = 3, outlier channels = 4,
             upstream gradient dO (for the backward) = 5
  normal draws: rng.standard_normal((L, d), float32)
  Student-t draws: rng.standard_t(3, (L, d)) in float64, cast to float32
  scaling (1/sqrt(d) on Q, x20 on outlier channels) is a float32 multiply;
  the key offset (one N(0, variance 2) value per head and channel) is added
  in float64 and cast to float32;
  float32 -> BF16 with round-to-nearest-even on the bit pattern.
The BF16 bit patterns (uint16) are the inputs of both the GPU path and the
oracle.
"""

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

D = 128
TID_Q, TID_K, TID_V, TID_OFFSET, TID_OUTLIER, TID_DOUT = 0, 1, 2, 3, 4, 5
TID_LIN_X, TID_LIN_W, TID_LIN_OUTLIER = 6, 7, 8
N_OUTLIER_CHANNELS = 3          # round(0.02 * 128)
OUTLIER_GAIN = np.float32(20.0)


class Config(object):
    def __init__(self, name, H, L, seed, scale, q_dist, k_dist, v_dist,
                 q_prescale=False, k_offset=False, outliers=False, desc=""):
        self.name = name
        self.H = H
        self.L = L
        self.seed = seed
        self.scale = scale
        self.q_dist = q_dist
        self.k_dist = k_dist
        self.v_dist = v_dist
        self.q_prescale = q_prescale
        self.k_offset = k_offset
        self.outliers = outliers
        self.desc = desc

    def with_shape(self, H=None, L=None):
        c = Config(**{k: getattr(self, k) for k in (
            "name", "H", "L", "seed", "scale", "q_dist", "k_dist", "v_dist",
            "q_prescale", "k_offset", "outliers", "desc")})
        if H is not None:
            c.H = H
        if L is not None:
            c.L = L
        return c


INV_SQRT_D = 1.0 / math.sqrt(D)

CONFIGS = {
    "tiny": Config("tiny", 2, 1024, 0, INV_SQRT_D, "normal", "normal", "normal",
                   k_offset=True,
                   desc="H=2 L=1024: N(0,1) Q/K/V, K plus a per-(head,channel) N(0,2) offset"),
    "mid": Config("mid", 24, 8192, 1, 1.0, "normal", "normal", "normal",
                  q_prescale=True,
                  desc="H=24 L=8192: N(0,1), Q pre-scaled by 1/sqrt(d), sigma=1"),
    "clip5s": Config("clip5s", 40, 36480, 2, INV_SQRT_D, "normal", "normal", "normal",
                     desc="H=40 L=36480: N(0,1) Q/K/V"),
    "clip15s": Config("clip15s", 40, 109000, 3, INV_SQRT_D, "normal", "normal", "normal",
                      outliers=True,
                      desc="H=40 L=109000: N(0,1), 3 of 128 channels x20 on Q and K"),
    "fp4": Config("fp4", 40, 109000, 4, INV_SQRT_D, "t3", "t3", "normal",
                  outliers=True,
                  desc="H=40 L=109000: Student-t(3) Q/K with 3 channels x20, N(0,1) V"),
}


def f32_to_bf16_bits(x):
    """float32 array -> BF16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed, tid, head):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, head])))


def outlier_channels(cfg, head):
    rng = _rng(cfg.seed, TID_OUTLIER, head)
    return np.sort(rng.choice(D, N_OUTLIER_CHANNELS, replace=False))


def _draw(dist, rng, L):
    if dist == "normal":
        return rng.standard_normal((L, D), dtype=np.float32)
    if dist == "t3":
        return rng.standard_t(3, size=(L, D)).astype(np.float32)
    raise ValueError(dist)


def head_tensor(cfg, which, head):
    """One head of Q, K, V or dO (N(0,1)) as BF16 bits [L, d]."""
    tid = {"q": TID_Q, "k": TID_K, "v": TID_V, "do": TID_DOUT}[which]
    dist = {"q": cfg.q_dist, "k": cfg.k_dist, "v": cfg.v_dist, "do": "normal"}[which]
    x = _draw(dist, _rng(cfg.seed, tid, head), cfg.L)
    return _finish(cfg, which, head, x)


def _finish(cfg, which, head, x):
    """Row-wise scaling and offset of float32 draws x [n, d], then BF16 bits."""
    if which == "q" and cfg.q_prescale:
        x *= np.float32(INV_SQRT_D)
    if which in ("q", "k") and cfg.outliers:
        ch = outlier_channels(cfg, head)
        x[:, ch] *= OUTLIER_GAIN
    if which == "k" and cfg.k_offset:
        off = _rng(cfg.seed, TID_OFFSET, head).normal(0.0, math.sqrt(2.0), D)
        x = (x.astype(np.float64) + off[None, :]).astype(np.float32)
    return f32_to_bf16_bits(x)


# A single long head (millions of tokens) is drawn in chunks of LONG_CHUNK
# rows, chunk c from Generator(PCG64(SeedSequence([seed, tensor_id, head,
# LONG_TAG + c]))), in a thread pool; the distribution, scaling, offset and
# rounding are those of head_tensor (a different stream of the same law).
LONG_CHUNK = 1 << 18
LONG_TAG = 1 << 20


def long_head_tensor(cfg, which, head=0):
    """One head of Q, K, V or dO as BF16 bits [L, d], drawn chunk-wise."""
    tid = {"q": TID_Q, "k": TID_K, "v": TID_V, "do": TID_DOUT}[which]
    dist = {"q": cfg.q_dist, "k": cfg.k_dist, "v": cfg.v_dist, "do": "normal"}[which]
    out = np.empty((cfg.L, D), dtype=np.uint16)

    def fill(c):
        r0 = c * LONG_CHUNK
        n = min(LONG_CHUNK, cfg.L - r0)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, tid, head, LONG_TAG + c])))
        out[r0:r0 + n] = _finish(cfg, which, head, _draw(dist, rng, n))

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range((cfg.L + LONG_CHUNK - 1) // LONG_CHUNK)))
    return out


def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make_tensor(cfg, which, heads=None, out=None):
    """BF16 bits [len(heads), L, d] for tensor ``which`` in {q, k, v, do}."""
    hs = list(range(cfg.H)) if heads is None else list(heads)
    if out is None:
        out = np.empty((len(hs), cfg.L, D), dtype=np.uint16)

    def fill(i):
        out[i] = head_tensor(cfg, which, hs[i])

    if len(hs) == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(len(hs))))
    return out


def make_inputs(name_or_cfg, heads=None, H=None, L=None):
    """Q, K, V BF16 bits for a named configuration (optionally resized)."""
    cfg = CONFIGS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    if H is not None or L is not None:
        cfg = cfg.with_shape(H=H, L=L)
    return {
        "cfg": cfg,
        "q": make_tensor(cfg, "q", heads),
        "k": make_tensor(cfg, "k", heads),
        "v": make_tensor(cfg, "v", heads),
        "scale": cfg.scale,
    }


# Toy heads of the section "FP4 attention": 64 channels (four 16-value
# blocks), 32 keys, Gaussian values, one bias per channel shared by every key,
# two channels scaled up.  The pages give no magnitudes; these are the ones of
# the long-clip inputs above (bias N(0, variance 2), gain x10 on Q and K) and
# 32 queries per head.
TOY_D = 64
TOY_LEN = 32
TOY_OUTLIERS = 2
TOY_GAIN = np.float32(10.0)


def toy_heads(n_heads, seed=5):
    """Q, K, V BF16 bits [n_heads, 32, 64] of the toy heads; per head h the
    same recipe as above with rng streams (seed, tensor_id, h)."""
    out = {w: np.empty((n_heads, TOY_LEN, TOY_D), np.uint16) for w in ("q", "k", "v")}
    for h in range(n_heads):
        ch = np.sort(_rng(seed, TID_OUTLIER, h).choice(TOY_D, TOY_OUTLIERS, replace=False))
        off = _rng(seed, TID_OFFSET, h).normal(0.0, math.sqrt(2.0), TOY_D)
        for w, tid in (("q", TID_Q), ("k", TID_K), ("v", TID_V)):
            x = _rng(seed, tid, h).standard_normal((TOY_LEN, TOY_D), dtype=np.float32)
            if w != "v":
                x[:, ch] *= TOY_GAIN
            if w == "k":
                x = (x.astype(np.float64) + off[None, :]).astype(np.float32)
            out[w][h] = f32_to_bf16_bits(x)
    return out


def sample_rows(L, n_random, seed=12345, tiles=(64, 128, 256)):
    """Query rows for sampled parity at large L: the first and last rows of
    every tile size in ``tiles`` around the start and the ragged end, plus
    ``n_random`` seeded rows.  Sorted, unique, all in [0, L)."""
    fixed = {0, 1, L - 1, L - 2}
    for t in tiles:
        last = (L - 1) // t * t
        for r in (t - 1, t, t + 1, last - 1, last, last + 1):
            if 0 <= r < L:
                fixed.add(r)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, L])))
    rand = rng.choice(L, size=min(n_random, L), replace=False)
    return np.array(sorted(fixed.union(int(r) for r in rand)), dtype=np.int64)


# Operands of a linear layer of the same transformer (section "NVFP4 QAD":
# every attention and feed-forward linear takes 4-bit weights and
# activations).  The hidden size is the head configuration above (40 x 128 =
# 5120).  Activations X [M, K]: N(0,1) values with 2% of the K channels
# (chosen per seed) scaled x20, the outlier channels of a transformer's hidden
# state; weights W [N, K]: N(0, 1/K).  Rows are drawn in chunks of LIN_CHUNK
# rows, chunk c from rng (seed, tensor_id, c), so any row can be regenerated
# alone; float32 -> BF16 round to nearest even as above.
LIN_CHUNK = 4096
LIN_OUTLIER_FRAC = 0.02


def linear_outlier_channels(K, seed):
    n = max(1, int(round(LIN_OUTLIER_FRAC * K)))
    return np.sort(_rng(seed, TID_LIN_OUTLIER, 0).choice(K, n, replace=False))


def _linear_chunk(kind, rows, K, seed, c):
    n = min(LIN_CHUNK, rows - c * LIN_CHUNK)
    if kind == "x":
        x = _rng(seed, TID_LIN_X, c).standard_normal((n, K), dtype=np.float32)
        x[:, linear_outlier_channels(K, seed)] *= OUTLIER_GAIN
    else:
        x = _rng(seed, TID_LIN_W, c).standard_normal((n, K), dtype=np.float32)
        x *= np.float32(1.0 / math.sqrt(K))
    return f32_to_bf16_bits(x)


def linear_operand(kind, rows, K, seed, row_ids=None):
    """BF16 bits of X (kind "x", [rows, K]) or W (kind "w", [rows, K]); with
    ``row_ids`` only those rows (regenerating just their chunks)."""
    if kind not in ("x", "w"):
        raise ValueError(kind)
    if row_ids is not None:
        row_ids = np.asarray(row_ids, dtype=np.int64)
        out = np.empty((len(row_ids), K), dtype=np.uint16)
        for c in np.unique(row_ids // LIN_CHUNK):
            sel = np.nonzero(row_ids // LIN_CHUNK == c)[0]
            out[sel] = _linear_chunk(kind, rows, K, seed, int(c))[row_ids[sel] - c * LIN_CHUNK]
        return out
    out = np.empty((rows, K), dtype=np.uint16)
    nchunks = (rows + LIN_CHUNK - 1) // LIN_CHUNK

    def fill(c):
        out[c * LIN_CHUNK:(c + 1) * LIN_CHUNK] = _linear_chunk(kind, rows, K, seed, c)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(nchunks)))
    return out
