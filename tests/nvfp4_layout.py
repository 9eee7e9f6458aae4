"""Test helper (not a test module): the tiled NVFP4 code layout as a plain
index permutation of the row-major bytes, for comparing the GPU's tiled
output with the oracle's row-major codes.  Chunks (256-row tile, 64-value
stage), tile-major, each holding its rows' 32 code bytes (4 scale bytes) in
row order; zero padding at the ragged ends."""

import numpy as np

TILE_ROWS, STAGE = 256, 64


def to_tiled(codes, scales):
    """Row-major codes [R, K/2] and scales [R, K/16] -> the tiled byte order:
    chunks (256-row tile, 64-value stage), tile-major, each holding its rows'
    32 code bytes (4 scale bytes) in row order; zero padding."""
    R, kc = codes.shape
    T, S = -(-R // TILE_ROWS), -(-(2 * kc) // STAGE)
    out = []
    for a, per in ((codes, STAGE // 2), (scales, STAGE // 16)):
        pad = np.zeros((T * TILE_ROWS, S * per), dtype=np.uint8)
        pad[:R, :a.shape[1]] = a
        out.append(pad.reshape(T, TILE_ROWS, S, per).transpose(0, 2, 1, 3).reshape(-1))
    return out


def from_tiled(codes, scales, R, K):
    T, S = -(-R // TILE_ROWS), -(-K // STAGE)
    out = []
    for a, per, width in ((codes, STAGE // 2, K // 2), (scales, STAGE // 16, K // 16)):
        full = a.reshape(T, S, TILE_ROWS, per).transpose(0, 2, 1, 3).reshape(T * TILE_ROWS, S * per)
        out.append(full[:R, :width])
    return out
