"""CPU checks of the tests' own tiled-layout permutation (tests/nvfp4_layout.py)."""

import numpy as np

from nvfp4_layout import from_tiled, to_tiled


def test_tiled_layout_is_a_permutation():
    # the test's own re-layout: round trip, padding zero, chunk placement
    rng = np.random.default_rng(3)
    c = rng.integers(0, 256, (300, 40), dtype=np.uint8)
    s_ = rng.integers(0, 127, (300, 5), dtype=np.uint8)
    tc, ts = to_tiled(c, s_)
    assert tc.size == 2 * 2 * 8192 and ts.size == 2 * 2 * 1024
    back_c, back_s = from_tiled(tc, ts, 300, 80)
    assert np.array_equal(back_c, c) and np.array_equal(back_s, s_)
    assert np.array_equal(tc[8192:8192 + 32][:8], c[0, 32:40])          # tile 0, stage 1, row 0
    assert np.all(tc[8192 + 32 * 0 + 8:8192 + 32] == 0)                  # K padding of stage 1
    assert np.all(tc[3 * 8192 + 32 * 44:] == 0)                          # rows past 300 in tile 1
