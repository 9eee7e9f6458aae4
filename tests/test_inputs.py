"""The seeded input generators: determinism, per-head independence, BF16
rounding, and the shape/structure of each workload (CPU only)."""

import numpy as np

from long_sequence_dense_amd import inputs


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9, -2.5, 0.0, -0.0],
                 dtype=np.float32)
    b = inputs.f32_to_bf16_bits(x)
    back = inputs.bf16_bits_to_f32(b)
    # 1+2^-8 is a tie between 1 and 1+2^-7 -> even (1); 1+3*2^-8 -> 1+2^-6
    assert list(back) == [1.0, 1.0, 1.0 + 2.0 ** -6, 1.0, -2.5, 0.0, -0.0]
    assert b[6] == 0x8000
    rng = np.random.default_rng(0)
    y = rng.standard_normal(10000).astype(np.float32)
    err = np.abs(inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(y)) - y)
    assert np.all(err <= np.abs(y) * 2.0 ** -8)


def test_deterministic_and_head_independent():
    cfg = inputs.CONFIGS["tiny"]
    a = inputs.make_tensor(cfg, "k")
    b = inputs.make_tensor(cfg, "k", heads=[1])
    assert np.array_equal(a[1], b[0])
    assert np.array_equal(a, inputs.make_tensor(cfg, "k"))
    assert not np.array_equal(a[0], a[1])


def test_tiny_key_offset():
    d = inputs.make_inputs("tiny")
    k = inputs.bf16_bits_to_f32(d["k"]).astype(np.float64)
    q = inputs.bf16_bits_to_f32(d["q"]).astype(np.float64)
    assert d["k"].shape == (2, 1024, 128)
    # per-channel means of K carry the N(0, 2) offset, Q's do not
    assert np.std(k.mean(axis=1)) > 0.8
    assert np.std(q.mean(axis=1)) < 0.1


def test_outlier_structure_small():
    cfg = inputs.CONFIGS["fp4"].with_shape(H=3, L=2048)
    q = inputs.bf16_bits_to_f32(inputs.make_tensor(cfg, "q")).astype(np.float64)
    v = inputs.bf16_bits_to_f32(inputs.make_tensor(cfg, "v")).astype(np.float64)
    for h in range(3):
        ch = inputs.outlier_channels(cfg, h)
        assert len(ch) == 3
        med = np.median(np.abs(q[h]), axis=0)
        others = np.setdiff1d(np.arange(128), ch)
        assert np.all(med[ch] > 10 * np.max(med[others]))
    assert abs(np.std(v) - 1.0) < 0.05


def test_sample_rows():
    r = inputs.sample_rows(109000, 64)
    assert r.min() >= 0 and r.max() == 108999 and len(set(r)) == len(r)
    for t in (64, 128, 256):
        assert (108999 // t) * t in r


def test_toy_heads_structure():
    t = inputs.toy_heads(8)
    assert t["q"].shape == (8, 32, 64) and t["k"].shape == (8, 32, 64) and t["v"].shape == (8, 32, 64)
    again = inputs.toy_heads(8)
    for w in ("q", "k", "v"):
        assert np.array_equal(t[w], again[w])
    assert np.array_equal(inputs.toy_heads(3)["k"], t["k"][:3])        # heads independent of the count
    q = inputs.bf16_bits_to_f32(t["q"]).astype(np.float64)
    k = inputs.bf16_bits_to_f32(t["k"]).astype(np.float64)
    v = inputs.bf16_bits_to_f32(t["v"]).astype(np.float64)
    for h in range(8):
        rms_q = np.sqrt((q[h] ** 2).mean(axis=0))
        big = np.argsort(rms_q)[-2:]
        assert np.all(rms_q[big] > 4 * np.median(rms_q))                # two scaled-up channels
        centred = k[h] - k[h].mean(axis=0)
        assert np.all(np.sqrt((centred[:, big] ** 2).mean(axis=0)) > 4)  # same channels on K
    # every key of a head shares one bias per channel: the column means of K
    # spread far more than those of Q (outlier channels aside)
    assert np.std(k.mean(axis=1)) > 2 * np.std(np.median(q, axis=1))
    assert abs(np.std(v) - 1.0) < 0.1


def test_linear_operands_rows_regenerate():
    # any row set regenerates alone (chunked seeding), X carries its outlier
    # channels, W has variance about 1/K
    x = inputs.linear_operand("x", 5000, 64, 3)
    rows = [0, 4095, 4096, 4999]
    assert np.array_equal(inputs.linear_operand("x", 5000, 64, 3, row_ids=rows), x[rows])
    xf = inputs.bf16_bits_to_f32(x)
    ch = inputs.linear_outlier_channels(64, 3)
    assert len(ch) == 1
    assert 15 < np.std(xf[:, ch]) < 25 and 0.9 < np.std(np.delete(xf, ch, axis=1)) < 1.1
    w = inputs.bf16_bits_to_f32(inputs.linear_operand("w", 256, 1024, 4))
    assert abs(np.var(w) * 1024 - 1) < 0.05


def test_long_head_chunks():
    """The chunked generator of one long head: deterministic, each chunk its
    own stream (regenerated alone here), the ragged last chunk, and the
    outlier channels of the 15-second structure."""
    cfg = inputs.CONFIGS["clip15s"].with_shape(H=1, L=2 * inputs.LONG_CHUNK + 1000)
    a = inputs.long_head_tensor(cfg, "q")
    assert a.shape == (cfg.L, 128) and a.dtype == np.uint16
    assert np.array_equal(a, inputs.long_head_tensor(cfg, "q"))
    ch = inputs.outlier_channels(cfg, 0)
    for c, n in ((1, inputs.LONG_CHUNK), (2, 1000)):
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(
            [cfg.seed, inputs.TID_Q, 0, inputs.LONG_TAG + c])))
        x = rng.standard_normal((n, 128), dtype=np.float32)
        x[:, ch] *= np.float32(20.0)
        r0 = c * inputs.LONG_CHUNK
        assert np.array_equal(a[r0:r0 + n], inputs.f32_to_bf16_bits(x))
    assert not np.array_equal(a[:1000], a[inputs.LONG_CHUNK:inputs.LONG_CHUNK + 1000])
    q = inputs.bf16_bits_to_f32(a).astype(np.float64)
    med = np.median(np.abs(q), axis=0)
    others = np.setdiff1d(np.arange(128), ch)
    assert np.all(med[ch] > 10 * np.max(med[others]))
    v = inputs.bf16_bits_to_f32(inputs.long_head_tensor(cfg, "v")).astype(np.float64)
    assert abs(np.std(v) - 1.0) < 0.01
