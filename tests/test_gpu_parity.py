"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars (from the method's own acceptance criteria): NVFP4 codes, scales and the
mean key bit-exact; attention outputs within max-abs 2e-2 and mean-abs 2e-3 of
the fp64 oracle on the same seeded inputs (the FP4-QK path against the oracle
attention on the oracle's own quantized Q/K).  Small shapes are compared
element by element in full; the full-size workloads (40 heads x 36,480 or
109,000 tokens, the launch configuration the benchmark times) on sampled query
rows and heads, tile edges and the ragged tail included.
"""

import math
import os
import sys

import numpy as np
import pytest

from long_sequence_dense_amd import inputs

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
MEAN_ABS = 2e-3
# The LSE output is m + ln(sum_j p_j) over the BF16-rounded weights p_j that
# O is normalized with (consistent with O); each p_j is within BF16's unit
# roundoff 2^-8 of its exact value, so the LSE is within ln(1 + 2^-8) of the
# exact one, plus 1e-3 for fp32 scores and rounding.
LSE_TOL = math.log1p(2.0 ** -8) + 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available()
    from long_sequence_dense_amd import binding
    binding.load_library()
    return t


def dev(torch, arr):
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def bf16_dev(torch, bits):
    return dev(torch, bits.view(np.int16)).view(torch.bfloat16)


def out_f64(o):
    import torch
    bits = o.view(torch.int16).cpu().numpy().view(np.uint16)
    return inputs.bf16_bits_to_f32(bits).astype(np.float64)


def f64(bits):
    return inputs.bf16_bits_to_f32(bits).astype(np.float64)


def compare(name, got, want, max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    err = np.abs(got - want)
    mx, mn = float(err.max()), float(err.mean())
    say("  %-40s max-abs %.3e mean-abs %.3e (n=%d)" % (name, mx, mn, err.size))
    assert np.all(np.isfinite(got)), name
    assert mx <= max_abs, (name, mx)
    assert mn <= mean_abs, (name, mn)


def run_bf16(torch, d, lse=True):
    from long_sequence_dense_amd import binding
    q, k, v = (bf16_dev(torch, d[n]) for n in ("q", "k", "v"))
    H, L, _ = d["q"].shape
    o = torch.full((H, L, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    l = torch.full((H, L), float("nan"), dtype=torch.float32, device="cuda") if lse else None
    binding.attn_fwd_bf16(q, k, v, o, l, softmax_scale=d["scale"])
    torch.cuda.synchronize()
    return o, l


def check_attention(name, o, lse, oref, lref, rows=None, heads=None):
    got = out_f64(o)
    if heads is not None:
        got = got[heads]
    if rows is not None:
        got = got[:, rows]
    compare(name + " O", got, oref)
    if lse is not None:
        lg = lse.cpu().numpy().astype(np.float64)
        if heads is not None:
            lg = lg[heads]
        if rows is not None:
            lg = lg[:, rows]
        tol = LSE_TOL + 2e-6 * np.abs(lref)
        bad = np.abs(lg - lref) > tol
        say("  %-40s lse max-abs %.3e" % (name, float(np.abs(lg - lref).max())))
        assert not bad.any(), name


# ---------------------------------------------------------------- BF16 path ----

def test_bf16_tiny_full(torch):
    from oracle.attention import attention_fp64
    d = inputs.make_inputs("tiny")
    say("case tiny H=2 L=1024 bf16")
    o, l = run_bf16(torch, d)
    oref, lref = attention_fp64(f64(d["q"]), f64(d["k"]), f64(d["v"]), d["scale"])
    check_attention("tiny", o, l, oref, lref)


@pytest.mark.parametrize("L", [1, 2, 63, 64, 65, 127, 129, 200, 333])
def test_bf16_ragged_lengths(torch, L):
    from oracle.attention import attention_fp64
    d = inputs.make_inputs("tiny", H=3, L=L)
    say("case ragged H=3 L=%d bf16" % L)
    o, l = run_bf16(torch, d)
    oref, lref = attention_fp64(f64(d["q"]), f64(d["k"]), f64(d["v"]), d["scale"])
    check_attention("ragged L=%d" % L, o, l, oref, lref)


def test_bf16_deterministic_and_no_lse(torch):
    d = inputs.make_inputs("tiny", H=2, L=777)
    say("case determinism H=2 L=777")
    o1, l1 = run_bf16(torch, d)
    o2, _ = run_bf16(torch, d, lse=False)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_bf16_outliers_small(torch):
    from oracle.attention import attention_fp64
    d = inputs.make_inputs("clip15s", H=4, L=3000)
    say("case clip15s-structure H=4 L=3000 bf16")
    o, l = run_bf16(torch, d)
    oref, lref = attention_fp64(f64(d["q"]), f64(d["k"]), f64(d["v"]), d["scale"])
    check_attention("outliers H=4 L=3000", o, l, oref, lref)


@pytest.mark.parametrize("cfg,nrows,nheads", [("mid", 96, 24), ("clip5s", 48, 10), ("clip15s", 40, 8)])
def test_bf16_full_size_sampled(torch, cfg, nrows, nheads):
    from oracle.attention import attention_fp64
    c = inputs.CONFIGS[cfg]
    say("case %s H=%d L=%d bf16 (generate)" % (cfg, c.H, c.L))
    d = inputs.make_inputs(cfg)
    o, l = run_bf16(torch, d)
    heads = np.unique(np.linspace(0, c.H - 1, nheads).astype(int))
    rows = inputs.sample_rows(c.L, nrows)
    say("  oracle on %d heads x %d rows" % (len(heads), len(rows)))
    oref, lref = attention_fp64(f64(d["q"][heads]), f64(d["k"][heads]), f64(d["v"][heads]),
                                d["scale"], rows=rows)
    check_attention("%s sampled" % cfg, o, l, oref, lref, rows=rows, heads=heads)
    # nothing left unwritten anywhere
    assert not torch.isnan(o).any().item()
    assert not torch.isnan(l).any().item()


# ---------------------------------------------------------------- FP4 prep -----

def run_prep(torch, d):
    from long_sequence_dense_amd import binding
    q, k = bf16_dev(torch, d["q"]), bf16_dev(torch, d["k"])
    H, L, _ = d["q"].shape
    out = {
        "q_codes": torch.full((H, L, 64), 0xAB, dtype=torch.uint8, device="cuda"),
        "q_scales": torch.full((H, L, 8), 0xFF, dtype=torch.uint8, device="cuda"),
        "k_codes": torch.full((H, L, 64), 0xAB, dtype=torch.uint8, device="cuda"),
        "k_scales": torch.full((H, L, 8), 0xFF, dtype=torch.uint8, device="cuda"),
        "k_mean": torch.full((H, 128), float("nan"), dtype=torch.float32, device="cuda"),
    }
    binding.qk_prep_fp4(q, k, out=out)
    torch.cuda.synchronize()
    return out


def check_prep_exact(name, got, ref, heads=None, rows=None):
    for key in ("q_codes", "q_scales", "k_codes", "k_scales"):
        g = got[key].cpu().numpy()
        if heads is not None:
            g = g[heads]
        if rows is not None:
            g = g[:, rows]
        nbad = int((g != ref[key]).sum())
        say("  %-40s %s mismatches %d of %d" % (name, key, nbad, g.size))
        assert nbad == 0, (name, key)
    km = got["k_mean"].cpu().numpy()
    if heads is not None:
        km = km[heads]
    assert np.array_equal(km.view(np.uint32), ref["k_mean"].view(np.uint32)), name


def test_prep_tiny_exact(torch):
    from oracle.nvfp4 import qk_prep_fp4
    d = inputs.make_inputs("tiny")
    say("case prep tiny")
    got = run_prep(torch, d)
    check_prep_exact("prep tiny", got, qk_prep_fp4(d["q"], d["k"]))


@pytest.mark.parametrize("H,L", [(1, 1), (3, 17), (2, 129), (5, 1000)])
def test_prep_ragged_exact(torch, H, L):
    from oracle.nvfp4 import qk_prep_fp4
    d = inputs.make_inputs("fp4", H=H, L=L)
    say("case prep fp4-structure H=%d L=%d" % (H, L))
    got = run_prep(torch, d)
    check_prep_exact("prep H=%d L=%d" % (H, L), got, qk_prep_fp4(d["q"], d["k"]))


def test_prep_special_values_exact(torch):
    # zero rows, signed zeros, subnormal BF16, huge and tiny magnitudes,
    # constant keys (K - mean is exactly zero), a single token
    from oracle.nvfp4 import qk_prep_fp4
    rng = np.random.default_rng(5)
    H, L = 3, 96
    q = inputs.f32_to_bf16_bits((rng.standard_t(3, (H, L, 128)) * 0.01).astype(np.float32))
    k = inputs.f32_to_bf16_bits((rng.standard_t(3, (H, L, 128)) * 50).astype(np.float32))
    q[0, 0] = 0
    q[0, 1] = 0x8000                                 # all -0
    q[0, 2, :] = 0x0001                              # smallest subnormal BF16
    q[0, 3, ::3] = 0x8001
    q[1, 4, :] = 0x7F00                              # 2^127 .. butterfly overflow region avoided below
    q[1, 4, 1:] = 0
    q[1, 5, :] = 0x6000
    k[2] = k[2, 0]                                   # every key of head 2 identical
    k[1, :, 7] = 0x0001
    k[1, ::2, 9] = 0x8002
    d = {"q": q, "k": k}
    say("case prep special values")
    got = run_prep(torch, d)
    check_prep_exact("prep special", got, qk_prep_fp4(q, k))


def test_prep_mean_combination_rounds(torch):
    """Column partials that are each exact but whose fp64 combination rounds:
    channel 3 of the one head holds 2^22 and 2^-2 on rows 0 and 16 (one
    partial) and 2^-31 on rows 4 and 8 (two others).  Added pairwise in fp64
    the two 2^-31 fall on ties and are lost, leaving 2^22 + 2^-2, whose mean
    over 64 rows is an fp32 tie that rounds down; the exact sum carries 2^-30
    more and its mean rounds up.  A final reduction that trusted the fp64 sum
    without checking it would be one fp32 ulp low."""
    from oracle.nvfp4 import qk_prep_fp4
    rng = np.random.default_rng(11)
    H, L = 1, 64
    q = inputs.f32_to_bf16_bits(rng.standard_normal((H, L, 128)).astype(np.float32))
    k = np.zeros((H, L, 128), np.uint16)
    k[0, 0, 3], k[0, 16, 3] = 0x4A80, 0x3E80          # 2^22, 2^-2
    k[0, 4, 3] = k[0, 8, 3] = 0x3000                   # 2^-31
    d = {"q": q, "k": k}
    ref = qk_prep_fp4(q, k)
    assert ref["k_mean"][0, 3] == np.float32(2.0 ** 16 + 2.0 ** -7)    # the exact sum's mean, rounded once
    say("case prep mean combination rounds")
    got = run_prep(torch, d)
    check_prep_exact("prep mean combination", got, ref)


def test_prep_deterministic(torch):
    d = inputs.make_inputs("fp4", H=2, L=2000)
    a = run_prep(torch, d)
    b = run_prep(torch, d)
    for key in a:
        assert torch.equal(a[key], b[key]), key


def test_prep_full_size_exact_all_heads(torch):
    """Every code, scale and mean of the full-size FP4 workload (40 heads x
    109,000 tokens: 1.1e9 codes) against the oracle, head by head."""
    from concurrent.futures import ThreadPoolExecutor
    from oracle.nvfp4 import qk_prep_fp4
    c = inputs.CONFIGS["fp4"]
    say("case prep fp4 H=40 L=109000 (generate)")
    d = inputs.make_inputs("fp4")
    got = run_prep(torch, d)
    g = {key: got[key].cpu().numpy() for key in got}
    assert not np.any((g["q_scales"] & 0x7F) == 0x7F)    # no NaN scale codes anywhere
    assert not np.any((g["k_scales"] & 0x7F) == 0x7F)

    def one(h):
        ref = qk_prep_fp4(d["q"][h:h + 1], d["k"][h:h + 1])
        bad = {key: int((g[key][h] != ref[key][0]).sum()) for key in ("q_codes", "q_scales", "k_codes", "k_scales")}
        bad["k_mean"] = int((g["k_mean"][h].view(np.uint32) != ref["k_mean"][0].view(np.uint32)).sum())
        return h, bad

    say("  oracle prep on all %d heads (all rows)" % c.H)
    total = 0
    with ThreadPoolExecutor(max(1, min(16, len(os.sched_getaffinity(0))))) as ex:
        for h, bad in ex.map(one, range(c.H)):
            total += sum(bad.values())
            if h % 8 == 7 or any(bad.values()):
                say("  head %2d mismatches %s" % (h, bad))
    assert total == 0


# ---------------------------------------------------------------- FP4-QK -------

def fp4_oracle(d, heads=None, rows=None):
    """oracle prep -> exact dequant -> fp64 attention (Q rows subset)."""
    from oracle.attention import attention_fp64
    from oracle.nvfp4 import dequant_nvfp4, qk_prep_fp4
    hs = list(range(d["q"].shape[0])) if heads is None else list(heads)
    prep = qk_prep_fp4(d["q"][hs], d["k"][hs])
    qh = dequant_nvfp4(prep["q_codes"], prep["q_scales"])
    kh = dequant_nvfp4(prep["k_codes"], prep["k_scales"])
    return attention_fp64(qh, kh, f64(d["v"][hs]), d["scale"], rows=rows)


def run_fp4(torch, d):
    from long_sequence_dense_amd import binding
    prep = run_prep(torch, d)
    v = bf16_dev(torch, d["v"])
    H, L, _ = d["v"].shape
    o = torch.full((H, L, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    l = torch.full((H, L), float("nan"), dtype=torch.float32, device="cuda")
    binding.attn_fwd_fp4qk(prep["q_codes"], prep["q_scales"], prep["k_codes"], prep["k_scales"],
                           v, o, l, softmax_scale=d["scale"])
    torch.cuda.synchronize()
    return o, l


def test_fp4qk_tiny_full(torch):
    d = inputs.make_inputs("tiny")
    say("case fp4qk tiny")
    o, l = run_fp4(torch, d)
    oref, lref = fp4_oracle(d)
    check_attention("fp4qk tiny", o, l, oref, lref)


@pytest.mark.parametrize("L", [1, 65, 200])
def test_fp4qk_ragged(torch, L):
    d = inputs.make_inputs("fp4", H=2, L=L)
    say("case fp4qk ragged L=%d" % L)
    o, l = run_fp4(torch, d)
    oref, lref = fp4_oracle(d)
    check_attention("fp4qk L=%d" % L, o, l, oref, lref)


def test_fp4qk_structure_mid(torch):
    d = inputs.make_inputs("fp4", H=3, L=4000)
    say("case fp4qk fp4-structure H=3 L=4000")
    o, l = run_fp4(torch, d)
    oref, lref = fp4_oracle(d)
    check_attention("fp4qk H=3 L=4000", o, l, oref, lref)


def test_fp4qk_full_size_sampled(torch):
    c = inputs.CONFIGS["fp4"]
    say("case fp4qk fp4 H=40 L=109000 (generate)")
    d = inputs.make_inputs("fp4")
    o, l = run_fp4(torch, d)
    heads = [0, 13, 39]
    rows = inputs.sample_rows(c.L, 48)
    say("  oracle prep + attention on heads %s x %d rows" % (heads, len(rows)))
    oref, lref = fp4_oracle(d, heads=heads, rows=rows)
    check_attention("fp4qk full-size sampled", o, l, oref, lref, rows=rows, heads=heads)
    assert not torch.isnan(o).any().item()


@pytest.mark.parametrize("H,L", [(2, 1024), (2, 65), (1, 200), (3, 4000)])
def test_fp4qk_equals_bf16_on_dequantized(torch, H, L):
    """The FP4-QK attention is the BF16 attention on the exactly dequantized
    Q-hat, K-hat: every E2M1 x E4M3 value is exact in BF16 (and in the FP16 the
    FP4 kernel multiplies in), the products are exact, and the sums run in the
    same order, so O and the LSE agree bit for bit."""
    from long_sequence_dense_amd import binding
    from oracle.nvfp4 import dequant_nvfp4
    d = inputs.make_inputs("fp4", H=H, L=L)
    say("case fp4qk == bf16 on dequantized H=%d L=%d" % (H, L))
    o4, l4 = run_fp4(torch, d)
    prep = run_prep(torch, d)
    hat = {}
    for n in ("q", "k"):
        vals = dequant_nvfp4(prep[n + "_codes"].cpu().numpy(), prep[n + "_scales"].cpu().numpy())
        bits = inputs.f32_to_bf16_bits(vals.astype(np.float32))
        assert np.array_equal(f64(bits), vals), n          # exact in BF16
        hat[n] = bits
    ob, lb = run_bf16(torch, {"q": hat["q"], "k": hat["k"], "v": d["v"], "scale": d["scale"]})
    same_o = torch.equal(o4.view(torch.int16), ob.view(torch.int16))
    same_l = torch.equal(l4, lb)
    say("  O bit-identical %s, LSE bit-identical %s" % (same_o, same_l))
    assert same_o and same_l


def test_bf16_max_head_length(torch):
    """The longest head the library accepts, L = 2^23 - 1 = 8,388,607 tokens
    (one head of the 15-second input structure, drawn chunk-wise; 2 GiB -
    256 B per BF16 tensor): the last K/V tile starts 16 KiB before 2^31 bytes
    into the head and is ragged (63 of its 64 keys).  BF16 attention on
    sampled query rows (the first and last rows of every tile size at both
    ends included) against the fp64 oracle over all keys; no output left
    unwritten."""
    from oracle.attention import attention_fp64
    L = (1 << 23) - 1
    c = inputs.CONFIGS["clip15s"].with_shape(H=1, L=L)
    say("case max head length: clip15s structure H=1 L=%d (generate)" % L)
    d = {w: inputs.long_head_tensor(c, w)[None] for w in ("q", "k", "v")}
    d["scale"] = c.scale
    say("  bf16 attention")
    o, l = run_bf16(torch, d)
    assert not torch.isnan(o).any().item()
    assert not torch.isnan(l).any().item()
    rows = inputs.sample_rows(L, 24)
    say("  oracle on %d rows over %d keys" % (len(rows), L))
    oref, lref = attention_fp64(f64(d["q"][:, rows]), f64(d["k"]), f64(d["v"]), d["scale"])
    check_attention("bf16 L=2^23-1 sampled", o, l, oref, lref, rows=rows)


def test_offsets_beyond_2gib(torch):
    """80 heads of the 15-second FP4 workload: every BF16 tensor is 2.23 GB,
    so the last heads start past 2^31 bytes.  BF16 attention, the prep (every
    code, scale and mean of the checked heads) and FP4-QK attention on the
    first and the last head."""
    from long_sequence_dense_amd import binding
    from oracle.attention import attention_fp64
    from oracle.nvfp4 import dequant_nvfp4, qk_prep_fp4
    H, L = 80, 109000
    heads = [0, H - 1]
    rows = inputs.sample_rows(L, 24)
    say("case offsets beyond 2 GiB: fp4 structure H=%d L=%d (generate)" % (H, L))
    d = inputs.make_inputs("fp4", H=H, L=L)
    assert (H - 1) * L * 128 * 2 > 2 ** 31

    say("  bf16 attention")
    o, l = run_bf16(torch, d)
    oref, lref = attention_fp64(f64(d["q"][heads]), f64(d["k"][heads]), f64(d["v"][heads]), d["scale"], rows=rows)
    check_attention("bf16 H=80 sampled", o, l, oref, lref, rows=rows, heads=heads)
    assert not torch.isnan(o).any().item()
    del o, l

    say("  prep + fp4qk attention")
    prep = run_prep(torch, d)
    ref = qk_prep_fp4(d["q"][heads], d["k"][heads])
    check_prep_exact("prep H=80 heads %s" % heads, prep, ref, heads=heads)
    v = bf16_dev(torch, d["v"])
    o = torch.full((H, L, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    l = torch.full((H, L), float("nan"), dtype=torch.float32, device="cuda")
    binding.attn_fwd_fp4qk(prep["q_codes"], prep["q_scales"], prep["k_codes"], prep["k_scales"],
                           v, o, l, softmax_scale=d["scale"])
    torch.cuda.synchronize()
    qh = dequant_nvfp4(ref["q_codes"], ref["q_scales"])
    kh = dequant_nvfp4(ref["k_codes"], ref["k_scales"])
    oref, lref = attention_fp64(qh, kh, f64(d["v"][heads]), d["scale"], rows=rows)
    check_attention("fp4qk H=80 sampled", o, l, oref, lref, rows=rows, heads=heads)
    assert not torch.isnan(o).any().item()
