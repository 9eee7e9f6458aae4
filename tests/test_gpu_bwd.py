"""GPU parity of the attention backward (attn_bwd_bf16, attn_bwd_fp4qk) against
the fp64 gradient oracle.

The bar is tied to the gradient's own size: every element of dQ, dK and dV
within 2e-2 of the largest magnitude of the same tensor of the same head
(the method's 2e-2 attention bar, taken relative to the gradient's scale),
and the sums softmax fixes (sum over keys of dK is zero, of dV the sum over
queries of dO) within 1e-2 of the summed row norms they add.

The HIP training forward supplies its fp32 O and row statistics (as a
training step would); the oracle computes the exact gradients of the same
BF16 inputs (for the FP4 path, of the dequantized codes, with the quantizer
passed straight through).  The training forwards themselves are checked
against the plain forwards: the same O and LSE bit for bit, an fp32 O that
rounds to that O, and row statistics that give the LSE.  Small
shapes are compared in full; the full-size workloads (40 heads x 109,000
tokens as the benchmark times them, and 80 heads, whose last rows lie past
2^31 bytes) on sampled dQ rows, every element of dK and dV of sampled key
rows of a head (which needs the oracle's LSE and D over all queries of that
head), and the key sums of every key.
"""

import sys

import numpy as np
import pytest

from long_sequence_dense_amd import inputs
from oracle_pool import map_rows

pytestmark = pytest.mark.gpu

REL = 2e-2          # elementwise, relative to the tensor's largest magnitude (per head)
SUM_REL = 1e-2      # key sums, relative to the summed magnitudes


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


def bf16_dev(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits.view(np.int16))).cuda().view(torch.bfloat16)


def f64(bits):
    return inputs.bf16_bits_to_f32(bits).astype(np.float64)


def to_f64(t):
    import torch
    return inputs.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)


def compare(name, got, want):
    """got, want [H, n, d] (or [n, d]): per head, max |got - want| <= REL *
    max |want|."""
    got, want = np.asarray(got), np.asarray(want)
    if got.ndim == 2:
        got, want = got[None], want[None]
    assert np.all(np.isfinite(got)), name
    worst = 0.0
    for h in range(want.shape[0]):
        err = np.abs(got[h] - want[h])
        scale = float(np.max(np.abs(want[h])))
        r = float(err.max()) / max(scale, 1e-30) if err.max() > 0 else 0.0
        if r > worst:
            worst, wh, we, ws = r, h, float(err.max()), scale
    if worst == 0.0:
        say("  %-32s exact" % name)
        return
    say("  %-32s max-abs %.3e  max|ref| %.3e  rel-max %.3e (head %d)" % (name, we, ws, worst, wh))
    # Diagnostic (not a bar): the worst error relative to its own row, over
    # the rows whose gradient is at least 1e-3 of the head's largest; rows
    # below that are numerically zero gradients (a softmax row saturated on
    # one key), where fp32 scores leave an absolute floor.
    g2, w2 = got.reshape(-1, got.shape[-1]), want.reshape(-1, want.shape[-1])
    rmax = np.abs(w2).max(axis=1)
    big = rmax >= 1e-3 * float(np.abs(w2).max())
    if big.any():
        rr = (np.abs(g2 - w2).max(axis=1)[big] / rmax[big])
        say("  %-32s row-relative max %.3e over %d of %d rows" % ("", float(rr.max()), int(big.sum()), big.size))
    assert worst <= REL, name


def run_bwd(torch, d, dout_bits):
    from long_sequence_dense_amd import binding
    q, k, v = (bf16_dev(torch, d[n]) for n in ("q", "k", "v"))
    H, L, _ = d["q"].shape
    o, o32, ml = binding.attn_fwd_bf16_train(q, k, v, softmax_scale=d["scale"])
    del o
    do = bf16_dev(torch, dout_bits)
    grads = [torch.full((H, L, 128), float("nan"), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    binding.attn_bwd_bf16(q, k, v, o32, ml, do, *grads, softmax_scale=d["scale"])
    torch.cuda.synchronize()
    return grads


def check_train_outputs(torch, name, o_ref, lse_ref, o, lse, o32, ml):
    """The training forward against the plain one: o and lse bit for bit, o32
    rounds (to nearest even) to o, and (m + log2 l) ln 2 is the LSE up to the
    fp32 roundings of the two formulas."""
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), name
    assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32)), name
    assert torch.equal(o32.to(torch.bfloat16).view(torch.int16), o.view(torch.int16)), name
    m, l = ml[..., 0].double(), ml[..., 1].double()
    assert bool((l >= 1.0).all()), name          # the row's largest weight is at least 1
    lse2 = (m + torch.log2(l)) * np.log(2.0)
    err = float(((lse2 - lse.double()).abs() / (1.0 + lse.double().abs())).max())
    say("  %s: o, lse identical; o32 rounds to o; LSE from (m, l) within %.2e (relative)" % (name, err))
    assert err <= 1e-6, name


@pytest.mark.parametrize("cfg,H,L", [("tiny", 2, 1), ("tiny", 3, 333), ("clip15s", 2, 3000), ("fp4", 2, 4000)])
def test_train_forward_bf16(torch, cfg, H, L):
    from long_sequence_dense_amd import binding
    d = inputs.make_inputs(cfg, H=H, L=L)
    say("case train forward bf16 %s H=%d L=%d" % (cfg, H, L))
    q, k, v = (bf16_dev(torch, d[n]) for n in ("q", "k", "v"))
    o_ref = binding.attn_fwd_bf16(q, k, v, softmax_scale=d["scale"])
    lse_ref = torch.empty((H, L), dtype=torch.float32, device="cuda")
    binding.attn_fwd_bf16(q, k, v, None, lse_ref, softmax_scale=d["scale"])
    lse = torch.empty((H, L), dtype=torch.float32, device="cuda")
    o, o32, ml = binding.attn_fwd_bf16_train(q, k, v, None, lse, softmax_scale=d["scale"])
    torch.cuda.synchronize()
    check_train_outputs(torch, "bf16 %s L=%d" % (cfg, L), o_ref, lse_ref, o, lse, o32, ml)


@pytest.mark.parametrize("cfg,H,L", [("fp4", 2, 1000), ("tiny", 1, 65)])
def test_train_forward_fp4qk(torch, cfg, H, L):
    from long_sequence_dense_amd import binding
    d = inputs.make_inputs(cfg, H=H, L=L)
    say("case train forward fp4qk %s H=%d L=%d" % (cfg, H, L))
    q, k, v = (bf16_dev(torch, d[n]) for n in ("q", "k", "v"))
    p = binding.qk_prep_fp4(q, k)
    codes = (p["q_codes"], p["q_scales"], p["k_codes"], p["k_scales"])
    lse_ref = torch.empty((H, L), dtype=torch.float32, device="cuda")
    o_ref = binding.attn_fwd_fp4qk(*codes, v, None, lse_ref, softmax_scale=d["scale"])
    lse = torch.empty((H, L), dtype=torch.float32, device="cuda")
    o, o32, ml = binding.attn_fwd_fp4qk_train(*codes, v, None, lse, softmax_scale=d["scale"])
    torch.cuda.synchronize()
    check_train_outputs(torch, "fp4qk %s L=%d" % (cfg, L), o_ref, lse_ref, o, lse, o32, ml)


@pytest.mark.parametrize("cfg,H,L", [("tiny", 2, 1024), ("tiny", 2, 1), ("tiny", 3, 33), ("tiny", 2, 200),
                                     ("clip15s", 2, 3000), ("fp4", 1, 777)])
def test_bwd_small_full(torch, cfg, H, L):
    from oracle.attention_bwd import attention_bwd_fp64
    d = inputs.make_inputs(cfg, H=H, L=L)
    dob = inputs.make_tensor(d["cfg"], "do")
    say("case bwd %s H=%d L=%d" % (cfg, H, L))
    dq, dk, dv = run_bwd(torch, d, dob)
    refs = attention_bwd_fp64(f64(d["q"]), f64(d["k"]), f64(d["v"]), f64(dob), d["scale"])
    if L == 1:
        check_single_key(d, dob, (dq, dk, dv), refs)
        return
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        compare("%s %s L=%d" % (name, cfg, L), to_f64(g), r)


def check_single_key(d, dob, grads, refs):
    """One key per head: P = 1, so dV = dO exactly and dQ = dK = 0.  The
    computed dS = P (dP - D) is the difference of two fp32 dot products of
    the same 128 terms dO_c V_c (O = V exactly), each within
    gamma_128 sum_c |dO_c V_c| of the exact value (gamma_n = n u / (1 - n u),
    u = 2^-24, the textbook bound for any summation order), so dQ and dK are
    bounded by sigma * 2 gamma_128 sum|dO V| * max|K| (max|Q|), with a factor
    (1 + 2^-7) for the BF16 roundings of dS and of the result."""
    dq, dk, dv = (to_f64(g) for g in grads)
    u = 2.0 ** -24
    gamma = 128 * u / (1 - 128 * u)
    do, v, q, k = f64(dob), f64(d["v"]), f64(d["q"]), f64(d["k"])
    ds_bound = 2 * gamma * np.abs(do * v).sum(axis=2, keepdims=True)          # [H, 1, 1]
    for name, g, x in (("dq", dq, k), ("dk", dk, q)):
        bound = d["scale"] * ds_bound * np.abs(x).max(axis=2, keepdims=True) * (1 + 2.0 ** -7)
        say("  %s single key: max |%s| %.3e, bound %.3e" % (name, name, float(np.abs(g).max()), float(bound.min())))
        assert np.all(np.abs(g) <= bound), name
    assert np.array_equal(dv, refs[2]), "dv single key"


def test_bwd_mid_full(torch):
    """Every gradient of two heads of 8192 tokens (256 key tiles, 64 query
    tiles of the kernels), outlier channels on Q and K."""
    from oracle.attention_bwd import attention_bwd_fp64
    d = inputs.make_inputs("clip15s", H=2, L=8192)
    dob = inputs.make_tensor(d["cfg"], "do")
    say("case bwd clip15s H=2 L=8192")
    dq, dk, dv = run_bwd(torch, d, dob)
    refs = attention_bwd_fp64(f64(d["q"]), f64(d["k"]), f64(d["v"]), f64(dob), d["scale"])
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        compare("%s L=8192" % name, to_f64(g), r)


def test_bwd_peaked_rows_full(torch):
    """The FP4 workload's structure (Student-t(3) with x20 channels) at
    H = 2, L = 4000: many rows put nearly all their weight on one key, so dS
    is nearly zero there and only a D formed with the weights of P (from the
    forward's fp32 O, not its BF16 O) keeps the
    gradient's relative accuracy."""
    from oracle.attention_bwd import attention_bwd_fp64
    d = inputs.make_inputs("fp4", H=2, L=4000)
    dob = inputs.make_tensor(d["cfg"], "do")
    say("case bwd fp4-structure (BF16 path) H=2 L=4000")
    dq, dk, dv = run_bwd(torch, d, dob)
    refs = attention_bwd_fp64(f64(d["q"]), f64(d["k"]), f64(d["v"]), f64(dob), d["scale"])
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        compare("%s peaked L=4000" % name, to_f64(g), r)


def test_bwd_deterministic(torch):
    d = inputs.make_inputs("tiny", H=2, L=1500)
    dob = inputs.make_tensor(d["cfg"], "do")
    a = run_bwd(torch, d, dob)
    b = run_bwd(torch, d, dob)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_bwd_full_size(torch):
    """40 heads x 109,000 tokens: dQ on sampled rows of three heads, dK and dV
    on sampled key rows of head 0, key sums of every key."""
    bwd_sampled(torch, 40)


def test_bwd_beyond_2gib(torch):
    """The same checks at 80 heads (2.23 GB per BF16 tensor): the last heads'
    rows lie past 2^31 bytes; dK and dV checked on sampled keys of the last
    head."""
    assert 79 * 109000 * 128 * 2 > 2 ** 31
    bwd_sampled(torch, 80)


def key_rows_oracle(qh, kh, vh, doh, scale, keys):
    """dK, dV of sampled keys of one head: the per-query LSE and D over all
    queries (row-local, in a thread pool), then every query's contribution."""
    from oracle.attention_bwd import attention_bwd_keys_fp64, attention_row_stats_fp64
    lse, dsum = map_rows(lambda sl: attention_row_stats_fp64(qh[sl], kh, vh, doh[sl], scale), qh.shape[0])
    return attention_bwd_keys_fp64(qh, kh, vh, doh, scale, keys, lse, dsum)


def bwd_sampled(torch, H):
    from oracle.attention_bwd import attention_bwd_dq_rows_fp64
    c = inputs.CONFIGS["clip15s"].with_shape(H=H)
    say("case bwd clip15s H=%d L=%d (generate)" % (c.H, c.L))
    d = inputs.make_inputs(c)
    dob = inputs.make_tensor(c, "do")
    dq, dk, dv = run_bwd(torch, d, dob)
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert not torch.isnan(g).any().item(), name
    rows = inputs.sample_rows(c.L, 512)
    heads = [0, H * 21 // 40, H - 1]
    gq = to_f64(dq[heads][:, rows])
    rq = np.stack([attention_bwd_dq_rows_fp64(f64(d["q"][h][rows]), f64(d["k"][h]), f64(d["v"][h]),
                                              f64(dob[h][rows]), d["scale"]) for h in heads])
    compare("dq sampled rows", gq, rq)
    h = 0 if H == 40 else H - 1
    keys = inputs.sample_rows(c.L, 256, seed=99)
    say("  oracle row statistics over all queries of head %d, then %d keys" % (h, len(keys)))
    rk, rv = key_rows_oracle(f64(d["q"][h]), f64(d["k"][h]), f64(d["v"][h]), f64(dob[h]), d["scale"], keys)
    compare("dk sampled keys head %d" % h, to_f64(dk[h][keys]), rk)
    compare("dv sampled keys head %d" % h, to_f64(dv[h][keys]), rv)
    check_key_sums(torch, "", dob, dk, dv)


def check_key_sums(torch, tag, dob, dk, dv):
    """sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i (softmax rows sum to one),
    per head, as vectors over the channels: the 2-norm of the residue within
    SUM_REL of the sum of the 2-norms of the rows it adds.  (The 2-norm is
    the one the Hadamard rotation of the FP4 path preserves; on the FP4
    workload a head's key gradient sits on a handful of keys whose
    contributions cancel, so a per-channel ratio would divide their rounding
    by a small sum.)"""
    dkd = dk.double()
    kr = float((dkd.sum(dim=1).norm(dim=1) / dkd.norm(dim=2).sum(dim=1).clamp_min(1e-300)).max())
    say("  %ssum over keys of dK: max ||sum|| / sum ||dK_j|| = %.3e" % (tag, kr))
    assert kr <= SUM_REL
    do = torch.from_numpy(f64(dob)).cuda()
    dvd = dv.double()
    vr = float(((dvd.sum(dim=1) - do.sum(dim=1)).norm(dim=1)
                / (dvd.norm(dim=2).sum(dim=1) + do.norm(dim=2).sum(dim=1))).max())
    say("  %ssum over keys of dV vs sum of dO: max ||diff|| / norms = %.3e" % (tag, vr))
    assert vr <= SUM_REL


# ---------------------------------------------- training-time FP4-QK backward --

def run_fp4_bwd(torch, d, dout_bits, flags):
    from long_sequence_dense_amd import binding
    q, k, v = (bf16_dev(torch, d[n]) for n in ("q", "k", "v"))
    H, L, _ = d["q"].shape
    prep = binding.qk_prep_fp4_ex(q, k, flags)
    codes = (prep["q_codes"], prep["q_scales"], prep["k_codes"], prep["k_scales"])
    o, o32, ml = binding.attn_fwd_fp4qk_train(*codes, v, softmax_scale=d["scale"])
    del o
    do = bf16_dev(torch, dout_bits)
    grads = [torch.full((H, L, 128), float("nan"), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    binding.attn_bwd_fp4qk(*codes, v, o32, ml, do, *grads, softmax_scale=d["scale"], flags=flags)
    torch.cuda.synchronize()
    return grads, prep


@pytest.mark.parametrize("cfg,H,L,flags", [("fp4", 2, 1000, 3), ("tiny", 2, 300, 3), ("fp4", 1, 65, 0),
                                           ("fp4", 2, 257, 2), ("tiny", 1, 130, 1), ("fp4", 2, 4000, 3)])
def test_fp4_bwd_small_full(torch, cfg, H, L, flags):
    from oracle.attention_bwd import fp4qk_bwd_ste_fp64
    from oracle.nvfp4 import qk_prep_fp4
    d = inputs.make_inputs(cfg, H=H, L=L)
    dob = inputs.make_tensor(d["cfg"], "do")
    say("case fp4 bwd %s H=%d L=%d flags=%d" % (cfg, H, L, flags))
    (dq, dk, dv), _ = run_fp4_bwd(torch, d, dob, flags)
    smooth, rotate = bool(flags & 1), bool(flags & 2)
    p = qk_prep_fp4(d["q"], d["k"], smooth=smooth, rotate=rotate)
    rq, rk, rv = fp4qk_bwd_ste_fp64(p["q_codes"], p["q_scales"], p["k_codes"], p["k_scales"], f64(d["v"]),
                                    f64(dob), d["scale"], rotate=rotate, smooth=smooth)
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        compare("fp4 %s %s L=%d f=%d" % (name, cfg, L, flags), to_f64(g), r)


def test_fp4_bwd_full_size(torch):
    """40 heads x 109,000 tokens of the FP4 workload: dQ on 1,000 sampled rows
    of two heads, dK and dV on 256 sampled key rows of head 0 (row-local oracle
    at the dequantized Q, K, rotated back), key sums of every key."""
    from oracle.attention_bwd import attention_bwd_dq_rows_fp64, hadamard_orthonormal
    from oracle.nvfp4 import dequant_nvfp4, qk_prep_fp4
    c = inputs.CONFIGS["fp4"]
    say("case fp4 bwd fp4 H=40 L=109000 (generate)")
    d = inputs.make_inputs("fp4")
    dob = inputs.make_tensor(c, "do")
    (dq, dk, dv), prep = run_fp4_bwd(torch, d, dob, 3)
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert not torch.isnan(g).any().item(), name
    # most rows of this workload put all their weight on one key (their
    # gradient is numerically zero), so the sample is large enough to hold
    # rows with a real gradient
    rows = inputs.sample_rows(c.L, 1024)
    heads = [0, 39]
    r = hadamard_orthonormal(128)
    refs, deq = [], {}
    for h in heads:
        p = qk_prep_fp4(d["q"][h:h + 1], d["k"][h:h + 1])
        qh = dequant_nvfp4(p["q_codes"][0], p["q_scales"][0])
        kh = dequant_nvfp4(p["k_codes"][0], p["k_scales"][0])
        deq[h] = (qh, kh)
        refs.append(attention_bwd_dq_rows_fp64(qh[rows], kh, f64(d["v"][h]), f64(dob[h][rows]), d["scale"]) @ r)
    compare("fp4 dq sampled rows", to_f64(dq[heads][:, rows]), np.stack(refs))
    keys = inputs.sample_rows(c.L, 256, seed=99)
    say("  oracle row statistics over all queries of head 0, then %d keys" % len(keys))
    qh, kh = deq[0]
    rk, rv = key_rows_oracle(qh, kh, f64(d["v"][0]), f64(dob[0]), d["scale"], keys)
    # sum over keys of dK is exactly zero, so the mean-key Jacobian adds nothing
    compare("fp4 dk sampled keys head 0", to_f64(dk[0][keys]), rk @ r)
    compare("fp4 dv sampled keys head 0", to_f64(dv[0][keys]), rv)
    check_key_sums(torch, "fp4 ", dob, dk, dv)
