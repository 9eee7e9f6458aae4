"""GPU parity of the attention backward (attn_bwd_bf16, attn_bwd_fp4qk) against
the fp64 gradient oracle, element by element within the error bound of the
kernels' BF16 arithmetic.  That arithmetic is the usual flash backward's: D =
rowsum(dO * O) is formed from the BF16 output O, so on strongly peaked rows
(one key takes almost all the weight, as the Student-t inputs with x20
channels produce) the true dS is nearly zero and the D error, which the bound
carries, can exceed it.

The HIP forward supplies O and the LSE (as a training step would); the oracle
computes the exact gradients of the same BF16 inputs.  Small shapes are
compared element by element in full; the full-size workload (40 heads x
109,000 tokens, as timed by the benchmark) on sampled dQ rows, and dK, dV
through the sums softmax fixes at any size (sum over keys of dK is zero, of
dV is the sum over queries of dO).
"""

import sys

import numpy as np
import pytest

from long_sequence_dense_amd import inputs

pytestmark = pytest.mark.gpu


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


def run_bwd(torch, d, dout_bits):
    from long_sequence_dense_amd import binding
    q, k, v = (bf16_dev(torch, d[n]) for n in ("q", "k", "v"))
    H, L, _ = d["q"].shape
    o = torch.empty((H, L, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((H, L), dtype=torch.float32, device="cuda")
    binding.attn_fwd_bf16(q, k, v, o, lse, softmax_scale=d["scale"])
    do = bf16_dev(torch, dout_bits)
    grads = [torch.full((H, L, 128), float("nan"), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    binding.attn_bwd_bf16(q, k, v, o, lse, do, *grads, softmax_scale=d["scale"])
    torch.cuda.synchronize()
    return grads, o


# The bar: every element within twice the error bound that the BF16
# arithmetic of the kernels implies (oracle.attention_bwd.attention_bwd_bound_fp64:
# D from the BF16 output O, P and dS rounded to BF16 for the products, fp32
# sums, BF16 outputs); the factor 2 covers what the model leaves out (the
# hardware exp2, the fp32 LSE).  A wrong index, operand or term gives errors
# of the order of the gradient itself, far above it.
BOUND_FACTOR = 2.0
UNDERFLOW = 2.0 ** -100   # exact values below the fp32 normal range flush to zero in the kernels


def compare(name, got, want, bound):
    err = np.abs(got - want)
    bound = bound + UNDERFLOW
    scale = np.max(np.abs(want))
    # an exactly zero bound (e.g. a K channel that quantizes to zero) admits no error
    ratio = float(np.max(np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))))
    say("  %-30s max-abs %.3e  max|ref| %.3e  rel-max %.3e  max err/bound %.3f" % (
        name, err.max(), scale, err.max() / max(scale, 1e-30), ratio))
    if ratio > BOUND_FACTOR:
        r = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))
        idx = np.unravel_index(np.argmax(r), r.shape)
        say("  worst element %s: got %.6e ref %.6e bound %.3e" % (idx, got[idx], want[idx], bound[idx]))
    assert np.all(np.isfinite(got)), name
    assert ratio <= BOUND_FACTOR, name


@pytest.mark.parametrize("cfg,H,L", [("tiny", 2, 1024), ("tiny", 2, 1), ("tiny", 3, 33), ("tiny", 2, 200),
                                     ("clip15s", 2, 3000), ("fp4", 1, 777)])
def test_bwd_small_full(torch, cfg, H, L):
    from oracle.attention_bwd import attention_bwd_bound_fp64, attention_bwd_fp64
    d = inputs.make_inputs(cfg, H=H, L=L)
    dob = inputs.make_tensor(d["cfg"], "do")
    say("case bwd %s H=%d L=%d" % (cfg, H, L))
    (dq, dk, dv), _ = run_bwd(torch, d, dob)
    args = (f64(d["q"]), f64(d["k"]), f64(d["v"]), f64(dob), d["scale"])
    refs, bounds = attention_bwd_fp64(*args), attention_bwd_bound_fp64(*args)
    for name, g, r, b in zip(("dq", "dk", "dv"), (dq, dk, dv), refs, bounds):
        compare("%s %s L=%d" % (name, cfg, L), to_f64(g), r, b)


def test_bwd_mid_full(torch):
    """Every gradient of two heads of 8192 tokens (256 key tiles, 64 query
    tiles of the two kernels), outlier channels on Q and K."""
    from oracle.attention_bwd import attention_bwd_bound_fp64, attention_bwd_fp64
    d = inputs.make_inputs("clip15s", H=2, L=8192)
    dob = inputs.make_tensor(d["cfg"], "do")
    say("case bwd clip15s H=2 L=8192")
    (dq, dk, dv), _ = run_bwd(torch, d, dob)
    args = (f64(d["q"]), f64(d["k"]), f64(d["v"]), f64(dob), d["scale"])
    refs, bounds = attention_bwd_fp64(*args), attention_bwd_bound_fp64(*args)
    for name, g, r, b in zip(("dq", "dk", "dv"), (dq, dk, dv), refs, bounds):
        compare("%s L=8192" % name, to_f64(g), r, b)


def test_bwd_deterministic(torch):
    d = inputs.make_inputs("tiny", H=2, L=1500)
    dob = inputs.make_tensor(d["cfg"], "do")
    a, _ = run_bwd(torch, d, dob)
    b, _ = run_bwd(torch, d, dob)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_bwd_full_size(torch):
    """40 heads x 109,000 tokens: dQ on sampled rows of sampled heads against
    the row-local oracle; dK and dV of every key through the sums that softmax
    fixes (sum over keys of dK = 0, of dV = sum over queries of dO)."""
    bwd_sampled(torch, 40)


def test_bwd_beyond_2gib(torch):
    """The same checks at 80 heads (2.23 GB per BF16 tensor): the last heads'
    rows lie past 2^31 bytes."""
    assert 79 * 109000 * 128 * 2 > 2 ** 31
    bwd_sampled(torch, 80)


def bwd_sampled(torch, H):
    from oracle.attention_bwd import attention_bwd_dq_bound_rows_fp64, attention_bwd_dq_rows_fp64
    c = inputs.CONFIGS["clip15s"].with_shape(H=H)
    say("case bwd clip15s H=%d L=%d (generate)" % (c.H, c.L))
    d = inputs.make_inputs(c)
    dob = inputs.make_tensor(c, "do")
    (dq, dk, dv), o = run_bwd(torch, d, dob)
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert not torch.isnan(g).any().item(), name
    rows = inputs.sample_rows(c.L, 40)
    heads = [0, H * 21 // 40, H - 1]
    gq = to_f64(dq[heads][:, rows])
    a = [(f64(d["q"][h][rows]), f64(d["k"][h]), f64(d["v"][h]), f64(dob[h][rows]), d["scale"]) for h in heads]
    rq = np.stack([attention_bwd_dq_rows_fp64(*x) for x in a])
    bq = np.stack([attention_bwd_dq_bound_rows_fp64(*x) for x in a])
    compare("dq sampled rows", gq, rq, bq)
    check_key_sums(torch, "", d["q"], dob, dk, dv, d["scale"], o=o)


def check_key_sums(torch, tag, q_bits_or_dev, dob, dk, dv, scale, o=None):
    """sum_j dK_j = -scale sum_i dD_i q_i and sum_j dV_j = sum_i dO_i up to
    rounding, where dD_i is the error of D_i = dO_i . O_i formed from the BF16
    output O.  Round-to-nearest errors are taken as independent, uniform in
    +-u |x| (variance u^2 x^2 / 3), and each sum is required within six
    standard deviations of its predicted spread:
      dK: sd^2 = (scale u)^2 / 3 sum_i q_ic^2 sum_c' (dO_ic' O_ic')^2   (the D errors)
               + u^2 / 3 sum_j dK_jc^2                                   (the dK roundings)
      dV: sd^2 = u^2 / 3 (sum_j dV_jc^2 + sum_i dO_ic^2 sum_j P_ij^2), the
          second term bounded by sum_i dO_ic^2 (P rounded to BF16)."""
    u = 2.0 ** -8
    do = torch.from_numpy(f64(dob)).cuda()
    q = q_bits_or_dev if isinstance(q_bits_or_dev, torch.Tensor) else torch.from_numpy(f64(q_bits_or_dev)).cuda()
    dkd = dk.double()
    ksum = dkd.sum(dim=1)
    var = u * u / 3.0 * (dkd * dkd).sum(dim=1)
    if o is not None:
        a2 = ((do * o.double()) ** 2).sum(dim=2, keepdim=True)
        var = var + (scale * u) ** 2 / 3.0 * (a2 * q * q).sum(dim=1)
    kr = float((ksum.abs() / (6.0 * var.sqrt())).max())
    say("  %ssum over keys of dK: max |sum| / 6 sd = %.3f (max |sum| / sum|dK| = %.3e)" % (
        tag, kr, float((ksum.abs() / dkd.abs().sum(dim=1)).max())))
    assert kr <= 1.0
    dvd = dv.double()
    vvar = u * u / 3.0 * ((dvd * dvd).sum(dim=1) + (do * do).sum(dim=1))
    vr = float(((dvd.sum(dim=1) - do.sum(dim=1)).abs() / (6.0 * vvar.sqrt())).max())
    say("  %ssum over keys of dV vs sum of dO: max |diff| / 6 sd = %.3f" % (tag, vr))
    assert vr <= 1.0


# ---------------------------------------------- training-time FP4-QK backward --

def run_fp4_bwd(torch, d, dout_bits, flags):
    from long_sequence_dense_amd import binding
    q, k, v = (bf16_dev(torch, d[n]) for n in ("q", "k", "v"))
    H, L, _ = d["q"].shape
    prep = binding.qk_prep_fp4_ex(q, k, flags)
    o = torch.empty((H, L, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((H, L), dtype=torch.float32, device="cuda")
    binding.attn_fwd_fp4qk(prep["q_codes"], prep["q_scales"], prep["k_codes"], prep["k_scales"], v, o, lse,
                           softmax_scale=d["scale"])
    do = bf16_dev(torch, dout_bits)
    grads = [torch.full((H, L, 128), float("nan"), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    binding.attn_bwd_fp4qk(prep["q_codes"], prep["q_scales"], prep["k_codes"], prep["k_scales"], v, o, lse, do,
                           *grads, softmax_scale=d["scale"], flags=flags)
    torch.cuda.synchronize()
    return grads, prep, o


def dequant_dev(torch, codes, scales):
    """Exact NVFP4 values as float64 on the GPU (test-side table lookup)."""
    from oracle.nvfp4 import e2m1_decode_table, e4m3_decode_table
    e2 = torch.from_numpy(e2m1_decode_table()).cuda()
    e4 = torch.from_numpy(e4m3_decode_table()).cuda()
    lo = (codes & 0xF).long()
    hi = (codes >> 4).long()
    vals = torch.stack([e2[lo], e2[hi]], dim=-1).reshape(codes.shape[:-1] + (codes.shape[-1] * 2,))
    sv = e4[scales.long()]
    return (vals.reshape(vals.shape[:-1] + (scales.shape[-1], 16)) * sv[..., None]).reshape(vals.shape)


def hadamard_dev(torch, n=128):
    h = torch.ones((1, 1), dtype=torch.float64, device="cuda")
    while h.shape[0] < n:
        h = torch.cat([torch.cat([h, h], 1), torch.cat([h, -h], 1)], 0)
    return h / np.sqrt(n)


@pytest.mark.parametrize("cfg,H,L,flags", [("fp4", 2, 1000, 3), ("tiny", 2, 300, 3), ("fp4", 1, 65, 0),
                                           ("fp4", 2, 257, 2), ("tiny", 1, 130, 1)])
def test_fp4_bwd_small_full(torch, cfg, H, L, flags):
    from oracle.attention_bwd import attention_bwd_bound_fp64, fp4qk_bwd_ste_fp64, rotate_bound
    from oracle.nvfp4 import dequant_nvfp4, qk_prep_fp4
    d = inputs.make_inputs(cfg, H=H, L=L)
    dob = inputs.make_tensor(d["cfg"], "do")
    say("case fp4 bwd %s H=%d L=%d flags=%d" % (cfg, H, L, flags))
    (dq, dk, dv), _, _ = run_fp4_bwd(torch, d, dob, flags)
    smooth, rotate = bool(flags & 1), bool(flags & 2)
    p = qk_prep_fp4(d["q"], d["k"], smooth=smooth, rotate=rotate)
    codes = (p["q_codes"], p["q_scales"], p["k_codes"], p["k_scales"], f64(d["v"]), f64(dob), d["scale"])
    rq, rk, rv = fp4qk_bwd_ste_fp64(*codes, rotate=rotate, smooth=smooth)
    # the kernel leaves out the mean-key Jacobian's term (zero in exact arithmetic)
    omitted = fp4qk_bwd_ste_fp64(*codes, rotate=rotate, smooth=False)[1] - rk
    bq, bk, bv = attention_bwd_bound_fp64(dequant_nvfp4(p["q_codes"], p["q_scales"]),
                                          dequant_nvfp4(p["k_codes"], p["k_scales"]), f64(d["v"]), f64(dob), d["scale"])
    if rotate:
        bq, bk = rotate_bound(bq, rq), rotate_bound(bk, rk, omitted=omitted)
    else:
        bk = bk + np.abs(omitted)
    for name, g, r, b in (("dq", dq, rq, bq), ("dk", dk, rk, bk), ("dv", dv, rv, bv)):
        compare("fp4 %s %s L=%d f=%d" % (name, cfg, L, flags), to_f64(g), r, b)


def test_fp4_bwd_full_size(torch):
    """40 heads x 109,000 tokens of the FP4 workload: dQ on sampled rows
    (row-local oracle at the dequantized Q, K, rotated back), dK and dV of every
    key through the softmax sums."""
    from oracle.attention_bwd import attention_bwd_dq_bound_rows_fp64, attention_bwd_dq_rows_fp64, rotate_bound
    from oracle.nvfp4 import dequant_nvfp4, qk_prep_fp4
    c = inputs.CONFIGS["fp4"]
    say("case fp4 bwd fp4 H=40 L=109000 (generate)")
    d = inputs.make_inputs("fp4")
    dob = inputs.make_tensor(c, "do")
    (dq, dk, dv), prep, o = run_fp4_bwd(torch, d, dob, 3)
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert not torch.isnan(g).any().item(), name
    rows = inputs.sample_rows(c.L, 24)
    heads = [0, 39]
    hm = np.array([[1.0]])
    while hm.shape[0] < 128:
        hm = np.block([[hm, hm], [hm, -hm]])
    hm /= np.sqrt(128)
    refs, bounds = [], []
    for h in heads:
        p = qk_prep_fp4(d["q"][h:h + 1], d["k"][h:h + 1])
        qh = dequant_nvfp4(p["q_codes"][0], p["q_scales"][0])
        kh = dequant_nvfp4(p["k_codes"][0], p["k_scales"][0])
        x = (qh[rows], kh, f64(d["v"][h]), f64(dob[h][rows]), d["scale"])
        refs.append(attention_bwd_dq_rows_fp64(*x) @ hm)
        bounds.append(rotate_bound(attention_bwd_dq_bound_rows_fp64(*x), refs[-1]))
    compare("fp4 dq sampled rows", to_f64(dq[heads][:, rows]), np.stack(refs), np.stack(bounds))
    # the key sums in the rotated basis of the quantized values: dKh = dK R
    r = hadamard_dev(torch)
    qh = dequant_dev(torch, prep["q_codes"], prep["q_scales"])
    check_key_sums(torch, "fp4 ", qh, dob, dk.double() @ r, dv, d["scale"], o=o)
