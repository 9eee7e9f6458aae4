"""GPU parity of the NVFP4 W4A4 linear layer (nvfp4_quantize, nvfp4_linear)
against the fp64 oracle (oracle.nvfp4_linear).

The quantizer's codes and scales are compared bit for bit, in both code
layouts (row-major, and the product's tiled load order: a plain permutation
of the row-major bytes with zero padding, rebuilt here from the oracle's
row-major codes).  The product is
compared element by element within twice the error bound of the kernel's
arithmetic (exact BF16 operands, fp32 sums, fp32 scaling, BF16 output);
the oracle quantizes the same BF16 inputs itself, so no GPU value is an
oracle input.  Small and ragged shapes (M, N not multiples of the 256 x 256
output tile, K not a multiple of the 64-value stage, N not a multiple of 4)
are compared in full; the full-size workload (109,000 tokens x 5120 -> 5120,
one attention projection at the 40 x 128 hidden size) on sampled token rows,
with every weight code checked.
"""

import sys

import numpy as np
import pytest

from long_sequence_dense_amd import inputs
from nvfp4_layout import from_tiled, to_tiled
from oracle import nvfp4_linear as ref

pytestmark = pytest.mark.gpu

E4M3_MAX = 448.0
E2M1_MAX = 6.0


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


def calibrated(bits):
    """Static global scale from a calibration pass over the tensor itself:
    its largest magnitude maps to the largest code, 6 * 448 (a float32
    quotient, as a host-side calibration would compute it)."""
    amax = np.float32(np.max(np.abs(inputs.bf16_bits_to_f32(bits))))
    return float(amax / np.float32(E2M1_MAX * E4M3_MAX))


ROWS, TILED = 0, 1
def gpu_quantize(torch, bits, g, layout=ROWS):
    from long_sequence_dense_amd import binding
    x = bf16_dev(torch, bits)
    rows, cols = bits.shape
    cshape = (rows, cols // 2) if layout == ROWS else (binding.nvfp4_codes_bytes(rows, cols, layout),)
    sshape = (rows, cols // 16) if layout == ROWS else (binding.nvfp4_scales_bytes(rows, cols, layout),)
    codes = torch.full(cshape, 0xA5, dtype=torch.uint8, device="cuda")
    scales = torch.full(sshape, 0xA5, dtype=torch.uint8, device="cuda")
    binding.nvfp4_quantize(x, g, codes, scales, layout=layout)
    torch.cuda.synchronize()
    return codes, scales


def check_codes(tag, got_c, got_s, bits, g, layout=ROWS):
    """Compare with the oracle's codes (in the layout's byte order); returns
    the oracle's row-major codes and scales."""
    want_c, want_s = ref.quantize(inputs.bf16_bits_to_f32(bits), g)
    rc, rs = want_c, want_s
    if layout == TILED:
        want_c, want_s = to_tiled(want_c, want_s)
    gc, gs = got_c.cpu().numpy(), got_s.cpu().numpy()
    nc, ns = int(np.sum(gc != want_c)), int(np.sum(gs != want_s))
    say("  %-28s codes %d/%d differ, scales %d/%d differ" % (tag, nc, gc.size, ns, gs.size))
    assert nc == 0 and ns == 0
    return rc, rs


QUANT_CASES = [
    # rows, cols, seed, scale choice
    (1, 16, 1, "one"),
    (37, 48, 2, "calibrated"),
    (300, 5120, 3, "calibrated"),
    (129, 160, 4, "pow2"),            # g = 2^-3: codes as for g = 1 with the scales shifted
    (64, 256, 5, "clip"),             # g far below calibration: saturation at 6 * 448
    (1000, 64, 6, "odd"),             # an arbitrary float32 g
]


@pytest.mark.parametrize("layout", [ROWS, TILED])
@pytest.mark.parametrize("rows,cols,seed,gsel", QUANT_CASES)
def test_quantize_bit_exact(torch, rows, cols, seed, gsel, layout):
    bits = inputs.linear_operand("x", rows, cols, seed)
    g = {"one": 1.0, "calibrated": calibrated(bits), "pow2": 0.125, "clip": calibrated(bits) / 50.0,
         "odd": float(np.float32(0.0123456))}[gsel]
    say("case quantize rows=%d cols=%d seed=%d g=%s (%r) layout=%d" % (rows, cols, seed, gsel, g, layout))
    c, s = gpu_quantize(torch, bits, g, layout)
    check_codes("x %dx%d" % (rows, cols), c, s, bits, g, layout)


def e4m3_value(j):
    """OCP E4M3 value of the positive code j (1 <= j <= 126), from the bit
    fields: exponent j >> 3 (bias 7), mantissa j & 7, subnormals m * 2^-9."""
    e, m = j >> 3, j & 7
    return 2.0 ** (e - 7) * (1 + m / 8) if e else m * 2.0 ** -9


def tie_blocks(seed=9):
    """One 16-value block per row that puts the quantizer's decisions on and
    next to every rounding boundary (all of them are BF16 values: each has at
    most 7 significant bits):
      - scale boundaries: block max = 6 x the midpoint of neighbouring E4M3
        values, and the BF16 values just below and above it;
      - code boundaries: for every scale v (block max 6 v, so the scale is v
        exactly) the E2M1 midpoints times v, and the BF16 values around them;
      - saturation: block maxima at, just above and far above 6 x 448.
    Signs, positions and the filler values are seeded."""
    rng = np.random.default_rng(seed)
    to_bits = lambda a: inputs.f32_to_bf16_bits(np.atleast_1d(np.asarray(a, np.float32)))
    one = lambda x: int(to_bits(x)[0])
    up = lambda b: b + 1                      # next BF16 magnitude (positive bit patterns)
    down = lambda b: b - 1
    rows = []

    def block(amax_bits, others_bits):
        vals = np.zeros(16, np.uint16)
        pos = rng.permutation(16)
        vals[pos[0]] = amax_bits
        for i, b in enumerate(others_bits[:15]):
            vals[pos[1 + i]] = b
        signs = rng.integers(0, 2, 16).astype(np.uint16) << 15
        rows.append(vals | signs)

    vs = [e4m3_value(j) for j in range(1, 127)]
    for c in range(0, 126):                   # scale midpoints between codes c and c + 1
        lo = vs[c - 1] if c else 0.0
        mid6 = 3.0 * (lo + vs[c])
        b = one(mid6)
        assert float(inputs.bf16_bits_to_f32(np.uint16(b))) == mid6
        for a in (b, down(b), up(b)):
            filler = to_bits(rng.uniform(0, 1, 15) * float(inputs.bf16_bits_to_f32(np.uint16(a))))
            block(a, list(filler))
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    for v in vs:                              # code midpoints at every scale
        amax = one(6.0 * v)
        ties = [one(t * v) for t in mids]
        assert all(float(inputs.bf16_bits_to_f32(np.uint16(b))) == t * v for b, t in zip(ties, mids))
        near = [up(b) for b in ties] + [down(b) for b in ties]
        block(amax, ties + near[:8])
        block(amax, near[8:] + [0, 0x8000, one(v / 64)] + list(to_bits(rng.uniform(0, 6 * v, 6))))
    for amax in (2688.0, 2700.0, 3000.0, 1.0e6):
        b = one(amax)
        block(b, list(to_bits([2688.0, 2600.0, 2500.0, 2400.0, 448.0 * 5, 448.0 * 5.5, 1.0, 0.0])))
    return np.stack(rows)


@pytest.mark.parametrize("layout", [ROWS, TILED])
def test_quantize_every_rounding_boundary(torch, layout):
    bits = tie_blocks()
    say("case quantize rounding boundaries rows=%d layout=%d" % (bits.shape[0], layout))
    c, s = gpu_quantize(torch, bits, 1.0, layout)
    check_codes("boundaries", c, s, bits, 1.0, layout)


@pytest.mark.parametrize("layout", [ROWS, TILED])
def test_quantize_quotient_next_to_decisions(torch, layout):
    """Blocks whose exact x / g lies next to the rounding boundary beside a
    code or scale threshold (tests/quotient_cases.py, each with its own odd
    float32 g): only the correctly rounded quotient RN32(x / g) gives the
    oracle's codes and scales on all of them."""
    from quotient_cases import quotient_cases
    cases = quotient_cases(60)
    say("case quantize quotient next to decisions: %d blocks, layout=%d" % (len(cases), layout))
    for i, (bits, g, kind, tau) in enumerate(cases):
        c, s = gpu_quantize(torch, bits[None], float(g), layout)
        check_codes("quotient case %d (%s)" % (i, kind), c, s, bits[None], float(g), layout)


def test_quantize_overflowing_quotient_saturates(torch):
    """x / g beyond the float32 range (the largest BF16 values with g < 1):
    scale 448 and code +-6, as for any value past 6 * 448 * g."""
    x = np.zeros((2, 32), np.uint16)
    x[0, :4] = [0x7F7F, 0xFF7F, 0x7F00, 0x3F80]        # +-3.39e38, 1.7e38, 1.0
    x[1, 16:19] = [0x7F7F, 0x0001, 0x8000]             # and a subnormal and -0 beside it
    for g in (0.5, float(np.float32(0.9999)), float(np.float32(1e-30))):
        say("case quantize overflowing quotient g=%r" % g)
        for layout in (ROWS, TILED):
            c, s = gpu_quantize(torch, x, g, layout)
            check_codes("overflow g=%r" % g, c, s, x, g, layout)


def test_quantize_subnormal_quotients(torch):
    """Quotients in float32's subnormal range, among them exact rounding ties
    (15 * 2^-133 / (3 * 2^17) = 2.5 * 2^-149) and values below half the
    smallest subnormal: the values of a block scaled so small that its scale
    is a subnormal E4M3 value or zero."""
    rng = np.random.default_rng(17)
    x = np.zeros((3, 32), np.uint16)
    x[0, :16] = 0x000F                                 # 15 * 2^-133 (BF16 subnormal)
    x[0, 16:] = rng.integers(1, 0x80, 16)              # BF16 subnormals
    x[1] = inputs.f32_to_bf16_bits((rng.standard_normal(32) * 1e-38).astype(np.float32))
    x[2] = rng.integers(0, 0x0300, 32).astype(np.uint16) | (rng.integers(0, 2, 32).astype(np.uint16) << 15)
    for g in (float(3 * 2 ** 17), float(np.float32(7.77e5)), 1.0):
        say("case quantize subnormal quotients g=%r" % g)
        for layout in (ROWS, TILED):
            c, s = gpu_quantize(torch, x, g, layout)
            check_codes("subnormal g=%r" % g, c, s, x, g, layout)


def compare(tag, got, want, bound):
    err = np.abs(got - want)
    ratio = float(np.max(err / (2.0 * bound + 2.0 ** -120)))
    say("  %-28s max-abs %.3e  max|ref| %.3e  max err/(2 bound) %.3f"
        % (tag, float(err.max()), float(np.abs(want).max()), ratio))
    assert np.all(np.isfinite(got))
    assert ratio <= 1.0


def to_f64(torch, y):
    return inputs.bf16_bits_to_f32(y.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)


LINEAR_CASES = [
    # M, N, K
    (1, 1, 16),
    (33, 17, 48),                     # everything ragged, N odd (scalar stores)
    (300, 260, 320),                  # 2 x 2 tiles, ragged M and N, K = 5 stages
    (512, 512, 1024),                 # whole tiles
    (257, 301, 80),                   # ragged K stage (80 = 64 + 16), N % 4 = 1
    (700, 1030, 5120),                # the hidden size as K
]


@pytest.mark.parametrize("layout", [ROWS, TILED])
@pytest.mark.parametrize("M,N,K", LINEAR_CASES)
def test_linear_small_full(torch, M, N, K, layout):
    from long_sequence_dense_amd import binding
    say("case linear M=%d N=%d K=%d layout=%d" % (M, N, K, layout))
    xb = inputs.linear_operand("x", M, K, 20 + M)
    wb = inputs.linear_operand("w", N, K, 30 + N)
    gx, gw = calibrated(xb), calibrated(wb)
    xc, xs = gpu_quantize(torch, xb, gx, layout)
    wc, ws = gpu_quantize(torch, wb, gw, layout)
    rxc, rxs = check_codes("x", xc, xs, xb, gx, layout)
    rwc, rws = check_codes("w", wc, ws, wb, gw, layout)
    y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    binding.nvfp4_linear(xc, xs, gx, wc, ws, gw, y, layout=layout, M=M, N=N, K=K)
    torch.cuda.synchronize()
    want = ref.linear(rxc, rxs, gx, rwc, rws, gw)
    bound = ref.linear_bound(rxc, rxs, gx, rwc, rws, gw)
    compare("y %dx%dx%d" % (M, N, K), to_f64(torch, y), want, bound)


def test_linear_deterministic_and_layouts_agree(torch):
    from long_sequence_dense_amd import binding
    M, N, K = 600, 520, 640
    say("case linear deterministic M=%d N=%d K=%d" % (M, N, K))
    xb, wb = inputs.linear_operand("x", M, K, 41), inputs.linear_operand("w", N, K, 42)
    xc, xs = gpu_quantize(torch, xb, 0.01)
    wc, ws = gpu_quantize(torch, wb, 0.001)
    a = binding.nvfp4_linear(xc, xs, 0.01, wc, ws, 0.001)
    b = binding.nvfp4_linear(xc, xs, 0.01, wc, ws, 0.001)
    txc, txs = gpu_quantize(torch, xb, 0.01, TILED)
    twc, tws = gpu_quantize(torch, wb, 0.001, TILED)
    t = binding.nvfp4_linear(txc, txs, 0.01, twc, tws, 0.001, layout=TILED, M=M, N=N, K=K)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # the same products summed in the same order: identical bits
    assert torch.equal(a.view(torch.int16), t.view(torch.int16))


FULL_M, FULL_N, FULL_K = 109000, 5120, 5120


@pytest.mark.parametrize("layout", [TILED, ROWS])
def test_linear_full_size(torch, layout):
    """Full-size projection as the benchmark runs it (tiled) and row-major:
    all weight codes bit exact, sampled token rows' codes bit exact and their
    outputs within the bound."""
    linear_sampled(torch, layout, FULL_M, FULL_N, FULL_K, "full")


@pytest.mark.parametrize("layout", [ROWS, TILED])
def test_linear_output_beyond_2gib(torch, layout):
    """A 300,000 x 4096 BF16 output (2.46 GB): output rows past 2^31 bytes,
    checked as in the full-size case."""
    assert 300000 * 4096 * 2 > 2 ** 31
    linear_sampled(torch, layout, 300000, 4096, 1024, "output past 2 GiB")


def linear_sampled(torch, layout, M, N, K, tag):
    from long_sequence_dense_amd import binding
    say("case linear %s M=%d N=%d K=%d layout=%d (generate)" % (tag, M, N, K, layout))
    xb = inputs.linear_operand("x", M, K, 7)
    wb = inputs.linear_operand("w", N, K, 8)
    gx, gw = calibrated(xb), calibrated(wb)
    xc, xs = gpu_quantize(torch, xb, gx, layout)
    del xb
    wc, ws = gpu_quantize(torch, wb, gw, layout)
    rwc, rws = check_codes("w all rows", wc, ws, wb, gw, layout)
    y = binding.nvfp4_linear(xc, xs, gx, wc, ws, gw, layout=layout, M=M, N=N, K=K)
    torch.cuda.synchronize()
    rows = inputs.sample_rows(M, 48, seed=77, tiles=(256,))
    xr = inputs.linear_operand("x", M, K, 7, row_ids=rows)
    if layout == TILED:
        gxc, gxs = from_tiled(xc.cpu().numpy(), xs.cpu().numpy(), M, K)
        gxc, gxs = gxc[rows], gxs[rows]
    else:
        idx = torch.from_numpy(rows).cuda()
        gxc, gxs = xc.index_select(0, idx).cpu().numpy(), xs.index_select(0, idx).cpu().numpy()
    rxc, rxs = ref.quantize(inputs.bf16_bits_to_f32(xr), gx)
    nc, ns = int(np.sum(gxc != rxc)), int(np.sum(gxs != rxs))
    say("  %-28s codes %d/%d differ, scales %d/%d differ" % ("x sampled rows", nc, rxc.size, ns, rxs.size))
    assert nc == 0 and ns == 0
    want = ref.linear(rxc, rxs, gx, rwc, rws, gw)
    bound = ref.linear_bound(rxc, rxs, gx, rwc, rws, gw)
    idx = torch.from_numpy(rows).cuda()
    compare("y sampled rows", to_f64(torch, y.index_select(0, idx)), want, bound)
