"""GPU: the ablation variants of the Q/K preparation (qk_prep_fp4_ex) and the
FP4-QK attention error they lead to.

Method: "Pika H3 Flex in FastVideo: 7x Faster, and Near Real Time in 4-bit",
section "FP4 attention": plain NVFP4 Q/K against NVFP4 after smoothing K and
the shared Hadamard rotation (its per-layer error table puts plain FP4 above
the transformed variant).  Codes, scales and the mean of every variant are
compared bit-exactly with the oracle; the error of the HIP path's FP4-QK
output against its BF16 output is compared with the oracle's exact error on
sampled rows, and the pages' ordering is checked at the full size.
"""

import ctypes
import sys

import numpy as np
import pytest

from long_sequence_dense_amd import inputs

pytestmark = pytest.mark.gpu

FLAGS = [0, 1, 2, 3]          # bit 0: smooth K, bit 1: rotate
NAMES = {0: "plain", 1: "smooth", 2: "rotate", 3: "smooth+rotate"}


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


def sentinel_outputs(torch, H, L):
    return {
        "q_codes": torch.full((H, L, 64), 0xAB, dtype=torch.uint8, device="cuda"),
        "q_scales": torch.full((H, L, 8), 0xFF, dtype=torch.uint8, device="cuda"),
        "k_codes": torch.full((H, L, 64), 0xAB, dtype=torch.uint8, device="cuda"),
        "k_scales": torch.full((H, L, 8), 0xFF, dtype=torch.uint8, device="cuda"),
        "k_mean": torch.full((H, 128), float("nan"), dtype=torch.float32, device="cuda"),
    }


def run_prep_ex(torch, q, k, flags):
    from long_sequence_dense_amd import binding
    H, L, _ = q.shape
    out = sentinel_outputs(torch, H, L)
    binding.qk_prep_fp4_ex(q, k, flags, out=out)
    torch.cuda.synchronize()
    return out


def check_exact(name, got, ref, heads=None, rows=None):
    for key in ("q_codes", "q_scales", "k_codes", "k_scales"):
        g = got[key].cpu().numpy()
        if heads is not None:
            g = g[heads]
        if rows is not None:
            g = g[:, rows]
        nbad = int((g != ref[key]).sum())
        say("  %-36s %-8s mismatches %d of %d" % (name, key, nbad, g.size))
        assert nbad == 0, (name, key)
    km = got["k_mean"].cpu().numpy()
    if heads is not None:
        km = km[heads]
    assert np.array_equal(km.view(np.uint32), ref["k_mean"].view(np.uint32)), name


@pytest.mark.parametrize("flags", FLAGS)
@pytest.mark.parametrize("cfg,H,L", [("fp4", 3, 1000), ("tiny", 2, 1024), ("fp4", 1, 1), ("fp4", 2, 129)])
def test_prep_variant_exact(torch, flags, cfg, H, L):
    from oracle.nvfp4 import qk_prep_fp4
    d = inputs.make_inputs(cfg, H=H, L=L)
    say("case prep_ex %s flags=%d (%s) H=%d L=%d" % (cfg, flags, NAMES[flags], H, L))
    got = run_prep_ex(torch, bf16_dev(torch, d["q"]), bf16_dev(torch, d["k"]), flags)
    ref = qk_prep_fp4(d["q"], d["k"], smooth=bool(flags & 1), rotate=bool(flags & 2))
    check_exact("%s flags=%d" % (cfg, flags), got, ref)


def test_prep_ex_full_method_equals_qk_prep(torch):
    from long_sequence_dense_amd import binding
    d = inputs.make_inputs("fp4", H=2, L=5000)
    q, k = bf16_dev(torch, d["q"]), bf16_dev(torch, d["k"])
    say("case prep_ex flags=3 vs qk_prep_fp4 H=2 L=5000")
    a = run_prep_ex(torch, q, k, 3)
    b = sentinel_outputs(torch, 2, 5000)
    binding.qk_prep_fp4(q, k, out=b)
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key], b[key]), key


@pytest.mark.parametrize("flags", [0, 2])
def test_prep_variant_without_mean_or_workspace(torch, flags):
    # Without smoothing the C ABI takes NULL for k_mean and the workspace.
    from long_sequence_dense_amd import binding
    from oracle.nvfp4 import qk_prep_fp4
    d = inputs.make_inputs("fp4", H=2, L=300)
    q, k = bf16_dev(torch, d["q"]), bf16_dev(torch, d["k"])
    out = sentinel_outputs(torch, 2, 300)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    say("case prep_ex flags=%d NULL k_mean and workspace" % flags)
    st = binding.load_library().qk_prep_fp4_ex(
        p(q), p(k), p(out["q_codes"]), p(out["q_scales"]), p(out["k_codes"]), p(out["k_scales"]),
        ctypes.c_void_p(0), ctypes.c_void_p(0), 0, 2, 300, 128, flags,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    ref = qk_prep_fp4(d["q"], d["k"], smooth=False, rotate=bool(flags & 2))
    out["k_mean"] = torch.zeros(2, 128, dtype=torch.float32, device="cuda")   # not written
    check_exact("NULL mean flags=%d" % flags, out, ref)


@pytest.mark.parametrize("flags", [0, 1, 2])
def test_prep_variant_full_size_sampled(torch, flags):
    """40 heads x 109,000 tokens: sampled rows of every head (of 3 heads when
    the oracle needs the exact mean over all rows)."""
    from oracle.nvfp4 import qk_prep_fp4
    c = inputs.CONFIGS["fp4"]
    say("case prep_ex fp4 H=40 L=109000 flags=%d (generate)" % flags)
    d = inputs.make_inputs("fp4")
    got = run_prep_ex(torch, bf16_dev(torch, d["q"]), bf16_dev(torch, d["k"]), flags)
    rows = inputs.sample_rows(c.L, 256)
    heads = [0, 17, 39] if flags & 1 else list(range(c.H))
    ref = qk_prep_fp4(d["q"], d["k"], heads=heads, rows=rows, smooth=bool(flags & 1), rotate=bool(flags & 2))
    check_exact("full-size flags=%d" % flags, got, ref, heads=heads, rows=rows)


def fp4_output(torch, binding, q, k, v, flags, scale):
    prep = run_prep_ex(torch, q, k, flags)
    o = binding.attn_fwd_fp4qk(prep["q_codes"], prep["q_scales"], prep["k_codes"], prep["k_scales"], v,
                               softmax_scale=scale)
    torch.cuda.synchronize()
    return o


def rel_err(torch, a, b):
    a = a.double()
    b = b.double()
    return float(torch.linalg.vector_norm(a - b) / torch.linalg.vector_norm(b))


def test_error_harness_matches_oracle(torch):
    """The HIP path's FP4-QK error (against its BF16 output) tracks the
    oracle's exact error on the same rows: the kernels' BF16 roundings are far
    below the quantization error."""
    from long_sequence_dense_amd import binding
    from oracle.fp4_error import fp4_outputs, relative_error
    d = inputs.make_inputs("fp4", H=3, L=4096)
    q, k, v = (bf16_dev(torch, d[n]) for n in ("q", "k", "v"))
    o_bf16 = binding.attn_fwd_bf16(q, k, v, softmax_scale=d["scale"])
    rows = inputs.sample_rows(4096, 48)
    for flags in FLAGS:
        o = fp4_output(torch, binding, q, k, v, flags, d["scale"])
        idx = torch.as_tensor(rows, device="cuda")
        e_gpu = rel_err(torch, o[:, idx], o_bf16[:, idx])
        o_ref, o_fp4 = fp4_outputs(d["q"], d["k"], d["v"], d["scale"], bool(flags & 1), bool(flags & 2), rows=rows)
        e_or = relative_error(o_fp4, o_ref)
        say("  flags=%d %-14s error GPU %.4f  oracle %.4f" % (flags, NAMES[flags], e_gpu, e_or))
        assert abs(e_gpu - e_or) <= 0.03 * e_or, (flags, e_gpu, e_or)


def test_error_ordering_full_size(torch):
    """The pages' ordering on the full-size FP4 workload (40 x 109,000): FP4-QK
    after smoothing and rotation is closer to BF16 attention than plain FP4."""
    from long_sequence_dense_amd import binding
    say("case ablation error fp4 H=40 L=109000 (generate)")
    d = inputs.make_inputs("fp4")
    q, k, v = (bf16_dev(torch, d[n]) for n in ("q", "k", "v"))
    o_bf16 = binding.attn_fwd_bf16(q, k, v, softmax_scale=d["scale"])
    err = {}
    for flags in FLAGS:
        o = fp4_output(torch, binding, q, k, v, flags, d["scale"])
        err[flags] = rel_err(torch, o, o_bf16)
        say("  full-size error %-14s %.4f" % (NAMES[flags], err[flags]))
        del o
    assert err[3] < 0.9 * err[0], err
