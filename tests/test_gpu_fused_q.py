"""GPU parity of the fused-Q FP4 path: qk_prep_fp4_ex with LSD_PREP_K_ONLY
(K's codes, scales and mean) followed by attn_fwd_fp4qk_fused_q (Q rotated
and quantized inside the attention kernel) against the two-call path
qk_prep_fp4 + attn_fwd_fp4qk, which the other tests compare with the oracle.
The fused kernel applies the prep's arithmetic to Q, so the results must be
bit-identical: K's outputs, O and the LSE.  The tiny workload is also
compared with the oracle directly."""

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


def both_paths(torch, d):
    from long_sequence_dense_amd import binding as b
    q, k, v = (bf16_dev(torch, d[n]) for n in ("q", "k", "v"))
    H, L, _ = d["q"].shape
    full = b.qk_prep_fp4(q, k)
    o1 = torch.full((H, L, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    l1 = torch.full((H, L), float("nan"), dtype=torch.float32, device="cuda")
    b.attn_fwd_fp4qk(full["q_codes"], full["q_scales"], full["k_codes"], full["k_scales"], v, o1, l1,
                     softmax_scale=d["scale"])
    kon = b.qk_prep_fp4_ex(None, k, b.PREP_K_ONLY | b.PREP_SMOOTH_K | b.PREP_ROTATE)
    o2 = torch.full((H, L, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    l2 = torch.full((H, L), float("nan"), dtype=torch.float32, device="cuda")
    b.attn_fwd_fp4qk_fused_q(q, kon["k_codes"], kon["k_scales"], v, o2, l2, softmax_scale=d["scale"])
    torch.cuda.synchronize()
    assert "q_codes" not in kon
    for key in ("k_codes", "k_scales", "k_mean"):
        assert torch.equal(full[key].view(torch.uint8), kon[key].view(torch.uint8)), key
    assert not torch.isnan(o2).any().item()
    same_o = torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    same_l = torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    nd = int((o1.view(torch.int16) != o2.view(torch.int16)).sum().item())
    say("  H=%d L=%d: O bit-identical %s (%d differ), LSE bit-identical %s" % (H, L, same_o, nd, same_l))
    assert same_o and same_l
    return o2, l2


@pytest.mark.parametrize("cfg,H,L", [("fp4", 2, 1), ("fp4", 2, 65), ("tiny", 3, 300), ("fp4", 3, 4000),
                                     ("clip15s", 2, 2500)])
def test_fused_q_bit_identical_small(torch, cfg, H, L):
    say("case fused-Q %s H=%d L=%d" % (cfg, H, L))
    both_paths(torch, inputs.make_inputs(cfg, H=H, L=L))


def test_fused_q_tiny_against_oracle(torch):
    from oracle.attention import attention_fp64
    from oracle.nvfp4 import dequant_nvfp4, qk_prep_fp4
    d = inputs.make_inputs("tiny")
    say("case fused-Q tiny against the oracle")
    o, _ = both_paths(torch, d)
    ref = qk_prep_fp4(d["q"], d["k"])
    qh = dequant_nvfp4(ref["q_codes"], ref["q_scales"])
    kh = dequant_nvfp4(ref["k_codes"], ref["k_scales"])
    oref, _ = attention_fp64(qh, kh, inputs.bf16_bits_to_f32(d["v"]).astype(np.float64), d["scale"])
    got = inputs.bf16_bits_to_f32(o.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    err = np.abs(got - oref)
    say("  max-abs %.3e mean-abs %.3e" % (err.max(), err.mean()))
    assert err.max() <= 2e-2 and err.mean() <= 2e-3


def test_fused_q_full_size_bit_identical(torch):
    c = inputs.CONFIGS["fp4"]
    say("case fused-Q fp4 H=%d L=%d (generate)" % (c.H, c.L))
    both_paths(torch, inputs.make_inputs("fp4"))
