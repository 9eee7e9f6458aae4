"""GPU test of qk_prep_fp4_noalloc (the prep with the library's static
scratch, for callers that cannot allocate) against qk_prep_fp4 (the same
prep with a caller workspace), through the C ABI: bit-identical codes,
scales and mean on two calls in a row, the second one smaller, so that the
scratch left by the first call is reused; then once more after the
workspace entry point has run in between."""

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


def outputs(torch, H, L, fill):
    return {
        "q_codes": torch.full((H, L, 64), fill, dtype=torch.uint8, device="cuda"),
        "q_scales": torch.full((H, L, 8), fill, dtype=torch.uint8, device="cuda"),
        "k_codes": torch.full((H, L, 64), fill, dtype=torch.uint8, device="cuda"),
        "k_scales": torch.full((H, L, 8), fill, dtype=torch.uint8, device="cuda"),
        "k_mean": torch.full((H, 128), float("nan"), dtype=torch.float32, device="cuda"),
    }


def case(torch, cfg, H, L):
    from long_sequence_dense_amd import binding
    d = inputs.make_inputs(cfg, H=H, L=L)
    q = torch.from_numpy(d["q"].view(np.int16)).cuda().view(torch.bfloat16)
    k = torch.from_numpy(d["k"].view(np.int16)).cuda().view(torch.bfloat16)
    say("case noalloc prep %s H=%d L=%d" % (cfg, H, L))
    got = binding.qk_prep_fp4_noalloc(q, k, outputs(torch, H, L, 0xAB))
    torch.cuda.synchronize()
    want = binding.qk_prep_fp4(q, k, out=outputs(torch, H, L, 0x5C))
    torch.cuda.synchronize()
    for key in got:
        assert torch.equal(got[key].view(torch.uint8), want[key].view(torch.uint8)), key
    return q, k


def test_noalloc_matches_workspace_entry_two_calls(torch):
    from long_sequence_dense_amd import binding
    case(torch, "fp4", 40, 109000)              # the full-size workload: 27 chunks per head
    q, k = case(torch, "tiny", 3, 5000)         # smaller, ragged: reuses the first call's scratch
    # and again with the workspace entry point having run in between
    again = binding.qk_prep_fp4_noalloc(q, k, outputs(torch, 3, 5000, 0x11))
    ref = binding.qk_prep_fp4(q, k, out=outputs(torch, 3, 5000, 0x22))
    torch.cuda.synchronize()
    for key in again:
        assert torch.equal(again[key].view(torch.uint8), ref[key].view(torch.uint8)), key


def test_noalloc_rejects_beyond_scratch(torch):
    from long_sequence_dense_amd import binding
    H, L = 4097, 1
    q = torch.zeros((H, L, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(binding.LsdError) as e:
        binding.qk_prep_fp4_noalloc(q, q, outputs(torch, H, L, 0))
    assert e.value.status == 5
