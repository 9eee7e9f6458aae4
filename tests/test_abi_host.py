"""The C-ABI library on the host (no GPU needed): it loads, exports every
symbol include/lsd_attn.h declares, and rejects bad arguments with the
documented status before anything is enqueued (no compute calls here)."""

import ctypes
import os
import re

import pytest

from long_sequence_dense_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lsd_attn.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("library not built")
    return binding.load_library()


def test_header_and_binding_agree():
    assert header_functions() == sorted(binding.SIGNATURES)


def test_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.lsd_abi_version() == 5 == binding.ABI_VERSION
    assert "#define LSD_ABI_VERSION 5\n" in open(HEADER).read()
    for st in range(9):
        assert lib.lsd_status_str(st).decode()
    assert lib.lsd_status_str(99).decode() == "unknown status"


def test_workspace_query(lib):
    # exact fp64 partial sums: 16 per 4096-row chunk per (head, channel)
    assert lib.qk_prep_fp4_workspace_bytes(40, 109000, 128) == 40 * 128 * 27 * 16 * 8
    assert lib.qk_prep_fp4_workspace_bytes(2, 4096, 128) == 2 * 128 * 1 * 16 * 8
    assert lib.qk_prep_fp4_workspace_bytes(2, 4097, 128) == 2 * 128 * 2 * 16 * 8
    assert lib.qk_prep_fp4_workspace_bytes(1, 1, 128) == 128 * 16 * 8
    assert lib.qk_prep_fp4_workspace_bytes(0, 10, 128) == 0
    assert lib.qk_prep_fp4_workspace_bytes(1, 10, 64) == 0


A = ctypes.c_void_p(0x100000)       # fake, 16-byte aligned, never dereferenced
B = ctypes.c_void_p(0x100008)       # 8-byte aligned only
N = ctypes.c_void_p(0)


def test_attn_bf16_argument_errors(lib):
    f = lib.attn_fwd_bf16
    assert f(A, A, A, A, N, 2, 16, 64, 0.1, N) == 3            # d
    assert f(A, A, A, A, N, 0, 16, 128, 0.1, N) == 2           # H
    assert f(A, A, A, A, N, 2, 0, 128, 0.1, N) == 2            # L
    assert f(A, A, A, A, N, 70000, 70000, 128, 0.1, N) == 2    # H*L overflow
    assert f(A, A, A, A, N, 1, 1 << 23, 128, 0.1, N) == 2      # one head too long for 32-bit offsets
    assert f(N, A, A, A, N, 2, 16, 128, 0.1, N) == 1           # null q
    assert f(A, A, A, N, N, 2, 16, 128, 0.1, N) == 1           # null o
    assert f(A, B, A, A, N, 2, 16, 128, 0.1, N) == 4           # misaligned k
    assert f(A, A, A, A, A, 2, 16, 128, 0.0, N) == 7           # scale 0
    assert f(A, A, A, A, A, 2, 16, 128, float("nan"), N) == 7
    assert f(A, A, A, A, A, 2, 16, 128, float("inf"), N) == 7


def test_prep_argument_errors(lib):
    f = lib.qk_prep_fp4
    ws = ctypes.c_void_p(0x200000)
    need = lib.qk_prep_fp4_workspace_bytes(2, 16, 128)
    assert f(A, A, A, A, A, A, A, ws, need, 2, 16, 64, N) == 3
    assert f(A, A, A, A, A, A, N, ws, need, 2, 16, 128, N) == 1          # null k_mean
    assert f(A, A, A, B, A, A, A, ws, need, 2, 16, 128, N) == 4          # misaligned scales
    assert f(A, A, A, A, A, A, A, N, need, 2, 16, 128, N) == 5           # null workspace
    assert f(A, A, A, A, A, A, A, ws, need - 1, 2, 16, 128, N) == 5      # too small
    assert f(A, A, A, A, A, A, A, ctypes.c_void_p(0x200010), need, 2, 16, 128, N) == 5  # not 256-aligned


def test_prep_ex_argument_errors(lib):
    f = lib.qk_prep_fp4_ex
    ws = ctypes.c_void_p(0x200000)
    need = lib.qk_prep_fp4_workspace_bytes(2, 16, 128)
    assert f(A, A, A, A, A, A, A, ws, need, 2, 16, 128, 8, N) == 8         # unknown flag bit
    assert f(A, A, A, A, A, A, A, ws, need, 2, 16, 128, -1, N) == 8
    assert f(A, A, A, A, A, A, A, ws, need, 2, 16, 64, 3, N) == 3
    assert f(A, A, A, A, A, A, N, ws, need, 2, 16, 128, 1, N) == 1         # smoothing needs k_mean
    assert f(A, A, A, A, A, A, A, N, 0, 2, 16, 128, 3, N) == 5             # ... and the workspace
    assert f(A, A, A, A, A, A, B, N, 0, 2, 16, 128, 2, N) == 4             # misaligned optional k_mean
    assert f(A, A, N, A, A, A, N, N, 0, 2, 16, 128, 0, N) == 1             # null q_codes


def test_noalloc_prep_argument_errors(lib):
    # every rejection happens on the host, before the scratch is looked up
    f = lib.qk_prep_fp4_noalloc
    ok = [A] * 7
    assert f(*ok, 2, 16, 64, N) == 3                                    # d
    assert f(*ok, 0, 16, 128, N) == 2                                   # H
    for i in range(7):                                                  # every pointer is required
        args = list(ok)
        args[i] = N
        assert f(*args, 2, 16, 128, N) == 1, i
    args = list(ok)
    args[6] = B                                                         # k_mean misaligned
    assert f(*args, 2, 16, 128, N) == 4
    # beyond the static scratch: H * ceil(L / 4096) > 4096
    assert f(*ok, 4097, 16, 128, N) == 5
    assert f(*ok, 40, 4096 * 103, 128, N) == 5
    assert lib.qk_prep_fp4_workspace_bytes(40, 4096 * 102, 128) == 4080 * 128 * 16 * 8 <= 64 << 20


def test_fp4qk_argument_errors(lib):
    f = lib.attn_fwd_fp4qk
    assert f(A, A, A, A, A, A, N, 2, 16, 128, -1.0, N) == 7
    assert f(A, A, N, A, A, A, N, 2, 16, 128, 0.1, N) == 1
    assert f(A, A, A, A, A, B, N, 2, 16, 128, 0.1, N) == 4
    assert f(A, A, A, A, A, A, N, 2, 16, 256, 0.1, N) == 3


def test_fused_q_argument_errors(lib):
    f = lib.attn_fwd_fp4qk_fused_q
    ok = [A] * 5
    assert f(*ok, N, 2, 16, 256, 0.1, N) == 3                           # d
    assert f(*ok, N, 2, 1 << 23, 128, 0.1, N) == 2                      # one head too long
    for i in range(5):
        args = list(ok)
        args[i] = N
        assert f(*args, N, 2, 16, 128, 0.1, N) == 1, i
    args = list(ok)
    args[0] = B
    assert f(*args, N, 2, 16, 128, 0.1, N) == 4
    assert f(*ok, ctypes.c_void_p(0x100002), 2, 16, 128, 0.1, N) == 4   # lse alignment
    assert f(*ok, N, 2, 16, 128, float("inf"), N) == 7


def test_k_only_prep_flag_errors(lib):
    f = lib.qk_prep_fp4_ex
    ws = ctypes.c_void_p(0x200000)
    need = lib.qk_prep_fp4_workspace_bytes(2, 16, 128)
    # K's pointers stay required; an unknown bit is still rejected
    assert f(N, N, N, N, N, A, A, ws, need, 2, 16, 128, 7, N) == 1      # k NULL
    assert f(N, A, N, N, A, N, A, ws, need, 2, 16, 128, 7, N) == 1      # k_scales NULL
    assert f(N, A, N, N, A, A, N, ws, need, 2, 16, 128, 7, N) == 1      # k_mean NULL with smoothing
    assert f(N, A, N, N, A, A, A, ws, need, 2, 16, 128, 15, N) == 8     # unknown bit 8
    assert f(N, A, N, N, A, A, A, ws, need - 1, 2, 16, 128, 7, N) == 5  # workspace


def test_missing_library_raises(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        binding.load_library(str(tmp_path / "nope.so"))


def test_bwd_workspace_queries(lib):
    assert lib.attn_bwd_bf16_workspace_bytes(40, 109000, 128) == 3 * 40 * 109000 * 4
    assert lib.attn_bwd_bf16_workspace_bytes(2, 16, 64) == 0
    assert lib.attn_bwd_fp4qk_workspace_bytes(2, 16, 128) == 4 * 2 * 16 * 128 * 2 + 3 * 2 * 16 * 4
    assert lib.attn_bwd_fp4qk_workspace_bytes(0, 16, 128) == 0


def test_train_forward_argument_errors(lib):
    C = ctypes.c_void_p(0x100004)       # 4-byte aligned only
    for f, nin in ((lib.attn_fwd_bf16_train, 3), (lib.attn_fwd_fp4qk_train, 5)):
        ins = [A] * nin
        # after the inputs: o, lse (optional), o_f32, row_ml; no call here passes every check
        assert f(*ins, A, N, A, A, 2, 16, 256, 0.1, N) == 3             # d
        assert f(*ins, A, N, A, A, 2, 1 << 23, 128, 0.1, N) == 2        # one head too long
        assert f(*ins, A, N, N, A, 2, 16, 128, 0.1, N) == 1             # o_f32 required
        assert f(*ins, A, N, A, N, 2, 16, 128, 0.1, N) == 1             # row_ml required
        assert f(*ins, N, N, A, A, 2, 16, 128, 0.1, N) == 1             # o required
        assert f(*ins, A, N, B, A, 2, 16, 128, 0.1, N) == 4             # o_f32 needs 16 bytes
        assert f(*ins, A, N, A, C, 2, 16, 128, 0.1, N) == 4             # row_ml needs 8 bytes
        assert f(*ins, A, C, A, A, 2, 16, 128, 0.0, N) == 7             # scale
        for i in range(nin):
            args = list(ins)
            args[i] = N
            assert f(*args, A, N, A, A, 2, 16, 128, 0.1, N) == 1, i


def test_bwd_bf16_argument_errors(lib):
    f = lib.attn_bwd_bf16
    ws = ctypes.c_void_p(0x200000)
    need = lib.attn_bwd_bf16_workspace_bytes(2, 16, 128)
    ok = [A] * 9        # q, k, v, o_f32, row_ml, dout, dq, dk, dv
    assert f(*ok, ws, need, 2, 16, 64, 0.1, N) == 3                     # d
    assert f(*ok, ws, need, 2, 1 << 23, 128, 0.1, N) == 2               # one head too long
    for i in range(9):                                                   # every pointer is required
        args = list(ok)
        args[i] = N
        assert f(*args, ws, need, 2, 16, 128, 0.1, N) == 1, i
    args = list(ok)
    args[4] = ctypes.c_void_p(0x100004)                                  # row_ml needs 8-byte alignment
    assert f(*args, ws, need, 2, 16, 128, 0.1, N) == 4
    args[4] = B
    args[3] = B                                                          # o_f32 misaligned
    assert f(*args, ws, need, 2, 16, 128, 0.1, N) == 4
    args[3] = A
    args[6] = B                                                          # dq misaligned
    assert f(*args, ws, need, 2, 16, 128, 0.1, N) == 4
    assert f(*ok, ws, need, 2, 16, 128, 0.0, N) == 7                    # scale
    assert f(*ok, N, need, 2, 16, 128, 0.1, N) == 5                     # workspace
    assert f(*ok, ws, need - 1, 2, 16, 128, 0.1, N) == 5


def test_bwd_fp4qk_argument_errors(lib):
    f = lib.attn_bwd_fp4qk
    ws = ctypes.c_void_p(0x200000)
    need = lib.attn_bwd_fp4qk_workspace_bytes(2, 16, 128)
    ok = [A] * 11       # 4 code/scale tensors, v, o_f32, row_ml, dout, dq, dk, dv
    assert f(*ok, ws, need, 2, 16, 128, 0.1, 4, N) == 8                 # unknown flag bit
    assert f(*ok, ws, need, 2, 16, 256, 0.1, 3, N) == 3
    for i in range(11):
        args = list(ok)
        args[i] = N
        assert f(*args, ws, need, 2, 16, 128, 0.1, 3, N) == 1, i
    args = list(ok)
    args[6] = ctypes.c_void_p(0x100004)                                  # row_ml
    assert f(*args, ws, need, 2, 16, 128, 0.1, 3, N) == 4
    assert f(*ok, ws, need, 2, 16, 128, float("nan"), 3, N) == 7
    assert f(*ok, ws, need - 1, 2, 16, 128, 0.1, 3, N) == 5
    assert f(*ok, ctypes.c_void_p(0x200010), need, 2, 16, 128, 0.1, 3, N) == 5


def test_nvfp4_buffer_sizes(lib):
    assert lib.nvfp4_codes_bytes(109000, 5120, 0) == 109000 * 2560
    assert lib.nvfp4_scales_bytes(109000, 5120, 0) == 109000 * 320
    # tiled: 256-row tiles x 64-value stages, 8192 code and 1024 scale bytes each
    assert lib.nvfp4_codes_bytes(109000, 5120, 1) == 426 * 80 * 8192
    assert lib.nvfp4_scales_bytes(109000, 5120, 1) == 426 * 80 * 1024
    assert lib.nvfp4_codes_bytes(1, 16, 1) == 8192 and lib.nvfp4_scales_bytes(257, 80, 1) == 2 * 2 * 1024
    assert lib.nvfp4_codes_bytes(0, 16, 0) == 0 and lib.nvfp4_codes_bytes(4, 24, 1) == 0
    assert lib.nvfp4_codes_bytes(4, 32, 2) == 0 and lib.nvfp4_scales_bytes(4, 32, -1) == 0


def test_nvfp4_quantize_argument_errors(lib):
    f = lib.nvfp4_quantize
    for layout in (0, 1):
        assert f(A, A, A, 0, 32, 1.0, layout, N) == 2                   # rows
        assert f(A, A, A, 4, 8, 1.0, layout, N) == 2                    # cols < 16
        assert f(A, A, A, 4, 40, 1.0, layout, N) == 2                   # cols not a multiple of 16
        assert f(A, A, A, 1 << 40, 16, 1.0, layout, N) == 2             # too many blocks for the grid
        assert f(N, A, A, 4, 32, 1.0, layout, N) == 1
        assert f(A, A, N, 4, 32, 1.0, layout, N) == 1
        assert f(B, A, A, 4, 32, 1.0, layout, N) == 4                   # x misaligned
        assert f(A, B, A, 4, 32, 1.0, layout, N) == 4                   # codes misaligned
        assert f(A, A, B, 4, 32, 1.0, layout, N) == 4                   # scales misaligned
        assert f(A, A, A, 4, 32, 0.0, layout, N) == 7
        assert f(A, A, A, 4, 32, -2.0, layout, N) == 7
        assert f(A, A, A, 4, 32, float("inf"), layout, N) == 7
    assert f(A, A, A, 4, 32, 1.0, 2, N) == 8                            # unknown layout
    assert f(A, A, A, 4, 32, 1.0, -1, N) == 8


def test_nvfp4_linear_argument_errors(lib):
    f = lib.nvfp4_linear
    for layout in (0, 1):
        assert f(A, A, 1.0, A, A, 1.0, A, 0, 8, 64, layout, N) == 2     # M
        assert f(A, A, 1.0, A, A, 1.0, A, 8, 0, 64, layout, N) == 2     # N
        assert f(A, A, 1.0, A, A, 1.0, A, 2 ** 31 - 255, 8, 64, layout, N) == 2    # M: tile count overflows
        assert f(A, A, 1.0, A, A, 1.0, A, 8, 2 ** 31 - 1, 64, layout, N) == 2      # N: tile count overflows
        assert f(A, A, 1.0, A, A, 1.0, A, 8, 8, 8, layout, N) == 2      # K < 16
        assert f(A, A, 1.0, A, A, 1.0, A, 8, 8, 72, layout, N) == 2     # K not a multiple of 16
        assert f(A, A, 1.0, A, A, 1.0, A, 8, 8, (1 << 20) + 16, layout, N) == 2    # K too large
        for i in (0, 1, 3, 4, 6):
            args = [A, A, 1.0, A, A, 1.0, A]
            args[i] = N
            assert f(*args, 8, 8, 64, layout, N) == 1, i
        assert f(B, A, 1.0, A, A, 1.0, A, 8, 8, 64, layout, N) == 4     # x codes misaligned
        assert f(A, A, 1.0, B, A, 1.0, A, 8, 8, 64, layout, N) == 4
        assert f(A, B, 1.0, A, A, 1.0, A, 8, 8, 64, layout, N) == 4     # x scales misaligned
        assert f(A, A, 1.0, A, B, 1.0, A, 8, 8, 64, layout, N) == 4     # w scales misaligned
        assert f(A, A, 1.0, A, A, 1.0, ctypes.c_void_p(0x100004), 8, 8, 64, layout, N) == 4    # y needs 8 bytes
        assert f(A, A, 0.0, A, A, 1.0, A, 8, 8, 64, layout, N) == 7
        assert f(A, A, 1.0, A, A, float("nan"), A, 8, 8, 64, layout, N) == 7
    assert f(A, A, 1.0, A, A, 1.0, A, 8, 8, 64, 5, N) == 8              # unknown layout
