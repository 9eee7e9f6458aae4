"""long_sequence_dense_amd - dense long-sequence attention for AMD MI355X (gfx950).

The product is liblsd_attn.so (C ABI in include/lsd_attn.h, HIP kernels in
csrc/).  ``binding`` exposes the same entry points to Python through ctypes;
``inputs`` draws the seeded synthetic workloads.  Importing the package does not
load the library; the first call does, and raises if it is not built.

Build with ``python -m long_sequence_dense_amd.build``.  Typical use, with
q, k, v torch BF16 tensors [H, L, 128] on the GPU:

    o = attn_fwd_bf16(q, k, v)                       # BF16 path
    prep = qk_prep_fp4(q, k)                         # mean-K, Hadamard, NVFP4
    o4 = attn_fwd_fp4qk(prep["q_codes"], prep["q_scales"],
                        prep["k_codes"], prep["k_scales"], v)   # FP4-QK path

and, for training, attn_bwd_bf16 / attn_bwd_fp4qk (which need the forward's
LSE: pass ``lse=`` to the forward), and for the W4A4 linear layers
nvfp4_quantize / nvfp4_linear.
"""

from .binding import (  # noqa: F401
    NVFP4_ROWS,
    NVFP4_TILED,
    PREP_ROTATE,
    PREP_SMOOTH_K,
    LsdError,
    attn_bwd_bf16,
    attn_bwd_fp4qk,
    attn_fwd_bf16,
    attn_fwd_fp4qk,
    load_library,
    nvfp4_linear,
    nvfp4_quantize,
    qk_prep_fp4,
    qk_prep_fp4_ex,
    qk_prep_fp4_workspace_bytes,
    status_str,
)
