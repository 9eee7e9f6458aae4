"""Plain, slow CPU oracle for dense long-sequence attention and its FP4-QK variant.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
GPU library (``long_sequence_dense_amd``) never imports it, and it imports
nothing from the GPU library: the two share no code.

Contents
--------
``oracle.attention``  fp64 softmax attention (the plain definition).
``oracle.nvfp4``      the Q/K preparation for FP4 attention (mean key, Hadamard
                      rotation, NVFP4 block quantization), the E4M3/E2M1 codecs
                      and exact dequantization; switches for the ablation
                      variants (no smoothing, no rotation).
``oracle.fp4_error``  relative attention error of the FP4-QK variants against
                      exact attention.
``oracle.attention_bwd`` fp64 gradients of attention (dQ, dK, dV), and of the
                      FP4-QK attention with a straight-through quantizer.
``oracle.nvfp4_linear``  NVFP4 W4A4 linear layer (quantizer with a global
                      scale, exact product).

Source: "Pika H3 Flex in FastVideo: 7x Faster, and Near Real Time in 4-bit"
(haoailab blog), sections "Faster at BF16" and "FP4 attention".  Every function
names the passage it follows.  Parity pins live in ``tests/test_oracle_*.py``.
No function here is "parity unpinned"; see the pin list in each module header.
"""

from .attention import attention_fp64, attention_rows_fp64  # noqa: F401
from .nvfp4 import (  # noqa: F401
    bf16_bits_to_f64,
    e2m1_decode_table,
    e4m3_decode_table,
    kmean_exact,
    hadamard_butterfly_fp32,
    hadamard_scale_f32,
    HADAMARD_SCALE_F32,
    e4m3_scale_code,
    e2m1_codes,
    qk_prep_fp4,
    dequant_nvfp4,
)
from .fp4_error import fp4_attention_error, fp4_outputs, relative_error  # noqa: F401
from .attention_bwd import attention_bwd_fp64, attention_bwd_dq_rows_fp64  # noqa: F401
