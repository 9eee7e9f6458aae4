"""long_sequence_dense_amd - dense long-sequence attention for AMD MI355X (gfx950).

The product is liblsd_attn.so (C ABI in include/lsd_attn.h, HIP kernels in
csrc/).  ``binding`` exposes the same entry points to Python through ctypes;
``inputs`` draws the seeded synthetic workloads.  Importing the package does not
load the library; the first call does, and raises if it is not built.
"""

from .binding import (  # noqa: F401
    LsdError,
    attn_fwd_bf16,
    attn_fwd_fp4qk,
    load_library,
    qk_prep_fp4,
    qk_prep_fp4_workspace_bytes,
    status_str,
)
