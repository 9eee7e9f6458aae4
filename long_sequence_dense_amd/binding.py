"""ctypes binding of liblsd_attn.so: same names as the C ABI, argument
marshalling only.  Every computation runs in the library's HIP kernels; there
is no fallback of any kind: if the library is missing or fails to load, every
call raises.

Tensors are torch tensors on a ROCm device (torch provides device memory and
the current stream, nothing else).  BF16 tensors may be torch.bfloat16 or
torch.uint16/int16 holding BF16 bit patterns.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblsd_attn.so")
HEAD_DIM = 128
ABI_VERSION = 5         # LSD_ABI_VERSION of include/lsd_attn.h, which SIGNATURES mirrors

STATUS = {
    0: "LSD_OK", 1: "LSD_ERR_NULL", 2: "LSD_ERR_SHAPE", 3: "LSD_ERR_UNSUPPORTED_D",
    4: "LSD_ERR_ALIGN", 5: "LSD_ERR_WORKSPACE", 6: "LSD_ERR_LAUNCH", 7: "LSD_ERR_SCALE",
    8: "LSD_ERR_FLAGS",
}
PREP_SMOOTH_K = 1       # lsd_prep_flags
PREP_ROTATE = 2
PREP_K_ONLY = 4
NVFP4_ROWS = 0          # lsd_nvfp4_layout
NVFP4_TILED = 1

# name -> (restype, argtypes); mirrors include/lsd_attn.h
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_S = ctypes.c_size_t
SIGNATURES = {
    "lsd_abi_version": (_I, []),
    "lsd_status_str": (ctypes.c_char_p, [_I]),
    "attn_fwd_bf16": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _F, _P]),
    "attn_fwd_bf16_train": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _F, _P]),
    "qk_prep_fp4_workspace_bytes": (_S, [_I, _I, _I]),
    "qk_prep_fp4": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _S, _I, _I, _I, _P]),
    "qk_prep_fp4_ex": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _S, _I, _I, _I, _I, _P]),
    "qk_prep_fp4_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _P]),
    "attn_fwd_fp4qk": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _F, _P]),
    "attn_fwd_fp4qk_train": (_I, [_P] * 9 + [_I, _I, _I, _F, _P]),
    "attn_fwd_fp4qk_fused_q": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _F, _P]),
    "attn_bwd_bf16_workspace_bytes": (_S, [_I, _I, _I]),
    "attn_bwd_bf16": (_I, [_P] * 10 + [_S, _I, _I, _I, _F, _P]),
    "attn_bwd_fp4qk_workspace_bytes": (_S, [_I, _I, _I]),
    "attn_bwd_fp4qk": (_I, [_P] * 12 + [_S, _I, _I, _I, _F, _I, _P]),
    "nvfp4_codes_bytes": (_S, [ctypes.c_longlong, _I, _I]),
    "nvfp4_scales_bytes": (_S, [ctypes.c_longlong, _I, _I]),
    "nvfp4_quantize": (_I, [_P, _P, _P, ctypes.c_longlong, _I, _F, _I, _P]),
    "nvfp4_linear": (_I, [_P, _P, _F, _P, _P, _F, _P, _I, _I, _I, _I, _P]),
}

_lib = None


class LsdError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__("%s failed: %s (%s)" % (fn, STATUS.get(status, status), msg))
        self.status = status


def load_library(path=None):
    """Load (once) and return the ctypes handle; raises if it is not built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError("liblsd_attn.so is not built (%s); run "
                           "`python -m long_sequence_dense_amd.build`" % p)
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    if lib.lsd_abi_version() != ABI_VERSION:
        raise RuntimeError("%s has ABI version %d, this binding expects %d; rebuild it with "
                           "`python -m long_sequence_dense_amd.build`" % (p, lib.lsd_abi_version(), ABI_VERSION))
    if path is None:
        _lib = lib
    return lib


def status_str(status):
    return load_library().lsd_status_str(int(status)).decode()


def _check(fn, st):
    if st != 0:
        raise LsdError(fn, st, status_str(st))


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(t, name, dtypes, shape):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on the GPU, got %s" % (name, t.device))
    if t.dtype not in dtypes:
        raise TypeError("%s: dtype %s not in %s" % (name, t.dtype, dtypes))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s: shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _bf16_types():
    import torch
    return (torch.bfloat16, torch.uint16, torch.int16)


def attn_fwd_bf16(q, k, v, o=None, lse=None, softmax_scale=None, stream=None):
    """O = softmax(scale * Q K^T) V per head; q, k, v [H, L, 128] BF16."""
    import torch
    H, L, d = q.shape
    for n, t in (("q", q), ("k", k), ("v", v)):
        _need(t, n, _bf16_types(), (H, L, d))
    if o is None:
        o = torch.empty((H, L, d), dtype=torch.bfloat16, device=q.device)
    _need(o, "o", _bf16_types(), (H, L, d))
    if lse is not None:
        _need(lse, "lse", (torch.float32,), (H, L))
    scale = float(d) ** -0.5 if softmax_scale is None else float(softmax_scale)
    st = load_library().attn_fwd_bf16(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                      H, L, d, scale, _stream(stream))
    _check("attn_fwd_bf16", st)
    return o


def _train_outputs(H, L, d, device, o32, ml):
    import torch
    if o32 is None:
        o32 = torch.empty((H, L, d), dtype=torch.float32, device=device)
    if ml is None:
        ml = torch.empty((H, L, 2), dtype=torch.float32, device=device)
    _need(o32, "o32", (torch.float32,), (H, L, d))
    _need(ml, "ml", (torch.float32,), (H, L, 2))
    return o32, ml


def attn_fwd_bf16_train(q, k, v, o=None, lse=None, o32=None, ml=None, softmax_scale=None, stream=None):
    """attn_fwd_bf16 that also returns the backward's inputs: (o, o32, ml)
    with o32 [H, L, 128] float32 and ml [H, L, 2] float32 (row max m, row sum
    l)."""
    import torch
    H, L, d = q.shape
    for n, t in (("q", q), ("k", k), ("v", v)):
        _need(t, n, _bf16_types(), (H, L, d))
    if o is None:
        o = torch.empty((H, L, d), dtype=torch.bfloat16, device=q.device)
    _need(o, "o", _bf16_types(), (H, L, d))
    if lse is not None:
        _need(lse, "lse", (torch.float32,), (H, L))
    o32, ml = _train_outputs(H, L, d, q.device, o32, ml)
    scale = float(d) ** -0.5 if softmax_scale is None else float(softmax_scale)
    st = load_library().attn_fwd_bf16_train(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(o32), _ptr(ml),
                                            H, L, d, scale, _stream(stream))
    _check("attn_fwd_bf16_train", st)
    return o, o32, ml


def qk_prep_fp4_workspace_bytes(H, L, d=HEAD_DIM):
    return int(load_library().qk_prep_fp4_workspace_bytes(H, L, d))


def _prep_outputs(q, k, out, with_q=True):
    import torch
    H, L, d = k.shape
    if with_q:
        _need(q, "q", _bf16_types(), (H, L, d))
    _need(k, "k", _bf16_types(), (H, L, d))
    dev = k.device
    sides = ("q", "k") if with_q else ("k",)
    if out is None:
        out = {"k_mean": torch.empty((H, d), dtype=torch.float32, device=dev)}
        for x in sides:
            out[x + "_codes"] = torch.empty((H, L, d // 2), dtype=torch.uint8, device=dev)
            out[x + "_scales"] = torch.empty((H, L, d // 16), dtype=torch.uint8, device=dev)
    for x in sides:
        _need(out[x + "_codes"], x + "_codes", (torch.uint8,), (H, L, d // 2))
        _need(out[x + "_scales"], x + "_scales", (torch.uint8,), (H, L, d // 16))
    _need(out["k_mean"], "k_mean", (torch.float32,), (H, d))
    return out


def qk_prep_fp4(q, k, out=None, workspace=None, stream=None):
    """Mean-K, Hadamard and NVFP4 quantization of Q and K ([H, L, 128] BF16).
    Returns dict(q_codes, q_scales, k_codes, k_scales, k_mean)."""
    import torch
    H, L, d = q.shape
    out = _prep_outputs(q, k, out)
    need = qk_prep_fp4_workspace_bytes(H, L, d)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = load_library().qk_prep_fp4(
        _ptr(q), _ptr(k), _ptr(out["q_codes"]), _ptr(out["q_scales"]), _ptr(out["k_codes"]),
        _ptr(out["k_scales"]), _ptr(out["k_mean"]), _ptr(workspace),
        workspace.numel() * workspace.element_size(), H, L, d, _stream(stream))
    _check("qk_prep_fp4", st)
    return out


def qk_prep_fp4_ex(q, k, flags, out=None, workspace=None, stream=None):
    """qk_prep_fp4 with the transforms switched by ``flags`` (PREP_SMOOTH_K |
    PREP_ROTATE = the full method).  Without smoothing no workspace is used and
    k_mean is written with zeros.  With PREP_K_ONLY only K is prepared (``q``
    may be None; the result has no q_codes / q_scales)."""
    import torch
    H, L, d = k.shape
    with_q = not flags & PREP_K_ONLY
    out = _prep_outputs(q, k, out, with_q)
    if workspace is None:
        need = qk_prep_fp4_workspace_bytes(H, L, d) if flags & PREP_SMOOTH_K else 0
        workspace = torch.empty(need, dtype=torch.uint8, device=k.device) if need else None
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load_library().qk_prep_fp4_ex(
        _ptr(q if with_q else None), _ptr(k), _ptr(out.get("q_codes")), _ptr(out.get("q_scales")),
        _ptr(out["k_codes"]),
        _ptr(out["k_scales"]), _ptr(out["k_mean"]), _ptr(workspace), nbytes, H, L, d, int(flags),
        _stream(stream))
    _check("qk_prep_fp4_ex", st)
    return out


def qk_prep_fp4_noalloc(q, k, out, stream=None):
    """qk_prep_fp4 with the library's static scratch instead of a workspace;
    ``out`` (the dict of qk_prep_fp4's outputs) must be given: nothing is
    allocated."""
    H, L, d = q.shape
    if out is None:
        raise ValueError("qk_prep_fp4_noalloc allocates nothing: pass the output tensors")
    out = _prep_outputs(q, k, out)
    st = load_library().qk_prep_fp4_noalloc(
        _ptr(q), _ptr(k), _ptr(out["q_codes"]), _ptr(out["q_scales"]), _ptr(out["k_codes"]),
        _ptr(out["k_scales"]), _ptr(out["k_mean"]), H, L, d, _stream(stream))
    _check("qk_prep_fp4_noalloc", st)
    return out


def attn_fwd_fp4qk(q_codes, q_scales, k_codes, k_scales, v, o=None, lse=None,
                   softmax_scale=None, stream=None):
    """Attention with scores from NVFP4 Q/K (as written by qk_prep_fp4)."""
    import torch
    H, L, d = v.shape
    _need(v, "v", _bf16_types(), (H, L, d))
    for n, t in (("q_codes", q_codes), ("k_codes", k_codes)):
        _need(t, n, (torch.uint8,), (H, L, d // 2))
    for n, t in (("q_scales", q_scales), ("k_scales", k_scales)):
        _need(t, n, (torch.uint8,), (H, L, d // 16))
    if o is None:
        o = torch.empty((H, L, d), dtype=torch.bfloat16, device=v.device)
    _need(o, "o", _bf16_types(), (H, L, d))
    if lse is not None:
        _need(lse, "lse", (torch.float32,), (H, L))
    scale = float(d) ** -0.5 if softmax_scale is None else float(softmax_scale)
    st = load_library().attn_fwd_fp4qk(_ptr(q_codes), _ptr(q_scales), _ptr(k_codes), _ptr(k_scales),
                                       _ptr(v), _ptr(o), _ptr(lse), H, L, d, scale, _stream(stream))
    _check("attn_fwd_fp4qk", st)
    return o


def attn_fwd_fp4qk_train(q_codes, q_scales, k_codes, k_scales, v, o=None, lse=None, o32=None, ml=None,
                         softmax_scale=None, stream=None):
    """attn_fwd_fp4qk that also returns the backward's inputs: (o, o32, ml)."""
    import torch
    H, L, d = v.shape
    _need(v, "v", _bf16_types(), (H, L, d))
    for n, t in (("q_codes", q_codes), ("k_codes", k_codes)):
        _need(t, n, (torch.uint8,), (H, L, d // 2))
    for n, t in (("q_scales", q_scales), ("k_scales", k_scales)):
        _need(t, n, (torch.uint8,), (H, L, d // 16))
    if o is None:
        o = torch.empty((H, L, d), dtype=torch.bfloat16, device=v.device)
    _need(o, "o", _bf16_types(), (H, L, d))
    if lse is not None:
        _need(lse, "lse", (torch.float32,), (H, L))
    o32, ml = _train_outputs(H, L, d, v.device, o32, ml)
    scale = float(d) ** -0.5 if softmax_scale is None else float(softmax_scale)
    st = load_library().attn_fwd_fp4qk_train(_ptr(q_codes), _ptr(q_scales), _ptr(k_codes), _ptr(k_scales),
                                             _ptr(v), _ptr(o), _ptr(lse), _ptr(o32), _ptr(ml), H, L, d, scale,
                                             _stream(stream))
    _check("attn_fwd_fp4qk_train", st)
    return o, o32, ml


def attn_fwd_fp4qk_fused_q(q, k_codes, k_scales, v, o=None, lse=None, softmax_scale=None, stream=None):
    """attn_fwd_fp4qk with Q ([H, L, 128] BF16) rotated and quantized inside
    the attention kernel; K as prepared by qk_prep_fp4_ex(..., PREP_K_ONLY |
    PREP_SMOOTH_K | PREP_ROTATE)."""
    import torch
    H, L, d = v.shape
    for n, t in (("q", q), ("v", v)):
        _need(t, n, _bf16_types(), (H, L, d))
    _need(k_codes, "k_codes", (torch.uint8,), (H, L, d // 2))
    _need(k_scales, "k_scales", (torch.uint8,), (H, L, d // 16))
    if o is None:
        o = torch.empty((H, L, d), dtype=torch.bfloat16, device=v.device)
    _need(o, "o", _bf16_types(), (H, L, d))
    if lse is not None:
        _need(lse, "lse", (torch.float32,), (H, L))
    scale = float(d) ** -0.5 if softmax_scale is None else float(softmax_scale)
    st = load_library().attn_fwd_fp4qk_fused_q(_ptr(q), _ptr(k_codes), _ptr(k_scales), _ptr(v), _ptr(o), _ptr(lse),
                                               H, L, d, scale, _stream(stream))
    _check("attn_fwd_fp4qk_fused_q", st)
    return o


def attn_bwd_bf16_workspace_bytes(H, L, d=HEAD_DIM):
    return int(load_library().attn_bwd_bf16_workspace_bytes(H, L, d))


def attn_bwd_bf16(q, k, v, o32, ml, dout, dq=None, dk=None, dv=None, softmax_scale=None,
                  workspace=None, stream=None):
    """Gradients (dq, dk, dv) of attn_fwd_bf16; o32 and ml as returned by
    attn_fwd_bf16_train."""
    import torch
    H, L, d = q.shape
    for n, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _need(t, n, _bf16_types(), (H, L, d))
    _need(o32, "o32", (torch.float32,), (H, L, d))
    _need(ml, "ml", (torch.float32,), (H, L, 2))
    outs = []
    for n, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is None:
            t = torch.empty((H, L, d), dtype=torch.bfloat16, device=q.device)
        _need(t, n, _bf16_types(), (H, L, d))
        outs.append(t)
    if workspace is None:
        workspace = torch.empty(attn_bwd_bf16_workspace_bytes(H, L, d), dtype=torch.uint8, device=q.device)
    scale = float(d) ** -0.5 if softmax_scale is None else float(softmax_scale)
    st = load_library().attn_bwd_bf16(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o32), _ptr(ml), _ptr(dout), _ptr(outs[0]), _ptr(outs[1]), _ptr(outs[2]),
        _ptr(workspace), workspace.numel() * workspace.element_size(), H, L, d, scale, _stream(stream))
    _check("attn_bwd_bf16", st)
    return tuple(outs)


def attn_bwd_fp4qk_workspace_bytes(H, L, d=HEAD_DIM):
    return int(load_library().attn_bwd_fp4qk_workspace_bytes(H, L, d))


def attn_bwd_fp4qk(q_codes, q_scales, k_codes, k_scales, v, o32, ml, dout, dq=None, dk=None, dv=None,
                   softmax_scale=None, flags=PREP_SMOOTH_K | PREP_ROTATE, workspace=None, stream=None):
    """Straight-through gradients (dq, dk, dv) of attn_fwd_fp4qk with respect
    to the original Q, K and V; o32 and ml as returned by
    attn_fwd_fp4qk_train."""
    import torch
    H, L, d = v.shape
    for n, t in (("v", v), ("dout", dout)):
        _need(t, n, _bf16_types(), (H, L, d))
    for n, t in (("q_codes", q_codes), ("k_codes", k_codes)):
        _need(t, n, (torch.uint8,), (H, L, d // 2))
    for n, t in (("q_scales", q_scales), ("k_scales", k_scales)):
        _need(t, n, (torch.uint8,), (H, L, d // 16))
    _need(o32, "o32", (torch.float32,), (H, L, d))
    _need(ml, "ml", (torch.float32,), (H, L, 2))
    outs = []
    for n, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is None:
            t = torch.empty((H, L, d), dtype=torch.bfloat16, device=v.device)
        _need(t, n, _bf16_types(), (H, L, d))
        outs.append(t)
    if workspace is None:
        workspace = torch.empty(attn_bwd_fp4qk_workspace_bytes(H, L, d), dtype=torch.uint8, device=v.device)
    scale = float(d) ** -0.5 if softmax_scale is None else float(softmax_scale)
    st = load_library().attn_bwd_fp4qk(
        _ptr(q_codes), _ptr(q_scales), _ptr(k_codes), _ptr(k_scales), _ptr(v), _ptr(o32), _ptr(ml), _ptr(dout),
        _ptr(outs[0]), _ptr(outs[1]), _ptr(outs[2]), _ptr(workspace), workspace.numel() * workspace.element_size(),
        H, L, d, scale, int(flags), _stream(stream))
    _check("attn_bwd_fp4qk", st)
    return tuple(outs)


def nvfp4_codes_bytes(rows, cols, layout=NVFP4_ROWS):
    return int(load_library().nvfp4_codes_bytes(int(rows), int(cols), int(layout)))


def nvfp4_scales_bytes(rows, cols, layout=NVFP4_ROWS):
    return int(load_library().nvfp4_scales_bytes(int(rows), int(cols), int(layout)))


def _nvfp4_shapes(rows, cols, layout):
    if layout == NVFP4_ROWS:
        return (rows, cols // 2), (rows, cols // 16)
    return (nvfp4_codes_bytes(rows, cols, layout),), (nvfp4_scales_bytes(rows, cols, layout),)


def nvfp4_quantize(x, global_scale=1.0, codes=None, scales=None, layout=NVFP4_ROWS, stream=None):
    """NVFP4 codes and E4M3 block scales of a [rows, cols] BF16 matrix
    quantized with per-tensor global scale g: row-major ([rows, cols/2],
    [rows, cols/16]) or, with layout=NVFP4_TILED, 1-D buffers in the product's
    tiled load order."""
    import torch
    if x.dim() != 2:
        raise ValueError("x must be [rows, cols]")
    rows, cols = x.shape
    _need(x, "x", _bf16_types(), (rows, cols))
    cshape, sshape = _nvfp4_shapes(rows, cols, layout)
    if codes is None:
        codes = torch.empty(cshape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(sshape, dtype=torch.uint8, device=x.device)
    _need(codes, "codes", (torch.uint8,), cshape)
    _need(scales, "scales", (torch.uint8,), sshape)
    st = load_library().nvfp4_quantize(_ptr(x), _ptr(codes), _ptr(scales), rows, cols, float(global_scale),
                                       int(layout), _stream(stream))
    _check("nvfp4_quantize", st)
    return codes, scales


def nvfp4_linear(x_codes, x_scales, x_global_scale, w_codes, w_scales, w_global_scale, y=None, stream=None,
                 layout=NVFP4_ROWS, M=None, N=None, K=None):
    """Y [M, N] BF16 = (X^ g_x)(W^ g_w)^T from NVFP4 operands X [M, K] and
    W [N, K].  Row-major operands carry M, N, K in their shapes; tiled ones
    need them passed."""
    import torch
    if layout == NVFP4_ROWS:
        M, K = x_codes.shape[0], 2 * x_codes.shape[1]
        N = w_codes.shape[0]
    elif M is None or N is None or K is None:
        raise ValueError("tiled operands need M, N and K")
    xcs, xss = _nvfp4_shapes(M, K, layout)
    wcs, wss = _nvfp4_shapes(N, K, layout)
    _need(x_codes, "x_codes", (torch.uint8,), xcs)
    _need(x_scales, "x_scales", (torch.uint8,), xss)
    _need(w_codes, "w_codes", (torch.uint8,), wcs)
    _need(w_scales, "w_scales", (torch.uint8,), wss)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x_codes.device)
    _need(y, "y", _bf16_types(), (M, N))
    st = load_library().nvfp4_linear(_ptr(x_codes), _ptr(x_scales), float(x_global_scale), _ptr(w_codes),
                                     _ptr(w_scales), float(w_global_scale), _ptr(y), M, N, K, int(layout),
                                     _stream(stream))
    _check("nvfp4_linear", st)
    return y
