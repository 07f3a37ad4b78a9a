"""ctypes binding of libflash_attn.so (include/flash_attn.h).

Argument marshalling only: shape, dtype, device and contiguity checks,
allocation of the outputs with torch, and the current torch stream.  Every
step of the attention computation runs in the library's HIP kernels; there is
no fallback.  If the library has not been built, the first call raises.
"""

import ctypes
import math
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libflash_attn.so"

FA_OK = 0
FA_ERR_INVALID_ARG = 1
FA_ERR_UNSUPPORTED = 2
FA_ERR_HIP = 3
FA_DTYPE_BF16 = 0
FA_DTYPE_FP32 = 1
FA_BWD_PREPROCESS = 1
FA_BWD_MAIN = 2
FA_BWD_FINALIZE = 4
FA_BWD_ALL = 7
FA_SPARSE_BLOCK = 128
FA_SPARSE_MAX_N = 65536
FA_DECODE_MAX_Q = 16
FA_BWD_NOALLOC_MAX_BYTES = 64 << 20

_lib = None


class FlashAttnError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {flash_attn_status_string(status)} (status {status})"
                         + (f" [{_raw().flash_attn_last_hip_error().decode()}]"
                            if status == FA_ERR_HIP else ""))


def library_path():
    return os.path.join(PKG_DIR, LIB_NAME)


def _raw():
    """The loaded CDLL with argument and result types declared."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m io_aware_tiled_attn_amd.build` "
            "(there is no non-HIP implementation)")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.flash_attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
    lib.flash_attn_fwd.restype = i
    lib.flash_attn_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp, i]
    lib.flash_attn_fwd_ex.restype = i
    lib.flash_attn_bwd_workspace_size.argtypes = [i, i, i, i]
    lib.flash_attn_bwd_workspace_size.restype = sz
    lib.flash_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, i, vp]
    lib.flash_attn_bwd.restype = i
    lib.flash_attn_bwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, i, vp, i]
    lib.flash_attn_bwd_ex.restype = i
    lib.flash_attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
    lib.flash_attn_bwd_noalloc.restype = i
    lib.flash_attn_fwd_blocksparse.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
    lib.flash_attn_fwd_blocksparse.restype = i
    lib.flash_attn_bwd_blocksparse.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, i, vp]
    lib.flash_attn_bwd_blocksparse.restype = i
    lib.flash_attn_decode_workspace_size.argtypes = [i, i, i, i]
    lib.flash_attn_decode_workspace_size.restype = sz
    lib.flash_attn_decode.argtypes = [vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, f, i, i, vp]
    lib.flash_attn_decode.restype = i
    lib.flash_attn_fwd_fp8.argtypes = [vp, vp, vp, f, f, f, vp, vp, i, i, i, i, f, i, vp]
    lib.flash_attn_fwd_fp8.restype = i
    lib.flash_attn_merge.argtypes = [vp, vp, vp, vp, vp, ctypes.c_longlong, i, vp]
    lib.flash_attn_merge.restype = i
    lib.flash_attn_device_info.argtypes = [i, ctypes.POINTER(i), ctypes.POINTER(i)]
    lib.flash_attn_device_info.restype = i
    lib.flash_attn_status_string.argtypes = [i]
    lib.flash_attn_status_string.restype = ctypes.c_char_p
    lib.flash_attn_last_hip_error.argtypes = []
    lib.flash_attn_last_hip_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def flash_attn_status_string(status):
    return _raw().flash_attn_status_string(int(status)).decode()


def flash_attn_bwd_workspace_size(B, H, N, d):
    return int(_raw().flash_attn_bwd_workspace_size(int(B), int(H), int(N), int(d)))


def _torch():
    import torch
    return torch


def _check(t, name, dtype, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return FA_DTYPE_BF16
    if t.dtype == torch.float32:
        return FA_DTYPE_FP32
    raise ValueError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _stream_ptr(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def flash_attn_fwd_ex(q, k, v, causal=False, scale=None, block_n=0, out=None, lse=None, stream=None):
    """Forward pass on [B, H, N, d] tensors; returns (O, LSE).

    q, k, v: contiguous GPU tensors, bfloat16 or float32, same shape.
    scale defaults to 1/sqrt(d).  LSE is float32 [B, H, N].
    block_n forces the key-tile width (0 = default).
    """
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    code = _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, name, q.dtype, q.shape)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", q.dtype, q.shape)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        _check(lse, "lse", torch.float32, (B, H, N))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = _raw().flash_attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                  B, H, N, d, float(scale), int(bool(causal)), code, _stream_ptr(stream),
                                  int(block_n))
    if st != FA_OK:
        raise FlashAttnError(st, "flash_attn_fwd")
    return out, lse


def flash_attn_fwd(q, k, v, causal=False, scale=None, out=None, lse=None, stream=None):
    """Forward pass; see flash_attn_fwd_ex."""
    return flash_attn_fwd_ex(q, k, v, causal=causal, scale=scale, block_n=0, out=out, lse=lse, stream=stream)


def flash_attn_fwd_fp8(q, k, v, q_descale, k_descale, v_descale, causal=False, scale=None, out=None, lse=None,
                       stream=None):
    """FP8 forward on [B, H, N, d] E4M3 codes; returns (O bf16, LSE fp32).

    q, k, v: contiguous GPU tensors of dtype uint8 (the codes) or
    float8_e4m3fn, same shape; the *_descale floats give each tensor's
    values as code value * descale.  scale defaults to 1/sqrt(d).
    """
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    if q.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise ValueError(f"q has dtype {q.dtype}, expected uint8 or float8_e4m3fn")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, name, q.dtype, q.shape)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q.device)
    else:
        _check(out, "out", torch.bfloat16, (B, H, N, d))
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        _check(lse, "lse", torch.float32, (B, H, N))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = _raw().flash_attn_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), float(q_descale), float(k_descale),
                                   float(v_descale), out.data_ptr(), lse.data_ptr(), B, H, N, d, float(scale),
                                   int(bool(causal)), _stream_ptr(stream))
    if st != FA_OK:
        raise FlashAttnError(st, "flash_attn_fwd_fp8")
    return out, lse


def flash_attn_device_info(device=0):
    """(compute units, peak clock in MHz) of a HIP device."""
    cus, khz = ctypes.c_int(0), ctypes.c_int(0)
    st = _raw().flash_attn_device_info(int(device), ctypes.byref(cus), ctypes.byref(khz))
    if st != FA_OK:
        raise FlashAttnError(st, "flash_attn_device_info")
    return cus.value, khz.value / 1000.0


def flash_attn_merge(o_acc, lse_acc, o_part, lse_part, out=None, stream=None):
    """Fold a partial result (o_part bf16 [..., N, d], lse_part fp32 [..., N])
    over another set of keys into the running result (o_acc fp32, lse_acc
    fp32, same shapes), in place; out (bf16, optional) receives the merged O.
    Returns out (or None)."""
    torch = _torch()
    shape = tuple(o_part.shape)
    d = shape[-1]
    rows = o_part.numel() // d
    _check(o_acc, "o_acc", torch.float32, shape)
    _check(lse_acc, "lse_acc", torch.float32, shape[:-1])
    _check(o_part, "o_part", torch.bfloat16, shape)
    _check(lse_part, "lse_part", torch.float32, shape[:-1])
    if out is not None:
        _check(out, "out", torch.bfloat16, shape)
    st = _raw().flash_attn_merge(o_acc.data_ptr(), lse_acc.data_ptr(), o_part.data_ptr(), lse_part.data_ptr(),
                                 None if out is None else out.data_ptr(), rows, d, _stream_ptr(stream))
    if st != FA_OK:
        raise FlashAttnError(st, "flash_attn_merge")
    return out


def flash_attn_bwd_ex(q, k, v, o, lse, do, causal=False, scale=None, workspace=None, stream=None,
                      dq=None, dk=None, dv=None, phases=FA_BWD_ALL):
    """Backward pass (bfloat16); returns (dQ, dK, dV).

    o and lse come from flash_attn_fwd with the same causal flag and scale.
    workspace, if given, is a uint8 GPU tensor of at least
    flash_attn_bwd_workspace_size(B, H, N, d) bytes; otherwise one is
    allocated with torch for this call.  `phases` selects which of the three
    backward kernels run (FA_BWD_* bits); callers running them one at a time
    pass the same workspace and output tensors to each call.
    """
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    code = _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check(t, name, q.dtype, q.shape)
    _check(lse, "lse", torch.float32, (B, H, N))
    need = flash_attn_bwd_workspace_size(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    else:
        _check(workspace, "workspace", torch.uint8)
    outs = []
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is None:
            t = torch.empty_like(q)
        else:
            _check(t, name, q.dtype, q.shape)
        outs.append(t)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = _raw().flash_attn_bwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                  lse.data_ptr(), outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(),
                                  workspace.data_ptr(), workspace.numel(), B, H, N, d, float(scale),
                                  int(bool(causal)), code, _stream_ptr(stream), int(phases))
    if st != FA_OK:
        raise FlashAttnError(st, "flash_attn_bwd")
    return tuple(outs)


def flash_attn_bwd(q, k, v, o, lse, do, causal=False, scale=None, workspace=None, stream=None,
                   dq=None, dk=None, dv=None):
    """Backward pass (all three kernels); see flash_attn_bwd_ex."""
    return flash_attn_bwd_ex(q, k, v, o, lse, do, causal=causal, scale=scale, workspace=workspace,
                             stream=stream, dq=dq, dk=dk, dv=dv, phases=FA_BWD_ALL)


def _check_block_mask(block_mask, B, H, N, device):
    torch = _torch()
    nb = (N + FA_SPARSE_BLOCK - 1) // FA_SPARSE_BLOCK
    _check(block_mask, "block_mask", torch.uint8, (B, H, nb, nb))
    if block_mask.device != device:
        raise ValueError("block_mask must be on the same device as q")


def flash_attn_fwd_blocksparse(q, k, v, block_mask, causal=False, scale=None, out=None, lse=None, stream=None):
    """Block-sparse forward (bfloat16); returns (O, LSE).

    block_mask: uint8 GPU tensor [B, H, nb, nb], nb = ceil(N / 128); entry
    [b, h, i, j] != 0 keeps (query block i, key block j).  Rows left with no
    key get O = 0 and LSE = -inf.
    """
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    code = _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, name, q.dtype, q.shape)
    _check_block_mask(block_mask, B, H, N, q.device)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", q.dtype, q.shape)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        _check(lse, "lse", torch.float32, (B, H, N))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = _raw().flash_attn_fwd_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                           lse.data_ptr(), block_mask.data_ptr(), B, H, N, d, float(scale),
                                           int(bool(causal)), code, _stream_ptr(stream))
    if st != FA_OK:
        raise FlashAttnError(st, "flash_attn_fwd_blocksparse")
    return out, lse


def flash_attn_bwd_blocksparse(q, k, v, o, lse, do, block_mask, causal=False, scale=None, workspace=None,
                               stream=None, dq=None, dk=None, dv=None):
    """Block-sparse backward (bfloat16); returns (dQ, dK, dV).  o, lse and
    block_mask as given to / returned by flash_attn_fwd_blocksparse."""
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    code = _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check(t, name, q.dtype, q.shape)
    _check(lse, "lse", torch.float32, (B, H, N))
    _check_block_mask(block_mask, B, H, N, q.device)
    need = flash_attn_bwd_workspace_size(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    else:
        _check(workspace, "workspace", torch.uint8)
    outs = []
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is None:
            t = torch.empty_like(q)
        else:
            _check(t, name, q.dtype, q.shape)
        outs.append(t)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = _raw().flash_attn_bwd_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                           lse.data_ptr(), block_mask.data_ptr(), outs[0].data_ptr(),
                                           outs[1].data_ptr(), outs[2].data_ptr(), workspace.data_ptr(),
                                           workspace.numel(), B, H, N, d, float(scale), int(bool(causal)), code,
                                           _stream_ptr(stream))
    if st != FA_OK:
        raise FlashAttnError(st, "flash_attn_bwd_blocksparse")
    return tuple(outs)


def flash_attn_decode_workspace_size(B, H, Nk, d):
    return int(_raw().flash_attn_decode_workspace_size(int(B), int(H), int(Nk), int(d)))


def flash_attn_decode(q, k, v, causal=False, scale=None, out=None, lse=None, workspace=None, stream=None):
    """Decoding against a key/value cache (bfloat16); returns (O, LSE).

    q: [B, H, Nq, d] with 1 <= Nq <= 16; k, v: [B, H, Nk, d], Nk >= Nq.
    The queries are the cache's last Nq positions (causal: query i sees keys
    j <= Nk - Nq + i).  workspace, if given, is a uint8 GPU tensor of at
    least flash_attn_decode_workspace_size(B, H, Nk, d) bytes.
    """
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [B, H, N, d]")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    code = _dtype_code(q)
    _check(q, "q", q.dtype)
    _check(k, "k", q.dtype, (B, H, Nk, d))
    _check(v, "v", q.dtype, (B, H, Nk, d))
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", q.dtype, q.shape)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    else:
        _check(lse, "lse", torch.float32, (B, H, Nq))
    need = flash_attn_decode_workspace_size(B, H, Nk, d)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    else:
        _check(workspace, "workspace", torch.uint8)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = _raw().flash_attn_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                  workspace.data_ptr(), workspace.numel(), B, H, Nq, Nk, d, float(scale),
                                  int(bool(causal)), code, _stream_ptr(stream))
    if st != FA_OK:
        raise FlashAttnError(st, "flash_attn_decode")
    return out, lse


def flash_attn_bwd_noalloc(q, k, v, o, lse, do, causal=False, scale=None, dq=None, dk=None, dv=None,
                           stream=None):
    """Backward pass whose workspace is the library's static device scratch
    (FA_BWD_NOALLOC_MAX_BYTES per GPU): the library allocates nothing.
    Pass dq, dk, dv to keep this wrapper from allocating the outputs with
    torch.  Calls that overlap on one GPU share the scratch and race; calls
    on one stream are ordered.  Returns (dQ, dK, dV)."""
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    code = _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check(t, name, q.dtype, q.shape)
    _check(lse, "lse", torch.float32, (B, H, N))
    outs = []
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is None:
            t = torch.empty_like(q)
        else:
            _check(t, name, q.dtype, q.shape)
        outs.append(t)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = _raw().flash_attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                       lse.data_ptr(), outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(),
                                       B, H, N, d, float(scale), int(bool(causal)), code, _stream_ptr(stream))
    if st != FA_OK:
        raise FlashAttnError(st, "flash_attn_bwd_noalloc")
    return tuple(outs)
