"""Exact tiled attention (FlashAttention) for AMD Instinct MI355X (gfx950).

The compute lives in hand-written HIP kernels behind a C-ABI shared library,
libflash_attn.so, built from csrc/.  The Python names below are thin ctypes
wrappers over that library's entry points; they marshal torch tensors and
streams and nothing else.  Importing the package does not load the library;
the first call does, and it raises if the library has not been built.
"""

__all__ = [
    "flash_attn_fwd",
    "flash_attn_fwd_ex",
    "flash_attn_fwd_fp8",
    "flash_attn_bwd",
    "flash_attn_bwd_ex",
    "flash_attn_bwd_noalloc",
    "flash_attn_fwd_blocksparse",
    "flash_attn_bwd_blocksparse",
    "flash_attn_decode",
    "flash_attn_merge",
    "flash_attn_decode_workspace_size",
    "flash_attn_bwd_workspace_size",
    "flash_attn_status_string",
    "flash_attn_device_info",
    "FlashAttnError",
    "library_path",
]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
