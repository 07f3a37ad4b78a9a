"""The C-ABI library on the CPU: it loads, exports every function the header
declares, and rejects bad arguments before touching the GPU (no call here
reaches a kernel launch)."""

import ctypes
import os
import re
import subprocess

import pytest

from io_aware_tiled_attn_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flash_attn.h")

lib_missing = not os.path.exists(binding.library_path())
pytestmark = pytest.mark.skipif(lib_missing, reason="libflash_attn.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(flash_attn_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert names == sorted(["flash_attn_fwd", "flash_attn_fwd_ex", "flash_attn_bwd", "flash_attn_bwd_ex",
                            "flash_attn_bwd_workspace_size", "flash_attn_status_string",
                            "flash_attn_last_hip_error", "flash_attn_fwd_blocksparse",
                            "flash_attn_bwd_blocksparse", "flash_attn_decode",
                            "flash_attn_decode_workspace_size", "flash_attn_fwd_fp8",
                            "flash_attn_merge", "flash_attn_device_info", "flash_attn_bwd_noalloc"])


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", binding.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(binding._raw(), name)


def test_status_strings_never_null():
    for code in (-5, 0, 1, 2, 3, 4, 1000):
        s = binding.flash_attn_status_string(code)
        assert isinstance(s, str) and s
    assert binding.flash_attn_status_string(0) == "ok"


def test_workspace_size_is_linear_in_n():
    f = binding.flash_attn_bwd_workspace_size
    # per row: D and the two row terms (fp32), the fp16 copies of Q, dO, K,
    # V; per 256-row chunk four maxima; per head four factors
    rows = 4 * 32 * 4096
    assert f(4, 32, 4096, 128) >= rows * (12 + 8 * 128)
    assert f(4, 32, 4096, 128) < rows * (12 + 8 * 128) * 1.01
    assert f(4, 32, 4096, 128) % 256 == 0
    assert f(1, 1, 2048, 64) * 2 - f(1, 1, 4096, 64) < 1024
    assert f(0, 1, 1, 64) == 0 and f(1, 1, -1, 64) == 0


FAKE = ctypes.c_void_p(0x1000)       # aligned, never dereferenced: validation fails first
MISALIGNED = ctypes.c_void_p(0x1004)


def fwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, N=16, d=64, scale=0.125,
             causal=0, dtype=binding.FA_DTYPE_BF16, stream=None, block_n=0)
    a.update(kw)
    return binding._raw().flash_attn_fwd_ex(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"],
                                            a["d"], a["scale"], a["causal"], a["dtype"], a["stream"],
                                            a["block_n"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), binding.FA_ERR_INVALID_ARG),
    (dict(o=None), binding.FA_ERR_INVALID_ARG),
    (dict(B=0), binding.FA_ERR_INVALID_ARG),
    (dict(H=-1), binding.FA_ERR_INVALID_ARG),
    (dict(N=0), binding.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), binding.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), binding.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), binding.FA_ERR_INVALID_ARG),
    (dict(scale=-1.0), binding.FA_ERR_INVALID_ARG),
    (dict(causal=2), binding.FA_ERR_INVALID_ARG),
    (dict(k=MISALIGNED), binding.FA_ERR_INVALID_ARG),
    (dict(B=4096, H=4096, N=4096), binding.FA_ERR_INVALID_ARG),
    (dict(d=96), binding.FA_ERR_UNSUPPORTED),
    (dict(d=256), binding.FA_ERR_UNSUPPORTED),
    (dict(dtype=7), binding.FA_ERR_UNSUPPORTED),
    (dict(block_n=48), binding.FA_ERR_UNSUPPORTED),
    (dict(block_n=128), binding.FA_ERR_UNSUPPORTED),
    (dict(block_n=64, dtype=binding.FA_DTYPE_FP32), binding.FA_ERR_UNSUPPORTED),
    (dict(lse=MISALIGNED), binding.FA_ERR_INVALID_ARG),
])
def test_forward_rejects_bad_arguments(kw, code):
    assert fwd(**kw) == code


def test_per_head_size_limit():
    """N d = 2^30 in one head is refused by every dense entry point (the
    in-head 32-bit byte offsets); the backward's phases are refused alike."""
    assert fwd(N=1 << 23, d=128) == binding.FA_ERR_UNSUPPORTED
    assert fwd(N=1 << 24, d=64, dtype=binding.FA_DTYPE_FP32) == binding.FA_ERR_UNSUPPORTED
    a = [FAKE] * 9 + [ctypes.c_void_p(0x10000), 1 << 40, 1, 1, 1 << 23, 128, 0.125, 1,
                      binding.FA_DTYPE_BF16, None, binding.FA_BWD_MAIN]
    assert binding._raw().flash_attn_bwd_ex(*a) == binding.FA_ERR_UNSUPPORTED


def bwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE,
             ws=ctypes.c_void_p(0x10000), ws_bytes=1 << 40, B=1, H=1, N=16, d=64, scale=0.125, causal=1,
             dtype=binding.FA_DTYPE_BF16, stream=None)
    a.update(kw)
    return binding._raw().flash_attn_bwd(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"],
                                         a["dv"], a["ws"], a["ws_bytes"], a["B"], a["H"], a["N"], a["d"],
                                         a["scale"], a["causal"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(do=None), binding.FA_ERR_INVALID_ARG),
    (dict(lse=None), binding.FA_ERR_INVALID_ARG),
    (dict(ws=None), binding.FA_ERR_INVALID_ARG),
    (dict(ws_bytes=16), binding.FA_ERR_INVALID_ARG),
    (dict(ws=ctypes.c_void_p(0x10010)), binding.FA_ERR_INVALID_ARG),
    (dict(dv=MISALIGNED), binding.FA_ERR_INVALID_ARG),
    (dict(N=0), binding.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), binding.FA_ERR_INVALID_ARG),
    (dict(d=32), binding.FA_ERR_UNSUPPORTED),
    (dict(dtype=binding.FA_DTYPE_FP32), binding.FA_ERR_UNSUPPORTED),
    (dict(o=MISALIGNED), binding.FA_ERR_INVALID_ARG),
    # one head's fp32 dQ accumulator (4 N d bytes) must be addressable with
    # 32-bit offsets: N d = 2^30 is refused, even though B H N d < 2^31
    (dict(N=1 << 23, d=128), binding.FA_ERR_UNSUPPORTED),
    (dict(N=1 << 24, d=64), binding.FA_ERR_UNSUPPORTED),
])
def test_backward_rejects_bad_arguments(kw, code):
    assert bwd(**kw) == code


@pytest.mark.parametrize("phases", [0, 8, -1, 15])
def test_backward_rejects_bad_phase_masks(phases):
    a = [FAKE] * 9 + [ctypes.c_void_p(0x10000), 1 << 40, 1, 1, 16, 64, 0.125, 1, binding.FA_DTYPE_BF16, None,
                      phases]
    assert binding._raw().flash_attn_bwd_ex(*a) == binding.FA_ERR_INVALID_ARG


def test_python_binding_requires_gpu_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        binding.flash_attn_fwd(q, q, q)


def fwd_sparse(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, mask=FAKE, B=1, H=1, N=16, d=64, scale=0.125, causal=0,
             dtype=binding.FA_DTYPE_BF16, stream=None)
    a.update(kw)
    return binding._raw().flash_attn_fwd_blocksparse(a["q"], a["k"], a["v"], a["o"], a["lse"], a["mask"], a["B"],
                                                     a["H"], a["N"], a["d"], a["scale"], a["causal"], a["dtype"],
                                                     a["stream"])


def bwd_sparse(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, mask=FAKE, dq=FAKE, dk=FAKE, dv=FAKE,
             ws=ctypes.c_void_p(0x10000), ws_bytes=1 << 40, B=1, H=1, N=16, d=64, scale=0.125, causal=1,
             dtype=binding.FA_DTYPE_BF16, stream=None)
    a.update(kw)
    return binding._raw().flash_attn_bwd_blocksparse(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["mask"],
                                                     a["dq"], a["dk"], a["dv"], a["ws"], a["ws_bytes"], a["B"],
                                                     a["H"], a["N"], a["d"], a["scale"], a["causal"], a["dtype"],
                                                     a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(mask=None), binding.FA_ERR_INVALID_ARG),
    (dict(q=None), binding.FA_ERR_INVALID_ARG),
    (dict(N=0), binding.FA_ERR_INVALID_ARG),
    (dict(N=binding.FA_SPARSE_MAX_N + 1), binding.FA_ERR_UNSUPPORTED),
    (dict(dtype=binding.FA_DTYPE_FP32), binding.FA_ERR_UNSUPPORTED),
    (dict(d=96), binding.FA_ERR_UNSUPPORTED),
    (dict(scale=-1.0), binding.FA_ERR_INVALID_ARG),
    (dict(o=MISALIGNED), binding.FA_ERR_INVALID_ARG),
])
def test_sparse_forward_rejects_bad_arguments(kw, code):
    assert fwd_sparse(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(mask=None), binding.FA_ERR_INVALID_ARG),
    (dict(ws=None), binding.FA_ERR_INVALID_ARG),
    (dict(ws_bytes=16), binding.FA_ERR_INVALID_ARG),
    (dict(N=binding.FA_SPARSE_MAX_N + 1), binding.FA_ERR_UNSUPPORTED),
    (dict(dtype=binding.FA_DTYPE_FP32), binding.FA_ERR_UNSUPPORTED),
    (dict(causal=2), binding.FA_ERR_INVALID_ARG),
    (dict(dk=MISALIGNED), binding.FA_ERR_INVALID_ARG),
])
def test_sparse_backward_rejects_bad_arguments(kw, code):
    assert bwd_sparse(**kw) == code


def decode(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, ws=ctypes.c_void_p(0x10000), ws_bytes=1 << 40, B=1, H=1,
             Nq=1, Nk=64, d=128, scale=0.125, causal=0, dtype=binding.FA_DTYPE_BF16, stream=None)
    a.update(kw)
    return binding._raw().flash_attn_decode(a["q"], a["k"], a["v"], a["o"], a["lse"], a["ws"], a["ws_bytes"],
                                            a["B"], a["H"], a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"],
                                            a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), binding.FA_ERR_INVALID_ARG),
    (dict(ws=None), binding.FA_ERR_INVALID_ARG),
    (dict(ws_bytes=16), binding.FA_ERR_INVALID_ARG),
    (dict(ws=ctypes.c_void_p(0x10010)), binding.FA_ERR_INVALID_ARG),
    (dict(Nq=0), binding.FA_ERR_INVALID_ARG),
    (dict(Nq=65), binding.FA_ERR_INVALID_ARG),           # more queries than cache entries
    (dict(Nq=17, Nk=100), binding.FA_ERR_UNSUPPORTED),
    (dict(d=96), binding.FA_ERR_UNSUPPORTED),
    (dict(dtype=binding.FA_DTYPE_FP32), binding.FA_ERR_UNSUPPORTED),
    (dict(causal=3), binding.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), binding.FA_ERR_INVALID_ARG),
    (dict(k=MISALIGNED), binding.FA_ERR_INVALID_ARG),
])
def test_decode_rejects_bad_arguments(kw, code):
    assert decode(**kw) == code


def test_decode_workspace_size():
    f = binding.flash_attn_decode_workspace_size
    assert f(16, 32, 8192, 128) > 0 and f(16, 32, 8192, 128) % 256 == 0
    assert f(1, 1, 1, 64) > 0
    assert f(0, 1, 64, 64) == 0 and f(1, 1, 64, 96) == 0


def fwd_fp8(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, qd=0.01, kd=0.01, vd=0.01, o=FAKE, lse=FAKE, B=1, H=1, N=64, d=128,
             scale=0.125, causal=0, stream=None)
    a.update(kw)
    return binding._raw().flash_attn_fwd_fp8(a["q"], a["k"], a["v"], a["qd"], a["kd"], a["vd"], a["o"], a["lse"],
                                             a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), binding.FA_ERR_INVALID_ARG),
    (dict(o=None), binding.FA_ERR_INVALID_ARG),
    (dict(qd=0.0), binding.FA_ERR_INVALID_ARG),
    (dict(kd=-1.0), binding.FA_ERR_INVALID_ARG),
    (dict(vd=float("nan")), binding.FA_ERR_INVALID_ARG),
    (dict(vd=float("inf")), binding.FA_ERR_INVALID_ARG),
    (dict(N=0), binding.FA_ERR_INVALID_ARG),
    (dict(d=96), binding.FA_ERR_UNSUPPORTED),
    (dict(causal=2), binding.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), binding.FA_ERR_INVALID_ARG),
    (dict(v=MISALIGNED), binding.FA_ERR_INVALID_ARG),
    (dict(lse=MISALIGNED), binding.FA_ERR_INVALID_ARG),
])
def test_fp8_forward_rejects_bad_arguments(kw, code):
    assert fwd_fp8(**kw) == code


def merge(**kw):
    a = dict(oa=FAKE, la=FAKE, op=FAKE, lp=FAKE, oo=None, rows=64, d=128, stream=None)
    a.update(kw)
    return binding._raw().flash_attn_merge(a["oa"], a["la"], a["op"], a["lp"], a["oo"], a["rows"], a["d"],
                                           a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(oa=None), binding.FA_ERR_INVALID_ARG),
    (dict(lp=None), binding.FA_ERR_INVALID_ARG),
    (dict(rows=0), binding.FA_ERR_INVALID_ARG),
    (dict(rows=1 << 25), binding.FA_ERR_INVALID_ARG),   # rows * d >= 2^31
    (dict(d=96), binding.FA_ERR_UNSUPPORTED),
    (dict(op=MISALIGNED), binding.FA_ERR_INVALID_ARG),
    (dict(oo=MISALIGNED), binding.FA_ERR_INVALID_ARG),
])
def test_merge_rejects_bad_arguments(kw, code):
    assert merge(**kw) == code


def test_device_info_rejects_bad_arguments():
    x = ctypes.c_int(0)
    f = binding._raw().flash_attn_device_info
    assert f(0, None, ctypes.byref(x)) == binding.FA_ERR_INVALID_ARG
    assert f(-1, ctypes.byref(x), ctypes.byref(x)) == binding.FA_ERR_INVALID_ARG


def bwd_noalloc(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, B=1, H=1, N=16, d=64,
             scale=0.125, causal=1, dtype=binding.FA_DTYPE_BF16, stream=None)
    a.update(kw)
    return binding._raw().flash_attn_bwd_noalloc(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"],
                                                 a["dk"], a["dv"], a["B"], a["H"], a["N"], a["d"], a["scale"],
                                                 a["causal"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dq=None), binding.FA_ERR_INVALID_ARG),
    (dict(lse=None), binding.FA_ERR_INVALID_ARG),
    (dict(dv=MISALIGNED), binding.FA_ERR_INVALID_ARG),
    (dict(N=0), binding.FA_ERR_INVALID_ARG),
    (dict(causal=3), binding.FA_ERR_INVALID_ARG),
    (dict(d=96), binding.FA_ERR_UNSUPPORTED),
    (dict(dtype=binding.FA_DTYPE_FP32), binding.FA_ERR_UNSUPPORTED),
    # the workspace of B4 H16 N2048 d64 (69 MB) exceeds the static scratch
    (dict(B=4, H=16, N=2048, d=64), binding.FA_ERR_UNSUPPORTED),
])
def test_noalloc_backward_rejects_bad_arguments(kw, code):
    assert bwd_noalloc(**kw) == code


def test_noalloc_limit_matches_the_workspace_size():
    """Shapes are accepted exactly while their workspace fits the scratch."""
    f = binding.flash_attn_bwd_workspace_size
    assert f(2, 16, 2048, 64) <= binding.FA_BWD_NOALLOC_MAX_BYTES
    assert f(4, 16, 2048, 64) > binding.FA_BWD_NOALLOC_MAX_BYTES
    assert f(1, 1, 1 << 17, 128) > binding.FA_BWD_NOALLOC_MAX_BYTES
    assert bwd_noalloc(N=1 << 17, d=128) == binding.FA_ERR_UNSUPPORTED
