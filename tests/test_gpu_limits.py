"""GPU parity at the size limit of the ABI: B*H*N*d just below 2^31
elements per tensor (B256 H64 N1023 d128, bf16, causal, about 4.3 GB per
tensor), where the per-head offsets of the last heads exceed 32 bits.  Inputs
are drawn on the GPU (seeded); the heads checked are copied back and given
to the float64 oracle as they are."""

import numpy as np
import pytest

import oracle
from io_aware_tiled_attn_amd import workloads as wl
from tests.gpu_util import TOL, announce, max_err, to_f64, torch_cuda

pytestmark = pytest.mark.gpu

SHAPE = (256, 64, 1023, 128)
HEADS = [(0, 0), (127, 31), (255, 63)]   # first, middle and last head


def fa():
    torch_cuda()
    import io_aware_tiled_attn_amd as pkg
    return pkg


def test_shape_is_just_below_the_limit():
    B, H, N, d = SHAPE
    assert B * H * N * d < 2 ** 31 and B * H * (N + 1) * d > 2 ** 31 - 1


def test_forward_and_backward_near_element_limit():
    torch = torch_cuda()
    announce(f"forward+backward near the element limit {SHAPE} causal")
    q, k, v, do = (wl.gpu_normal_bf16(SHAPE, 20000 + i) for i in range(4))
    o, lse = fa().flash_attn_fwd(q, k, v, causal=True)
    dq, dk, dv = fa().flash_attn_bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    worst = {"o": 0.0, "lse": 0.0, "dq": 0.0, "dk": 0.0, "dv": 0.0}
    for b, h in HEADS:
        qh, kh, vh, doh = (to_f64(t[b, h]) for t in (q, k, v, do))
        ro, rl = oracle.attention_forward_head(qh, kh, vh, causal=True)
        rdq, rdk, rdv, _ = oracle.attention_backward_head(qh, kh, vh, doh, causal=True)
        for name, got, ref in (("o", o, ro), ("lse", lse, rl), ("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
            worst[name] = max(worst[name], max_err(to_f64(got[b, h]), ref))
    print("  max err " + " ".join(f"{n}={e:.3e}" for n, e in worst.items()), flush=True)
    assert worst["lse"] <= 1e-4
    for n in ("o", "dq", "dk", "dv"):
        assert worst[n] <= TOL["bf16"], n
    del q, k, v, do, o, lse, dq, dk, dv
    torch.cuda.empty_cache()
