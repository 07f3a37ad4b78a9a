"""GPU parity of the persistent launches, through the C ABI.

With B*H a multiple of 8 (and a dense mask) the bf16 forward and the two
backward main kernels launch as many workgroups per XCD as run at once, and
each works through a fixed share of its XCD's list of (tile, head) items.
The shapes here give every XCD more items than it has resident workgroups,
with N not a multiple of any tile, so workgroups take two or more items,
among them partial last tiles, and the LDS and registers carried from one
item to the next are exercised.  Whole heads, chosen to cover every XCD and
both ends of its list, are compared with the float64 oracle."""

import numpy as np
import pytest

import oracle
from io_aware_tiled_attn_amd import workloads as wl
from tests.gpu_util import TOL, announce, f64, max_err, to_f64, to_gpu, torch_cuda

pytestmark = pytest.mark.gpu


def fa():
    torch_cuda()
    import io_aware_tiled_attn_amd as pkg
    return pkg


def heads_over_xcds(B, H):
    """The first and the last head of each XCD's list (heads x, x + 8, ...
    go to XCD x), as (batch, head) pairs."""
    bh_all = B * H
    pick = sorted({x for x in range(8)} | {bh_all - 8 + x for x in range(8)})
    return [(bh // H, bh % H) for bh in pick]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(4, 16, 1100, 128), (8, 16, 1100, 64)])
def test_forward_persistent_several_items(shape, causal):
    # d = 128: 96-key tiles, one workgroup per CU, 8 heads x 5 query tiles
    # = 40 items per XCD for 32 resident workgroups.  d = 64: two
    # workgroups per CU, 16 x 5 = 80 items for 64.
    announce(f"fwd persistent shape={shape} causal={causal}")
    inp = wl.make_inputs(shape, 6100 + shape[3], "bf16")
    q, k, v = (to_gpu(inp[n], "bf16") for n in ("q", "k", "v"))
    o, lse = fa().flash_attn_fwd(q, k, v, causal=causal)
    torch_cuda().cuda.synchronize()
    o64, lse64 = to_f64(o), to_f64(lse)
    assert np.isfinite(o64).all() and np.isfinite(lse64).all()
    worst_o = worst_l = 0.0
    for b, h in heads_over_xcds(shape[0], shape[1]):
        qh, kh, vh = (f64(inp[n][b, h], "bf16") for n in ("q", "k", "v"))
        ro, rl = oracle.attention_forward_head(qh, kh, vh, causal=causal)
        worst_o = max(worst_o, max_err(o64[b, h], ro))
        worst_l = max(worst_l, max_err(lse64[b, h], rl))
    print(f"  max|dO|={worst_o:.3e} max|dLSE|={worst_l:.3e} (tol {TOL['bf16']})", flush=True)
    assert worst_o <= TOL["bf16"] and worst_l <= TOL["bf16"]


@pytest.mark.parametrize("causal", [False, True])
def test_backward_persistent_several_items(causal):
    # 8 heads x 9 tiles of 128 rows = 72 items per XCD for 32 resident
    # workgroups, in both the dK/dV and the dQ kernel.
    shape = (4, 16, 1100, 128)
    announce(f"bwd persistent shape={shape} causal={causal}")
    inp = wl.make_inputs(shape, 6300, "bf16", with_grad=True)
    q, k, v, do = (to_gpu(inp[n], "bf16") for n in ("q", "k", "v", "do"))
    o, lse = fa().flash_attn_fwd(q, k, v, causal=causal)
    grads = fa().flash_attn_bwd(q, k, v, o, lse, do, causal=causal)
    torch_cuda().cuda.synchronize()
    g64 = [to_f64(t) for t in grads]
    for g in g64:
        assert np.isfinite(g).all()
    picks = heads_over_xcds(shape[0], shape[1])
    picks = [picks[i] for i in range(0, len(picks), 2)]   # 8 heads, one per XCD
    worst = [0.0, 0.0, 0.0]
    for b, h in picks:
        qh, kh, vh, doh = (f64(inp[n][b, h], "bf16") for n in ("q", "k", "v", "do"))
        ref = oracle.attention_backward_head(qh, kh, vh, doh, causal=causal)[:3]
        for i in range(3):
            worst[i] = max(worst[i], max_err(g64[i][b, h], ref[i]))
    print(f"  max err dQ={worst[0]:.3e} dK={worst[1]:.3e} dV={worst[2]:.3e} (tol {TOL['bf16']})", flush=True)
    for i in range(3):
        assert worst[i] <= TOL["bf16"], ("dQ", "dK", "dV")[i]
