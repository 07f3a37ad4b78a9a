"""GPU parity of block-sparse attention (forward and backward) against the
float64 oracle with the same block mask, through the C ABI.

Bound: 2e-2 absolute, the dense bound, on every element whose oracle value
is below 8 in magnitude; 2e-2 plus 2^-8 of the oracle's magnitude on the
elements at or above 8.  A block mask can leave a query block with very few
keys (here: only the one valid key of a ragged last block), and then a
gradient is the plain sum of up to 128 dO rows, magnitude ~25, and from 8
up the bf16 rounding of the output alone (half an ulp: 2^-5 in [8, 16),
2^-4 in [16, 32)) exceeds 2e-2 whatever the arithmetic; 2^-8 |ref| covers
that half ulp, the 2e-2 the arithmetic before it.  Each check prints how
many elements took the wider bound."""

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


def mask_gpu(mask):
    torch = torch_cuda()
    return torch.from_numpy(np.ascontiguousarray(mask)).cuda()


def run(inp, mask, causal, backward=True):
    q, k, v, do = (to_gpu(inp[n], "bf16") for n in ("q", "k", "v", "do"))
    m = mask_gpu(mask)
    o, lse = fa().flash_attn_fwd_blocksparse(q, k, v, m, causal=causal)
    grads = None
    if backward:
        grads = fa().flash_attn_bwd_blocksparse(q, k, v, o, lse, do, m, causal=causal)
    torch_cuda().cuda.synchronize()
    return o, lse, grads


WIDE_FROM = 8.0     # |ref| from which half a bf16 ulp (2^-5 at 8) exceeds 2e-2
WIDE_COUNT = [0]


def rel_err(gpu, ref):
    """max of |gpu - ref| - allowance, the allowance being 2^-8 |ref| where
    |ref| >= 8 and 0 elsewhere (0 for an empty array); compared with 2e-2."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    if gpu.size == 0:
        return 0.0
    assert np.all(np.isfinite(gpu)), "non-finite values in GPU output"
    wide = np.abs(ref) >= WIDE_FROM
    WIDE_COUNT[0] += int(wide.sum())
    return float(np.max(np.abs(gpu - ref) - np.where(wide, 2.0 ** -8 * np.abs(ref), 0.0)))


def check(inp, mask, causal, o, lse, grads, heads):
    o64, l64 = to_f64(o), to_f64(lse)
    g64 = [to_f64(t) for t in grads] if grads is not None else None
    worst = {"o": 0.0, "lse": 0.0, "dq": 0.0, "dk": 0.0, "dv": 0.0}
    for b, h in heads:
        qh, kh, vh, doh = (f64(inp[n][b, h], "bf16") for n in ("q", "k", "v", "do"))
        ro, rl = oracle.attention_forward_head(qh, kh, vh, causal=causal, block_mask=mask[b, h])
        empty = np.isinf(rl)
        # Rows that see no key: exactly zero output and -inf LSE.
        assert np.all(o64[b, h][empty] == 0.0)
        assert np.all(l64[b, h][empty] == -np.inf)
        worst["o"] = max(worst["o"], rel_err(o64[b, h], ro))
        worst["lse"] = max(worst["lse"], max_err(l64[b, h][~empty], rl[~empty]))
        if g64 is not None:
            ref = oracle.attention_backward_head(qh, kh, vh, doh, causal=causal, block_mask=mask[b, h])[:3]
            for name, g, r in zip(("dq", "dk", "dv"), g64, ref):
                worst[name] = max(worst[name], rel_err(g[b, h], r))
            assert np.all(g64[0][b, h][empty] == 0.0)
    print("  max err (beyond the allowance) " + " ".join(f"{k}={v:.3e}" for k, v in worst.items())
          + f"; elements at |ref| >= {WIDE_FROM:g}: {WIDE_COUNT[0]}", flush=True)
    WIDE_COUNT[0] = 0
    for k2, v2 in worst.items():
        assert v2 <= TOL["bf16"], k2
    return worst


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [200, 300, 513])
def test_blocksparse_random_masks(N, d, causal):
    shape = (1, 3, N, d)
    announce(f"blocksparse fwd+bwd shape={shape} causal={causal}")
    inp = wl.make_inputs(shape, 5000 + N + d, "bf16", with_grad=True)
    mask = wl.random_block_mask(1, 3, N, 6000 + N + d, density=0.5)
    mask[0, 1] = 1      # head 1: dense
    mask[0, 2, 0, :] = 0  # head 2: query block 0 sees nothing
    o, lse, grads = run(inp, mask, causal)
    check(inp, mask, causal, o, lse, grads, [(0, 0), (0, 1), (0, 2)])


@pytest.mark.parametrize("causal", [False, True])
def test_full_mask_matches_dense_kernels(causal):
    """All pairs kept: the sparse kernels visit every tile the dense kernels
    visit, in the same order, so O, LSE, dQ, dK and dV are bit-identical."""
    torch = torch_cuda()
    shape = (2, 2, 384, 64)
    announce(f"blocksparse full mask vs dense shape={shape} causal={causal}")
    inp = wl.make_inputs(shape, 7100, "bf16", with_grad=True)
    q, k, v, do = (to_gpu(inp[n], "bf16") for n in ("q", "k", "v", "do"))
    ones = mask_gpu(np.ones((2, 2, 3, 3), np.uint8))
    o1, l1 = fa().flash_attn_fwd(q, k, v, causal=causal)
    o2, l2 = fa().flash_attn_fwd_blocksparse(q, k, v, ones, causal=causal)
    g1 = fa().flash_attn_bwd(q, k, v, o1, l1, do, causal=causal)
    g2 = fa().flash_attn_bwd_blocksparse(q, k, v, o2, l2, do, ones, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_empty_mask_gives_zeros():
    shape = (1, 2, 300, 128)
    announce(f"blocksparse empty mask shape={shape}")
    inp = wl.make_inputs(shape, 7200, "bf16", with_grad=True)
    mask = np.zeros((1, 2, 3, 3), np.uint8)
    o, lse, (dq, dk, dv) = run(inp, mask, False)
    torch = torch_cuda()
    assert torch.count_nonzero(o).item() == 0
    assert bool(torch.all(lse == -float("inf")))
    for g in (dq, dk, dv):
        assert torch.count_nonzero(g).item() == 0


def test_block_diagonal_equals_independent_blocks():
    """Only diagonal blocks kept: each 128-row block is ordinary attention
    over its own keys; compared with the dense GPU kernel run on each block
    as a separate sequence, and with the oracle."""
    torch = torch_cuda()
    shape = (1, 2, 512, 64)
    announce(f"blocksparse block-diagonal shape={shape}")
    inp = wl.make_inputs(shape, 7300, "bf16", with_grad=True)
    mask = np.broadcast_to(np.eye(4, dtype=np.uint8), (1, 2, 4, 4)).copy()
    o, lse, grads = run(inp, mask, False)
    check(inp, mask, False, o, lse, grads, [(0, 0), (0, 1)])
    q, k, v = (to_gpu(inp[n], "bf16") for n in ("q", "k", "v"))
    for blk in range(4):
        r = slice(128 * blk, 128 * (blk + 1))
        ob, lb = fa().flash_attn_fwd(q[:, :, r].contiguous(), k[:, :, r].contiguous(), v[:, :, r].contiguous())
        torch.cuda.synchronize()
        assert max_err(to_f64(o[:, :, r]), to_f64(ob)) <= TOL["bf16"]
        assert max_err(to_f64(lse[:, :, r]), to_f64(lb)) <= 1e-4


@pytest.mark.parametrize("d", [64, 128])
def test_blocksparse_causal_band(d):
    """Causal local band + global column over a ragged length: each
    workgroup's list ends on its own diagonal, where all its waves but the
    last two have visited tiles past their last query (at d = 128 those are
    skipped per wave).  Whole heads against the oracle."""
    shape = (1, 2, 1000, d)
    announce(f"blocksparse causal band shape={shape}")
    inp = wl.make_inputs(shape, 7700 + d, "bf16", with_grad=True)
    mask = wl.local_global_block_mask(1, 2, 1000, band=1)
    o, lse, grads = run(inp, mask, True)
    check(inp, mask, True, o, lse, grads, [(0, 0), (0, 1)])


def test_sparse_workload_sampled():
    """The benchmark's block-sparse workload (B4 H32 N4096 d128, local band
    + global column) at full size: every output and gradient of three heads
    against the oracle."""
    w = wl.SPARSE_WORKLOAD
    announce(f"blocksparse workload {w.name} shape={w.shape}")
    inp = wl.make_inputs(w.shape, w.seed, "bf16", with_grad=True)
    mask = wl.local_global_block_mask(w.B, w.H, w.N)
    o, lse, grads = run(inp, mask, w.causal)
    check(inp, mask, w.causal, o, lse, grads, [(0, 0), (1, 17), (3, 31)])


@pytest.mark.parametrize("pattern", ["stair", "ramp"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_blocksparse_forward_live_rescale(d, causal, pattern):
    """Scores that climb across the visited key tiles (tests/rescale_cases.py)
    under a random block mask: the kernel raises its running max with l and
    O live (shown on the CPU by tests/test_rescale_model.py for these inputs
    and this mask)."""
    from tests import rescale_cases as rc
    from tests.test_rescale_model import sparse_case_mask
    N = 520
    announce(f"block-sparse fwd climbing scores pattern={pattern} d={d} causal={causal}")
    inp = rc.climbing_bf16((1, 2, N, d), 13, pattern)
    inp["do"] = np.zeros_like(inp["q"])
    mask = sparse_case_mask(N)
    o, lse, _ = run(inp, mask, causal, backward=False)
    check(inp, mask, causal, o, lse, None, [(0, 0), (0, 1)])
