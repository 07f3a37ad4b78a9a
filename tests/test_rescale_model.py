"""The inputs of the live-rescale GPU tests provably reach the forward
kernels' rescale of a live partial result.

`tests/lazy_max_model.py` replays the kernels' lazy-max trigger rule (lane
sums of P against the running reference, the wave vote, the raise) on the
exact values each GPU test feeds the kernel.  Every rising input must make
some query rescale an l and O that already hold mass, for every tile width
the GPU test runs; the falling control must make none.  Without such inputs
a kernel that dropped `l *= alpha` or `O *= alpha` would still pass every
GPU test, since with N(0, 1) inputs later tiles never climb far enough past
the first tile's max."""

import numpy as np
import pytest

from io_aware_tiled_attn_amd import workloads as wl
from tests import lazy_max_model as lm
from tests import rescale_cases as rc

SHAPE_N = 520          # the GPU tests' sequence length (ragged: not a tile multiple)


def _head(inp, dtype, name, h=0):
    if dtype == "fp8":
        import oracle
        return oracle.dequantize(inp[name][0, h], inp[name + "_descale"])
    return wl.values(inp[name][0, h], dtype).astype(np.float64)


@pytest.mark.parametrize("pattern", rc.PATTERNS)
@pytest.mark.parametrize("block_n", [0, 32, 64])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_bf16_forward_inputs_reach_live_rescale(d, causal, block_n, pattern):
    inp = rc.climbing_bf16((1, 2, SHAPE_N, d), 11, pattern)
    for h in range(2):
        r = lm.count_live_rescales(_head(inp, "bf16", "q", h), _head(inp, "bf16", "k", h),
                                   1.0 / np.sqrt(d), causal, "bf16", block_n)
        if pattern == "falling":
            assert r["live_any"] == 0, r
        else:
            assert r["live"] >= 32, r


@pytest.mark.parametrize("pattern", rc.PATTERNS)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_fp8_forward_inputs_reach_live_rescale(d, causal, pattern):
    inp = rc.climbing_fp8((1, 2, SHAPE_N, d), 12, pattern)
    for h in range(2):
        q, k = _head(inp, "fp8", "q", h), _head(inp, "fp8", "k", h)
        r = lm.count_live_rescales(q, k, 1.0 / np.sqrt(d), causal, "fp8")
        if pattern == "falling":
            assert r["live_any"] == 0, r
        else:
            assert r["live"] >= 32, r


def sparse_case_mask(N, seed=21):
    """Block mask of the block-sparse live-rescale test: random pairs kept
    with probability 0.6, plus the diagonal (so no row is empty)."""
    m = wl.random_block_mask(1, 2, N, seed, density=0.6)
    nb = m.shape[-1]
    m[..., np.arange(nb), np.arange(nb)] = 1
    return m


@pytest.mark.parametrize("pattern", ["stair", "ramp"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_blocksparse_forward_inputs_reach_live_rescale(d, causal, pattern):
    inp = rc.climbing_bf16((1, 2, SHAPE_N, d), 13, pattern)
    mask = sparse_case_mask(SHAPE_N)
    for h in range(2):
        r = lm.count_live_rescales(_head(inp, "bf16", "q", h), _head(inp, "bf16", "k", h),
                                   1.0 / np.sqrt(d), causal, "bf16", 0, block_mask=mask[0, h])
        assert r["live"] >= 32, r


@pytest.mark.parametrize("kernel,block_n,d", [("bf16", 0, 64), ("bf16", 32, 64), ("bf16", 64, 64),
                                              ("bf16", 0, 128), ("bf16", 32, 128), ("bf16", 64, 128),
                                              ("fp8", 0, 64), ("fp8", 0, 128)])
def test_worked_example_across_tiles_raises_the_max(kernel, block_n, d):
    """Query 0 of the worked-example head: its first tile holds scores
    6 * (2, 1), a later tile 6 * (3, 0); the raise happens with l > 0."""
    if kernel == "fp8":
        inp = rc.worked_across_tiles_fp8(d)
        q, k = _head(inp, "fp8", "q"), _head(inp, "fp8", "k")
    else:
        q, k, _ = rc.worked_across_tiles_f32(d)
        q, k = q[0, 0].astype(np.float64), k[0, 0].astype(np.float64)
    r = lm.count_live_rescales(q, k, rc.WORKED_SCALE, False, kernel, block_n)
    assert r["live"] >= 1, r


def test_model_counts_no_rescale_for_plain_normal_inputs():
    """The reason these inputs exist: N(0, 1) inputs at the default scale
    give no live rescale at all (the first tile's max is never exceeded by
    enough)."""
    for d in (64, 128):
        inp = wl.make_inputs((1, 2, SHAPE_N, d), 1000 + d, "bf16")
        for causal in (False, True):
            r = lm.count_live_rescales(_head(inp, "bf16", "q"), _head(inp, "bf16", "k"),
                                       1.0 / np.sqrt(d), causal, "bf16", 0)
            assert r["live_any"] == 0, r


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_planted_rescale_mistakes_exceed_the_tolerance(d, causal):
    """Carried out in float64, the kernels' lazy update on these inputs
    equals the oracle (it is exact in exact arithmetic; 1e-6 allows for the
    factor scale * log2 e rounded to fp32 as the kernels use it), and each
    planted mistake in the rescale branch moves O, on the stair or the ramp
    input, by far more than the 2e-2 bound the GPU tests apply: so the GPU
    tests reaching the branch would catch such a mistake in the kernel.
    (The stair is the one that shows a wrongly based alpha: the ramp's
    rescaled mass is too small to matter.)"""
    import oracle
    scale = 1.0 / np.sqrt(d)
    worst = {mut: 0.0 for mut in lm.MUTATIONS}
    for pattern in ("stair", "ramp"):
        inp = rc.climbing_bf16((1, 1, SHAPE_N, d), 11, pattern)
        q, k, v = (_head(inp, "bf16", n) for n in "qkv")
        ref, _ = oracle.attention_forward_head(q, k, v, causal=causal)
        for block_n in (0, 32):
            good = lm.count_live_rescales(q, k, scale, causal, "bf16", block_n, v=v)["o"]
            assert np.max(np.abs(good - ref)) < 1e-6
            for mut in lm.MUTATIONS:
                bad = lm.count_live_rescales(q, k, scale, causal, "bf16", block_n, v=v, mutation=mut)["o"]
                worst[mut] = max(worst[mut], float(np.max(np.abs(bad - ref))))
    for mut, err in worst.items():
        assert err > 0.1, (mut, err)
