"""GPU parity of the forward pass against the float64 oracle, through the
C ABI (ctypes binding).  Every case prints its name before the GPU step."""

import math

import numpy as np
import pytest

import oracle
from io_aware_tiled_attn_amd import workloads as wl
from tests import rescale_cases as rc
from tests.gpu_util import TOL, announce, f64, max_err, to_f64, to_gpu, torch_cuda

pytestmark = pytest.mark.gpu


def fa():
    torch_cuda()
    import io_aware_tiled_attn_amd as pkg
    return pkg


def run_fwd(inp, dtype, causal, scale=None, block_n=0):
    q, k, v = (to_gpu(inp[n], dtype) for n in ("q", "k", "v"))
    o, lse = fa().flash_attn_fwd_ex(q, k, v, causal=causal, scale=scale, block_n=block_n)
    torch_cuda().cuda.synchronize()
    return o, lse


def check_heads(inp, dtype, causal, o, lse, heads, scale=None, rows=None):
    """Compare whole heads (or selected rows of them) with the oracle."""
    tol = TOL[dtype]
    o64, lse64 = to_f64(o), to_f64(lse)
    worst_o = worst_l = 0.0
    for b, h in heads:
        qh, kh, vh = (f64(inp[n][b, h], dtype) for n in ("q", "k", "v"))
        ro, rl = oracle.attention_forward_head(qh, kh, vh, scale=scale, causal=causal, rows=rows)
        sel = slice(None) if rows is None else rows
        worst_o = max(worst_o, max_err(o64[b, h][sel], ro))
        worst_l = max(worst_l, max_err(lse64[b, h][sel], rl))
    print(f"  max|dO|={worst_o:.3e} max|dLSE|={worst_l:.3e} (tol {tol})", flush=True)
    assert worst_o <= tol
    assert worst_l <= tol
    return worst_o, worst_l


# --------------------------------------------------------------------------
# Small shapes: whole tensors against the oracle.  N values span several
# query and key tiles and leave ragged tails.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 17, 255, 300, 513])
def test_forward_small_bf16(N, d, causal):
    shape = (2, 2, N, d)
    announce(f"fwd bf16 shape={shape} causal={causal}")
    inp = wl.make_inputs(shape, 1000 + N + d, "bf16")
    o, lse = run_fwd(inp, "bf16", causal)
    check_heads(inp, "bf16", causal, o, lse, [(b, h) for b in range(2) for h in range(2)])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 33, 300])
def test_forward_small_fp32(N, d, causal):
    shape = (1, 2, N, d)
    announce(f"fwd fp32 shape={shape} causal={causal}")
    inp = wl.make_inputs(shape, 2000 + N + d, "fp32")
    o, lse = run_fwd(inp, "fp32", causal)
    check_heads(inp, "fp32", causal, o, lse, [(0, 0), (0, 1)])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_block_size_never_changes_answer(d, causal):
    """The pages' assertion that block size does not move the result
    (vibeengines.com, "Solve it yourself"), on the GPU: every key-tile width
    agrees with the oracle and with the others.  block_n = 0 is the default
    tile: 96 keys for dense d = 128, whose tiles do not divide the 256-query
    tiles or N = 390."""
    shape = (1, 3, 390, d)
    inp = wl.make_inputs(shape, 3000 + d, "bf16")
    outs = []
    for bn in (0, 32, 64):
        announce(f"fwd bf16 shape={shape} causal={causal} block_n={bn}")
        o, lse = run_fwd(inp, "bf16", causal, block_n=bn)
        check_heads(inp, "bf16", causal, o, lse, [(0, h) for h in range(3)])
        outs.append((to_f64(o), to_f64(lse)))
    for o2, l2 in outs[1:]:
        assert max_err(o2, outs[0][0]) <= TOL["bf16"]
        assert max_err(l2, outs[0][1]) <= 1e-4


def test_explicit_scale():
    shape = (1, 2, 200, 64)
    inp = wl.make_inputs(shape, 77, "bf16")
    for scale in (0.05, 0.3):
        announce(f"fwd bf16 shape={shape} scale={scale}")
        o, lse = run_fwd(inp, "bf16", True, scale=scale)
        check_heads(inp, "bf16", True, o, lse, [(0, 0), (0, 1)], scale=scale)


# --------------------------------------------------------------------------
# Pins carried onto the GPU.
# --------------------------------------------------------------------------
def _worked_example_inputs(n_keys, pad_value):
    """Row [2, 1, 3, 0] of the pages' worked example as scores of query 0:
    q_0 = e_0, k_j = s_j e_0, V_j = e_j, scale 1; extra keys (if any) get
    k_j = pad_value e_0 so that exp(pad - 3) underflows to 0 in fp32."""
    d = 64
    s = [2.0, 1.0, 3.0, 0.0]
    q = np.zeros((1, 1, n_keys, d), np.float32); q[0, 0, 0, 0] = 1.0
    k = np.zeros((1, 1, n_keys, d), np.float32)
    k[0, 0, :, 0] = pad_value
    k[0, 0, :4, 0] = s
    v = np.zeros((1, 1, n_keys, d), np.float32)
    for j in range(n_keys):
        v[0, 0, j, j % d] = 1.0
    return q, k, v


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("n_keys", [4, 64])
def test_worked_example_on_gpu(golden_dir, dtype, n_keys):
    import json, os
    g = json.load(open(os.path.join(golden_dir, "worked_example.json")))
    q, k, v = _worked_example_inputs(n_keys, -1024.0)
    if dtype == "bf16":
        inp = {n: wl.f32_to_bf16_bits(a) for n, a in zip("qkv", (q, k, v))}
    else:
        inp = dict(zip("qkv", (q, k, v)))
    announce(f"fwd {dtype} worked example n_keys={n_keys}")
    o, lse = run_fwd(inp, dtype, False, scale=1.0)
    o0 = to_f64(o)[0, 0, 0, :4]
    lse0 = float(to_f64(lse)[0, 0, 0])
    page_half_ulp = 0.5 * 10.0 ** -g["printed_decimals"]
    out_round = 2.0 ** -9 if dtype == "bf16" else 1e-6     # half-ulp of bf16 below 1
    np.testing.assert_allclose(o0, g["weights"], atol=page_half_ulp + out_round)
    m, l_page = g["after_block_2"]["m"], g["after_block_2"]["l"]
    assert abs(lse0 - (m + math.log(l_page))) <= page_half_ulp / l_page + 1e-5
    assert np.all(to_f64(o)[0, 0, 0, 4:] == 0.0)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_toy_example_on_gpu(golden_dir, dtype):
    """The page's 4 x 2 toy Q, K, V, zero-padded to d = 64 (zero features do
    not change Q K^T), scale 1/sqrt(2) passed explicitly."""
    import json, os
    g = json.load(open(os.path.join(golden_dir, "toy_example.json")))
    Q, K, V = (np.array(g[n], np.float32) for n in ("Q", "K", "V"))
    pads = []
    for a in (Q, K, V):
        p = np.zeros((1, 1, 4, 64), np.float32)
        p[0, 0, :, :2] = a
        pads.append(p)
    inp = ({n: wl.f32_to_bf16_bits(a) for n, a in zip("qkv", pads)} if dtype == "bf16"
           else dict(zip("qkv", pads)))
    announce(f"fwd {dtype} toy example")
    o, lse = run_fwd(inp, dtype, False, scale=1.0 / math.sqrt(2.0))
    ro, rl = oracle.attention_forward_head(Q, K, V)
    assert max_err(to_f64(o)[0, 0, :, :2], ro) <= TOL[dtype]
    assert max_err(to_f64(lse)[0, 0], rl) <= TOL[dtype]


@pytest.mark.parametrize("causal", [False, True])
def test_unit_values_give_unit_output(causal):
    """Rows of P sum to 1, so V = 1 gives O = 1 (within one bf16 ulp)."""
    shape = (1, 4, 700, 128)
    inp = wl.make_inputs(shape, 55, "bf16")
    inp["v"] = wl.f32_to_bf16_bits(np.ones(shape, np.float32))
    announce(f"fwd bf16 V=1 shape={shape} causal={causal}")
    o, _ = run_fwd(inp, "bf16", causal)
    assert max_err(to_f64(o), np.ones(shape)) <= 2.0 ** -7


def test_zero_keys_closed_form():
    """K = 0 gives uniform weights: causal O_i = mean of V_0..V_i and
    LSE_i = ln(i + 1)."""
    shape = (1, 2, 300, 64)
    inp = wl.make_inputs(shape, 56, "bf16")
    inp["k"] = np.zeros(shape, np.uint16)
    announce(f"fwd bf16 K=0 shape={shape}")
    o, lse = run_fwd(inp, "bf16", True)
    v = f64(inp["v"], "bf16")
    cum = np.cumsum(v, axis=2) / np.arange(1, 301)[None, None, :, None]
    assert max_err(to_f64(o), cum) <= TOL["bf16"]
    assert max_err(to_f64(lse), np.broadcast_to(np.log(np.arange(1, 301)), (1, 2, 300))) <= 1e-5


def test_forward_is_deterministic():
    shape = (2, 4, 1000, 128)
    inp = wl.make_inputs(shape, 57, "bf16")
    announce(f"fwd bf16 determinism shape={shape}")
    q, k, v = (to_gpu(inp[n], "bf16") for n in ("q", "k", "v"))
    o1, l1 = fa().flash_attn_fwd(q, k, v, causal=True)
    for _ in range(5):
        o2, l2 = fa().flash_attn_fwd(q, k, v, causal=True)
        torch = torch_cuda()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


# --------------------------------------------------------------------------
# The online-softmax update with live state: scores that climb from one key
# tile to the next, so the running max is raised while l and O already hold
# mass (vibeengines.com, "The math, worked with real numbers": "Rescale old
# l", "Absorb new block").  tests/test_rescale_model.py shows on the CPU that
# these exact inputs make the kernel's rescale branch run for live rows at
# every tile width used here; "falling" is the control without a raise.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("pattern", rc.PATTERNS)
@pytest.mark.parametrize("block_n", [0, 32, 64])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_forward_live_rescale(d, causal, block_n, pattern):
    shape = (1, 2, 520, d)
    announce(f"fwd bf16 climbing scores pattern={pattern} shape={shape} causal={causal} block_n={block_n}")
    inp = rc.climbing_bf16(shape, 11, pattern)
    o, lse = run_fwd(inp, "bf16", causal, block_n=block_n)
    check_heads(inp, "bf16", causal, o, lse, [(0, 0), (0, 1)])


@pytest.mark.parametrize("dtype,d,block_n", [("bf16", 64, 0), ("bf16", 64, 32), ("bf16", 64, 64),
                                             ("bf16", 128, 0), ("bf16", 128, 32), ("bf16", 128, 64),
                                             ("fp32", 64, 0), ("fp32", 128, 0)])
def test_worked_example_across_tiles(dtype, d, block_n):
    """The page's worked example with its two blocks in different key tiles
    (keys 0, 1 and 96, 97), scores multiplied by 6 through the scale
    argument so that the second block's max forces the raise of the running
    max with the first block's l and O live.  O_0[0:4] are the weights
    softmax(6 * [2, 1, 3, 0]) in the page's order; LSE_0 = 18 + ln of the
    sum of e^(6 s - 18)."""
    q, k, v = rc.worked_across_tiles_f32(d)
    inp = ({n: wl.f32_to_bf16_bits(a) for n, a in zip("qkv", (q, k, v))} if dtype == "bf16"
           else dict(zip("qkv", (q, k, v))))
    announce(f"fwd {dtype} worked example across tiles d={d} block_n={block_n}")
    o, lse = run_fwd(inp, dtype, False, scale=rc.WORKED_SCALE, block_n=block_n)
    z = [math.exp(rc.WORKED_SCALE * s - 18.0) for s in rc.WORKED_SCORES]
    weights = np.array(z) / sum(z)
    out_round = 2.0 ** -9 if dtype == "bf16" else 1e-6
    o64 = to_f64(o)
    np.testing.assert_allclose(o64[0, 0, 0, :4], weights, atol=out_round)
    assert np.all(o64[0, 0, 0, 4:] == 0.0)
    assert abs(float(to_f64(lse)[0, 0, 0]) - (18.0 + math.log(sum(z)))) <= 1e-5
    check_heads(inp, dtype, False, o, lse, [(0, 0)], scale=rc.WORKED_SCALE)


# --------------------------------------------------------------------------
# The five workloads at full size.  Small ones are compared whole; large ones
# on sampled heads (whole heads) plus sampled rows of every head.
# --------------------------------------------------------------------------
def _sampled_rows(N, count, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, 1, N - 1], rng.integers(0, N, count)]))


@pytest.mark.parametrize("name", ["fp32_single_head", "bf16_n1k_d64"])
def test_workload_whole(name):
    w = wl.WORKLOADS[name]
    announce(f"fwd workload {name}")
    inp = wl.workload_inputs(name, with_grad=False)
    o, lse = run_fwd(inp, w.dtype, w.causal)
    check_heads(inp, w.dtype, w.causal, o, lse, [(b, h) for b in range(w.B) for h in range(w.H)])


@pytest.mark.parametrize("name,heads", [
    ("bf16_n4k_d128_causal", [(0, 0), (3, 31)]),
    ("bf16_n16k_d64_causal", [(0, 5)]),
    ("bf16_n2k_d64_causal_fwdbwd", [(0, 0), (1, 7), (3, 15)]),
])
def test_workload_sampled(name, heads):
    w = wl.WORKLOADS[name]
    announce(f"fwd workload {name}")
    inp = wl.workload_inputs(name, with_grad=False)
    o, lse = run_fwd(inp, w.dtype, w.causal)
    check_heads(inp, w.dtype, w.causal, o, lse, heads)
    rows = _sampled_rows(w.N, 24, 9)
    every = [(b, h) for b in range(w.B) for h in range(w.H)]
    rng = np.random.default_rng(10)
    pick = [every[i] for i in rng.choice(len(every), size=min(len(every), 12), replace=False)]
    check_heads(inp, w.dtype, w.causal, o, lse, pick, rows=rows)


def test_long_context_extra_memory_is_linear():
    """N = 16384: the call allocates nothing; the only extra memory is the
    O and LSE buffers, far below one N x N score matrix (8.6 GB in bf16)."""
    torch = torch_cuda()
    w = wl.WORKLOADS["bf16_n16k_d64_causal"]
    announce("fwd memory check N=16384")
    inp = wl.workload_inputs(w.name, with_grad=False)
    q, k, v = (to_gpu(inp[n], "bf16") for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    fa().flash_attn_fwd(q, k, v, causal=True, out=o, lse=lse)     # warm-up: module load
    torch.cuda.synchronize()
    free_before, _ = torch.cuda.mem_get_info()
    torch.cuda.reset_peak_memory_stats()
    alloc_before = torch.cuda.max_memory_allocated()
    fa().flash_attn_fwd(q, k, v, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    free_after, _ = torch.cuda.mem_get_info()
    assert torch.cuda.max_memory_allocated() == alloc_before
    assert free_before - free_after < 64 << 20
