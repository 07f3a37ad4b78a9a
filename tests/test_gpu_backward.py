"""GPU parity of the backward pass (dQ, dK, dV) against the float64 oracle's
analytic gradients, through the C ABI.  The GPU backward consumes the GPU
forward's O and LSE, as a training step would; the oracle recomputes
everything from the bf16 inputs."""

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


def run_fwd_bwd(inp, causal, scale=None):
    q, k, v, do = (to_gpu(inp[n], "bf16") for n in ("q", "k", "v", "do"))
    o, lse = fa().flash_attn_fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa().flash_attn_bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch_cuda().cuda.synchronize()
    return dq, dk, dv


def check_grads(inp, causal, grads, heads, scale=None):
    g64 = [to_f64(t) for t in grads]
    worst = [0.0, 0.0, 0.0]
    for b, h in heads:
        qh, kh, vh, doh = (f64(inp[n][b, h], "bf16") for n in ("q", "k", "v", "do"))
        ref = oracle.attention_backward_head(qh, kh, vh, doh, scale=scale, causal=causal)[:3]
        for i in range(3):
            worst[i] = max(worst[i], max_err(g64[i][b, h], ref[i]))
    print(f"  max err dQ={worst[0]:.3e} dK={worst[1]:.3e} dV={worst[2]:.3e} (tol {TOL['bf16']})", flush=True)
    for i in range(3):
        assert worst[i] <= TOL["bf16"], ("dQ", "dK", "dV")[i]
    return worst


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 40, 300, 520])
def test_backward_small(N, d, causal):
    shape = (1, 2, N, d)
    announce(f"bwd shape={shape} causal={causal}")
    inp = wl.make_inputs(shape, 4000 + N + d, "bf16", with_grad=True)
    grads = run_fwd_bwd(inp, causal)
    check_grads(inp, causal, grads, [(0, 0), (0, 1)])


def test_backward_phases_equal_one_call():
    """Running the three backward kernels one call at a time (as the
    benchmark does to time them) gives the same result as one call."""
    torch = torch_cuda()
    from io_aware_tiled_attn_amd import binding
    shape = (2, 2, 333, 128)
    announce(f"bwd phases shape={shape}")
    inp = wl.make_inputs(shape, 4400, "bf16", with_grad=True)
    q, k, v, do = (to_gpu(inp[n], "bf16") for n in ("q", "k", "v", "do"))
    o, lse = fa().flash_attn_fwd(q, k, v, causal=True)
    ref = fa().flash_attn_bwd(q, k, v, o, lse, do, causal=True)
    ws = torch.empty(fa().flash_attn_bwd_workspace_size(*shape), dtype=torch.uint8, device="cuda")
    outs = [torch.empty_like(q) for _ in range(3)]
    for ph in (binding.FA_BWD_PREPROCESS, binding.FA_BWD_MAIN, binding.FA_BWD_FINALIZE):
        fa().flash_attn_bwd_ex(q, k, v, o, lse, do, causal=True, workspace=ws, dq=outs[0], dk=outs[1],
                               dv=outs[2], phases=ph)
    torch.cuda.synchronize()
    # Every gradient row is written once, by one workgroup, in a fixed
    # order: identical.
    for got, want in zip(outs, ref):
        assert torch.equal(got, want)


def test_backward_explicit_scale():
    """A non-default scale must reach every product (a scale applied twice
    or not at all moves the gradients far beyond the bound); 0.1 at d = 64
    is softer than the default 1/8 (test_backward_sharp_scale takes 0.2)."""
    shape = (1, 2, 260, 64)
    inp = wl.make_inputs(shape, 4100, "bf16", with_grad=True)
    announce(f"bwd shape={shape} scale=0.1")
    grads = run_fwd_bwd(inp, True, scale=0.1)
    check_grads(inp, True, grads, [(0, 0), (0, 1)], scale=0.1)


@pytest.mark.parametrize("causal", [True, False])
def test_backward_sharp_scale(causal):
    """Sharper attention, scale 0.2 at d = 64 (1.6x the default 1/8): the
    largest dK of this input is about 4.5, where half a bf16 step is 0.016,
    so the output rounding alone takes most of the 2e-2 bound and the
    arithmetic before it (fp16 P and dS, D from the bf16 O) must stay
    within the rest."""
    shape = (1, 2, 260, 64)
    inp = wl.make_inputs(shape, 4100, "bf16", with_grad=True)
    announce(f"bwd shape={shape} scale=0.2 causal={causal}")
    grads = run_fwd_bwd(inp, causal, scale=0.2)
    check_grads(inp, causal, grads, [(0, 0), (0, 1)], scale=0.2)


@pytest.mark.parametrize("d", [64, 128])
def test_backward_chunks_of_different_magnitude(d):
    """The preprocessing converts each 256-row chunk of Q and dO to fp16
    with the chunk's own power-of-two factor and then converts again, with
    the head's factor, every chunk whose factor differs.  Rows 256-511 of Q
    scaled by 2^-6 and rows 512-767 of dO by 2^-5 (exact in bf16) give
    those chunks factors 64 and 32 times the head's: a chunk left at its own
    factor would scale its scores or its dO by that much."""
    shape = (1, 2, 1100, d)
    inp = wl.make_inputs(shape, 4500 + d, "bf16", with_grad=True)
    q = f64(inp["q"], "bf16")
    g = f64(inp["do"], "bf16")
    q[:, :, 256:512] *= 2.0 ** -6
    g[:, :, 512:768] *= 2.0 ** -5
    inp = dict(inp, q=wl.f32_to_bf16_bits(q.astype(np.float32)), do=wl.f32_to_bf16_bits(g.astype(np.float32)))
    assert np.array_equal(f64(inp["q"], "bf16"), q) and np.array_equal(f64(inp["do"], "bf16"), g)
    announce(f"bwd shape={shape} chunk magnitudes")
    for causal in (True, False):
        grads = run_fwd_bwd(inp, causal)
        check_grads(inp, causal, grads, [(0, 0), (0, 1)])


def _invariants(inp, grads, causal):
    """Properties at any size: rows of dS sum to 0 so the key gradients sum
    to 0; rows of P sum to 1 so sum_j dV_j = sum_i dO_i; causal row 0 sees
    only key 0, so dQ_0 = 0.  Bounds allow for bf16 rounding of each term."""
    dq, dk, dv = (to_f64(t) for t in grads)
    do = f64(inp["do"], "bf16")
    N = dk.shape[2]
    ulp = 2.0 ** -8
    s_dk = np.abs(dk.sum(axis=2))
    assert np.all(s_dk <= 4 * ulp * np.sqrt(N) * np.abs(dk).max(axis=2) + 1e-3)
    s_dv = np.abs(dv.sum(axis=2) - do.sum(axis=2))
    assert np.all(s_dv <= 4 * ulp * np.sqrt(N) * np.abs(dv).max(axis=2) + 1e-3)
    if causal:
        assert np.abs(dq[:, :, 0, :]).max() <= 1e-3


@pytest.mark.parametrize("name,heads", [
    ("bf16_n2k_d64_causal_fwdbwd", [(0, 0), (1, 9), (2, 3), (3, 15)]),
    ("bf16_n4k_d128_causal", [(0, 0), (2, 0), (3, 31)]),
])
def test_workload_backward(name, heads):
    w = wl.WORKLOADS[name]
    announce(f"bwd workload {name}")
    inp = wl.workload_inputs(name, with_grad=True)
    grads = run_fwd_bwd(inp, w.causal)
    check_grads(inp, w.causal, grads, heads)
    _invariants(inp, grads, w.causal)
