"""GPU parity of decoding against a key/value cache (split-KV) with the
float64 oracle's decoding form, through the C ABI."""

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


def run(inp, causal):
    q, k, v = (to_gpu(inp[n], "bf16") for n in ("q", "k", "v"))
    o, lse = fa().flash_attn_decode(q, k, v, causal=causal)
    torch_cuda().cuda.synchronize()
    return o, lse


def check(inp, causal, o, lse, heads):
    o64, l64 = to_f64(o), to_f64(lse)
    eo = el = 0.0
    for b, h in heads:
        qh, kh, vh = (f64(inp[n][b, h], "bf16") for n in ("q", "k", "v"))
        ro, rl = oracle.attention_decode_head(qh, kh, vh, causal=causal)
        eo = max(eo, max_err(o64[b, h], ro))
        el = max(el, max_err(l64[b, h], rl))
    print(f"  max err O={eo:.3e} LSE={el:.3e}", flush=True)
    assert eo <= TOL["bf16"] and el <= 1e-4


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("nq,nk", [(1, 1), (1, 31), (3, 100), (16, 16), (16, 513), (5, 2048)])
def test_decode_small(nq, nk, d, causal):
    announce(f"decode B2 H3 Nq={nq} Nk={nk} d={d} causal={causal}")
    inp = wl.decode_inputs(2, 3, nq, nk, d, 8000 + nq + nk + d)
    o, lse = run(inp, causal)
    check(inp, causal, o, lse, [(b, h) for b in range(2) for h in range(3)])


@pytest.mark.parametrize("causal", [False, True])
def test_decode_equals_last_rows_of_forward(causal):
    """The last Nq queries decoded against the whole cache match the last Nq
    rows of the forward kernel run on the full sequence (prefill)."""
    torch = torch_cuda()
    B, H, N, d, nq = 2, 2, 600, 128, 7
    announce(f"decode vs forward last rows N={N} nq={nq} causal={causal}")
    inp = wl.make_inputs((B, H, N, d), 8100, "bf16")
    q, k, v = (to_gpu(inp[n], "bf16") for n in ("q", "k", "v"))
    of, lf = fa().flash_attn_fwd(q, k, v, causal=causal)
    od, ld = fa().flash_attn_decode(q[:, :, N - nq:].contiguous(), k, v, causal=causal)
    torch.cuda.synchronize()
    assert max_err(to_f64(od), to_f64(of[:, :, N - nq:])) <= TOL["bf16"]
    assert max_err(to_f64(ld), to_f64(lf[:, :, N - nq:])) <= 1e-4


def test_decode_workload_sampled():
    """The benchmark's decoding workload at full size, sampled heads."""
    w = wl.DECODE_WORKLOAD
    announce(f"decode workload {w.name}")
    inp = wl.decode_inputs(w.B, w.H, w.Nq, w.Nk, w.d, w.seed)
    o, lse = run(inp, w.causal)
    check(inp, w.causal, o, lse, [(0, 0), (7, 13), (15, 31)])
