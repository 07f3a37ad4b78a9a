"""The ABI's stream and threading promises: every call enqueues its kernels
on the stream it is given (results match the default-stream ones and are
complete once that stream alone is synchronised), and calls from several
host threads, each on its own stream, give the same results as serial
calls.  Every output is bit-reproducible: each element is written once, by
one workgroup, after a fixed order of operations."""

import threading

import pytest

from io_aware_tiled_attn_amd import workloads as wl
from tests.gpu_util import announce, to_gpu, torch_cuda

pytestmark = pytest.mark.gpu


def fa():
    torch_cuda()
    import io_aware_tiled_attn_amd as pkg
    return pkg


def _inputs(seed, shape=(2, 4, 700, 128)):
    inp = wl.make_inputs(shape, seed, "bf16", with_grad=True)
    return [to_gpu(inp[n], "bf16") for n in ("q", "k", "v", "do")]


def _run(q, k, v, do, stream=None):
    torch = torch_cuda()
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    fa().flash_attn_fwd(q, k, v, causal=True, out=o, lse=lse, stream=stream)
    dq, dk, dv = fa().flash_attn_bwd(q, k, v, o, lse, do, causal=True, stream=stream)
    return o, lse, dq, dk, dv


def _same(got, ref):
    torch = torch_cuda()
    o, lse, dq, dk, dv = got
    ro, rl, rdq, rdk, rdv = ref
    for a, b in ((o, ro), (lse, rl), (dq, rdq), (dk, rdk), (dv, rdv)):
        assert torch.equal(a, b)


def test_calls_run_on_the_given_stream():
    torch = torch_cuda()
    announce("forward + backward on a side stream")
    q, k, v, do = _inputs(40000)
    ref = _run(q, k, v, do)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        got = _run(q, k, v, do, stream=s)
    s.synchronize()                       # that stream alone
    _same(got, ref)


def test_calls_from_several_host_threads():
    torch = torch_cuda()
    announce("forward + backward from four host threads")
    inputs = [_inputs(40100 + t, (1, 2, 300 + 100 * t, 64 if t % 2 else 128)) for t in range(4)]
    refs = [_run(*x) for x in inputs]
    torch.cuda.synchronize()
    results, errors = [None] * 4, []

    def work(t):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(3):
                    results[t] = _run(*inputs[t], stream=s)
            s.synchronize()
        except Exception as e:  # reported below, in the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for got, ref in zip(results, refs):
        _same(got, ref)
