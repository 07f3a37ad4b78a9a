"""The allocation-free backward entry point (flash_attn_bwd_noalloc, whose
workspace is the library's static device scratch) against the ordinary
entry point (flash_attn_bwd, caller-owned workspace) and the oracle, through
the C ABI: two calls in a row on the same GPU, the second with a smaller
input, so the second runs on scratch the first left behind."""

import pytest

import oracle
from io_aware_tiled_attn_amd import binding
from io_aware_tiled_attn_amd import workloads as wl
from tests.gpu_util import TOL, announce, f64, max_err, to_f64, to_gpu, torch_cuda

pytestmark = pytest.mark.gpu


def _case(shape, seed, causal):
    torch = torch_cuda()
    import io_aware_tiled_attn_amd as fa
    inp = wl.make_inputs(shape, seed, "bf16", with_grad=True)
    q, k, v, do = (to_gpu(inp[n], "bf16") for n in ("q", "k", "v", "do"))
    o, lse = fa.flash_attn_fwd(q, k, v, causal=causal)
    ref = fa.flash_attn_bwd(q, k, v, o, lse, do, causal=causal)
    torch.cuda.synchronize()
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    got = fa.flash_attn_bwd_noalloc(q, k, v, o, lse, do, causal=causal, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert got[0] is dq and got[1] is dk and got[2] is dv
    # The same kernels in the same order, each output written once by one
    # workgroup: bit-identical.
    assert torch.equal(dq, ref[0]) and torch.equal(dk, ref[1]) and torch.equal(dv, ref[2])
    # and both against the oracle on two heads
    for b, h in ((0, 0), (shape[0] - 1, shape[1] - 1)):
        qh, kh, vh, doh = (f64(inp[n][b, h], "bf16") for n in ("q", "k", "v", "do"))
        rdq, rdk, rdv, _ = oracle.attention_backward_head(qh, kh, vh, doh, causal=causal)
        for g, r in ((dq, rdq), (dk, rdk), (dv, rdv)):
            assert max_err(to_f64(g)[b, h], r) <= TOL["bf16"]


@pytest.mark.parametrize("causal", [True, False])
def test_noalloc_backward_two_calls_second_smaller(causal):
    first, second = (2, 16, 2048, 64), (1, 3, 333, 128)
    announce(f"bwd noalloc call 1 shape={first} causal={causal}")
    _case(first, 8100, causal)
    announce(f"bwd noalloc call 2 shape={second} causal={causal}")
    _case(second, 8101, causal)


def test_noalloc_backward_rejects_a_workspace_beyond_the_scratch():
    torch = torch_cuda()
    import io_aware_tiled_attn_amd as fa
    shape = (4, 16, 2048, 64)        # 69 MB of workspace
    assert fa.flash_attn_bwd_workspace_size(*shape) > binding.FA_BWD_NOALLOC_MAX_BYTES
    q = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(shape[:3], dtype=torch.float32, device="cuda")
    with pytest.raises(fa.FlashAttnError) as exc:
        fa.flash_attn_bwd_noalloc(q, q, q, q, lse, q)
    assert exc.value.status == binding.FA_ERR_UNSUPPORTED
