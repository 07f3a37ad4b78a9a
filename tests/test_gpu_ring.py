"""One GPU's part of a sequence-parallel (ring) schedule, run through the
library's own calls.

The sequence is cut into 2P chunks; device r of P holds query chunks r and
2P-1-r (zig-zag), and every key/value chunk visits it in turn.  Here the P
devices run one after another on the same GPU: flash_attn_fwd on each
(query chunk, visiting key/value chunk) pair -- causal on the diagonal
chunk, unmasked for an earlier chunk, skipped for a later one -- folded into
a running result with flash_attn_merge; then flash_attn_bwd on the same
pairs with the final O and LSE, whose per-pair gradients add up to the full
ones.  Compared with the float64 oracle's attention over the whole sequence.
The transfers between devices, and their overlap with compute, are what one
GPU cannot show."""

import numpy as np
import pytest

import oracle
from io_aware_tiled_attn_amd import workloads as wl
from tests.gpu_util import TOL, announce, max_err, to_f64, to_gpu, torch_cuda

pytestmark = pytest.mark.gpu


def fa():
    torch_cuda()
    import io_aware_tiled_attn_amd as pkg
    return pkg


def zigzag(P):
    return [[r, 2 * P - 1 - r] for r in range(P)]


def split(t, nc):
    c = t.shape[2] // nc
    return [t[:, :, i * c:(i + 1) * c].contiguous() for i in range(nc)]


def ring_forward(q, k, v, P, causal):
    torch = torch_cuda()
    nc = 2 * P
    qs, ks, vs = split(q, nc), split(k, nc), split(v, nc)
    out, lse = [None] * nc, [None] * nc
    pairs = []
    for dev in zigzag(P):
        n_pairs = 0
        for i in dev:
            o_acc = torch.zeros(qs[i].shape, dtype=torch.float32, device="cuda")
            l_acc = torch.full(qs[i].shape[:3], -float("inf"), dtype=torch.float32, device="cuda")
            o_out = torch.empty_like(qs[i])
            for step in range(nc):
                j = (i - step) % nc          # the chunk visiting at this step
                if causal and j > i:
                    continue
                o_p, l_p = fa().flash_attn_fwd(qs[i], ks[j], vs[j], causal=causal and j == i)
                fa().flash_attn_merge(o_acc, l_acc, o_p, l_p, out=o_out)
                n_pairs += 1
            out[i], lse[i] = o_out, l_acc
        pairs.append(n_pairs)
    return torch.cat(out, dim=2), torch.cat(lse, dim=2), pairs


def ring_backward(q, k, v, o, lse, do, P, causal):
    torch = torch_cuda()
    nc = 2 * P
    qs, ks, vs, os_, ls, dos = (split(t, nc) for t in (q, k, v, o, lse[..., None], do))
    ls = [t[..., 0].contiguous() for t in ls]
    dq = [torch.zeros(t.shape, dtype=torch.float32, device="cuda") for t in qs]
    dk = [torch.zeros(t.shape, dtype=torch.float32, device="cuda") for t in ks]
    dv = [torch.zeros(t.shape, dtype=torch.float32, device="cuda") for t in vs]
    for dev in zigzag(P):
        for i in dev:
            for j in range(nc):
                if causal and j > i:
                    continue
                gq, gk, gv = fa().flash_attn_bwd(qs[i], ks[j], vs[j], os_[i], ls[i], dos[i], causal=causal and j == i)
                dq[i] += gq.float()
                dk[j] += gk.float()
                dv[j] += gv.float()
    return (torch.cat(t, dim=2) for t in (dq, dk, dv))


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("P,N,d", [(2, 512, 64), (4, 1024, 128)])
def test_ring_forward_and_backward(P, N, d, causal):
    torch = torch_cuda()
    B, H = 1, 2
    announce(f"ring P={P} N={N} d={d} causal={causal}")
    inp = wl.make_inputs((B, H, N, d), 30000 + P + N + d, "bf16", with_grad=True)
    q, k, v, do = (to_gpu(inp[n], "bf16") for n in ("q", "k", "v", "do"))
    o, lse, pairs = ring_forward(q, k, v, P, causal)
    if causal:   # zig-zag: every device does the same number of chunk pairs
        assert len(set(pairs)) == 1, pairs
    dq, dk, dv = ring_backward(q, k, v, o, lse, do, P, causal)
    torch.cuda.synchronize()
    errs = {"o": 0.0, "lse": 0.0, "dq": 0.0, "dk": 0.0, "dv": 0.0}
    for h in range(H):
        qh, kh, vh, doh = (wl.values(inp[n][0, h], "bf16").astype(np.float64) for n in ("q", "k", "v", "do"))
        ro, rl = oracle.attention_forward_head(qh, kh, vh, causal=causal)
        rdq, rdk, rdv, _ = oracle.attention_backward_head(qh, kh, vh, doh, causal=causal)
        for name, got, ref in (("o", o, ro), ("lse", lse, rl), ("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
            errs[name] = max(errs[name], max_err(to_f64(got[0, h]), ref))
    print("  max err " + " ".join(f"{n}={e:.3e}" for n, e in errs.items()), flush=True)
    assert errs["lse"] <= 1e-4
    for n in ("o", "dq", "dk", "dv"):
        assert errs[n] <= TOL["bf16"], n


def test_merge_of_two_halves_equals_whole():
    """Keys split in two halves: merging the two partial results gives the
    forward over all keys (non-causal), and merging into an empty running
    result returns the part unchanged."""
    torch = torch_cuda()
    B, H, N, d = 2, 3, 384, 128
    announce("merge of two key halves")
    inp = wl.make_inputs((B, H, N, d), 30100, "bf16")
    q, k, v = (to_gpu(inp[n], "bf16") for n in ("q", "k", "v"))
    o_full, l_full = fa().flash_attn_fwd(q, k, v)
    # Queries attend to each half of the keys: pad each half into a square
    # problem would change N, so use the decoding form (Nq <= Nk).
    half = N // 2
    parts = []
    for lo in (0, half):
        kk, vv = k[:, :, lo:lo + half].contiguous(), v[:, :, lo:lo + half].contiguous()
        o_h = torch.empty_like(q)
        l_h = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        for c0 in range(0, N, 16):   # decoding takes up to 16 queries per head
            qq = q[:, :, c0:c0 + 16].contiguous()
            oo, ll = fa().flash_attn_decode(qq, kk, vv)
            o_h[:, :, c0:c0 + 16] = oo
            l_h[:, :, c0:c0 + 16] = ll
        parts.append((o_h, l_h))
    o_acc = torch.zeros(q.shape, dtype=torch.float32, device="cuda")
    l_acc = torch.full((B, H, N), -float("inf"), dtype=torch.float32, device="cuda")
    out = torch.empty_like(q)
    fa().flash_attn_merge(o_acc, l_acc, parts[0][0], parts[0][1], out=out)
    torch.cuda.synchronize()
    assert torch.equal(out, parts[0][0])                      # empty + part = part
    np.testing.assert_array_equal(l_acc.cpu().numpy(), parts[0][1].cpu().numpy())
    fa().flash_attn_merge(o_acc, l_acc, parts[1][0], parts[1][1], out=out)
    torch.cuda.synchronize()
    e_o = max_err(to_f64(out), to_f64(o_full))
    e_l = max_err(to_f64(l_acc), to_f64(l_full))
    print(f"  merged vs whole: O {e_o:.3e} LSE {e_l:.3e}", flush=True)
    assert e_o <= TOL["bf16"] and e_l <= 1e-4
