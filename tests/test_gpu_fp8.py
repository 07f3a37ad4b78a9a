"""GPU parity of the FP8 (E4M3) forward with the float64 oracle, through the
C ABI.

The oracle is exact attention of the dequantized inputs.  The kernel rounds
the softmax weights to E4M3 before the P V product, so O is compared against
a bound derived from that rounding rather than a fixed number:
  * per element (rigorous): with p_ij the exact weights and l_i the row's
    sum of exp(s - max), the weight rounding moves O_ic by at most
    sum_j e_ij |V_jc|, e_ij = max(2^-4 p_ij, min(p_ij, 2^-10 / l_i)) (half an
    E4M3 step: 2^-4 relative in the normal range, 2^-10 absolute below
    2^-6, and the kernel's reference max never exceeds the true one); the
    FP8 product's accumulation (under 2^-13 of sum |q k| in the probes) adds
    up to 2^-9 p_ij |V_jc|; the bf16 output rounding 2^-8 |O_ic|.
  * in aggregate: the roundings are unbiased and independent, so the RMS
    error stays within twice the predicted sqrt(sum_j (2^-4 p_ij V_jc)^2 / 3)
    (plus the bf16 output term), and the regression slope of the error on O
    stays near 0 (a wrong descale would show there).
  * LSE: only the score product's accumulation reaches it:
    |dLSE_i| <= 2^-12 max_j scale |q_i| . |k_j| + 1e-5.
"""

import numpy as np
import pytest

import oracle
from io_aware_tiled_attn_amd import workloads as wl
from tests import rescale_cases as rc
from tests.gpu_util import announce, to_f64, torch_cuda

pytestmark = pytest.mark.gpu


def fa():
    torch_cuda()
    import io_aware_tiled_attn_amd as pkg
    return pkg


def to_gpu_u8(a):
    torch = torch_cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def run(inp, causal, scale=None):
    q, k, v = (to_gpu_u8(inp[n]) for n in ("q", "k", "v"))
    o, lse = fa().flash_attn_fwd_fp8(q, k, v, inp["q_descale"], inp["k_descale"], inp["v_descale"],
                                     causal=causal, scale=scale)
    torch_cuda().cuda.synchronize()
    return to_f64(o), to_f64(lse)


def bounds(inp, b, h, causal, rows, scale=None):
    """Oracle O and LSE of the sampled rows, and their error bounds."""
    q8, k8, v8 = (inp[n][b, h] for n in ("q", "k", "v"))
    qd, kd, vd = inp["q_descale"], inp["k_descale"], inp["v_descale"]
    ro, rl = oracle.attention_forward_fp8_head(q8, k8, v8, qd, kd, vd, scale=scale, causal=causal, rows=rows)
    p = oracle.attention_weights_fp8_head(q8, k8, qd, kd, scale=scale, causal=causal, rows=rows)
    v = oracle.dequantize(v8, vd)
    l_row = 1.0 / p.max(axis=1)                        # sum of exp(s - max)
    e = np.maximum(2.0 ** -4 * p, np.minimum(p, 2.0 ** -10 / l_row[:, None]))
    bound_o = (e + 2.0 ** -9 * p) @ np.abs(v) + 2.0 ** -8 * np.abs(ro) + 1e-6
    sigma2 = (2.0 ** -8 / 3) * ((p ** 2) @ (v ** 2)) + (2.0 ** -18 / 3) * ro ** 2
    q = oracle.dequantize(q8, qd)[rows]
    k = oracle.dequantize(k8, kd)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[1])
    sabs = scale * (np.abs(q) @ np.abs(k).T)
    if causal:
        sabs = np.where(np.arange(k.shape[0])[None, :] > np.asarray(rows)[:, None], 0.0, sabs)
    bound_l = 2.0 ** -12 * sabs.max(axis=1) + 1e-5
    return ro, rl, bound_o, sigma2, bound_l


def check(inp, causal, o, lse, cases, scale=None, slope_check=True):
    errs, sig, prod, osq = [], [], 0.0, 0.0
    worst = 0.0
    for b, h, rows in cases:
        ro, rl, bo, s2, bl = bounds(inp, b, h, causal, rows, scale)
        go, gl = o[b, h][rows], lse[b, h][rows]
        assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl))
        err = go - ro
        worst = max(worst, float(np.max(np.abs(err) / bo)))
        assert np.all(np.abs(err) <= bo), f"O outside bound at head {(b, h)}: {np.max(np.abs(err) - bo):.3e}"
        assert np.all(np.abs(gl - rl) <= bl), f"LSE outside bound: {np.max(np.abs(gl - rl) - bl):.3e}"
        errs.append(err.ravel())
        sig.append(s2.ravel())
        prod += float(np.sum(err * ro))
        osq += float(np.sum(ro * ro))
    err = np.concatenate(errs)
    rms, rms_pred = float(np.sqrt(np.mean(err ** 2))), float(np.sqrt(np.mean(np.concatenate(sig))))
    slope = prod / osq if osq > 0 else 0.0
    print(f"  max |err|/bound={worst:.3f} rms={rms:.3e} predicted={rms_pred:.3e} slope={slope:.2e}", flush=True)
    assert rms <= 2.0 * rms_pred + 1e-7
    if slope_check:
        assert abs(slope) <= 5e-3


def all_rows(B, H, N):
    return [(b, h, np.arange(N)) for b in range(B) for h in range(H)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 63, 64, 65, 300, 1000])
def test_fp8_forward_small(N, d, causal):
    B, H = 2, 2
    announce(f"fp8 forward B{B} H{H} N={N} d={d} causal={causal}")
    inp = wl.fp8_inputs((B, H, N, d), 9000 + N + d)
    o, lse = run(inp, causal)
    check(inp, causal, o, lse, all_rows(B, H, N), slope_check=N * d * B * H >= 32768)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [383, 384, 385, 800])
def test_fp8_forward_around_query_tiles(N, causal):
    # d = 128 takes 384 queries per workgroup (three wave groups): N just
    # below, at and past one tile, and a second tile whose last waves lie
    # wholly past N, so they run no products.
    B, H, d = 1, 3, 128
    announce(f"fp8 forward B{B} H{H} N={N} d={d} causal={causal}")
    inp = wl.fp8_inputs((B, H, N, d), 9500 + N)
    o, lse = run(inp, causal)
    check(inp, causal, o, lse, all_rows(B, H, N), slope_check=True)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_forward_descales_and_scale(causal):
    """Descales far from 1 and an explicit softmax scale: all three fold into
    the kernel's factors."""
    B, H, N, d = 1, 3, 517, 128
    announce(f"fp8 forward descales N={N} causal={causal}")
    inp = wl.fp8_inputs((B, H, N, d), 9100)
    inp["q_descale"] *= 37.0
    inp["k_descale"] /= 11.0
    inp["v_descale"] *= 1000.0
    o, lse = run(inp, causal, scale=0.05)
    check(inp, causal, o, lse, all_rows(B, H, N), scale=0.05)


def test_fp8_forward_zero_queries():
    """All-zero Q codes: every visible key gets the same weight, so O is the
    running mean of V (causal) and LSE = ln(i + 1)."""
    B, H, N, d = 1, 2, 333, 64
    announce("fp8 forward zero queries")
    inp = wl.fp8_inputs((B, H, N, d), 9200)
    inp["q"] = np.zeros_like(inp["q"])
    o, lse = run(inp, True)
    check(inp, True, o, lse, all_rows(B, H, N))
    np.testing.assert_allclose(lse[0, 0], np.log(np.arange(1, N + 1)), atol=2e-6)


def test_fp8_forward_matches_bf16_path_on_shared_values():
    """Inputs whose values are exact in both E4M3 and bf16: the FP8 and
    bf16 forwards compute the same attention; their outputs differ only by
    the weights' rounding (E4M3 vs bf16), within the FP8 bound."""
    torch = torch_cuda()
    B, H, N, d = 1, 2, 700, 128
    announce("fp8 vs bf16 forward, shared values")
    inp = wl.fp8_inputs((B, H, N, d), 9300)
    # Power-of-two descales: code values times 2^k are exact in bf16.
    inp.update(q_descale=2.0 ** -8, k_descale=2.0 ** -7, v_descale=2.0 ** -6)
    vals = {n: oracle.dequantize(inp[n], inp[n + "_descale"]).astype(np.float32) for n in ("q", "k", "v")}
    o8, l8 = run(inp, True)
    bf = {n: torch.from_numpy(vals[n]).to(torch.bfloat16).cuda() for n in vals}
    for n in vals:   # the dequantized values must be exact in bf16 for the comparison to mean anything
        assert np.array_equal(bf[n].float().cpu().numpy(), vals[n])
    ob, lb = fa().flash_attn_fwd(bf["q"], bf["k"], bf["v"], causal=True)
    torch.cuda.synchronize()
    np.testing.assert_allclose(l8, to_f64(lb), atol=1e-3)
    check(inp, True, o8, l8, all_rows(B, H, N))


def test_fp8_forward_full_size_sampled():
    """The FP8 benchmark shape (B4 H32 N4096 d128 causal) in the launch
    configuration the benchmark times; sampled heads and rows against the
    oracle."""
    w = wl.FP8_WORKLOAD
    announce(f"fp8 forward full size {w.name}")
    inp = wl.fp8_inputs(w.shape, w.seed)
    o, lse = run(inp, w.causal)
    rng = np.random.default_rng(9400)
    rows = np.sort(np.concatenate([[0, 1, 255, 256, w.N - 1], rng.choice(w.N, 59, replace=False)]))
    cases = [(b, h, rows) for b, h in ((0, 0), (1, 7), (2, 19), (3, 31))]
    check(inp, w.causal, o, lse, cases)


@pytest.mark.parametrize("pattern", rc.PATTERNS)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_fp8_forward_live_rescale(d, causal, pattern):
    """Scores that climb across key tiles (tests/rescale_cases.py): the
    kernel raises its running max with l and O live (shown on the CPU by
    tests/test_rescale_model.py for these exact codes); "falling" is the
    control."""
    B, H, N = 1, 2, 520
    announce(f"fp8 forward climbing scores pattern={pattern} d={d} causal={causal}")
    inp = rc.climbing_fp8((B, H, N, d), 12, pattern)
    o, lse = run(inp, causal)
    check(inp, causal, o, lse, all_rows(B, H, N))


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_worked_example_across_tiles(d):
    """The page's worked example in two key tiles with exact E4M3 values
    (scores 6 * [2, 1, 3, 0] through the scale argument): O_0[0:4] are the
    weights, LSE_0 = 18 + ln of the sum of e^(6 s - 18)."""
    import math
    inp = rc.worked_across_tiles_fp8(d)
    announce(f"fp8 worked example across tiles d={d}")
    o, lse = run(inp, False, scale=rc.WORKED_SCALE)
    z = [math.exp(rc.WORKED_SCALE * s - 18.0) for s in rc.WORKED_SCORES]
    weights = np.array(z) / sum(z)
    # E4M3 rounding of P (2^-4 relative) and the bf16 output rounding.
    np.testing.assert_allclose(o[0, 0, 0, :4], weights, atol=2.0 ** -4 * weights.max() + 2.0 ** -9)
    assert abs(float(lse[0, 0, 0]) - (18.0 + math.log(sum(z)))) <= 1e-5
    check(inp, False, o, lse, [(0, 0, np.arange(rc.WORKED_N))], scale=rc.WORKED_SCALE, slope_check=False)


def test_fp8_forward_is_deterministic():
    """The kept FP8 kernel at the benchmark shape (B4 H32 N4096 d128 causal)
    gives bit-identical O and LSE over repeated calls: no call depends on
    the timing of the LDS copies or on the order the workgroups run in."""
    torch = torch_cuda()
    w = wl.FP8_WORKLOAD
    announce(f"fp8 forward determinism {w.name}")
    inp = wl.fp8_inputs(w.shape, w.seed)
    q, k, v = (to_gpu_u8(inp[n]) for n in ("q", "k", "v"))
    args = (inp["q_descale"], inp["k_descale"], inp["v_descale"])
    o1, l1 = fa().flash_attn_fwd_fp8(q, k, v, *args, causal=True)
    for _ in range(4):
        o2, l2 = fa().flash_attn_fwd_fp8(q, k, v, *args, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
