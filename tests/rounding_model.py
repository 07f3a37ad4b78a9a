"""A float64 model of where the bf16 path's rounding goes: the accuracy
budget of the forward and backward kernels, split by source.

Test infrastructure: it takes the exact reference from the oracle and
imports nothing from the product.  The kernels' arithmetic is written out
here in numpy with each rounding they take applied (round to nearest even)
and each one switchable on its own:
  forward  - S = scale q k^T, P = exp(S - m) against the row max, P rounded
             to bf16 for the P V product, l the sum of the unrounded P,
             O = (P V) / l, O rounded to bf16 on output;
  backward - D = rowsum(dO * O) from the saved bf16 O, P = exp(S - LSE),
             dP = dO V^T, dS = P (dP - D); P and dS rounded to fp16 for the
             dV, dK and dQ products (dS in the units the kernels hold it in:
             times the dO and V power-of-two factors), the gradients rounded
             to bf16 on output.
Not modelled: the fp16 copies of Q, K, V and dO (exact: a bf16 value times a
power of two), and the fp32 accumulation of the products (relative error
near 1e-7).  The lazy reference of the forward only changes the power of
two P is expressed against, which moves no rounding but the output's.

    python -m tests.rounding_model [N] [d] [heads]   # table at one shape
    python -m tests.rounding_model workload [heads]  # heads of the B4 H32 N4096
                                                     # d128 causal workload, picked
                                                     # as bench.py picks its sample
"""

import sys

import numpy as np

import oracle
from io_aware_tiled_attn_amd import workloads as wl


def round_bf16(x):
    """float64 -> nearest bfloat16 (ties to even), as float64."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    r = ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def round_fp16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def pow2_factor(amax):
    """The power of two that brings amax into [1, 2) (1 for 0)."""
    if not amax > 0:
        return 1.0
    return 2.0 ** (-np.floor(np.log2(amax)))


def _scores(q, k, scale, causal):
    s = scale * (q @ k.T)
    if causal:
        n = s.shape[0]
        s = np.where(np.tril(np.ones((n, n), dtype=bool)), s, -np.inf)
    return s


def forward(q, k, v, scale, causal, bf16_p=True, bf16_out=True):
    """(O, LSE) with the chosen roundings."""
    s = _scores(q, k, scale, causal)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1)
    o = (round_bf16(p) if bf16_p else p) @ v / l[:, None]
    lse = m[:, 0] + np.log(l)
    return (round_bf16(o) if bf16_out else o), lse


def backward(q, k, v, do, o_saved, lse, scale, causal, fp16_ps=True, bf16_out=True, ps_round=round_fp16):
    """(dQ, dK, dV) from the saved O and LSE with the chosen roundings
    (ps_round: how P and dS are rounded for the products when fp16_ps)."""
    d_row = (do * o_saved).sum(axis=1)
    p = np.exp(_scores(q, k, scale, causal) - lse[:, None])
    ds = p * (do @ v.T - d_row[:, None])
    if fp16_ps:
        f = pow2_factor(np.abs(do).max()) * pow2_factor(np.abs(v).max())
        p = ps_round(p)
        ds = ps_round(ds * f) / f
    dv = p.T @ do
    dk = scale * (ds.T @ q)
    dq = scale * (ds @ k)
    if bf16_out:
        dq, dk, dv = round_bf16(dq), round_bf16(dk), round_bf16(dv)
    return dq, dk, dv


SOURCES = ("P to bf16 in P V", "O to bf16", "D from the bf16 O", "P, dS to fp16", "gradients to bf16", "all")


def budget(q, k, v, do, scale, causal):
    """Max |error| against the exact result for O and for dQ, dK, dV, per
    source of rounding alone and for all of them together."""
    o_x, lse_x = oracle.attention_forward_head(q, k, v, scale=scale, causal=causal)
    grads_x = oracle.attention_backward_head(q, k, v, do, scale=scale, causal=causal)[:3]

    def err_o(o):
        return float(np.abs(o - o_x).max())

    def err_g(g):
        return [float(np.abs(a - b).max()) for a, b in zip(g, grads_x)]

    out = {}
    out["P to bf16 in P V"] = (err_o(forward(q, k, v, scale, causal, True, False)[0]), None)
    out["O to bf16"] = (err_o(round_bf16(o_x)), None)
    out["D from the bf16 O"] = (None, err_g(backward(q, k, v, do, round_bf16(o_x), lse_x, scale, causal, False, False)))
    out["P, dS to fp16"] = (None, err_g(backward(q, k, v, do, o_x, lse_x, scale, causal, True, False)))
    out["gradients to bf16"] = (None, err_g([round_bf16(g) for g in grads_x]))
    o_k, lse_k = forward(q, k, v, scale, causal)
    out["all"] = (err_o(o_k), err_g(backward(q, k, v, do, o_k, lse_k, scale, causal)))
    out["_largest"] = (float(np.abs(o_x).max()), [float(np.abs(g).max()) for g in grads_x])
    return out


def head_inputs(shape, seed, b, h):
    inp = wl.make_inputs(shape, seed, "bf16", with_grad=True)
    return [wl.values(inp[n][b, h], "bf16").astype(np.float64) for n in ("q", "k", "v", "do")]


def table(N=1024, d=128, heads=2, causal=True, seed=42, sample=None):
    """The per-source maxima over `heads` heads of seeded inputs, or over the
    given sample [(q, k, v, do), ...]."""
    lines = ["source                 |   O      |   dQ     |   dK     |   dV"]
    agg = {}
    if sample is None:
        sample = (head_inputs((1, heads, N, d), seed, 0, h) for h in range(heads))
    for qkvd in sample:
        r = budget(*qkvd, 1.0 / np.sqrt(qkvd[0].shape[1]), causal)
        for key in SOURCES + ("_largest",):
            eo, eg = r[key]
            prev = agg.get(key, (None, None))
            eo2 = None if eo is None else max(eo, prev[0] or 0.0)
            eg2 = None if eg is None else [max(a, b) for a, b in zip(eg, prev[1] or [0.0] * 3)]
            agg[key] = (eo2, eg2)
    for key in SOURCES + ("_largest",):
        eo, eg = agg[key]
        cells = ["%.2e" % eo if eo is not None else "   -    "] + (["%.2e" % x for x in eg] if eg else ["   -    "] * 3)
        lines.append("%-22s | %s" % (key if key != "_largest" else "largest |value|", " | ".join(cells)))
    return "\n".join(lines)


def workload_sample(heads=40, name="bf16_n4k_d128_causal"):
    """The heads bench.py compares on: every (B * H / heads)-th (b, h)."""
    w = wl.WORKLOADS[name]
    inp = wl.workload_inputs(name, with_grad=True)
    picks = [(b, h) for b in range(w.B) for h in range(w.H)][::max(1, (w.B * w.H) // heads)][:heads]
    for b, h in picks:
        yield [wl.values(inp[n][b, h], w.dtype).astype(np.float64) for n in ("q", "k", "v", "do")]


if __name__ == "__main__":
    if sys.argv[1:2] == ["workload"]:
        print(table(sample=workload_sample(*[int(a) for a in sys.argv[2:]])))
    else:
        print(table(*[int(a) for a in sys.argv[1:]]))
