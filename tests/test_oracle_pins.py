"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each test ties the oracle to a fact fixed outside it: values printed on the
pages' worked example, closed forms, pure-Python brute force, finite
differences, invariants of the softmax, and an independent library
implementation (torch's CPU float64 attention and autograd).  Between them a
dropped term, a wrong sign, an off-by-one in the causal mask, a transposed
operand or a missing scale factor fails at least one test
(test_oracle_mutants.py plants such mistakes and checks that).
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import (attention_backward, attention_backward_head,
                    attention_forward, attention_forward_head, blockwise_softmax,
                    safe_softmax, tiled_attention)


def _golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# Brute force: the definition as scalar Python loops, no numpy arithmetic.
# ---------------------------------------------------------------------------

def brute_attention(Q, K, V, scale, causal):
    out, lses = [], []
    for i, q in enumerate(Q):
        scores = []
        for j, k in enumerate(K):
            if causal and j > i:
                continue
            dot = 0.0
            for a, b in zip(q, k):
                dot += float(a) * float(b)
            scores.append((j, scale * dot))
        m = max(s for _, s in scores)
        total = 0.0
        for _, s in scores:
            total += math.exp(s - m)
        row = [0.0] * len(V[0])
        for j, s in scores:
            w = math.exp(s - m) / total
            for c in range(len(row)):
                row[c] += w * float(V[j][c])
        out.append(row)
        lses.append(m + math.log(total))
    return np.array(out), np.array(lses)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d,dv,seed", [(1, 1, 1, 0), (3, 2, 2, 1), (5, 4, 3, 2),
                                         (8, 3, 4, 3), (7, 4, 1, 4)])
def test_brute_force_tiny(n, d, dv, seed, causal):
    rng = np.random.default_rng(100 + seed)
    q = rng.standard_normal((n, d)) * 2
    k = rng.standard_normal((n, d)) * 2
    v = rng.standard_normal((n, dv))
    scale = 0.37 + seed * 0.1
    o, lse = attention_forward_head(q, k, v, scale=scale, causal=causal)
    bo, blse = brute_attention(q.tolist(), k.tolist(), v.tolist(), scale, causal)
    np.testing.assert_allclose(o, bo, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, blse, rtol=0, atol=1e-13)


def test_brute_force_rectangular_noncausal():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((3, 4))
    k = rng.standard_normal((6, 4))
    v = rng.standard_normal((6, 5))
    o, lse = attention_forward_head(q, k, v, scale=0.5)
    bo, blse = brute_attention(q.tolist(), k.tolist(), v.tolist(), 0.5, False)
    np.testing.assert_allclose(o, bo, atol=1e-13)
    np.testing.assert_allclose(lse, blse, atol=1e-13)


def test_default_scale_is_inverse_sqrt_d():
    rng = np.random.default_rng(8)
    q, k, v = (rng.standard_normal((4, 9)) for _ in range(3))
    o, lse = attention_forward_head(q, k, v)
    bo, blse = brute_attention(q.tolist(), k.tolist(), v.tolist(), 1.0 / 3.0, False)
    np.testing.assert_allclose(o, bo, atol=1e-13)
    np.testing.assert_allclose(lse, blse, atol=1e-13)


# ---------------------------------------------------------------------------
# The pages' worked example (vibeengines.com, "The math, worked with real
# numbers"): row [2, 1, 3, 0] in two blocks.
# ---------------------------------------------------------------------------

def test_worked_example_safe_softmax(golden_dir):
    g = _golden(golden_dir, "worked_example.json")
    w, m, l = safe_softmax(g["row"])
    half_ulp = 0.5 * 10.0 ** -g["printed_decimals"]
    assert m == g["after_block_2"]["m"]
    assert abs(l - g["after_block_2"]["l"]) <= half_ulp
    np.testing.assert_allclose(w, g["weights"], rtol=0, atol=half_ulp)


def test_worked_example_online_trace(golden_dir):
    g = _golden(golden_dir, "worked_example.json")
    half_ulp = 0.5 * 10.0 ** -g["printed_decimals"]
    w, m, l, trace = blockwise_softmax(g["row"], block=g["block"])
    (m1, l1), (m2, l2) = trace
    assert m1 == g["after_block_1"]["m"]
    assert abs(l1 - g["after_block_1"]["l"]) <= half_ulp
    # The page rounds 1.3679 * e^(2-3) to 0.5033 (exact: 0.50322).
    assert abs(l1 * math.exp(m1 - m2) - g["rescaled_l_before_block_2"]) <= 1.5e-4
    assert m2 == g["after_block_2"]["m"]
    assert abs(l2 - g["after_block_2"]["l"]) <= half_ulp
    np.testing.assert_allclose(w, g["weights"], atol=half_ulp)


def test_worked_example_through_attention(golden_dir):
    """Embed the row as scores: q_0 = e_0, k_j = s_j e_0, V = identity,
    scale 1.  Row 0 of O is then the softmax weights and LSE_0 = m + ln l."""
    g = _golden(golden_dir, "worked_example.json")
    s = np.array(g["row"])
    n = len(s)
    q = np.zeros((n, n)); q[0, 0] = 1.0
    k = np.zeros((n, n)); k[:, 0] = s
    v = np.eye(n)
    o, lse = attention_forward_head(q, k, v, scale=1.0)
    half_ulp = 0.5 * 10.0 ** -g["printed_decimals"]
    np.testing.assert_allclose(o[0], g["weights"], atol=half_ulp)
    l_page = g["after_block_2"]["l"]
    assert abs(lse[0] - (g["after_block_2"]["m"] + math.log(l_page))) <= half_ulp / l_page + 1e-12
    # Full-precision closed form of the same sum: e^-1 + e^-2 + e^0 + e^-3.
    assert abs(lse[0] - (3.0 + math.log(math.exp(-1) + math.exp(-2) + 1 + math.exp(-3)))) < 1e-14


# ---------------------------------------------------------------------------
# The pages' five assertions ("Solve it yourself"), on the float64 tiled
# reference and the oracle.
# ---------------------------------------------------------------------------

def _toy(golden_dir):
    g = _golden(golden_dir, "toy_example.json")
    return (np.array(g["Q"], float), np.array(g["K"], float),
            np.array(g["V"], float), g)


def test_assertion_online_equals_naive():
    rng = np.random.default_rng(11)
    for n in (1, 2, 5, 17):
        row = list(rng.standard_normal(n) * 3)
        w_naive, m, l = safe_softmax(row)
        for block in (1, 2, 3, n):
            w_on, m_on, l_on, _ = blockwise_softmax(row, block)
            np.testing.assert_allclose(w_on, w_naive, atol=1e-15)
            assert m_on == m
            assert abs(l_on - l) < 1e-13


@pytest.mark.parametrize("block", [1, 2, 3, 4])
def test_assertion_block_size_never_changes_answer(golden_dir, block):
    q, k, v, g = _toy(golden_dir)
    ref, ref_lse = tiled_attention(q, k, v, block=g["block"])
    o, lse = tiled_attention(q, k, v, block=block)
    assert np.max(np.abs(o - ref)) < 1e-14
    assert np.max(np.abs(lse - ref_lse)) < 1e-14


def test_assertion_flash_equals_standard_toy(golden_dir):
    q, k, v, g = _toy(golden_dir)
    std, std_lse = attention_forward_head(q, k, v)
    bo, blse = brute_attention(q.tolist(), k.tolist(), v.tolist(), 1 / math.sqrt(2), False)
    np.testing.assert_allclose(std, bo, atol=1e-14)
    for block in [g["block"]] + g["other_blocks"]:
        fl, fl_lse = tiled_attention(q, k, v, block=block)
        # The page reports a max difference of order 1e-16.
        assert np.max(np.abs(fl - std)) < 100 * g["max_difference_order"]
        assert np.max(np.abs(fl_lse - std_lse)) < 100 * g["max_difference_order"]


@pytest.mark.parametrize("causal", [False, True])
def test_assertion_flash_equals_standard_random(causal):
    rng = np.random.default_rng(12)
    q, k, v = (rng.standard_normal((37, 8)) for _ in range(3))
    std, std_lse = attention_forward_head(q, k, v, causal=causal)
    for block in (1, 5, 16, 37):
        fl, fl_lse = tiled_attention(q, k, v, block=block, causal=causal)
        assert np.max(np.abs(fl - std)) < 1e-13
        assert np.max(np.abs(fl_lse - std_lse)) < 1e-13


def test_assertion_valid_distribution():
    rng = np.random.default_rng(13)
    row = list(rng.standard_normal(23) * 5)
    for block in (1, 4, 23):
        w, _, _, _ = blockwise_softmax(row, block)
        assert abs(sum(w) - 1.0) < 1e-14
        assert min(w) > 0.0


def test_rows_of_p_sum_to_one_through_values():
    """V = 1 gives O = 1 when every row has probabilities summing to 1."""
    rng = np.random.default_rng(14)
    for causal in (False, True):
        q = rng.standard_normal((2, 3, 40, 16)) * 3
        k = rng.standard_normal((2, 3, 40, 16)) * 3
        v = np.ones((2, 3, 40, 5))
        o, _ = attention_forward(q, k, v, causal=causal)
        assert np.max(np.abs(o - 1.0)) < 1e-12


# ---------------------------------------------------------------------------
# Closed forms.
# ---------------------------------------------------------------------------

def test_zero_keys_give_uniform_average():
    rng = np.random.default_rng(15)
    n, d = 50, 8
    q = rng.standard_normal((n, d))
    k = np.zeros((n, d))
    v = rng.standard_normal((n, 3))
    o, lse = attention_forward_head(q, k, v)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(0), o.shape), atol=1e-13)
    np.testing.assert_allclose(lse, np.full(n, math.log(n)), atol=1e-13)
    oc, lsec = attention_forward_head(q, k, v, causal=True)
    cum = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    np.testing.assert_allclose(oc, cum, atol=1e-13)
    np.testing.assert_allclose(lsec, np.log(np.arange(1, n + 1)), atol=1e-13)


def test_single_key():
    q = np.array([[0.5, -2.0, 1.0]])
    k = np.array([[1.5, 0.25, -3.0]])
    v = np.array([[7.0, -1.0]])
    o, lse = attention_forward_head(q, k, v, scale=0.7)
    np.testing.assert_allclose(o, v, atol=1e-15)
    assert abs(lse[0] - 0.7 * float(q[0] @ k[0])) < 1e-15


def test_causal_row_zero_sees_only_key_zero():
    rng = np.random.default_rng(16)
    q, k, v = (rng.standard_normal((9, 4)) for _ in range(3))
    o, lse = attention_forward_head(q, k, v, scale=0.9, causal=True)
    np.testing.assert_allclose(o[0], v[0], atol=1e-15)
    assert abs(lse[0] - 0.9 * float(q[0] @ k[0])) < 1e-14


def test_key_shift_moves_only_lse():
    """k_j -> k_j + c shifts every score of row i by scale q_i.c: O is
    unchanged and LSE_i moves by exactly that amount, even for a shift so
    large that exp without the max subtraction would overflow."""
    rng = np.random.default_rng(17)
    q, k, v = (rng.standard_normal((12, 6)) for _ in range(3))
    c = rng.standard_normal(6) * 400.0
    for causal in (False, True):
        o1, l1 = attention_forward_head(q, k, v, causal=causal)
        o2, l2 = attention_forward_head(q, k + c, v, causal=causal)
        np.testing.assert_allclose(o2, o1, atol=1e-11)
        np.testing.assert_allclose(l2 - l1, (q @ c) / math.sqrt(6), atol=1e-9)


def test_permutation_equivariance():
    rng = np.random.default_rng(18)
    q, k, v = (rng.standard_normal((15, 5)) for _ in range(3))
    o, lse = attention_forward_head(q, k, v)
    pk = rng.permutation(15)
    o2, lse2 = attention_forward_head(q, k[pk], v[pk])
    np.testing.assert_allclose(o2, o, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, atol=1e-13)
    pq = rng.permutation(15)
    o3, lse3 = attention_forward_head(q[pq], k, v)
    np.testing.assert_allclose(o3, o[pq], atol=1e-13)
    np.testing.assert_allclose(lse3, lse[pq], atol=1e-13)


def test_row_selection_matches_full():
    rng = np.random.default_rng(19)
    q, k, v = (rng.standard_normal((1030, 8)) for _ in range(3))
    o, lse = attention_forward_head(q, k, v, causal=True)
    rows = np.array([0, 5, 511, 512, 513, 1029])
    o2, lse2 = attention_forward_head(q, k, v, causal=True, rows=rows)
    # BLAS may block the two products differently; rounding order only.
    np.testing.assert_allclose(o2, o[rows], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse2, lse[rows], rtol=0, atol=1e-14)


# ---------------------------------------------------------------------------
# Independent library: torch CPU float64 attention and autograd.
# ---------------------------------------------------------------------------

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("causal", [False, True])
def test_forward_matches_torch_sdpa(causal):
    rng = np.random.default_rng(20)
    shape = (2, 3, 37, 16)
    q, k, v = (rng.standard_normal(shape) for _ in range(3))
    scale = 0.3
    o, lse = attention_forward(q, k, v, scale=scale, causal=causal)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=causal, scale=scale)
    s = scale * torch.matmul(tq, tk.transpose(-1, -2))
    if causal:
        s = s.masked_fill(torch.ones(37, 37, dtype=torch.bool).triu(1), -math.inf)
    tlse = torch.logsumexp(s, dim=-1)
    np.testing.assert_allclose(o, to.numpy(), atol=1e-12)
    np.testing.assert_allclose(lse, tlse.numpy(), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_torch_autograd(causal):
    rng = np.random.default_rng(21)
    shape = (2, 2, 29, 8)
    q, k, v, do = (rng.standard_normal(shape) for _ in range(4))
    scale = 0.45
    dq, dk, dv = attention_backward(q, k, v, do, scale=scale, causal=causal)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=causal, scale=scale)
    to.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


# ---------------------------------------------------------------------------
# Backward: finite differences and invariants.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(1, 2), (4, 3), (6, 4)])
def test_backward_finite_differences(n, d, causal):
    rng = np.random.default_rng(200 + n * 10 + d)
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    scale = 0.8

    def f(qq, kk, vv):
        o, _ = attention_forward_head(qq, kk, vv, scale=scale, causal=causal)
        return float(np.sum(o * do))

    dq, dk, dv, _ = attention_backward_head(q, k, v, do, scale=scale, causal=causal)
    h = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        base = [q, k, v]
        num = np.zeros_like(grad)
        for idx in np.ndindex(*grad.shape):
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[which][idx] += h
            minus[which][idx] -= h
            num[idx] = (f(*plus) - f(*minus)) / (2 * h)
        np.testing.assert_allclose(grad, num, atol=1e-7)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_invariants(causal):
    rng = np.random.default_rng(22)
    n, d = 300, 16
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    dq, dk, dv, D = attention_backward_head(q, k, v, do, causal=causal)
    # Rows of dS sum to 0, so the key gradients sum to 0 for every feature.
    assert np.max(np.abs(dk.sum(0))) < 1e-10 * n
    # Rows of P sum to 1, so the value gradients sum to the output gradients.
    assert np.max(np.abs(dv.sum(0) - do.sum(0))) < 1e-10 * n
    o, _ = attention_forward_head(q, k, v, causal=causal)
    np.testing.assert_allclose(D, np.sum(do * o, axis=1), atol=1e-12)
    if causal:
        assert np.max(np.abs(dq[0])) < 1e-14


def test_oracle_exports():
    for name in ("attention_forward", "attention_backward", "safe_softmax",
                 "blockwise_softmax", "tiled_attention", "default_scale"):
        assert callable(getattr(oracle, name))
