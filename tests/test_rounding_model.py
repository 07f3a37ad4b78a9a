"""CPU checks of the accuracy budget (tests/rounding_model.py): the bf16
path's roundings, modelled in float64 against the oracle, fit the 2e-2
bound, and each source stays within the share the design gives it."""

import numpy as np

import oracle
from tests import rounding_model as rm

SHAPE = (1, 2, 512, 128)
SCALE = 1.0 / np.sqrt(128)


def _inputs(h):
    return rm.head_inputs(SHAPE, 7, 0, h)


def test_model_without_roundings_is_the_oracle():
    # The model's arithmetic is the same computation as the oracle's: with
    # every rounding off the two agree to float64 rounding.
    q, k, v, do = _inputs(0)
    o_x, lse_x = oracle.attention_forward_head(q, k, v, scale=SCALE, causal=True)
    g_x = oracle.attention_backward_head(q, k, v, do, scale=SCALE, causal=True)[:3]
    o, lse = rm.forward(q, k, v, SCALE, True, bf16_p=False, bf16_out=False)
    assert np.abs(o - o_x).max() < 1e-12 and np.abs(lse - lse_x).max() < 1e-12
    g = rm.backward(q, k, v, do, o, lse, SCALE, True, fp16_ps=False, bf16_out=False)
    for a, b in zip(g, g_x):
        assert np.abs(a - b).max() < 1e-11


def test_rounding_budget_fits_the_bound():
    for h in range(2):
        r = rm.budget(*_inputs(h), SCALE, True)
        o_all, g_all = r["all"]
        assert o_all <= 2e-2 and max(g_all) <= 2e-2, r
        # Each source's share: P to bf16 in P V and D from the bf16 O stay
        # well under the output rounding of values near 4; the fp16 P and dS
        # cost an order of magnitude less than either.
        assert r["P to bf16 in P V"][0] <= 4e-3
        assert max(r["D from the bf16 O"][1]) <= 1e-2
        assert max(r["P, dS to fp16"][1]) <= 1.5e-3
        largest = max(r["_largest"][1])
        assert max(r["gradients to bf16"][1]) <= largest * 2.0 ** -8


def test_fp16_p_and_ds_cost_less_than_bf16():
    # The reason the backward feeds fp16 P and dS: bf16 ones cost several
    # times more, a large part of the budget.
    q, k, v, do = _inputs(1)
    o_x, lse_x = oracle.attention_forward_head(q, k, v, scale=SCALE, causal=True)
    g_x = oracle.attention_backward_head(q, k, v, do, scale=SCALE, causal=True)[:3]

    def worst(ps_round):
        g = rm.backward(q, k, v, do, o_x, lse_x, SCALE, True, fp16_ps=True, bf16_out=False, ps_round=ps_round)
        return max(np.abs(a - b).max() for a, b in zip(g, g_x))

    assert worst(rm.round_bf16) >= 4 * worst(rm.round_fp16)


def test_rounding_helpers():
    # bf16: 8 significant bits, ties to even; fp16: 11.
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9, -2.5])
    assert list(rm.round_bf16(x)) == [1.0, 1.0, 1.0 + 2.0 ** -6, 1.0, -2.5]
    assert rm.round_fp16(1.0 + 2.0 ** -11) == 1.0 and rm.round_fp16(1.0 + 2.0 ** -10) == 1.0 + 2.0 ** -10
    assert rm.pow2_factor(4.9) == 0.25 and rm.pow2_factor(1.0) == 1.0 and rm.pow2_factor(0.0) == 1.0
