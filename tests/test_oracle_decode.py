"""Pins for the oracle's decoding form (Nq new queries against an Nk-entry
key/value cache; reading in oracle/attention.py): prefill consistency, the
unshifted causal rule at Nq = Nk, scalar brute force, and torch's masked
attention."""

import math

import numpy as np
import pytest
import torch

from oracle import attention_decode_head, attention_forward_head


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", [(1, 1), (1, 9), (3, 9), (16, 40), (8, 8)])
def test_decode_equals_last_rows_of_full_attention(nq, nk, causal):
    """Decoding the last nq queries equals the last nq rows of attention over
    all nk positions (the prefill of the same sequence)."""
    rng = np.random.default_rng(400 + nq * 10 + nk)
    q = rng.standard_normal((nk, 8))
    k, v = rng.standard_normal((nk, 8)), rng.standard_normal((nk, 5))
    o, lse = attention_decode_head(q[nk - nq:], k, v, scale=0.4, causal=causal)
    fo, flse = attention_forward_head(q, k, v, scale=0.4, causal=causal)
    np.testing.assert_allclose(o, fo[nk - nq:], atol=1e-14)
    np.testing.assert_allclose(lse, flse[nk - nq:], atol=1e-14)


def test_decode_brute_force():
    rng = np.random.default_rng(410)
    nq, nk, d = 3, 7, 4
    q, k, v = rng.standard_normal((nq, d)), rng.standard_normal((nk, d)), rng.standard_normal((nk, 2))
    for causal in (False, True):
        o, lse = attention_decode_head(q, k, v, scale=0.9, causal=causal)
        for i in range(nq):
            keys = [j for j in range(nk) if not (causal and j > nk - nq + i)]
            sc = [0.9 * sum(q[i, c] * k[j, c] for c in range(d)) for j in keys]
            m = max(sc)
            tot = sum(math.exp(x - m) for x in sc)
            ref = [sum(math.exp(x - m) / tot * v[j, c] for x, j in zip(sc, keys)) for c in range(2)]
            assert abs(lse[i] - (m + math.log(tot))) < 1e-13
            assert np.allclose(o[i], ref, atol=1e-13)


def test_decode_matches_torch_masked_attention():
    rng = np.random.default_rng(411)
    nq, nk, d = 5, 23, 8
    q, k, v = rng.standard_normal((nq, d)), rng.standard_normal((nk, d)), rng.standard_normal((nk, d))
    o, lse = attention_decode_head(q, k, v, scale=0.3, causal=True)
    allowed = np.arange(nk)[None, :] <= (nk - nq + np.arange(nq))[:, None]
    to = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k),
                                                          torch.from_numpy(v), attn_mask=torch.from_numpy(allowed),
                                                          scale=0.3)
    s = 0.3 * (torch.from_numpy(q) @ torch.from_numpy(k).T)
    tlse = torch.logsumexp(s.masked_fill(~torch.from_numpy(allowed), -math.inf), dim=-1)
    np.testing.assert_allclose(o, to.numpy(), atol=1e-12)
    np.testing.assert_allclose(lse, tlse.numpy(), atol=1e-12)
