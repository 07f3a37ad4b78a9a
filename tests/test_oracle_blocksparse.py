"""Pins for the oracle's block-sparse attention (a block mask over
(query block, key block) pairs; masked pairs get weight 0).

The pages name block-sparse FlashAttention as an approximate extension
(chorfi.xyz, "Main concepts to understand") without defining it; the reading
is the one stated in oracle/attention.py.  Each test ties the masked oracle to
something outside it: scalar brute force, the unmasked oracle on independent
sub-problems, torch's own masked attention and autograd, finite differences.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention_backward_head, attention_forward_head


def brute_masked(Q, K, V, scale, keep):
    """Scalar loops: row i attends to the keys j with keep(i, j)."""
    out, lses = [], []
    for i, q in enumerate(Q):
        scores = []
        for j, k in enumerate(K):
            if not keep(i, j):
                continue
            dot = 0.0
            for a, b in zip(q, k):
                dot += float(a) * float(b)
            scores.append((j, scale * dot))
        row = [0.0] * len(V[0])
        if not scores:
            out.append(row)
            lses.append(-math.inf)
            continue
        m = max(s for _, s in scores)
        total = sum(math.exp(s - m) for _, s in scores)
        for j, s in scores:
            w = math.exp(s - m) / total
            for c in range(len(row)):
                row[c] += w * float(V[j][c])
        out.append(row)
        lses.append(m + math.log(total))
    return np.array(out), np.array(lses)


def random_mask(rng, nqb, nkb, density=0.5):
    return (rng.random((nqb, nkb)) < density).astype(np.uint8)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,bq,bk,seed", [(5, 2, 2, 0), (7, 2, 3, 1), (8, 3, 2, 2), (6, 1, 4, 3)])
def test_block_mask_brute_force(n, bq, bk, seed, causal):
    rng = np.random.default_rng(300 + seed)
    q, k, v = (rng.standard_normal((n, 3)) * 1.5 for _ in range(3))
    mask = random_mask(rng, -(-n // bq), -(-n // bk))
    mask[0, 0] = 1 if seed % 2 else 0   # seeds 0 and 2 leave row block 0 possibly empty
    scale = 0.6
    o, lse = attention_forward_head(q, k, v, scale=scale, causal=causal, block_mask=mask, block=(bq, bk))

    def keep(i, j):
        return mask[i // bq, j // bk] != 0 and not (causal and j > i)

    bo, blse = brute_masked(q.tolist(), k.tolist(), v.tolist(), scale, keep)
    np.testing.assert_allclose(o, bo, rtol=0, atol=1e-13)
    np.testing.assert_array_equal(np.isinf(lse), np.isinf(blse))
    fin = np.isfinite(blse)
    np.testing.assert_allclose(lse[fin], blse[fin], rtol=0, atol=1e-13)


def test_full_mask_equals_dense():
    rng = np.random.default_rng(310)
    n, d = 300, 16
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    ones = np.ones((3, 3), dtype=np.uint8)
    for causal in (False, True):
        o0, l0 = attention_forward_head(q, k, v, causal=causal)
        o1, l1 = attention_forward_head(q, k, v, causal=causal, block_mask=ones)
        np.testing.assert_array_equal(o0, o1)
        np.testing.assert_array_equal(l0, l1)
        g0 = attention_backward_head(q, k, v, do, causal=causal)
        g1 = attention_backward_head(q, k, v, do, causal=causal, block_mask=ones)
        for a, b in zip(g0, g1):
            np.testing.assert_array_equal(a, b)


def test_block_diagonal_mask_is_independent_blocks():
    """With only diagonal blocks kept, each block is ordinary attention on its
    own rows and keys: the unmasked oracle on the sub-arrays is the answer."""
    rng = np.random.default_rng(311)
    n, d, blk = 300, 8, 128
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    nb = -(-n // blk)
    mask = np.eye(nb, dtype=np.uint8)
    o, lse = attention_forward_head(q, k, v, block_mask=mask, block=(blk, blk))
    dq, dk, dv, _ = attention_backward_head(q, k, v, do, block_mask=mask, block=(blk, blk))
    for b in range(nb):
        r = slice(b * blk, min(n, (b + 1) * blk))
        ob, lb = attention_forward_head(q[r], k[r], v[r])
        np.testing.assert_allclose(o[r], ob, atol=1e-13)
        np.testing.assert_allclose(lse[r], lb, atol=1e-13)
        gq, gk, gv, _ = attention_backward_head(q[r], k[r], v[r], do[r])
        np.testing.assert_allclose(dq[r], gq, atol=1e-13)
        np.testing.assert_allclose(dk[r], gk, atol=1e-13)
        np.testing.assert_allclose(dv[r], gv, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_block_mask_matches_torch_masked_attention(causal):
    """torch's masked scaled_dot_product_attention and its autograd, with the
    block mask expanded to an element mask (no row left empty)."""
    rng = np.random.default_rng(312)
    n, d, bq, bk = 40, 8, 8, 16
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    mask = random_mask(rng, n // bq, -(-n // bk))
    mask[:, 0] = 1   # every row keeps key block 0, which holds key 0
    scale = 0.5
    o, lse = attention_forward_head(q, k, v, scale=scale, causal=causal, block_mask=mask, block=(bq, bk))
    dq, dk, dv, _ = attention_backward_head(q, k, v, do, scale=scale, causal=causal, block_mask=mask,
                                            block=(bq, bk))
    allowed = mask[np.arange(n)[:, None] // bq, np.arange(n)[None, :] // bk] != 0
    if causal:
        allowed &= np.arange(n)[None, :] <= np.arange(n)[:, None]
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    ta = torch.from_numpy(allowed)
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=ta, scale=scale)
    to.backward(torch.from_numpy(do))
    s = scale * (tq.detach() @ tk.detach().T)
    tlse = torch.logsumexp(s.masked_fill(~ta, -math.inf), dim=-1)
    np.testing.assert_allclose(o, to.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(lse, tlse.numpy(), atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


def test_block_mask_finite_differences():
    rng = np.random.default_rng(313)
    n, d, bq, bk = 6, 3, 2, 3
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    mask = np.array([[1, 0], [0, 1], [1, 1]], dtype=np.uint8)
    scale = 0.7
    grads = attention_backward_head(q, k, v, do, scale=scale, block_mask=mask, block=(bq, bk))[:3]
    h = 1e-6
    for which, g in zip(range(3), grads):
        for i in range(n):
            for c in range(d):
                args = [q.copy(), k.copy(), v.copy()]
                args[which][i, c] += h
                fp = np.sum(attention_forward_head(*args, scale=scale, block_mask=mask, block=(bq, bk))[0] * do)
                args[which][i, c] -= 2 * h
                fm = np.sum(attention_forward_head(*args, scale=scale, block_mask=mask, block=(bq, bk))[0] * do)
                assert abs((fp - fm) / (2 * h) - g[i, c]) < 1e-7


def test_fully_masked_rows_are_zero_with_zero_gradients():
    rng = np.random.default_rng(314)
    n, d = 12, 4
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    mask = np.array([[0, 0, 0], [1, 0, 1], [0, 1, 0]], dtype=np.uint8)   # query block 0 sees nothing
    o, lse = attention_forward_head(q, k, v, block_mask=mask, block=(4, 4))
    dq, dk, dv, D = attention_backward_head(q, k, v, do, block_mask=mask, block=(4, 4))
    assert np.all(o[:4] == 0) and np.all(lse[:4] == -np.inf) and np.all(np.isfinite(lse[4:]))
    assert np.all(dq[:4] == 0) and np.all(D[:4] == 0)
    # Keys 4..7 (key block 1) are seen only by query block 2.
    dk2 = attention_backward_head(q[8:], k, v, do[8:], block_mask=mask[2:], block=(4, 4))[1]
    np.testing.assert_allclose(dk[4:8], dk2[4:8], atol=1e-13)
