"""The pages' block-by-block update rule, in float64, for tests only.

This is not the parity target (that is oracle.attention, the plain
definition).  It exists so the tests can check the pages' own claims about
the tiled method: that streaming a row in blocks of any size gives the safe
softmax of the whole row, and that the tiled attention output equals the
standard one.

The update rule (vibeengines.com "FlashAttention, explained", section "The
math, worked with real numbers"), applied per query row as each key block
arrives:
    m_new = max(m_old, max of the block's scores)
    l_new = l_old * exp(m_old - m_new) + sum over the block of exp(s - m_new)
    O_new = O_old * exp(m_old - m_new) + sum over the block of exp(s - m_new) V
and the result is O / l after the last block; the running state starts
empty (m = -inf, l = 0, O = 0).

Written here as a merge of two partial states.  A block is first summarised
on its own, (m_b, l_b, O_b) with l_b and O_b taken against the block's own
max m_b; folding it into the running state (m, l, O) gives
    m' = max(m, m_b),  l' = l e^(m - m') + l_b e^(m_b - m'),
    O' = O e^(m - m') + O_b e^(m_b - m'),
which is the rule above, since e^(m_b - m') sum e^(s - m_b) = sum e^(s - m').
A side whose max is -inf (nothing seen yet, or a block whose scores are all
masked) holds l = 0 and O = 0 and contributes nothing; its factor is taken
as 0 rather than evaluating e^(-inf + inf) (reading of the pages: their
rule leaves that case open).
"""

import math

import numpy as np


def _fold_weight(m_side, m_new):
    """e^(m_side - m_new), elementwise, with 0 where m_side is -inf."""
    m_side = np.asarray(m_side, np.float64)
    m_new = np.asarray(m_new, np.float64)
    safe_new = np.where(np.isfinite(m_new), m_new, 0.0)
    return np.where(np.isfinite(m_side), np.exp(np.where(np.isfinite(m_side), m_side, 0.0) - safe_new), 0.0)


def merge_states(a, b):
    """Fold partial state b = (m_b, l_b[, O_b]) into a = (m, l[, O]); arrays
    broadcast over rows (O with one more trailing axis).  Returns the merged
    state as a tuple of the same length."""
    m = np.maximum(a[0], b[0])
    wa, wb = _fold_weight(a[0], m), _fold_weight(b[0], m)
    out = [m, a[1] * wa + b[1] * wb]
    if len(a) > 2:
        out.append(a[2] * np.asarray(wa)[..., None] + b[2] * np.asarray(wb)[..., None])
    return tuple(out)


def block_state(scores, values=None):
    """Summary of one key block for each row: its max m_b, l_b = sum of
    exp(s - m_b) and, with values, O_b = sum of exp(s - m_b) V.
    scores: [rows, n] (masked entries -inf); values: [n, dv]."""
    s = np.asarray(scores, np.float64)
    m_b = np.max(s, axis=-1)
    w = np.exp(s - np.where(np.isfinite(m_b), m_b, 0.0)[..., None])
    w = np.where(np.isfinite(s), w, 0.0)
    state = (m_b, np.sum(w, axis=-1))
    if values is not None:
        state = state + (w @ np.asarray(values, np.float64),)
    return state


def blockwise_softmax(row, block=2):
    """Softmax of one row computed by streaming it in blocks of `block`.

    Returns (weights, m, l, trace) where trace lists (m, l) after each
    block, as the page's worked example prints them.
    """
    if block < 1:
        raise ValueError("block must be >= 1")
    s = np.asarray([float(x) for x in row], np.float64)
    state = (np.float64(-np.inf), np.float64(0.0))
    trace = []
    for lo in range(0, s.size, block):
        state = merge_states(state, block_state(s[lo:lo + block]))
        trace.append((float(state[0]), float(state[1])))
    m, l = float(state[0]), float(state[1])
    weights = [math.exp(x - m) / l if x != -math.inf else 0.0 for x in s]
    return weights, m, l, trace


def tiled_attention(q, k, v, block=2, scale=None, causal=False):
    """Attention for one head with the keys walked in blocks of `block`, all
    query rows at once, each block folded into the running (m, l, O) by the
    update rule.

    q: [Nq, d], k: [Nk, d], v: [Nk, dv].  Returns (O, LSE) in float64; a row
    that sees no key gets O = 0 and LSE = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[1])
    n_q, n_k = q.shape[0], k.shape[0]
    rows = np.arange(n_q)[:, None]
    state = (np.full(n_q, -np.inf), np.zeros(n_q), np.zeros((n_q, v.shape[1])))
    for lo in range(0, n_k, block):
        hi = min(lo + block, n_k)
        s = scale * (q @ k[lo:hi].T)
        if causal:
            s = np.where(np.arange(lo, hi)[None, :] > rows, -np.inf, s)
        state = merge_states(state, block_state(s, v[lo:hi]))
    m, l, acc = state
    seen = l > 0.0
    out = np.where(seen[:, None], acc / np.where(seen, l, 1.0)[:, None], 0.0)
    lse = np.where(seen, m + np.log(np.where(seen, l, 1.0)), -np.inf)
    return out, lse
