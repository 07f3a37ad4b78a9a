"""The pages' block-by-block update rule, in float64, for tests only.

This is not the parity target (that is oracle.attention, the plain
definition).  It exists so the tests can check the pages' own claims about
the tiled method: that streaming a row in blocks of any size gives the safe
softmax of the whole row, and that the tiled attention output equals the
standard one.

Update rule (vibeengines.com "FlashAttention, explained", section "The math,
worked with real numbers"), applied per query row as each key block arrives:
    m_new = max(m_old, max of the block's scores)
    l_new = l_old * exp(m_old - m_new) + sum over the block of exp(s - m_new)
    O_new = O_old * exp(m_old - m_new) + sum over the block of exp(s - m_new) V
and the result is O / l after the last block.  The running state starts at
m = -inf, l = 0, O = 0 (same page, section "Solve it yourself").

Reading: when every score seen so far is -inf (a fully masked block at the
start of a row), exp(m_old - m_new) would be exp(-inf + inf); the correction
factor is taken as 0 there, since l_old and O_old are still 0.
"""

import math

import numpy as np


def _correction(m_old, m_new):
    if m_old == -math.inf:
        return 0.0
    return math.exp(m_old - m_new)


def online_softmax(row, block=2):
    """Softmax of one row computed by streaming it in blocks of `block`.

    Returns (weights, m, l, trace) where trace lists (m, l) after each block.
    """
    row = [float(x) for x in row]
    if block < 1:
        raise ValueError("block must be >= 1")
    m, l = -math.inf, 0.0
    trace = []
    for start in range(0, len(row), block):
        part = row[start:start + block]
        m_new = max(m, max(part))
        if m_new == -math.inf:
            trace.append((m, l))
            continue
        l = l * _correction(m, m_new) + sum(math.exp(s - m_new) for s in part)
        m = m_new
        trace.append((m, l))
    weights = [math.exp(s - m) / l if s != -math.inf else 0.0 for s in row]
    return weights, m, l, trace


def tiled_attention(q, k, v, block=2, scale=None, causal=False):
    """Attention for one head, walking the keys in blocks of `block` and
    carrying (m, l, O) per query row with the update rule above.

    q: [Nq, d], k: [Nk, d], v: [Nk, dv].  Returns (O, LSE) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[1])
    n_q, n_k = q.shape[0], k.shape[0]
    out = np.zeros((n_q, v.shape[1]), dtype=np.float64)
    lse = np.full(n_q, -np.inf, dtype=np.float64)
    for i in range(n_q):
        m, l = -math.inf, 0.0
        acc = np.zeros(v.shape[1], dtype=np.float64)
        for j0 in range(0, n_k, block):
            j1 = min(j0 + block, n_k)
            s = scale * (k[j0:j1] @ q[i])
            if causal:
                s = np.where(np.arange(j0, j1) > i, -np.inf, s)
            m_new = max(m, float(np.max(s)))
            if m_new == -math.inf:
                continue
            alpha = _correction(m, m_new)
            w = np.exp(s - m_new)
            l = l * alpha + float(np.sum(w))
            acc = acc * alpha + w @ v[j0:j1]
            m = m_new
        if l > 0.0:
            out[i] = acc / l
            lse[i] = m + math.log(l)
    return out, lse
