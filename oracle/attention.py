"""Plain float64 attention: the definition the GPU path must reproduce.

Test infrastructure only (tests, the smoke entry and the benchmark's CPU
baseline).  Nothing here is blocked, fused or reordered: every output row is
the textbook formula evaluated with numpy matmuls.

Sources (FlashAttention, Dao et al., NeurIPS 2022, as explained on three web
pages):
  * "FlashAttention, explained" (vibeengines.com), section "The math, worked
    with real numbers": safe softmax, softmax(s_i) = exp(s_i - m) / l with
    m the row maximum and l the sum of exp(s - m) over the row.
  * same page, section "Solve it yourself": standard attention divides each
    query-key dot product by sqrt(d) before the softmax, then takes the
    softmax-weighted sum of the value rows.
  * same page, section "Exact, not approximate", and the chorfi.xyz study
    guide, section "Guarantees versus empirical results": the tiled method
    returns exactly softmax(QK^T)V in exact arithmetic, so the plain
    definition is the parity target.

Readings where the pages are silent:
  * scale: s_ij = scale * (q_i . k_j), default scale = 1/sqrt(d), applied
    before the max and the exponential.
  * causal: the pages only mention "masking settings" (chorfi.xyz, "What to
    inspect in the evaluation").  Causal means key j > query i is masked
    (probability exactly 0), queries and keys aligned at index 0.
  * LSE: the per-row log-sum-exp of the scaled, masked scores, natural log:
    LSE_i = m_i + ln(l_i).  A row with every key masked (impossible for
    causal with N_q = N_k, kept for completeness) gets O = 0, LSE = -inf.
  * block-sparse attention: the pages name block-sparse FlashAttention as
    an approximate extension (chorfi.xyz, "Main concepts to understand"; its
    Path-256 result in vibeengines.com's table of headline numbers) without
    defining it.  Reading: a block mask over (query block, key block) pairs;
    the scores of every pair whose mask entry is 0 are -inf (weight 0), the
    rest is ordinary attention.  Rows left with no key get O = 0, LSE = -inf
    and zero gradients.
  * decoding with a key/value cache: the pages only ask which parts of the
    speed-up carry over to autoregressive decoding with a KV cache
    (chorfi.xyz, "Discussion prompts").  Reading: Nq new queries attend to
    an Nk-entry cache (Nq <= Nk); they are the cache's last Nq positions, so
    under the causal mask query i sees keys j <= Nk - Nq + i (the same rule
    as above, shifted by Nk - Nq); without it every query sees every key.
  * backward: the pages only say the backward pass recomputes attention
    instead of storing it (chorfi.xyz "Study objectives"; modelfieldguide.com
    "An IO-aware rewrite").  The gradients below are the calculus of the
    forward definition for an upstream gradient dO:
        dV = P^T dO,  dP = dO V^T,  D_i = sum_k dO_ik O_ik,
        dS = P * (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q.

Pins: tests/test_oracle_pins.py checks these functions against the pages'
worked example, closed forms, brute-force loops, finite differences and an
independent library implementation.
"""

import math

import numpy as np

# Rows of S evaluated at once in the forward pass.  Each output row depends
# only on its own score row, so evaluating rows in groups changes nothing
# about the arithmetic; it only bounds memory for long sequences.
_ROW_CHUNK = 512


def default_scale(d):
    """1/sqrt(d), the factor of the pages' standard attention ("Solve it
    yourself", vibeengines.com)."""
    return 1.0 / math.sqrt(d)


def safe_softmax(s):
    """Safe softmax of one score row (vibeengines.com, "The math, worked with
    real numbers"): subtract the row max m, exponentiate, divide by the sum l.

    Returns (weights, m, l) in float64.  Entries equal to -inf get weight 0.
    """
    s = np.asarray(s, dtype=np.float64)
    m = np.max(s)
    if m == -np.inf:
        return np.zeros_like(s), m, 0.0
    e = np.exp(s - m)
    l = float(np.sum(e))
    return e / l, float(m), l


def _causal_mask(row_idx, n_keys, offset=0):
    """True where key j > query i + offset (masked)."""
    j = np.arange(n_keys)[None, :]
    return j > np.asarray(row_idx)[:, None] + offset


def _block_masked(row_idx, n_keys, block_mask, block):
    """True where (query row, key) falls in a (query block, key block) pair
    whose block-mask entry is 0."""
    bq, bk = block
    bm = np.asarray(block_mask) != 0
    qb = np.asarray(row_idx) // bq
    kb = np.arange(n_keys) // bk
    return ~bm[qb][:, kb]


def attention_forward_head(q, k, v, scale=None, causal=False, rows=None, block_mask=None, block=(128, 128),
                           causal_offset=0):
    """Exact attention for one head.

    q: [Nq, d], k: [Nk, d], v: [Nk, dv], any real dtype (promoted to float64).
    rows: optional index array of query rows to evaluate (default: all).
    block_mask: optional [ceil(Nq/bq), ceil(Nk/bk)] array for block-sparse
    attention, block = (bq, bk); pairs whose entry is 0 are masked.
    causal_offset: under the causal mask, query i sees keys j <= i + offset.
    Returns (O [len(rows), dv], LSE [len(rows)]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if scale is None:
        scale = default_scale(q.shape[-1])
    if rows is None:
        rows = np.arange(q.shape[0])
    rows = np.asarray(rows, dtype=np.int64)
    n_keys = k.shape[0]
    out = np.zeros((rows.shape[0], v.shape[1]), dtype=np.float64)
    lse = np.full(rows.shape[0], -np.inf, dtype=np.float64)
    for c0 in range(0, rows.shape[0], _ROW_CHUNK):
        r = rows[c0:c0 + _ROW_CHUNK]
        s = scale * (q[r] @ k.T)                       # scores, [rows, Nk]
        if causal:
            s[_causal_mask(r, n_keys, causal_offset)] = -np.inf
        if block_mask is not None:
            s[_block_masked(r, n_keys, block_mask, block)] = -np.inf
        m = np.max(s, axis=1)                          # row max
        live = m > -np.inf
        m_safe = np.where(live, m, 0.0)
        e = np.exp(s - m_safe[:, None])                # exp(s - m); masked -> 0
        l = np.sum(e, axis=1)                          # row sum
        p = np.zeros_like(e)
        p[live] = e[live] / l[live, None]              # softmax weights
        out[c0:c0 + r.shape[0]] = p @ v                # weighted sum of values
        lse[c0:c0 + r.shape[0]][live] = m[live] + np.log(l[live])
    return out, lse


def attention_forward(q, k, v, scale=None, causal=False, block_mask=None, block=(128, 128)):
    """Exact attention over [B, H, N, d] arrays; returns (O, LSE) float64
    with shapes [B, H, N, dv] and [B, H, N].  block_mask, if given, is
    [B, H, ceil(N/bq), ceil(N/bk)]."""
    q = np.asarray(q)
    B, H, N, _ = q.shape
    out = np.zeros((B, H, N, v.shape[-1]), dtype=np.float64)
    lse = np.zeros((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            out[b, h], lse[b, h] = attention_forward_head(
                q[b, h], k[b, h], v[b, h], scale=scale, causal=causal,
                block_mask=None if block_mask is None else block_mask[b, h], block=block)
    return out, lse


def attention_backward_head(q, k, v, do, scale=None, causal=False, block_mask=None, block=(128, 128)):
    """Analytic gradients of O = softmax(scale * q k^T [masked]) v for one head.

    q: [N, d], k: [N, d], v: [N, dv], do: [N, dv]; block_mask as in
    attention_forward_head.
    Returns (dq, dk, dv, D) in float64, where D_i = sum_k dO_ik O_ik.
    The N x N matrices are formed whole; callers keep N moderate.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    if scale is None:
        scale = default_scale(q.shape[-1])
    n_q, n_k = q.shape[0], k.shape[0]
    s = scale * (q @ k.T)
    if causal:
        s[_causal_mask(np.arange(n_q), n_k)] = -np.inf
    if block_mask is not None:
        s[_block_masked(np.arange(n_q), n_k, block_mask, block)] = -np.inf
    m = np.max(s, axis=1)
    live = m > -np.inf
    m_safe = np.where(live, m, 0.0)
    e = np.exp(s - m_safe[:, None])
    l = np.sum(e, axis=1)
    p = np.zeros_like(e)
    p[live] = e[live] / l[live, None]
    o = p @ v
    dv = p.T @ do                                      # dV = P^T dO
    dp = do @ v.T                                      # dP = dO V^T
    D = np.sum(do * o, axis=1)                         # D_i = <dO_i, O_i>
    ds = p * (dp - D[:, None])                         # softmax Jacobian
    dq = scale * (ds @ k)                              # dQ = scale dS K
    dk = scale * (ds.T @ q)                            # dK = scale dS^T Q
    return dq, dk, dv, D


def attention_backward(q, k, v, do, scale=None, causal=False, block_mask=None, block=(128, 128)):
    """Analytic gradients over [B, H, N, d] arrays; returns (dQ, dK, dV)."""
    B, H, N, d = np.asarray(q).shape
    dq = np.zeros((B, H, N, d), dtype=np.float64)
    dk = np.zeros((B, H, N, d), dtype=np.float64)
    dv = np.zeros((B, H, N, np.asarray(v).shape[-1]), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h], _ = attention_backward_head(
                q[b, h], k[b, h], v[b, h], do[b, h], scale=scale, causal=causal,
                block_mask=None if block_mask is None else block_mask[b, h], block=block)
    return dq, dk, dv


def attention_decode_head(q, k, v, scale=None, causal=False):
    """Nq new queries (the cache's last Nq positions) against an Nk-entry
    key/value cache: q [Nq, d], k [Nk, d], v [Nk, dv], Nq <= Nk.  Causal:
    query i sees keys j <= Nk - Nq + i.  Returns (O [Nq, dv], LSE [Nq])."""
    n_q, n_k = np.asarray(q).shape[0], np.asarray(k).shape[0]
    return attention_forward_head(q, k, v, scale=scale, causal=causal, causal_offset=n_k - n_q)
