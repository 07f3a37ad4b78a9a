"""CPU model of the forward kernels' lazy running max, used to show that a
GPU test reaches the kernels' rescale of a live partial result.

The kernels (bf16 `fa_fwd_bf16_kernel`, block-sparse included, and FP8
`fa_fwd_fp8_kernel`) keep, per query, a reference max m in log2 units, a
partial sum l and an output accumulator O.  Each wave owns 32 queries; each
query's scores of a key tile are split over two lanes (lane halves).  For
every visited key tile, in order:

  1. every lane sums P = exp2(s * c - m) over its keys of the tile
     (c = scale * log2 e; masked keys have s = -inf);
  2. if any lane of the wave has a sum that is not <= 256, the wave takes
     the rescale branch: per query m_new = max(m, c * tile max),
     alpha = exp2(m - m_new), l and O are multiplied by alpha and the
     exponentials are taken again against m_new;
  3. l += the lane's sum.

A "live rescale" is a query for which step 2 lowers alpha below 1 while its
l is already positive: exactly the case where dropping `l *= alpha` or
`O *= alpha`, or computing alpha wrongly, changes the result.  The model
replays that rule on the exact input values in float64 (the kernels use
fp32; a trigger counts as robust only when the lane sum passes 256 by at
least 2 %, far beyond that difference).

This is test infrastructure that mirrors the kernels' decision rule; it is
not the oracle and computes no attention output.
"""

import numpy as np

LIMIT = 256.0
LOG2E = 1.4426950408889634
BM = 256          # queries per workgroup (8 waves of 32)
SPARSE_BLOCK = 128


def default_block_n(d, kernel, sparse):
    if kernel == "fp8":
        return 64
    if kernel == "bf16" and d == 128 and not sparse:
        return 96
    return 64


def lane_keys(kernel, block_n):
    """[2, block_n // 2] key offsets within a tile held by lane half 0 and 1."""
    halves = []
    for lg in (0, 1):
        keys = []
        for mb in range(block_n // 32):
            for r in range(16):
                if kernel == "fp8":
                    keys.append(32 * mb + 16 * lg + r)
                else:
                    keys.append(32 * mb + 8 * (r >> 2) + 4 * lg + (r & 3))
        halves.append(keys)
    return np.array(halves)


MUTATIONS = ("drop_l_rescale", "drop_o_rescale", "alpha_base_e", "alpha_inverted")


def count_live_rescales(q, k, scale, causal, kernel="bf16", block_n=0, block_mask=None, v=None,
                        mutation=None):
    """Replay the trigger rule for one head.

    q, k        : [N, d] exact input values (for FP8, the dequantized values).
    block_mask  : [nb, nb] keep flags of (128-query block, 128-key block)
                  pairs, or None (dense).
    v           : [N, d] values; when given, the update is carried out in
                  float64 with P unrounded and the result O = O_acc / l is
                  returned under "o" (rows past N dropped).
    mutation    : one of MUTATIONS, a planted mistake in the rescale branch
                  (drop `l *= alpha`, drop `O *= alpha`, alpha = e^(m_old -
                  m_new) on the log2-unit m, alpha = 2^(m_new - m_old)), to
                  show that the tests reaching the branch would catch it.
    Returns a dict: "live" (robust live-rescale events, counted per query),
    "live_any" (all live events), "tiles" (tile visits modelled).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    N, d = q.shape
    sparse = block_mask is not None
    bn = block_n or default_block_n(d, kernel, sparse)
    c = float(np.float32(np.float32(scale) * np.float32(LOG2E)))
    keys_of = lane_keys(kernel, bn)                       # [2, bn/2]
    live = live_any = visits = 0
    out = np.zeros((-(-N // BM) * BM, d)) if v is not None else None
    if v is not None:
        v = np.asarray(v, np.float64)
    for qt in range(-(-N // BM)):
        q_tile_end = min(N, (qt + 1) * BM)
        key_end = q_tile_end if causal else N
        num_kt = -(-key_end // bn)
        tiles = []
        for t in range(num_kt):
            kb = t * bn // SPARSE_BLOCK
            if sparse:
                k0 = bool(block_mask[2 * qt, kb])
                k1 = bool(2 * qt + 1 < block_mask.shape[0] and block_mask[2 * qt + 1, kb])
                if k0 or k1:
                    tiles.append((t, (k0, k1)))
            else:
                tiles.append((t, (True, True)))
        for w in range(8):
            group = w // 4
            qi = qt * BM + 32 * w + np.arange(32)
            qrows = np.where(qi[:, None] < N, q[np.minimum(qi, N - 1)], 0.0)   # rows past N read zero
            qlim = np.minimum(qi, N - 1) if causal else np.full(32, N - 1)
            m = np.full(32, -np.inf)
            lsum = np.zeros((32, 2))
            oacc = np.zeros((32, d))
            for t, keep in tiles:
                visits += 1
                keys = t * bn + keys_of                      # [2, bn/2]
                kv = np.where((keys < N)[..., None], k[np.minimum(keys, N - 1)], 0.0)
                s = np.einsum("qc,hjc->qhj", qrows, kv)      # [32, 2, bn/2]
                masked = (keys[None] > qlim[:, None, None]) | (not keep[group])
                s = np.where(masked, -np.inf, s)

                def lane_sums(ref):
                    with np.errstate(invalid="ignore", over="ignore"):
                        # -inf - (-inf) is NaN, as in the kernels: a NaN sum fires
                        return np.exp2(s * c - ref[:, None, None]).sum(axis=2)   # [32, 2]

                rs = lane_sums(m)
                fire = ~(rs <= LIMIT)
                if fire.any():
                    mx = s.max(axis=(1, 2)) * c
                    m_new = np.maximum(m, mx)
                    with np.errstate(invalid="ignore"):
                        raised = np.isfinite(m) & (m_new > m) & (lsum.max(axis=1) > 0)
                    robust_wave = bool((np.isfinite(m) & (rs.max(axis=1) >= 1.02 * LIMIT)).any())
                    live_any += int(raised.sum())
                    if robust_wave:
                        live += int((raised & (m_new - m > 1e-3)).sum())
                    with np.errstate(invalid="ignore"):
                        diff = np.where(np.isfinite(m), m - m_new, -np.inf)
                        if mutation == "alpha_base_e":
                            diff = diff / LOG2E          # exp(diff) written as exp2
                        elif mutation == "alpha_inverted":
                            diff = np.where(np.isfinite(diff), -diff, diff)
                        alpha = np.where(m_new == -np.inf, 1.0, np.exp2(diff))
                    m = m_new
                    if mutation != "drop_l_rescale":
                        lsum = lsum * alpha[:, None]
                    if mutation != "drop_o_rescale":
                        oacc = oacc * alpha[:, None]
                    rs = lane_sums(np.where(m == -np.inf, 0.0, m))
                lsum = lsum + np.nan_to_num(rs, nan=0.0)
                if v is not None:
                    ref = np.where(m == -np.inf, 0.0, m)
                    with np.errstate(invalid="ignore", over="ignore"):
                        p = np.nan_to_num(np.exp2(s * c - ref[:, None, None]), nan=0.0)   # [32, 2, bn/2]
                    vk = np.where((keys < N)[..., None], v[np.minimum(keys, N - 1)], 0.0)   # [2, bn/2, d]
                    oacc = oacc + np.einsum("qhj,hjc->qc", p, vk)
            if v is not None:
                l_tot = lsum.sum(axis=1)
                with np.errstate(invalid="ignore", divide="ignore"):
                    out[qi] = np.where(l_tot[:, None] > 0, oacc / l_tot[:, None], 0.0)
    res = {"live": live, "live_any": live_any, "tiles": visits}
    if v is not None:
        res["o"] = out[:N]
    return res
