"""Inputs whose scores climb from one key tile to the next, so that the
forward kernels' online-softmax update has to raise the running max while
it already holds a partial sum and a partial output (vibeengines.com,
"FlashAttention, explained", section "The math, worked with real numbers":
the "Rescale old l" and "Absorb new block" rows and the update rule).

The kernels keep a lazy reference max: they raise it only when a tile's
exponentials against the current one would sum past 256 in some lane.  With
N(0, 1) inputs that never happens after the first tile, so these inputs put
a level in one feature: q[:, 0] = 4 and k[j, 0] = level(j), the other
features are N(0, 1) scaled by 1/4 (small noise), and V carries an indicator
of the key's quarter of the sequence in features 1..4, so that O shows
directly how much weight each part of the sequence received.  The patterns:

  * "stair": level 0 for about the first 3/4 of the keys, then one step
    up; the rows that see the step must rescale 10-20 % of their mass.
  * "ramp": level rising linearly with the key index; rows rescale many
    times.
  * "falling": the same ramp falling; the first tile holds the max, so no
    rescale happens after it (a control).

The step height is chosen per head size so that, at the default scale
1/sqrt(d), one lane's 16 keys of a 32-key block already sum past 256 against
the old max.  `tests/lazy_max_model.py` replays the kernels' trigger rule on
these exact inputs; the CPU test there asserts that each rising pattern
triggers live rescales, so the GPU tests that use them reach the rescale.

This module draws numbers and places them; it holds no attention
arithmetic.
"""

import numpy as np

from io_aware_tiled_attn_amd import workloads as wl

# Step height of the level feature per head size: 4 * L * scale * log2(e)
# = 4.33 (d = 64) and 4.59 (d = 128) in log2 units, so 16 keys at P ~ 2^4.3
# sum past 256.  Multiples of L up to 3L are exact in bf16 and E4M3.
STEP = {64: 6.0, 128: 9.0}
# Ramp slope per key (level units), about 0.15 in log2 units per key.
SLOPE = {64: 0.2, 128: 0.27}

PATTERNS = ("stair", "ramp", "falling")


def stair_cut(N):
    """First key of the step: about 3/4 of the way, on a multiple of 96 keys
    (a tile boundary for every tile width) when N allows."""
    cut = (3 * N) // 4
    return cut - cut % 96 if cut >= 96 else cut


def level(pattern, N, d):
    j = np.arange(N, dtype=np.float64)
    if pattern == "stair":
        return np.where(j >= stair_cut(N), STEP[d], 0.0)
    if pattern == "ramp":
        return SLOPE[d] * j
    if pattern == "falling":
        return SLOPE[d] * (N - 1 - j)
    raise ValueError(pattern)


def climbing_f32(shape, seed, pattern):
    """float32 Q, K, V of the pattern (before any rounding)."""
    B, H, N, d = shape
    q, k, v = wl.draw(tuple(shape), seed, 3)
    q *= np.float32(0.25)
    k *= np.float32(0.25)
    q[..., 0] = 4.0
    k[..., 0] = level(pattern, N, d).astype(np.float32)
    # V: noise plus an indicator of the key's quarter of the sequence, so
    # the weight each part of the sequence receives shows in O.
    quarter = np.minimum(4 * np.arange(N) // N, 3)
    v *= np.float32(0.5)
    for part in range(4):
        v[..., quarter == part, 1 + part] += np.float32(2.0)
    return q, k, v


def climbing_bf16(shape, seed, pattern):
    """{"q", "k", "v"}: bf16 bit patterns (uint16) of the pattern."""
    return {n: wl.f32_to_bf16_bits(a) for n, a in zip("qkv", climbing_f32(shape, seed, pattern))}


def climbing_fp8(shape, seed, pattern):
    """E4M3 codes and per-tensor descales of the pattern (the workloads'
    amax recipe)."""
    out = {}
    for name, a in zip("qkv", climbing_f32(shape, seed, pattern)):
        out[name], out[name + "_descale"] = wl.quantize_e4m3(a)
    return out


# The page's worked example spread over two key tiles: scores 2, 1 in the
# first block (keys 0, 1) and 3, 0 in the second (keys 96, 97), every other
# key padded far below.  Keys 96 and 97 sit in a later tile for every tile
# width the kernels use (32, 64, 96).  With the scores multiplied by 6 (the
# scale argument), the second block's max lifts P of key 96 to e^6 = 403
# against the first block's max, past the kernels' limit of 256, so the
# running max is raised with the first block's l and O live.
WORKED_SCORES = (2.0, 1.0, 3.0, 0.0)
WORKED_KEYS = (0, 1, 96, 97)
WORKED_SCALE = 6.0
WORKED_N = 128
WORKED_PAD = -64.0


def worked_across_tiles_f32(d=64):
    """float32 Q, K, V of one head [1, 1, 128, d]: q_0 = e_0, k_j = s_j e_0
    for the four keys of the example (padding k_j = -64 e_0 elsewhere), and
    V_j = e_t for the example's t-th key (0 elsewhere), so O_0[0:4] are the
    example's four weights in the page's order."""
    N = WORKED_N
    q = np.zeros((1, 1, N, d), np.float32)
    q[0, 0, :, 0] = 1.0
    k = np.zeros((1, 1, N, d), np.float32)
    k[0, 0, :, 0] = WORKED_PAD
    v = np.zeros((1, 1, N, d), np.float32)
    for t, (j, s) in enumerate(zip(WORKED_KEYS, WORKED_SCORES)):
        k[0, 0, j, 0] = s
        v[0, 0, j, t] = 1.0
    return q, k, v


def worked_across_tiles_fp8(d=64):
    """The same head as E4M3 codes with descales chosen so that every value
    is exact: q and v with descale 1 (codes 1.0), k with descale 1/4 (codes
    8, 4, 12, 0 and -256 for the padding)."""
    import torch
    q, k, v = worked_across_tiles_f32(d)
    out = {}
    for name, a, ds in (("q", q, 1.0), ("k", k, 0.25), ("v", v, 1.0)):
        y = torch.from_numpy(np.ascontiguousarray(a / np.float32(ds)))
        codes = y.to(torch.float8_e4m3fn)
        assert torch.equal(codes.float(), y), "worked example must be exact in E4M3"
        out[name] = codes.view(torch.uint8).numpy().copy()
        out[name + "_descale"] = ds
    return out
