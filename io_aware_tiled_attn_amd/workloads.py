"""Seeded synthetic inputs shared by the tests, the smoke entry and the bench.

This module draws random numbers and rounds them to the storage type; it
holds none of attention's arithmetic, so both the CPU oracle and the GPU
library can be fed from it without sharing any of the method's code.

Recipe (one per workload, seeded by its index):
  rng = numpy.random.default_rng(seed)                       # PCG64
  Q, K, V, dO = rng.standard_normal(shape, float32) x 4       # in this order
  bf16 workloads round each float32 value to bfloat16, round-to-nearest-even.
Values are N(0, 1) with no structure, standing in for the pages' training
workloads (BERT, GPT-2, Long-Range Arena, Path-X), whose data is not used.
"""

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "bf16" or "fp32"
    causal: bool
    backward: bool      # whether the workload includes the backward pass
    seed: int
    what: str

    @property
    def shape(self):
        return (self.B, self.H, self.N, self.d)


# The five workloads: a fp32 single head, a short non-causal batch, the
# N=4096 d=128 causal shape that the throughput metric is quoted on, a 16K
# causal long context, and a causal forward+backward.
WORKLOADS = {
    "fp32_single_head": Workload(
        "fp32_single_head", 1, 1, 256, 64, "fp32", False, False, 1,
        "fp32 single head B1 H1 N256 d64, non-causal, forward"),
    "bf16_n1k_d64": Workload(
        "bf16_n1k_d64", 8, 16, 1024, 64, "bf16", False, False, 2,
        "bf16 B8 H16 N1024 d64, non-causal, forward"),
    "bf16_n4k_d128_causal": Workload(
        "bf16_n4k_d128_causal", 4, 32, 4096, 128, "bf16", True, True, 3,
        "bf16 B4 H32 N4096 d128, causal, forward and backward"),
    "bf16_n16k_d64_causal": Workload(
        "bf16_n16k_d64_causal", 1, 16, 16384, 64, "bf16", True, False, 4,
        "bf16 B1 H16 N16384 d64, causal long context, forward"),
    "bf16_n2k_d64_causal_fwdbwd": Workload(
        "bf16_n2k_d64_causal_fwdbwd", 4, 16, 2048, 64, "bf16", True, True, 5,
        "bf16 B4 H16 N2048 d64, causal, forward and backward"),
}


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16 (round to nearest, ties to even) and
    return the 16-bit patterns as uint16.  Inputs must be finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits):
    """Exact widening of bfloat16 bit patterns (uint16) to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def draw(shape, seed, count=4):
    """The first `count` of Q, K, V, dO as float32 N(0, 1), drawn in order."""
    rng = np.random.default_rng(seed)
    return [rng.standard_normal(shape, dtype=np.float32) for _ in range(count)]


def make_inputs(shape, seed, dtype="bf16", with_grad=False):
    """Seeded inputs for one workload shape.

    Returns a dict with "q", "k", "v" (and "do" when with_grad) holding the
    stored representation: uint16 bf16 bit patterns for dtype "bf16", float32
    arrays for "fp32".  `values(inputs[name], dtype)` gives the exact values
    as float32.
    """
    arrays = draw(tuple(shape), seed, 4 if with_grad else 3)
    names = ["q", "k", "v", "do"][:len(arrays)]
    if dtype == "bf16":
        return {n: f32_to_bf16_bits(a) for n, a in zip(names, arrays)}
    if dtype == "fp32":
        return dict(zip(names, arrays))
    raise ValueError(f"unknown dtype {dtype!r}")


def values(stored, dtype):
    """Exact numeric values of a stored input as float32."""
    if dtype == "bf16":
        return bf16_bits_to_f32(stored)
    return np.asarray(stored, dtype=np.float32)


def workload_inputs(name, with_grad=None):
    w = WORKLOADS[name]
    if with_grad is None:
        with_grad = w.backward
    return make_inputs(w.shape, w.seed, w.dtype, with_grad)


# ---------------------------------------------------------------------------
# Block masks for block-sparse attention: one byte per (128-query block,
# 128-key block) pair, [B, H, nb, nb] with nb = ceil(N / 128); nonzero keeps
# the pair.  Structure only, no attention arithmetic.
# ---------------------------------------------------------------------------
SPARSE_BLOCK = 128


def random_block_mask(B, H, N, seed, density=0.5, block=SPARSE_BLOCK):
    """Each pair kept independently with probability `density` (PCG64)."""
    nb = -(-N // block)
    rng = np.random.default_rng(seed)
    return (rng.random((B, H, nb, nb)) < density).astype(np.uint8)


def local_global_block_mask(B, H, N, band=2, block=SPARSE_BLOCK):
    """A local band of blocks (|i - j| <= band) plus the first key block
    (a global column), the same for every head."""
    nb = -(-N // block)
    i = np.arange(nb)[:, None]
    j = np.arange(nb)[None, :]
    m = ((np.abs(i - j) <= band) | (j == 0)).astype(np.uint8)
    return np.ascontiguousarray(np.broadcast_to(m, (B, H, nb, nb)))


# Block-sparse workload the benchmark reports beside the dense one: the
# N=4096, d=128 shape with the local+global mask (6 of 32 key blocks per
# query block at most, about 17 % of the pairs), non-causal, forward and
# backward.
SPARSE_WORKLOAD = Workload("bf16_n4k_d128_blocksparse", 4, 32, 4096, 128, "bf16", False, True, 6,
                           "block-sparse (local band 2 + global first block), forward+backward")


# Decoding against a key/value cache: Nq new queries per head and an
# Nk-entry cache.  Recipe: rng = default_rng(seed); Q [B,H,Nq,d], then K and
# V [B,H,Nk,d], standard normal float32, rounded to bf16.
@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    causal: bool
    seed: int


DECODE_WORKLOAD = DecodeWorkload("bf16_decode_b16_h32_q1_nk8k_d128", 16, 32, 1, 8192, 128, False, 7)


def decode_inputs(B, H, Nq, Nk, d, seed):
    """bf16 bit patterns (uint16) of Q, K, V for a decoding call."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, Nq, d), dtype=np.float32)
    k = rng.standard_normal((B, H, Nk, d), dtype=np.float32)
    v = rng.standard_normal((B, H, Nk, d), dtype=np.float32)
    return {"q": f32_to_bf16_bits(q), "k": f32_to_bf16_bits(k), "v": f32_to_bf16_bits(v)}


# ---------------------------------------------------------------------------
# FP8 inputs.  Recipe: the same seeded N(0, 1) float32 draws as a workload
# (Q, K, V in that order); each tensor gets one descale factor
# s = max|x| / 448 (rounded to float32) and is stored as the E4M3 codes of
# x / s, rounded to nearest even by torch's float8_e4m3fn conversion (values
# clipped to +-448 first).  The stored tensor stands for codes * s.
# ---------------------------------------------------------------------------
E4M3_MAX = 448.0


def quantize_e4m3(x):
    """(uint8 E4M3 codes, float32 descale) of a float32 array, per tensor."""
    import torch
    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = float(np.abs(x).max()) if x.size else 0.0
    descale = float(np.float32(amax / E4M3_MAX)) if amax > 0 else 1.0
    y = np.clip(x / np.float32(descale), -E4M3_MAX, E4M3_MAX).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return codes, descale


def fp8_inputs(shape, seed):
    """E4M3 codes and descale factors of Q, K, V:
    {"q": codes, "q_descale": s, "k": ..., "k_descale": ..., "v": ..., "v_descale": ...}."""
    out = {}
    for name, a in zip(("q", "k", "v"), draw(tuple(shape), seed, 3)):
        out[name], out[name + "_descale"] = quantize_e4m3(a)
    return out


# FP8 forward reported beside the bf16 step: the N=4096, d=128 causal shape,
# quantized from the same draws (seed 3) as the bf16 workload.
FP8_WORKLOAD = Workload("fp8_n4k_d128_causal", 4, 32, 4096, 128, "fp8", True, False, 3,
                        "FP8 (E4M3, per-tensor descale) B4 H32 N4096 d128, causal, forward")


def gpu_normal_bf16(shape, seed, device="cuda"):
    """N(0, 1) values rounded to bf16, drawn on the GPU by torch's seeded
    Philox generator: for tensors too large to draw on the host in a test
    (the inputs near the library's element limit).  Tests copy the heads they
    check back to the host and give those exact values to the oracle."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
