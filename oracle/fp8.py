"""Oracle for the FP8 forward: exact attention of dequantized 8-bit inputs.

Test infrastructure only (tests, the smoke entry and the benchmark's CPU
baseline).

The pages name FP8 support only as part of FlashAttention-3's rebuild for
newer hardware (vibeengines.com, "FlashAttention, explained", section "Why it
still matters", the lineage table); they define no format, scaling or
tolerance.  Readings:
  * format: OCP 8-bit floating point, E4M3 variant (sign bit, 4 exponent bits
    with bias 7, 3 mantissa bits; exponent field 0 holds subnormals
    m/8 * 2^-6; no infinities; codes 0x7F and 0xFF are NaN; largest finite
    value 448).  This is the E4M3 encoding the gfx950 matrix cores read.
  * scaling: one float descale factor per tensor: the value of a stored code
    c of Q is e4m3(c) * q_descale, likewise for K and V.
  * what is computed: ordinary attention (attention.attention_forward_head,
    the plain definition) of those dequantized values, in float64.  The
    rounding the GPU applies inside the method (the probabilities fed to the
    second product in E4M3) is not modelled: the oracle is the exact result,
    and the test tolerance accounts for that rounding.

Pins: tests/test_oracle_fp8.py (the full code table against an independent
library decoder, hand-checked codes, closed forms of the descale factors,
brute force on tiny inputs, and planted mistakes).
"""

import numpy as np

from .attention import attention_forward_head, default_scale, safe_softmax

E4M3_MAX = 448.0
E4M3_BIAS = 7


def e4m3_to_float64(codes):
    """Decode E4M3 byte codes (any integer array) to float64 values."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    subnormal = m / 8.0 * 2.0 ** (1 - E4M3_BIAS)
    normal = (1.0 + m / 8.0) * np.exp2((e - E4M3_BIAS).astype(np.float64))
    val = np.where(e == 0, subnormal, normal)
    val = np.where((e == 0xF) & (m == 7), np.nan, val)
    return sign * val


def dequantize(codes, descale):
    """Values of a stored E4M3 tensor with a per-tensor descale factor."""
    return e4m3_to_float64(codes) * float(descale)


def attention_forward_fp8_head(q8, k8, v8, q_descale, k_descale, v_descale, scale=None, causal=False, rows=None):
    """Exact attention (O, LSE) of one head whose Q, K, V are stored as E4M3
    codes [N, d] with per-tensor descale factors."""
    q = dequantize(q8, q_descale)
    k = dequantize(k8, k_descale)
    v = dequantize(v8, v_descale)
    return attention_forward_head(q, k, v, scale=scale, causal=causal, rows=rows)


def attention_weights_fp8_head(q8, k8, q_descale, k_descale, scale=None, causal=False, rows=None):
    """Softmax weights [len(rows), N] (row i: the weights query rows[i] gives
    each key) of one head stored as E4M3 codes, from the safe softmax of each
    scaled, masked score row.  The tests use it to bound the effect of
    rounding the weights."""
    q = dequantize(q8, q_descale)
    k = dequantize(k8, k_descale)
    if scale is None:
        scale = default_scale(q.shape[-1])
    if rows is None:
        rows = np.arange(q.shape[0])
    w = np.zeros((len(rows), k.shape[0]), dtype=np.float64)
    for n, i in enumerate(rows):
        s = scale * (k @ q[i])
        if causal:
            s[i + 1:] = -np.inf
        w[n] = safe_softmax(s)[0]
    return w
