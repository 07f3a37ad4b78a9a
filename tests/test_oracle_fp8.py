"""Pins of the FP8 oracle (oracle/fp8.py), all on the CPU.

The E4M3 decoder is checked against torch's independent float8_e4m3fn
conversion over all 256 codes and against hand-derived codes of the OCP
E4M3 format; the attention of dequantized inputs against closed forms of the
descale factors and a pure-Python brute force; planted mistakes in a copy of
the module must each fail one of these checks.
"""

import math
import os
import types

import numpy as np
import pytest

import oracle
from io_aware_tiled_attn_amd import workloads as wl

torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "fp8.py")

# (code, value) pairs worked out by hand from the E4M3 layout: sign, 4-bit
# exponent (bias 7), 3-bit mantissa; exponent 0 = subnormal m/8 * 2^-6.
HAND = [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x0F, 1.875 * 2.0 ** -6),
    (0x30, 0.5), (0x38, 1.0), (0x3C, 1.5), (0x40, 2.0), (0x77, 240.0), (0x78, 256.0), (0x7E, 448.0),
    (0xB8, -1.0), (0xFE, -448.0), (0x81, -(2.0 ** -9)),
]


def _decoder_checks(dec):
    codes = np.arange(256)
    got = dec(codes)
    lib = torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(lib))
    fin = ~np.isnan(lib)
    assert np.array_equal(got[fin], lib[fin])
    for c, v in HAND:
        assert dec(np.array([c]))[0] == v, hex(c)
    assert np.isnan(dec(np.array([0x7F]))[0]) and np.isnan(dec(np.array([0xFF]))[0])
    assert math.copysign(1.0, dec(np.array([0x80]))[0]) == -1.0
    pos = dec(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0)


def _brute(q, k, v, scale, causal):
    out, lses = [], []
    for i in range(len(q)):
        sc = [(j, scale * sum(a * b for a, b in zip(q[i], k[j])))
              for j in range(len(k)) if not (causal and j > i)]
        m = max(s for _, s in sc)
        tot = sum(math.exp(s - m) for _, s in sc)
        out.append([sum(math.exp(s - m) / tot * v[j][c] for j, s in sc) for c in range(len(v[0]))])
        lses.append(m + math.log(tot))
    return np.array(out), np.array(lses)


def _attention_checks(mod):
    rng = np.random.default_rng(11)
    n, d = 9, 8
    codes = {t: wl.quantize_e4m3(rng.standard_normal((n, d), dtype=np.float32))[0] for t in "qkv"}
    lib = {t: torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy() for t, c in codes.items()}
    ds = {"q": 0.013, "k": 0.021, "v": 0.007}
    for causal in (False, True):
        o, lse = mod.attention_forward_fp8_head(codes["q"], codes["k"], codes["v"], ds["q"], ds["k"], ds["v"],
                                                causal=causal)
        ob, lb = _brute((lib["q"] * ds["q"]).tolist(), (lib["k"] * ds["k"]).tolist(),
                        (lib["v"] * ds["v"]).tolist(), 1 / math.sqrt(d), causal)
        np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(lse, lb, rtol=1e-12, atol=1e-15)
        # Q and K descales multiply the scores: same as unit descales with
        # scale * q_descale * k_descale.  The V descale multiplies O only.
        o1, l1 = mod.attention_forward_fp8_head(codes["q"], codes["k"], codes["v"], 1.0, 1.0, 1.0,
                                                scale=ds["q"] * ds["k"] / math.sqrt(d), causal=causal)
        np.testing.assert_allclose(o, o1 * ds["v"], rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(lse, l1, rtol=1e-12, atol=1e-15)
        # Weights: rows sum to 1, zero above the diagonal when causal, and
        # O = P V.
        w = mod.attention_weights_fp8_head(codes["q"], codes["k"], ds["q"], ds["k"], causal=causal)
        np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-13)
        if causal:
            assert np.all(np.triu(w, 1) == 0)
        np.testing.assert_allclose(w @ (lib["v"] * ds["v"]), o, rtol=1e-12, atol=1e-15)
        ws = mod.attention_weights_fp8_head(codes["q"], codes["k"], ds["q"], ds["k"], causal=causal, rows=[6, 2])
        np.testing.assert_array_equal(ws, w[[6, 2]])


def test_decoder_pins():
    _decoder_checks(oracle.e4m3_to_float64)


def test_attention_pins():
    _attention_checks(oracle.fp8)


def test_constant_values_give_exact_output():
    # Every V row the same code: O is that value for every query, whatever
    # the weights.
    rng = np.random.default_rng(12)
    q8, _ = wl.quantize_e4m3(rng.standard_normal((40, 16), dtype=np.float32))
    k8, _ = wl.quantize_e4m3(rng.standard_normal((40, 16), dtype=np.float32))
    v8 = np.full((40, 16), 0x3C, np.uint8)   # 1.5
    o, _ = oracle.attention_forward_fp8_head(q8, k8, v8, 0.01, 0.02, 2.0, causal=True)
    np.testing.assert_allclose(o, 3.0, rtol=1e-14)


def test_quantizer_round_trip():
    # Input generation: codes * descale recover x within half an E4M3 step
    # (relative 2^-4) for normal values, and max|x| maps to code 0x7E.
    rng = np.random.default_rng(13)
    x = rng.standard_normal(4096, dtype=np.float32)
    codes, s = wl.quantize_e4m3(x)
    back = oracle.dequantize(codes, s)
    big = np.abs(x) >= 2.0 ** -6 * s
    assert np.all(np.abs(back[big] - x[big]) <= 2.0 ** -4 * np.abs(x[big]) * (1 + 1e-6))
    assert codes[np.argmax(np.abs(x))] & 0x7F == 0x7E


MUTANTS = {
    "bias_8": ("E4M3_BIAS = 7", "E4M3_BIAS = 8"),
    "subnormal_as_normal": ("val = np.where(e == 0, subnormal, normal)", "val = normal"),
    "subnormal_scale": ("subnormal = m / 8.0 * 2.0 ** (1 - E4M3_BIAS)", "subnormal = m / 8.0 * 2.0 ** (-E4M3_BIAS)"),
    "mantissa_over_16": ("normal = (1.0 + m / 8.0)", "normal = (1.0 + m / 16.0)"),
    "nan_missing": ("val = np.where((e == 0xF) & (m == 7), np.nan, val)", "pass"),
    "sign_dropped": ("sign = np.where(c & 0x80, -1.0, 1.0)", "sign = 1.0"),
    "v_descale_on_k": ("k = dequantize(k8, k_descale)\n    v = dequantize(v8, v_descale)",
                       "k = dequantize(k8, v_descale)\n    v = dequantize(v8, k_descale)"),
    "weights_causal_off_by_one": ("s[i + 1:] = -np.inf", "s[i:] = -np.inf"),
}


def _load_mutant(old, new):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor not found once: {old!r}"
    mod = types.ModuleType("oracle.fp8_mutant")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), "oracle_fp8_mutant", "exec"), mod.__dict__)
    return mod


def test_unmutated_copy_passes():
    mod = _load_mutant("E4M3_BIAS = 7", "E4M3_BIAS = 7")
    _decoder_checks(mod.e4m3_to_float64)
    _attention_checks(mod)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _load_mutant(*MUTANTS[name])
    with pytest.raises((AssertionError, ValueError, FloatingPointError)):
        _decoder_checks(mod.e4m3_to_float64)
        _attention_checks(mod)
