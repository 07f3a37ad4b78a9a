"""The seeded input generators: determinism and bf16 rounding."""

import numpy as np
import pytest

from io_aware_tiled_attn_amd import workloads as wl


def test_bf16_rounding_matches_torch_rne():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0, -1.0, 0.0, 1.00390625, 1.01171875,
                                  3.0e38, -3.0e38, 1e-40], np.float32)])
    ours = wl.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = wl.bf16_bits_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_inputs_are_seeded_and_ordered():
    a = wl.make_inputs((1, 2, 8, 4), 3, "bf16", with_grad=True)
    b = wl.make_inputs((1, 2, 8, 4), 3, "bf16", with_grad=True)
    for n in ("q", "k", "v", "do"):
        np.testing.assert_array_equal(a[n], b[n])
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 2, 8, 4), dtype=np.float32)
    np.testing.assert_array_equal(wl.values(a["q"], "bf16"),
                                  wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(q)))
    f = wl.make_inputs((1, 1, 4, 2), 9, "fp32")
    assert f["q"].dtype == np.float32 and set(f) == {"q", "k", "v"}


def test_workload_table():
    w = wl.WORKLOADS["bf16_n4k_d128_causal"]
    assert w.shape == (4, 32, 4096, 128) and w.causal and w.dtype == "bf16"
    assert wl.WORKLOADS["fp32_single_head"].dtype == "fp32"
    assert len(wl.WORKLOADS) == 5
