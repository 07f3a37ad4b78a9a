"""Helpers shared by the GPU parity tests: moving seeded inputs to the GPU,
reading results back as float64, and the accuracy bounds.

The bounds are those of the parity contract: float32 inputs and outputs
within 1e-5 max absolute error of the float64 oracle; bfloat16 outputs and
gradients within 2e-2 (the oracle reads the same bf16-rounded inputs).
"""

import sys

import numpy as np
import pytest

from io_aware_tiled_attn_amd import workloads as wl

TOL = {"fp32": 1e-5, "bf16": 2e-2}


def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def announce(msg):
    """Name the case on stdout before a GPU step (flushes, so a fault that
    ends the process still leaves the case in the log)."""
    print(f"[gpu case] {msg}", flush=True)
    sys.stdout.flush()


def to_gpu(stored, dtype):
    torch = torch_cuda()
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(stored).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(stored, dtype=np.float32))
    return t.cuda()


def to_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def f64(stored, dtype):
    return wl.values(stored, dtype).astype(np.float64)


def max_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    if a.size == 0:
        return 0.0
    assert np.all(np.isfinite(a)), "non-finite values in GPU output"
    return float(np.max(np.abs(a - b)))
