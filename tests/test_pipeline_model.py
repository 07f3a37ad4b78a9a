"""CPU checks of the kernels' LDS tile layouts and buffer schedules.

* tests/layout_check.hip, compiled from the same index-math header as the
  kernels, replays every global -> LDS copy and every MFMA operand read of
  every tile shape the kernels launch (and of the wider shapes that were
  tried and set aside) and reports any read that is out of bounds,
  misaligned or returns another row or column than the operand layout
  asks for.
* tests/pipeline_model.py replays the barrier intervals of the forward's
  three-buffer ping-pong and of the two backward kernels and reports any
  read of a buffer whose copy is still in flight or already replaced.
Planted schedule mistakes show that the model catches such hazards."""

import ctypes
import os
import subprocess

import pytest

from tests import pipeline_model as pm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "layout_check.hip")
LIB = os.path.join(ROOT, "tests", "_build", "liblayout_check.so")
HEADER = os.path.join(ROOT, "io_aware_tiled_attn_amd", "csrc", "fa_layout.h")


def build_checker():
    """Compile the checker (host code only) when it is missing or older than
    its sources."""
    if os.path.exists(LIB) and os.path.getmtime(LIB) >= max(os.path.getmtime(SRC), os.path.getmtime(HEADER)):
        return LIB
    from io_aware_tiled_attn_amd import build as b
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    cmd = [b.hipcc_path(), f"--offload-arch={b.ARCH}", "-O2", "-std=c++17", "-fPIC", "-shared", "-x", "hip", SRC,
           "-o", LIB]
    subprocess.run(cmd, check=True, capture_output=True)
    return LIB


@pytest.fixture(scope="module")
def layout_report():
    lib = ctypes.CDLL(build_checker())
    buf = ctypes.create_string_buffer(1 << 16)
    n = lib.fa_layout_check(buf, len(buf))
    return n, buf.value.decode()


def test_tile_copies_and_operand_reads_agree(layout_report):
    n, text = layout_report
    print(text)
    assert n == 0, text


def test_launched_shapes_are_conflict_free_and_fit(layout_report):
    _, text = layout_report
    lines = [line for line in text.splitlines() if "(launched)" in line]
    assert len(lines) == 7                       # 5 bf16 tile shapes, 2 FP8
    for line in lines:
        assert "over 160 KB" not in line
        assert "conflict degree 1" in line and line.rstrip().endswith("read degree 1"), line
    assert "bwd D=128: LDS at most" in text


@pytest.mark.parametrize("preload", [False, True])
@pytest.mark.parametrize("num_kt", range(1, 10))
def test_forward_schedule_is_safe(num_kt, preload):
    assert pm.check(pm.forward_schedule(num_kt, preload)) == []


@pytest.mark.parametrize("num_kt", range(0, 14))
def test_fp8_three_group_schedule_is_safe(num_kt):
    # d = 128 FP8 forward: 12 waves, output rows staged over K0-K2, V0 (group
    # 0) and V1, V2 (group 1) once every group is past its last tile read.
    assert pm.check(pm.fp8_three_group_schedule(num_kt)) == []


@pytest.mark.parametrize("n_blk", range(0, 12))
def test_backward_schedules_are_safe(n_blk):
    assert pm.check(pm.dkdv_schedule(n_blk)) == []
    assert pm.check(pm.dq_schedule(n_blk)) == []


@pytest.mark.parametrize("preload", [False, True])
@pytest.mark.parametrize("num_kt", range(1, 10))
def test_earlier_forward_schedule_is_safe(num_kt, preload):
    # Tile t + 2 copied at the start of the matrix phase of step t.
    assert pm.check(pm.forward_schedule(num_kt, preload, ahead=2, copy_at="matrix")) == []


def test_model_catches_planted_schedule_mistakes():
    # Two buffers for a copy two tiles ahead: the copy overwrites a tile the
    # other group still reads.
    assert pm.check(pm.forward_schedule(6, False, ahead=2, copy_at="matrix", bufs=2))
    # Three tiles ahead from the start of the matrix phase: on the first
    # step, tile 3 lands in tile 0's buffer while the other group is still
    # taking its first scores from it.
    assert pm.check(pm.forward_schedule(6, False, ahead=3, copy_at="matrix"))
    # Three tiles ahead with only three buffers is safe only from the vector
    # phase; with two buffers it never is.
    assert pm.check(pm.forward_schedule(6, True, bufs=2))
    # No wait for the copies: tiles are read before they are known to be in.
    assert pm.check(pm.forward_schedule(6, False, waits=False))
    # Three groups: K copied four tiles ahead or V three ahead into three
    # buffers overwrites a tile a later group still reads; two buffers never
    # suffice.
    assert pm.check(pm.fp8_three_group_schedule(8, k_ahead=4))
    assert pm.check(pm.fp8_three_group_schedule(8, v_ahead=3))
    assert pm.check(pm.fp8_three_group_schedule(8, bufs=2))
    # Group 0 staging its rows over V0 two intervals before its last
    # barrier, while group 2 still takes its last P V products from V(6).
    early = pm.fp8_three_group_schedule(7)
    early[0].intervals[-4].clobbers.append("V0")
    assert pm.check(early)
    # The dK/dV kernel's next block copied during the matrix phase, which
    # still reads that buffer's previous block.
    assert pm.check(pm.dkdv_schedule(8, copy_in_vector=False))
    # The dQ kernel copying two steps ahead into two buffers.
    assert pm.check(pm.dq_schedule(8, bufs=2))
