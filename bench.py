#!/usr/bin/env python3
"""Throughput of exact tiled attention on one MI355X: forward + backward.

One step is the whole hot path once: the forward kernel (O and LSE) and the
backward phases (preprocessing: D and the per-head fp16 factors; the
key-major dK/dV kernel; the query-major dQ kernel) on one batch of seeded
synthetic input already resident in HBM.  The default workload is B=4, H=32, N=4096, d=128, bf16,
causal.  FLOPs follow the usual convention: forward 4*B*H*N^2*d, halved when
causal; backward 2.5x the forward (five products, including the recomputed
Q K^T); softmax work is not counted.  The backward's two main kernels
execute seven products between them (each recomputes Q K^T and dO V^T):
the dK/dV kernel four of the five counted ones, the dQ kernel the fifth plus
the two recomputed ones, which the convention does not count.

Prints one JSON line: the step's throughput and time, the forward and
backward kernels' figures, the roofline of the dominant kernel (achieved
against the published peak, with the HBM bytes per launch measured by the
hardware counters while the kernel sources are unchanged), the CPU oracle's
throughput on a sample of the same workload, and beside the dense step the
block-sparse step, the FP8 forward, KV-cache decoding and the bf16 forward
alone at other d = 128 shapes with N >= 4096 (causal and not).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def host_threads():
    """Host threads the CPU oracle uses: the cores this process may run on
    (its affinity mask), capped by an OMP_NUM_THREADS that the host already
    sets for this process's share of the machine."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return n


# The BLAS thread counts must be in the environment before numpy (or torch,
# which imports it) is first imported.
HOST_THREADS = host_threads()
for _var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ[_var] = str(HOST_THREADS)

METRIC = "attention fwd/bwd TFLOP/s and % of MI355X bf16 MFMA peak at N=4K,d=128"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published figure
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA, published figure
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
KERNEL_SOURCES = ["io_aware_tiled_attn_amd/csrc/fa_fwd.hip", "io_aware_tiled_attn_amd/csrc/fa_bwd.hip",
                  "io_aware_tiled_attn_amd/csrc/fa_fwd_fp8.hip",
                  "io_aware_tiled_attn_amd/csrc/fa_decode.hip", "io_aware_tiled_attn_amd/csrc/fa_common.h"]


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="bf16_n4k_d128_causal")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=40,
                    help="heads of the workload the CPU oracle is timed on")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the KV-cache decoding step reported beside the dense one")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the FP8 forward reported beside the dense step")
    ap.add_argument("--no-blocksparse", action="store_true",
                    help="skip the block-sparse step reported beside the dense one")
    ap.add_argument("--no-fwd-shapes", action="store_true",
                    help="skip the forward timings at the other d = 128 shapes with N >= 4096")
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="before the steps, copy a buffer of this many MiB once (device to device) so that "
                         "HBM byte counters can be scaled against a transfer of known size")
    return ap.parse_args()


def flops(w):
    fwd = 4.0 * w.B * w.H * w.N * w.N * w.d * (0.5 if w.causal else 1.0)
    return fwd, 2.5 * fwd


def bwd_kernel_flops(f_bwd):
    """Counted FLOPs of the dK/dV kernel (S, dP, dV, dK: four of the five
    products) and of the dQ kernel (dQ), and the dQ kernel's executed FLOPs
    (S, dP and dQ)."""
    prod = f_bwd / 5.0
    return 4.0 * prod, prod, 3.0 * prod


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch of one kernel on one workload, from the committed
    rocprofv3 counter summary; None when it holds no entry for them, or the
    kernel sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    if data.get("source_sha") != kernel_source_hash():
        return None
    entry = data.get("kernels", {}).get(kernel, {}).get(workload)
    return entry.get("bytes_per_launch") if entry else None


def device_info(torch):
    """The GPU's name, compute units and peak clock, and the dense bf16 MFMA
    peak they imply (units x clock x 4096 FLOP per cycle on gfx950)."""
    from io_aware_tiled_attn_amd import binding
    cus, mhz = binding.flash_attn_device_info(torch.cuda.current_device())
    props = torch.cuda.get_device_properties(torch.cuda.current_device())
    return {"name": props.name, "arch": getattr(props, "gcnArchName", ""), "compute_units": cus,
            "peak_clock_mhz": mhz, "bf16_peak_from_clock_tflops": round(cus * mhz * 1e6 * 4096 / 1e12, 1)}


def cpu_baseline(w, inp, gpu_out, heads):
    """Time the float64 oracle on `heads` whole heads of the same workload
    (forward and backward), and compare the GPU results on those heads."""
    import numpy as np
    import oracle
    from io_aware_tiled_attn_amd import workloads as wl
    cores = HOST_THREADS
    try:   # the BLAS pool numpy actually runs, when threadpoolctl can see it
        from threadpoolctl import threadpool_info
        pools = [p.get("num_threads", 0) for p in threadpool_info() if p.get("user_api") == "blas"]
        if pools:
            cores = max(pools)
    except Exception:
        pass
    picks = [(b, h) for b in range(w.B) for h in range(w.H)][::max(1, (w.B * w.H) // heads)][:heads]
    errs = {"o": 0.0, "lse": 0.0, "dq": 0.0, "dk": 0.0, "dv": 0.0}
    elapsed = 0.0
    for b, h in picks:
        q, k, v, do = (wl.values(inp[n][b, h], w.dtype).astype(np.float64) for n in ("q", "k", "v", "do"))
        t0 = time.perf_counter()
        o_ref, lse_ref = oracle.attention_forward_head(q, k, v, causal=w.causal)
        dq_ref, dk_ref, dv_ref, _ = oracle.attention_backward_head(q, k, v, do, causal=w.causal)
        elapsed += time.perf_counter() - t0
        for name, ref in (("o", o_ref), ("lse", lse_ref), ("dq", dq_ref), ("dk", dk_ref), ("dv", dv_ref)):
            errs[name] = max(errs[name], float(np.max(np.abs(gpu_out[name][b, h] - ref))))
    f_fwd, f_bwd = flops(w)
    per_head = (f_fwd + f_bwd) / (w.B * w.H)
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), cpu_model)
    except OSError:
        pass
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        blas = ", ".join(sorted({"%s %s" % (p.get("internal_api", "?"), p.get("version", "")) for p in threadpool_info()}))
    except Exception:
        pass
    return {
        "value": per_head * len(picks) / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": int(cores),
        "affinity_cores": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"{len(picks)} whole heads {picks} of the same workload, forward+backward, float64 numpy "
                  f"({elapsed:.1f} s); FLOPs counted with the GPU's convention (the oracle itself forms the "
                  f"full masked N x N matrices)",
        "seconds": elapsed,
        "cpu": cpu_model,
        "blas": blas,
        # the oracle forms the full masked N x N matrices: 4 N^2 d FLOP forward, 2.5x that backward
        "oracle_gflops_dense": round(4.0 * w.N * w.N * w.d * 3.5 * len(picks) / elapsed / 1e9, 2),
    }, errs


def blocksparse_step(q, k, v, do, o, lse, dq, dk, dv, ws, stream, dense_ms, warmup, steps):
    """The block-sparse workload (same shape, the local-band + global-column
    block mask, non-causal), forward + backward on the same tensors.  FLOPs
    are counted on the kept (128 x 128) blocks only, with the dense
    convention (forward 4 d per kept query-key pair, backward 2.5x)."""
    import numpy as np
    import torch
    import io_aware_tiled_attn_amd as fa
    from io_aware_tiled_attn_amd import workloads as wl
    w = wl.SPARSE_WORKLOAD
    B, H, N, d = q.shape
    mask_np = wl.local_global_block_mask(B, H, N)
    mask = torch.from_numpy(mask_np).cuda()
    kept = int(mask_np.astype(np.int64).sum())
    f_fwd = 4.0 * d * kept * wl.SPARSE_BLOCK * wl.SPARSE_BLOCK
    f_bwd = 2.5 * f_fwd

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        fa.flash_attn_fwd_blocksparse(q, k, v, mask, out=o, lse=lse)
        if ev:
            ev[1].record(stream)
        fa.flash_attn_bwd_blocksparse(q, k, v, o, lse, do, mask, workspace=ws, dq=dq, dk=dk, dv=dv)
        if ev:
            ev[2].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        step(events[i])
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    bwd_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in events]))
    tf = (f_fwd + f_bwd) / (ms * 1e-3) / 1e12
    return {
        "workload": "%s: B=%d H=%d N=%d d=%d bf16, non-causal, block mask local band 2 + global first key "
                    "block (128 x 128 blocks), same tensors as the dense step" % (w.name, B, H, N, d),
        "kept_block_fraction": round(kept / mask_np.size, 4),
        "ms_per_step": round(ms, 4),
        "fwd": {"ms": round(fwd_ms, 4), "tflops": round(f_fwd / (fwd_ms * 1e-3) / 1e12, 2),
                "frac_of_peak": round(f_fwd / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic("fa_fwd_bf16_kernel", w.name)},
        "bwd": {"ms": round(bwd_ms, 4), "tflops": round(f_bwd / (bwd_ms * 1e-3) / 1e12, 2),
                "frac_of_peak": round(f_bwd / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "dkdv_kernel_traffic": measured_traffic("fa_bwd_dkdv_kernel", w.name),
                "dq_kernel_traffic": measured_traffic("fa_bwd_dq_kernel", w.name)},
        "tflops": round(tf, 2),
        "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
        "unit": "TFLOP/s on kept blocks",
        "speedup_vs_dense_causal_step": round(dense_ms / ms, 3),
    }


def fp8_step(warmup, steps):
    """FP8 forward on the N=4096, d=128 causal shape: the same seeded draws
    quantized to E4M3 with one descale per tensor.  FLOPs are the forward's
    (4 N^2 d per head, halved by the causal mask), against the FP8 peak."""
    import numpy as np
    import torch
    import io_aware_tiled_attn_amd as fa
    from io_aware_tiled_attn_amd import workloads as wl
    w = wl.FP8_WORKLOAD
    inp = wl.fp8_inputs(w.shape, w.seed)
    q, k, v = (torch.from_numpy(inp[n]).cuda() for n in ("q", "k", "v"))
    o = torch.empty(w.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(w.shape[:3], dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    ds = (inp["q_descale"], inp["k_descale"], inp["v_descale"])

    def run():
        fa.flash_attn_fwd_fp8(q, k, v, *ds, causal=w.causal, out=o, lse=lse)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        run()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    f_fwd = flops(w)[0]
    tf = f_fwd / (ms * 1e-3) / 1e12
    return {
        "workload": "%s: B=%d H=%d N=%d d=%d, E4M3 inputs with per-tensor descales, bf16 output, causal"
                    % (w.name, w.B, w.H, w.N, w.d),
        "ms": round(ms, 4),
        "tflops": round(tf, 2),
        "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_FP8_TFLOPS, 4),
                     "traffic": measured_traffic("fa_fwd_fp8_g3_kernel", w.name)},
    }


# Forward-only timings at d = 128 and N >= 4096 besides the step's own shape:
# (B, H, N, causal), B * H * N fixed at 2^19 query rows.
FWD_SHAPES = ((4, 32, 4096, False), (2, 32, 8192, True), (2, 32, 8192, False), (1, 32, 16384, True),
              (1, 32, 16384, False))


def forward_shapes_step(warmup, steps):
    """The bf16 forward alone on seeded N(0,1) inputs of each shape in
    FWD_SHAPES (drawn on the device, rounded to bf16), timed with events on
    the launch stream; FLOPs 4 B H N^2 d, halved when causal."""
    import torch
    import io_aware_tiled_attn_amd as fa
    stream = torch.cuda.current_stream()
    gen = torch.Generator(device="cuda").manual_seed(4096)
    out = []
    for B, H, N, causal in FWD_SHAPES:
        q, k, v = (torch.randn((B, H, N, 128), generator=gen, device="cuda").to(torch.bfloat16) for _ in range(3))
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        for _ in range(warmup):
            fa.flash_attn_fwd(q, k, v, causal=causal, out=o, lse=lse)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(steps):
            fa.flash_attn_fwd(q, k, v, causal=causal, out=o, lse=lse)
        end.record(stream)
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / steps
        tf = 4.0 * B * H * N * N * 128 * (0.5 if causal else 1.0) / (ms * 1e-3) / 1e12
        out.append({"B": B, "H": H, "N": N, "d": 128, "causal": causal, "ms": round(ms, 4),
                    "tflops": round(tf, 2), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)})
        del q, k, v, o, lse
    return out


def decode_step(warmup, steps):
    """Decoding against a KV cache (split-KV): one new query per head of a
    B=16, H=32, 8192-entry d=128 cache, the inputs drawn with the workload's
    recipe.  HBM-bound: the roofline is bytes moved (Q, K, V read, O and LSE
    written, the split partials counted too) over the 8 TB/s HBM peak."""
    import numpy as np
    import torch
    import io_aware_tiled_attn_amd as fa
    from io_aware_tiled_attn_amd import workloads as wl
    w = wl.DECODE_WORKLOAD
    inp = wl.decode_inputs(w.B, w.H, w.Nq, w.Nk, w.d, w.seed)
    q, k, v = (torch.from_numpy(inp[n].view(np.int16)).view(torch.bfloat16).cuda() for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.flash_attn_decode_workspace_size(w.B, w.H, w.Nk, w.d), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fa.flash_attn_decode(q, k, v, causal=w.causal, out=o, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fa.flash_attn_decode(q, k, v, causal=w.causal, out=o, lse=lse, workspace=ws)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    # Algorithmic bytes: K and V read once, Q read, O and LSE written.  The
    # split partials (a few MB) are overhead of the method, not counted here;
    # the counters' figure for both kernels is reported as traffic.
    kv_bytes = 2.0 * w.B * w.H * w.Nk * w.d * 2
    qo_bytes = 2.0 * w.B * w.H * w.Nq * w.d * 2 + 4.0 * w.B * w.H * w.Nq
    gbs = (kv_bytes + qo_bytes) / (ms * 1e-3) / 1e9
    # Context for the roofline: what a plain device-to-device copy (HIP
    # runtime, 1 GiB read + 1 GiB written) sustains on this GPU.
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(5):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2.0 * src.numel() / (c0.elapsed_time(c1) / 5 * 1e-3) / 1e9
    del src, dst
    t_split = measured_traffic("fa_decode_split_kernel", w.name)
    t_merge = measured_traffic("fa_decode_merge_kernel", w.name)
    traffic = t_split + t_merge if t_split is not None and t_merge is not None else None
    return {
        "workload": "%s: B=%d H=%d Nq=%d Nk=%d d=%d bf16, %s" % (w.name, w.B, w.H, w.Nq, w.Nk, w.d,
                                                               "causal" if w.causal else "non-causal"),
        "ms": round(ms, 4),
        "tokens_per_s": round(w.B * w.Nq / (ms * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "bytes_per_launch": int(kv_bytes + qo_bytes), "traffic": traffic},
        "device_copy_gbs": round(copy_gbs, 1),
    }


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the library has no multi-GPU path. "
              "Every (batch, head) pair is independent, so across GPUs the work would be split by head.",
              file=sys.stderr)
        return 2
    import numpy as np
    import torch
    import io_aware_tiled_attn_amd as fa
    from io_aware_tiled_attn_amd import binding
    from io_aware_tiled_attn_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    w = wl.WORKLOADS[args.workload]
    if w.dtype != "bf16" or not w.backward:
        print("the benchmark step is forward+backward in bf16", file=sys.stderr)
        return 1
    print(f"[bench] workload {w.name}: generating inputs", file=sys.stderr, flush=True)
    inp = wl.workload_inputs(w.name, with_grad=True)

    def gpu(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    q, k, v, do = (gpu(inp[n]) for n in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(fa.flash_attn_bwd_workspace_size(w.B, w.H, w.N, w.d), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        fa.flash_attn_fwd(q, k, v, causal=w.causal, out=o, lse=lse)
        if ev:
            ev[1].record(stream)
        kw = dict(causal=w.causal, workspace=ws, dq=dq, dk=dk, dv=dv)
        fa.flash_attn_bwd_ex(q, k, v, o, lse, do, phases=binding.FA_BWD_PREPROCESS, **kw)
        if ev:
            ev[2].record(stream)
        fa.flash_attn_bwd_ex(q, k, v, o, lse, do, phases=binding.FA_BWD_MAIN, **kw)
        if ev:
            ev[3].record(stream)
        fa.flash_attn_bwd_ex(q, k, v, o, lse, do, phases=binding.FA_BWD_FINALIZE, **kw)
        if ev:
            ev[4].record(stream)

    if args.calibrate_copy_mb:
        src = torch.ones(args.calibrate_copy_mb << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(events[i])
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    per_kernel = {name: np.array([e[i].elapsed_time(e[i + 1]) for e in events])
                  for i, name in enumerate(("forward", "preprocess", "dkdv", "dq"))}
    fwd_ms, prep_ms, dkdv_ms, dq_ms = (float(per_kernel[n].mean()) for n in per_kernel)
    kernel_stats = {n: {"mean": round(float(a.mean()), 4), "median": round(float(np.median(a)), 4),
                        "min": round(float(a.min()), 4), "max": round(float(a.max()), 4),
                        "std": round(float(a.std()), 4)} for n, a in per_kernel.items()}

    f_fwd, f_bwd = flops(w)
    value = (f_fwd + f_bwd) / (ms_per_step * 1e-3) / 1e12
    fwd_tf = f_fwd / (fwd_ms * 1e-3) / 1e12
    bwd_ms = prep_ms + dkdv_ms + dq_ms
    bwd_tf = f_bwd / (bwd_ms * 1e-3) / 1e12
    f_dkdv, f_dq, f_dq_exec = bwd_kernel_flops(f_bwd)
    # Dominant kernel of the step: the one with the largest share of time,
    # priced at its counted FLOPs.
    dom, dom_ms, dom_flops = max((("fa_fwd_bf16_kernel", fwd_ms, f_fwd), ("fa_bwd_dkdv_kernel", dkdv_ms, f_dkdv),
                                  ("fa_bwd_dq_kernel", dq_ms, f_dq)), key=lambda t: t[1])
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12
    traffic = measured_traffic(dom, w.name)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) Q, K, V, dO (numpy PCG64, seed %d), rounded to bf16" % w.seed,
        "config": {"workload": "attention forward+backward, B=%d H=%d N=%d d=%d, bf16, %s"
                               % (w.B, w.H, w.N, w.d, "causal" if w.causal else "non-causal"),
                   "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "global_batch": w.B, "seq_len": w.N},
        "fwd": {"ms": round(fwd_ms, 4), "tflops": round(fwd_tf, 2),
                "frac_of_peak": round(fwd_tf / PEAK_BF16_TFLOPS, 4)},
        "bwd": {"ms": round(bwd_ms, 4), "tflops": round(bwd_tf, 2),
                "frac_of_peak": round(bwd_tf / PEAK_BF16_TFLOPS, 4),
                "kernels_ms": {"preprocess": round(prep_ms, 4), "dkdv": round(dkdv_ms, 4),
                               "dq": round(dq_ms, 4)},
                "dkdv_kernel_tflops": round(f_dkdv / (dkdv_ms * 1e-3) / 1e12, 2),
                "dq_kernel_tflops_executed": round(f_dq_exec / (dq_ms * 1e-3) / 1e12, 2)},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
        "kernel_ms": kernel_stats,
        "peak_basis": "MI355X dense bf16 MFMA 2.5 PFLOP/s (published); FLOPs: fwd 4BHN^2d (x1/2 causal), "
                      "bwd 2.5x fwd (dK/dV kernel 4/5 of it, dQ kernel 1/5 counted, 3/5 executed)",
        "device": device_info(torch),
    }
    if not args.no_blocksparse:
        print("[bench] block-sparse step", file=sys.stderr, flush=True)
        # Separate outputs: the dense step's results are still checked below.
        result["blocksparse"] = blocksparse_step(q, k, v, do, torch.empty_like(o), torch.empty_like(lse),
                                                 torch.empty_like(dq), torch.empty_like(dk), torch.empty_like(dv),
                                                 ws, stream, ms_per_step, max(5, args.warmup // 2),
                                                 max(10, args.steps // 2))
    if not args.no_fp8:
        print("[bench] FP8 forward", file=sys.stderr, flush=True)
        result["fp8_forward"] = fp8_step(max(5, args.warmup // 2), args.steps)
    if not args.no_fwd_shapes:
        print("[bench] forward at other d = 128 shapes", file=sys.stderr, flush=True)
        result["fwd_d128_shapes"] = forward_shapes_step(max(3, args.warmup // 4), max(10, args.steps // 2))
    if not args.no_decode:
        print("[bench] decoding step", file=sys.stderr, flush=True)
        result["decode"] = decode_step(max(5, args.warmup // 2), args.steps)
    if not args.no_cpu_baseline:
        print(f"[bench] CPU oracle baseline on {args.cpu_heads} heads", file=sys.stderr, flush=True)
        gpu_out = {"o": o.float().cpu().numpy(), "lse": lse.cpu().numpy(), "dq": dq.float().cpu().numpy(),
                   "dk": dk.float().cpu().numpy(), "dv": dv.float().cpu().numpy()}
        base, errs = cpu_baseline(w, inp, gpu_out, args.cpu_heads)
        result["cpu_baseline"] = {k2: (round(v2, 6) if isinstance(v2, float) else v2)
                                  for k2, v2 in base.items() if k2 != "seconds"}
        result["sample_max_abs_err"] = {k2: float("%.3e" % v2) for k2, v2 in errs.items()}
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
