"""Throughput of the fused smooth + rotate + MXFP4 quantization on one MI355X.

A step is one mxq_rotate_quant call over one batch of synthetic activations
(default workload: down_proj-input shape, bf16 8192 x 14336 with massive
outliers on 1% of tokens, outlier-aware Householder block, no smoothing).
Inputs sit in HBM before the timed region starts.  Consecutive steps use
different buffer sets (together > 3x the 256 MB last-level cache), so every
step reads its activations from HBM rather than from cache.

Prints one JSON line.  Besides the headline throughput it carries:
  roofline      the quantize kernel's algorithmic HBM bytes per launch
                (2 B read + 0.5 B codes + 1/32 B scale per element) over its
                mean launch time (HIP events around the timed region on the
                launch stream, divided by the step count), against the 8 TB/s
                HBM peak; traffic = bytes the kernel really moved,
                from committed rocprofv3 FETCH_SIZE/WRITE_SIZE counters when
                they were taken on the current kernel source, else null;
  cpu_baseline  the fp64 CPU oracle on the host cores, same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "rotate+MXFP4-quant throughput: Gelem/s, HBM GB/s, % of MI355X HBM peak"
HBM_PEAK_GBPS = 8000.0
BYTES_PER_ELEM = 2.0 + 0.5 + 1.0 / 32.0  # bf16/fp16 in, FP4 codes + E8M0 scales out
KERNEL_SOURCES = ("mxfp4_activation_rotation_amd/csrc/mxq.hip",
                  "mxfp4_activation_rotation_amd/csrc/mxq_device.h")
COUNTERS = {3: "profiles/rotate_quant_bf16_8192x14336_hbm_counters.txt",
            2: "profiles/rotate_quant_bf16_lambda_2048x4096_hbm_counters.txt",
            4: "profiles/rotate_quant_bf16_lambda_decode_16x8192_hbm_counters.txt",
            5: "profiles/rotate_quant_fp16_lambda_32768x8192_hbm_counters.txt"}
GEMM_SOURCES = ("mxfp4_activation_rotation_amd/csrc/mxq_gemm.hip",)
GEMM_COUNTERS = "profiles/gemm_mxfp4_tiled_8192x4096x14336_hbm_counters.txt"
DECODE_COUNTERS = {16: "profiles/gemm_mxfp4_tiled_decode_16x4096x14336_hbm_counters.txt"}
FP4_MFMA_PEAK_TFLOPS = 10100.0  # MI355X dense FP4 (E2M1) matrix-core peak
WORKLOAD_NAMES = {
    2: "QKV-input shape: bf16 2048x4096, 0.5% outlier channels x20, lognormal lambda, seeded orthogonal R",
    3: "down_proj-input shape: bf16 8192x14336, Student-t(3) background, +-U(500,2000) on 1% of tokens "
       "at channels 17/4099/9001/14000, outlier-aware Householder R (k from a 256-token slice), no lambda",
    4: "decode-shaped calls: bf16 16x8192 per call, 2 outlier channels x30, lognormal lambda, orthogonal R",
    5: "large prefill: fp16 32768x8192, 0.1% entries +-U(100,1000), 8 channels x25, "
       "lambda = amax^0.5 (512-token slice), outlier-aware Householder R",
}


def kernel_source_hash(sources=KERNEL_SOURCES) -> str:
    """Hash of a kernel's sources and the compile flags."""
    from mxfp4_activation_rotation_amd import _build
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    h.update(" ".join(_build.flags_for(sources[0])).encode())
    return h.hexdigest()[:16]


def read_counters(cfg: int, rel: str | None = None, sources=KERNEL_SOURCES):
    """Per-launch HBM bytes from the committed counter summary, or None when
    it is absent or was taken on a different kernel source."""
    rel = rel or COUNTERS.get(cfg)
    if not rel or not os.path.exists(os.path.join(ROOT, rel)):
        return None
    kv = {}
    for line in open(os.path.join(ROOT, rel)):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_hash") != kernel_source_hash(sources):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def host_cpu_model() -> str:
    """The host CPU's model name (first processor in /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, min_seconds: float):
    import oracle
    orc = oracle.default()
    elems = wl.tokens * wl.channels
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        orc.rotate_quant(wl.x, wl.lam, wl.r_hat)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start >= min_seconds and len(times) >= 3:
            break
    med = statistics.median(times)
    return {"value": round(elems / med / 1e9, 4), "unit": "Gelem/s", "cores": orc.num_threads(),
            "kind": "oracle", "cpu": host_cpu_model(),
            "sample": f"the full {wl.tokens}x{wl.channels} batch, {len(times)} repetitions "
                      f"({sum(times):.1f} s of CPU wall time), median {med * 1e3:.0f} ms each"}


def bench_calibration(args):
    """Greedy block search (128 steps max) on a 262144 x 32 fp64 block; each
    timed call starts from a fresh copy of the block (copied outside the
    events).  With pi/4 the scan kernel reads the block once per step and
    writes the two rotated columns of the previous step; with an angle grid
    (--angle-grid M) a step applies the previous rotation in one pass and
    scans every (candidate, angle) pair in ceil(M / 8) more."""
    import numpy as np
    import torch

    import mxfp4_activation_rotation_amd as mxq
    import workloads

    dev = torch.device("cuda:0")
    xw_host = workloads.calibration_block()
    pristine = torch.from_numpy(xw_host).to(dev)
    work = torch.empty_like(pristine)
    reps = max(1, min(args.steps, 20))
    times = []
    for i in range(3 + reps):
        work.copy_(pristine)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        if args.angle_grid:
            _, hist, done, _, _ = mxq.calib_givens_angles(work, 128, args.angle_grid)
        else:
            _, hist, done, _ = mxq.calib_givens(work, 128)
        e1.record()
        e1.synchronize()
        if i >= 3:
            times.append(e0.elapsed_time(e1))
    steps = int(done)
    ms = float(np.median(times))
    T = xw_host.shape[0]
    bytes_per_scan = T * 32 * 8
    if args.angle_grid:
        # init scan; per step executed (steps + 1, the last one refused or the
        # 128th): an apply pass (none before the first) and ceil(M / 8) angle scans
        executed = min(steps + 1, 128)
        scans = 1 + executed * (1 + -(-args.angle_grid // 8))
    else:
        scans = steps + 2  # init scan, one per step (the last step's pass finds no better candidate), final apply
    result = {
        "metric": "greedy block calibration time (DuQuant++ page sec. 3.2), GPU fp64",
        "value": round(ms, 3), "unit": "ms per search", "higher_is_better": False, "n_gpus": 1,
        "steps": reps, "data": "synthetic",
        "config": {"workload": "page-scale X_worst: 128 x 2048 tokens x 32 channels fp64, Student-t(3) "
                               "background, +-U(200,800) on 2000 tokens of channel 9",
                   "tokens": T, "max_steps": 128, "steps_taken": steps,
                   "angle": f"grid of {args.angle_grid} per candidate" if args.angle_grid else "pi/4"},
        "ms_per_step": round(ms / max(steps, 1), 4),
        "scan_bytes_per_step": bytes_per_scan,
        "achieved_GBps_all_launches": round(bytes_per_scan * scans / (ms * 1e-3) / 1e9, 1),
        "linf": [float(hist[0]), float(hist[steps])],
    }
    if not args.no_cpu_baseline:
        from oracle import calibration as CAL
        if args.angle_grid:
            # a whole search would take many minutes: time two steps, scale to the steps taken
            t0 = time.perf_counter()
            CAL.greedy_givens_angle(xw_host, 2, args.angle_grid)
            dt = (time.perf_counter() - t0) / 2 * max(steps, 1)
            sample = f"the same block, the first 2 steps (NumPy fp64), scaled to {steps} steps"
        else:
            t0 = time.perf_counter()
            CAL.greedy_givens(xw_host, 128)
            dt = time.perf_counter() - t0
            sample = "the same block, one search (NumPy fp64)"
        result["cpu_baseline"] = {"value": round(dt * 1e3, 1), "unit": "ms per search", "cores": 1,
                                  "kind": "oracle", "cpu": host_cpu_model(), "sample": sample}
    print(json.dumps(result), flush=True)


def bench_gemm(args):
    """The consumer: W4A4 MXFP4 product of the quantized down_proj input
    (8192 x 14336, from mxq_rotate_quant on the headline activations) with
    absorbed, quantized synthetic weights (4096 x 14336), bf16 output.  The
    operands (88 MB) are built once on the GPU before the timed region.
    With --decode, the activations are the first --rows tokens (1..64,
    default 16) of the same batch: the product is bound by reading the
    weights, so its roofline is HBM.  Without --decode, --rows (65..8192)
    takes the first rows of the batch as a shorter prefill.  Both
    operands are in the fragment-tiled layout (the activations written so by
    the quantizer, the weights repacked once offline); --row-layout times the
    row-layout operands instead."""
    import numpy as np
    import torch

    import mxfp4_activation_rotation_amd as mxq
    import workloads

    dev = torch.device("cuda:0")
    wl = workloads.make_config(3)
    w = workloads.linear_weights(workloads.DOWN_PROJ_OUT, wl.channels)
    r = wl.r_hat.to(dev)
    lam = torch.from_numpy(wl.lam).to(dev) if wl.lam is not None else None
    ac, asc = mxq.rotate_quant(wl.x.to(dev), r, lam)
    bc, bsc = mxq.absorb_quant(w.to(dev), r, lam)
    M, K, N = ac.shape[0], wl.channels, workloads.DOWN_PROJ_OUT
    weight_bytes = N * (K // 2 + K // 32)
    tiled = not args.row_layout
    if args.rows is not None:
        M = args.rows
        ac, asc = ac[:M].contiguous(), asc[:M].contiguous()
    if tiled:
        ta, tsa = mxq.rotate_quant_tiled(wl.x[:M].contiguous().to(dev), r, lam)
    weights = [mxq.tile_mxfp4(bc, bsc) if tiled else (bc, bsc)]
    if args.decode:
        # A decode step reads every layer's weights once: rotate through
        # enough weight copies (> 768 MB) that none is still cached from its
        # previous use, so the weights stream from HBM as they would there.
        weights += [(weights[0][0].clone(), weights[0][1].clone())
                    for _ in range(int(np.ceil(768e6 / weight_bytes)))]
    n_w = len(weights)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    flop = 2.0 * M * N * K

    def product(i):
        if tiled:
            mxq.gemm_mxfp4_tiled(ta, tsa, *weights[i % n_w], M, N, K, out=y)
        else:
            mxq.gemm_mxfp4(ac, asc, *weights[i % n_w], out=y)

    for i in range(args.warmup):
        product(i)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for i in range(args.steps):
        product(args.warmup + i)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean_launch_s = ev0.elapsed_time(ev1) / 1e3 / args.steps
    achieved = flop / mean_launch_s / 1e12
    if not tiled:
        hbm = None
    elif args.decode:
        hbm = read_counters(0, DECODE_COUNTERS.get(M, ""), GEMM_SOURCES)
    elif M == 8192:
        hbm = read_counters(0, GEMM_COUNTERS, GEMM_SOURCES)
    else:
        hbm = None
    result = {
        "metric": "W4A4 MXFP4 GEMM throughput (consumer of the quantized activations): TFLOP/s",
        "value": round(flop * args.steps / wall / 1e12, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp4",
        "data": "synthetic",
        "config": {"workload": f"down_proj product: activations bf16 {M}x14336 ("
                               + ("the headline batch" if M == 8192 else f"the first {M} tokens of the headline batch")
                               + ") rotated and MXFP4-quantized, times absorbed MXFP4 weights 4096x14336 "
                                 "(seeded N(0, 1/14336)); fp32 accumulation, bf16 output",
                   "M": M, "N": N, "K": K,
                   "operands": "E2M1 codes + E8M0 scales per 32 along K, " +
                               ("fragment-tiled records (16 rows x 128 positions)" if tiled else "row layout"),
                   "parallelism": "single GPU", "launch": "eager launches"},
        "launch_us_mean": round(mean_launch_s * 1e6, 3),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP4_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / FP4_MFMA_PEAK_TFLOPS, 4),
                     "traffic": None if hbm is None else round(hbm)},
        "kernel_source_hash": kernel_source_hash(GEMM_SOURCES),
    }
    if args.decode:
        algo = weight_bytes + M * (K // 2 + K // 32) + M * N * 2
        gbps = algo / mean_launch_s / 1e9
        result["metric"] = "decode-shaped W4A4 MXFP4 GEMM: GB/s of weights streamed"
        result["value"] = round(algo * args.steps / wall / 1e9, 1)
        result["unit"] = "GB/s"
        result["config"]["workload"] = (f"decode product: {M} token{'s' if M > 1 else ''} of the headline batch, "
                                        "rotated and MXFP4-quantized, times absorbed MXFP4 weights 4096x14336, "
                                        "bf16 output")
        result["config"]["weight_sets"] = n_w
        result["roofline"] = {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                              "frac": round(gbps / HBM_PEAK_GBPS, 4),
                              "traffic": None if hbm is None else round(hbm)}
    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.default()
        rows = min(64, M)
        a_s, as_s = ac[:rows].cpu().numpy(), asc[:rows].cpu().numpy()
        b_h, bs_h = bc.cpu().numpy(), bsc.cpu().numpy()
        times = []
        t_start = time.perf_counter()
        while True:
            t1 = time.perf_counter()
            oracle.gemm_mxfp4(a_s, as_s, b_h, bs_h, orc)
            times.append(time.perf_counter() - t1)
            if time.perf_counter() - t_start >= args.cpu_seconds and len(times) >= 3:
                break
        med = statistics.median(times)
        try:
            from threadpoolctl import threadpool_info
            blas = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"),
                       default=1)
        except Exception:  # pragma: no cover
            blas = 1
        cpu_value = (round((weight_bytes + rows * (K // 2 + K // 32) + rows * N * 2) / med / 1e9, 4)
                     if args.decode else round(2.0 * rows * N * K / med / 1e12, 5))
        result["cpu_baseline"] = {
            "value": cpu_value, "unit": "GB/s" if args.decode else "TFLOP/s",
            "cores": max(blas, orc.num_threads()), "kind": "oracle", "cpu": host_cpu_model(),
            "sample": f"the first {rows} activation rows against all {N} weight rows (exact dequantization, "
                      f"fp64 matmul), {len(times)} repetitions, median {med:.2f} s each"}
    print(json.dumps(result), flush=True)


NORM_SOURCES = ("mxfp4_activation_rotation_amd/csrc/mxq_norm.hip", "mxfp4_activation_rotation_amd/csrc/mxq_device.h")
NORM_COUNTERS = "profiles/norm_rotate_quant_bf16_8192x4096_hbm_counters.txt"


def bench_norm(args):
    """RMSNorm + smooth + rotate + MXFP4 in one pass (DuQuant++ page sec. 5.2
    item 1) on the QKV/gate-input shape: bf16 8192 x 4096 residual stream."""
    import numpy as np
    import torch

    import mxfp4_activation_rotation_amd as mxq
    import workloads

    dev = torch.device("cuda:0")
    wl = workloads.norm_workload()
    T, C = wl.x.shape
    step_bytes = T * C * BYTES_PER_ELEM
    n_buf = max(2, int(np.ceil(768e6 / step_bytes)) + 1)
    x0 = wl.x.to(dev)
    xs = [x0] + [x0.clone() for _ in range(n_buf - 1)]
    gamma = torch.from_numpy(wl.gamma).to(dev)
    lam = torch.from_numpy(wl.lam).to(dev)
    r = wl.r_hat.to(dev)
    outs = [(torch.empty((T, C // 2), dtype=torch.uint8, device=dev),
             torch.empty((T, C // 32), dtype=torch.uint8, device=dev)) for _ in range(n_buf)]

    def step(i):
        c, s = outs[i % n_buf]
        mxq.norm_rotate_quant(xs[i % n_buf], r, gamma, None, lam, norm="rms", eps=wl.eps, codes=c, scales=s)

    for i in range(args.warmup):
        step(i)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for i in range(args.steps):
        step(args.warmup + i)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean_launch_s = ev0.elapsed_time(ev1) / 1e3 / args.steps
    achieved = step_bytes / mean_launch_s / 1e9
    value = T * C * args.steps / wall / 1e9
    hbm = read_counters(0, NORM_COUNTERS, NORM_SOURCES)
    result = {
        "metric": "RMSNorm+rotate+MXFP4-quant throughput: Gelem/s",
        "value": round(value, 2), "unit": "Gelem/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "QKV-input shape after RMSNorm: bf16 8192x4096 residual stream (N(0,1), 4 channels "
                               "+-U(50,200) on 0.5% of tokens), gamma U(0.5,1.5), lognormal lambda, seeded "
                               "orthogonal R, eps 1e-5",
                   "tokens": T, "channels": C, "norm": "rms", "lambda": True, "buffer_sets": n_buf,
                   "parallelism": "single GPU", "launch": "eager launches"},
        "hbm_gbps": round(value * BYTES_PER_ELEM, 1),
        "launch_us_mean": round(mean_launch_s * 1e6, 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": None if hbm is None else round(hbm)},
        "kernel_source_hash": kernel_source_hash(NORM_SOURCES),
    }
    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.default()
        rows = 1024
        xs_h = wl.x[:rows]
        times = []
        t_start = time.perf_counter()
        while True:
            t1 = time.perf_counter()
            orc.norm_rotate_quant(xs_h, "rms", wl.gamma, None, wl.eps, wl.lam, wl.r_hat)
            times.append(time.perf_counter() - t1)
            if time.perf_counter() - t_start >= args.cpu_seconds and len(times) >= 3:
                break
        med = statistics.median(times)
        result["cpu_baseline"] = {"value": round(rows * C / med / 1e9, 4), "unit": "Gelem/s",
                                  "cores": orc.num_threads(), "kind": "oracle", "cpu": host_cpu_model(),
                                  "sample": f"the first {rows} rows of the batch, {len(times)} repetitions, "
                                            f"median {med * 1e3:.0f} ms each"}
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--workload", type=int, default=3, choices=[2, 3, 4, 5],
                    help="workload id (3 = the headline down_proj-input batch)")
    ap.add_argument("--buffers", type=int, default=0, help="buffer sets to rotate (0 = enough for > 768 MB)")
    ap.add_argument("--graph", action="store_true",
                    help="capture the K timed launches once as a HIP graph and time one replay "
                         "(how decode-shaped loops are driven; removes per-call host overhead)")
    ap.add_argument("--calibrate", action="store_true",
                    help="time the greedy block calibration (DuQuant++ page sec. 3.2) on a "
                         "page-scale block instead of the quantization path")
    ap.add_argument("--angle-grid", type=int, default=0,
                    help="with --calibrate: choose each candidate's angle from a grid of this many angles "
                         "(1..1024) instead of pi/4")
    ap.add_argument("--gemm", action="store_true",
                    help="time the consumer instead: the W4A4 MXFP4 product of the headline batch's codes "
                         "with absorbed, quantized weights (8192x14336 by 4096x14336)")
    ap.add_argument("--decode", action="store_true",
                    help="with --gemm: a few activation rows (decode), timed against HBM bandwidth")
    ap.add_argument("--rows", type=int, default=None,
                    help="with --gemm: activation rows, the first of the headline batch; with --decode "
                         "1..64 (default 16), otherwise 65..8192 (default 8192)")
    ap.add_argument("--row-layout", action="store_true",
                    help="with --gemm: row-layout operands instead of fragment-tiled ones")
    ap.add_argument("--norm", action="store_true",
                    help="time the norm-fused path instead: RMSNorm + smooth + rotate + MXFP4 on bf16 8192x4096")
    ap.add_argument("--block", type=int, default=0, choices=[0, 16, 32, 64, 128],
                    help="time the block-size variant kernel (DuQuant++ page sec. 4.3 ablation) with a seeded "
                         "random Hadamard block of this size instead of the workload's 32-wide block")
    ap.add_argument("--tiled", action="store_true",
                    help="quantizer output in the fragment-tiled layout (the tiled product's A operand)")
    ap.add_argument("--op", default="rotate", choices=["rotate", "quant", "dequant"],
                    help="rotate: mxq_rotate_quant (the headline); quant: mxq_quant (no smoothing, no "
                         "rotation); dequant: mxq_dequant of the batch's codes to bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra-workloads", action="store_true",
                    help="default run only: skip the extra lines of workloads 2, 4 and 5")
    ap.add_argument("--extra-steps", type=int, default=0,
                    help="timed calls of each extra workload (0 = 2000, 1024 and 400 for workloads 2, 4, 5)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: this path needs no cross-GPU exchange (each GPU quantizes its own "
              f"token shard), so the whole-job rate is the one-GPU rate times the GPU count, and the bench "
              f"does not launch on several GPUs (asked for --gpus {args.gpus}, WORLD_SIZE={world}).",
              file=sys.stderr)
        sys.exit(2)
    if args.decode:
        args.rows = 16 if args.rows is None else args.rows
        if not 1 <= args.rows <= 64:
            ap.error("--rows must be in 1..64 with --decode (the decode-shaped product kernel's range)")
    elif args.rows is not None and not 65 <= args.rows <= 8192:
        ap.error("--rows must be in 65..8192 without --decode (the headline batch has 8192 tokens)")

    import numpy as np
    import torch

    import mxfp4_activation_rotation_amd as mxq
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    mxq.load()
    if args.calibrate:
        bench_calibration(args)
        return
    if args.gemm:
        bench_gemm(args)
        return
    if args.norm:
        bench_norm(args)
        return
    result = time_quant(args, args.workload, args.steps, args.warmup, graph=args.graph)
    default_run = (args.workload == 3 and not (args.block or args.tiled or args.graph) and args.op == "rotate"
                   and not args.no_extra_workloads)
    if default_run:
        # the other seeded workloads of the same path, timed in the same process
        # (fewer steps; each its own buffer rotation and warm-up)
        extra = {}
        for wid, steps in ((2, 2000), (4, 1024), (5, 400)):
            steps = args.extra_steps or steps
            warm = min(args.warmup, 300)
            r = time_quant(args, wid, steps, warm, graph=False, core_only=True)
            if wid == 4:
                g = time_quant(args, wid, steps, warm, graph=True, core_only=True)
                r["graph_launch_us_mean"] = g["launch_us_mean"]
                r["graph_gelem_s"] = g["gelem_s"]
            extra[str(wid)] = r
        result["workloads"] = extra
    if not args.no_cpu_baseline and not args.block and args.op == "rotate":
        import workloads
        result["cpu_baseline"] = cpu_baseline(workloads.make_config(args.workload), args.cpu_seconds)
    print(json.dumps(result), flush=True)


def time_quant(args, wid, steps, warmup, graph=False, core_only=False):
    """Time `steps` calls of the quantize path on workload `wid` (buffer sets
    rotated so each call reads cold data; one event pair around the timed
    calls on the launch stream).  core_only: the per-workload fields only."""
    import numpy as np
    import torch

    import mxfp4_activation_rotation_amd as mxq
    import workloads

    dev = torch.device("cuda:0")
    wl = workloads.make_config(wid)
    call_tokens = workloads.SHAPES[4][0] if wid == 4 else wl.tokens
    C = wl.channels
    elems = call_tokens * C
    step_bytes = elems * BYTES_PER_ELEM

    n_buf = args.buffers or max(2, int(np.ceil(768e6 / step_bytes)) + 1)
    if wid == 4:
        n_buf = wl.tokens // call_tokens  # the 256 distinct decode inputs
    x_all = wl.x.to(dev)
    xs = [x_all[i * call_tokens:(i + 1) * call_tokens] for i in range(n_buf)] if wid == 4 \
        else [x_all] + [x_all.clone() for _ in range(n_buf - 1)]
    lam = torch.from_numpy(wl.lam).to(dev) if wl.lam is not None else None
    r = wl.r_hat.to(dev)
    if args.block:
        r = workloads.bf16_matrix(workloads.random_hadamard(np.random.default_rng(2005 + args.block),
                                                            args.block)).to(dev)
    if args.tiled:
        nc, ns = mxq.tiled_sizes(call_tokens, C)
        outs = [(torch.empty((nc,), dtype=torch.uint8, device=dev), torch.empty((ns,), dtype=torch.uint8, device=dev))
                for _ in range(n_buf)]
    else:
        outs = [(torch.empty((call_tokens, C // 2), dtype=torch.uint8, device=dev),
                 torch.empty((call_tokens, C // 32), dtype=torch.uint8, device=dev)) for _ in range(n_buf)]
    if args.op == "dequant":
        # codes and scales of every buffer set, decoded to bf16 (2.53125 B/elem moved as well:
        # 0.53125 read, 2 written)
        for i in range(n_buf):
            mxq.rotate_quant(xs[i], r, lam, codes=outs[i][0], scales=outs[i][1])
        ys = [torch.empty((call_tokens, C), dtype=torch.bfloat16, device=dev) for _ in range(n_buf)]
    torch.cuda.synchronize()

    def step(i):
        c, s = outs[i % n_buf]
        if args.op == "quant":
            mxq.quant(xs[i % n_buf], codes=c, scales=s)
        elif args.op == "dequant":
            mxq.dequant(c, s, torch.bfloat16, out=ys[i % n_buf])
        elif args.block:
            mxq.rotate_quant_block(xs[i % n_buf], r, lam, codes=c, scales=s)
        elif args.tiled:
            mxq.rotate_quant_tiled(xs[i % n_buf], r, lam, tcodes=c, tscales=s)
        else:
            mxq.rotate_quant(xs[i % n_buf], r, lam, codes=c, scales=s)

    for i in range(warmup):
        step(i)
    hip_graph = None
    if graph:
        # Capture exactly the K timed launches (same buffers, same order).
        torch.cuda.synchronize()
        hip_graph = torch.cuda.CUDAGraph()
        capture_stream = torch.cuda.Stream()
        capture_stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(capture_stream):
            hip_graph.capture_begin()
            for i in range(steps):
                step(warmup + i)
            hip_graph.capture_end()
        torch.cuda.current_stream().wait_stream(capture_stream)
        hip_graph.replay()  # one untimed replay after capture
    # One event pair brackets the timed region on the launch stream (the
    # binding launches on torch's current stream); events between launches
    # would add several microseconds of queue work to every step.
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    if hip_graph is not None:
        hip_graph.replay()
    else:
        for i in range(steps):
            step(warmup + i)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean_launch_s = ev0.elapsed_time(ev1) / 1e3 / steps

    achieved = step_bytes / mean_launch_s / 1e9
    value = elems * steps / wall / 1e9
    hbm = None if (args.block or args.tiled or args.op != "rotate") else read_counters(wid)
    core = {
        "workload": WORKLOAD_NAMES[wid], "tokens": call_tokens, "channels": C,
        "x_dtype": str(wl.x.dtype).replace("torch.", ""), "lambda": wl.lam is not None,
        "steps": steps, "gelem_s": round(value, 2), "hbm_gbps": round(value * BYTES_PER_ELEM, 1),
        "launch_us_mean": round(mean_launch_s * 1e6, 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": None if hbm is None else round(hbm)},
    }
    if wid == 4 and not graph:
        # decode-shaped calls: per-call latency, each call bracketed by its own
        # event pair (outside the timed region above)
        lat = []
        for i in range(n_buf):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            step(i)
            e1.record()
            e1.synchronize()
            lat.append(e0.elapsed_time(e1) * 1e3)
        core["call_latency_us"] = {"p50": round(float(np.percentile(lat, 50)), 2),
                                   "p99": round(float(np.percentile(lat, 99)), 2), "calls": len(lat)}
        core["aggregate_gbps"] = core["hbm_gbps"]
    if core_only:
        return core
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "Gelem/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(wall / steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.x.dtype == torch.bfloat16 else "fp16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[wid], "tokens": call_tokens, "channels": C,
                   "x_dtype": str(wl.x.dtype).replace("torch.", ""), "lambda": wl.lam is not None,
                   "r_hat": (f"seeded random Hadamard {args.block}x{args.block} (block-size variant kernel)"
                             if args.block else "bf16 32x32"),
                   "buffer_sets": n_buf, "parallelism": "single GPU",
                   "output_layout": "fragment-tiled records" if args.tiled else "row layout",
                   "launch": "hip graph of the K launches" if graph else "eager launches"},
        "hbm_gbps": core["hbm_gbps"],
        "pct_hbm_peak": round(100 * value * BYTES_PER_ELEM / HBM_PEAK_GBPS, 2),
        "launch_us_mean": core["launch_us_mean"],
        "roofline": core["roofline"],
        "kernel_source_hash": kernel_source_hash(),
    }
    for k in ("call_latency_us",):
        if k in core:
            result[k] = core[k]
    if args.block:
        result["kernel_source_hash"] = kernel_source_hash(("mxfp4_activation_rotation_amd/csrc/mxq_block.hip",
                                                           "mxfp4_activation_rotation_amd/csrc/mxq_device.h"))
    if args.op != "rotate":
        result["metric"] = ("plain MXFP4 quantization (mxq_quant) throughput: Gelem/s" if args.op == "quant"
                            else "MXFP4 dequantization to bf16 (mxq_dequant) throughput: Gelem/s")
        result["config"]["op"] = args.op
        result["kernel_source_hash"] = kernel_source_hash()
    return result


if __name__ == "__main__":
    main()
