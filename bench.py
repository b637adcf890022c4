"""Benchmark of the fused contraction + bias + activation on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one fused gemm_bias_act call over the resident inputs of the
workload (default: M = N = K = 4096, bf16 operands, fp32 bias, ReLU, bf16
output).  W untimed steps, then exactly K timed steps between two
synchronisations; rank 0 prints one JSON line.

Besides the headline, the line carries:
  roofline      the dominant kernel's achieved TFLOP/s (algorithmic flops per
                launch / mean launch time from HIP events on the launch stream)
                against the dense bf16 MFMA peak;
  cpu_baseline  the fp64 CPU oracle timed on a bounded sample of the same
                workload (a subset of output rows), on this host's cores;
  others        every workload, fused and two-kernel: eager back-to-back steps
                (mean), HIP-graph replays of R steps (median and minimum of 20
                trials, no host call cost), and for the HBM-bound workloads
                single steps after a 512 MiB cache flush; `tuned_path` is the
                path the library's own tuner records for the workload;
                `cpu_oracle` the fp64 oracle's rate on a bounded sample of
                it, on all host threads (and on one, for the small workloads);
  path_rule     the static fused-vs-two-kernel rule's case (the 4096^3 GEMM
                with a misaligned output): fused, two-kernel and auto calls;
  launch_floor  the per-call time of a trivial kernel on the same stream
                (eager and graph replays), next to which the latency-bound
                small workloads are read.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# dense MFMA, MI355X datasheet (int8: TOP/s)
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3, "i8": 5033.2}
PEAK_HBM_GBS = 8000.0

# Sources that define each kernel; a committed HBM-traffic record carries
# their hash and is reported only while they are unchanged.
KERNEL_SOURCES = {   # each kernel's source and every header it includes
    "gemm16_pp_kernel": ["gemm_pp.hpp", "epilogue.hpp", "device_common.hpp", "gemm_args.hpp",
                         "tile_map.hpp", "launch_kernel.hpp"],
    "conv16_halo_kernel": ["conv_halo.hpp", "epilogue.hpp", "launch.hpp", "launch_kernel.hpp",
                           "mfma_core.hpp", "device_common.hpp", "gemm_args.hpp", "tile_map.hpp"],
    "conv32_halo_kernel": ["conv_halo32.hpp", "epilogue.hpp", "launch.hpp", "launch_kernel.hpp",
                           "mfma_core.hpp", "device_common.hpp", "gemm_args.hpp", "tile_map.hpp"],
    "gemm_bias_act_kernel": ["kernels_impl.hpp", "mfma_core.hpp", "epilogue.hpp", "launch.hpp",
                             "launch_kernel.hpp", "device_common.hpp", "gemm_args.hpp", "tile_map.hpp"],
    "conv_bias_act_kernel": ["kernels_impl.hpp", "mfma_core.hpp", "epilogue.hpp", "launch.hpp",
                             "launch_kernel.hpp", "device_common.hpp", "gemm_args.hpp", "tile_map.hpp"],
}
TRAFFIC_RECORDS = os.path.join(ROOT, "profiles", "hbm_traffic.json")
TWO_KERNEL = "two-kernel: "


def kernel_name(desc: str) -> str:
    """Kernel function behind a last_tile_config() description (the first
    kernel of a two-kernel call)."""
    if desc.startswith(TWO_KERNEL):
        desc = desc[len(TWO_KERNEL):]
    if "ping-pong" in desc:
        return "gemm16_pp_kernel"
    if desc.startswith("conv-halo fp32"):
        return "conv32_halo_kernel"
    if desc.startswith("conv-halo"):
        return "conv16_halo_kernel"
    return "gemm_bias_act_kernel" if desc.startswith("gemm") else "conv_bias_act_kernel"


def kernel_fingerprint(kernel: str = "gemm16_pp_kernel") -> str:
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "conv_bias_activation_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(workload: str, tile: str, path: str):
    """HBM bytes per launch from the committed counter records (FETCH_SIZE and
    WRITE_SIZE scaled by a plain copy of known size) for this workload, kernel
    and tile (its last_tile_config() description) and path, or None if there
    is no such record or it was taken on other kernel sources."""
    try:
        with open(TRAFFIC_RECORDS) as f:
            recs = json.load(f)
    except (OSError, ValueError):
        return None
    kernel = kernel_name(tile)
    for rec in recs:
        if (rec.get("workload") == workload and rec.get("tile") == tile and
                rec.get("path", "fused") == path and rec.get("kernel") == kernel and
                rec.get("kernel_sources_sha256") == kernel_fingerprint(kernel)):
            return rec.get("bytes_per_launch")
    return None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="gemm_relu_4096_bf16")
    ap.add_argument("--no-others", action="store_true", help="skip the other workloads")
    ap.add_argument("--halo-variant", type=int, default=-1,
                    help="force the fp16/bf16 conv-halo variant (0 widest, 1 and 2 two per CU, 3 and 4 eight waves; -1 auto)")
    ap.add_argument("--path", choices=("fused", "2k"), default="fused",
                    help="time the fused kernel (default) or the two-kernel ablation for --workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target oracle sample time")
    ap.add_argument("--tile", type=int, default=-1, help="force a tile config (tuning)")
    ap.add_argument("--fingerprint", default=None, metavar="KERNEL",
                    help="print the source hash of a kernel (e.g. gemm16_pp_kernel) and exit")
    ap.add_argument("--launch-floor", action="store_true",
                    help="only measure the trivial-kernel launch floor (eager and graph replays) and exit")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a device copy of 256 MiB (read 256 MiB + write 256 MiB) --steps "
                         "times; its FETCH_SIZE / WRITE_SIZE counters scale the kernel's counters "
                         "to bytes")
    return ap.parse_args()


def to_device(words, dt):
    import torch
    if dt == "f32":
        return torch.from_numpy(np.ascontiguousarray(words).view(np.float32)).cuda()
    if dt in ("i8", "i32"):
        return torch.from_numpy(np.ascontiguousarray(words).view(np.int8 if dt == "i8" else np.int32)).cuda()
    t = torch.from_numpy(np.ascontiguousarray(words).view(np.int16))
    return t.view({"f16": torch.float16, "bf16": torch.bfloat16}[dt]).cuda()


def make_step(case, seed=0, path="fused"):
    """Returns (step_fn, n_kernel_launches) for one workload with resident inputs."""
    import torch
    import conv_bias_activation_amd as ba
    import workloads as wl
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "i32": torch.int32}
    if isinstance(case, wl.GemmCase):
        inp = wl.gen_gemm(case, seed)
        A = to_device(inp["A"].reshape(case.M, case.K), case.in_dtype)
        B = to_device(inp["B"].reshape(case.K, case.N), case.in_dtype)
        bias = None if inp["bias"] is None else to_device(inp["bias"], case.bias_dtype)
        C = torch.empty((case.M, case.N), dtype=tdt[case.out_dtype], device="cuda")
        alpha = float(np.float32(case.alpha))
        R = None if inp.get("R") is None else to_device(inp["R"].reshape(case.M, case.N),
                                                        case.out_dtype)
        if path == "fused":
            if R is not None:
                return (lambda: ba.gemm_bias_add_act(A, B, bias, R, C, case.act, alpha)), 1
            return (lambda: ba.gemm_bias_act(A, B, bias, C, case.act, alpha)), 1
        ws = torch.empty(ba.gemm_bias_act_workspace_size(case.M, case.N) // 4, dtype=torch.float32,
                         device="cuda")
        if R is not None:
            return (lambda: ba.gemm_bias_add_act_2k(A, B, bias, R, C, case.act, alpha,
                                                    workspace=ws)), 2
        return (lambda: ba.gemm_bias_act_2k(A, B, bias, C, case.act, alpha, workspace=ws)), 2
    inp = wl.gen_conv(case, seed)
    x = to_device(inp["x"].reshape(case.N, case.C, case.H, case.W), case.in_dtype)
    w = to_device(inp["w"].reshape(case.Co, case.C, case.kh, case.kw), case.in_dtype)
    bias = None if inp["bias"] is None else to_device(inp["bias"], case.bias_dtype)
    Ho, Wo = case.out_hw()
    y = torch.empty((case.N, case.Co, Ho, Wo), dtype=tdt[case.out_dtype], device="cuda")
    args = (case.strides, case.pads, case.dilations, case.act)
    R = None if inp.get("R") is None else to_device(inp["R"].reshape(case.N, case.Co, Ho, Wo),
                                                    case.out_dtype)
    if path == "fused":
        if R is not None:
            return (lambda: ba.conv2d_bias_add_act(x, w, bias, R, y, *args)), 1
        return (lambda: ba.conv2d_bias_act(x, w, bias, y, *args)), 1
    n = ba.conv2d_bias_act_workspace_size(case.N, case.C, case.H, case.W, case.Co, case.kh, case.kw,
                                          case.strides, case.pads, case.dilations)
    ws = torch.empty(n // 4, dtype=torch.float32, device="cuda")
    if R is not None:
        return (lambda: ba.conv2d_bias_add_act_2k(x, w, bias, R, y, *args, workspace=ws)), 2
    return (lambda: ba.conv2d_bias_act_2k(x, w, bias, y, *args, workspace=ws)), 2


def tune_case(case, reps=20):
    """The library's own fused-vs-two-kernel choice for this workload
    (biasact_tune_*: both paths timed on these buffers, the faster recorded)."""
    import torch
    import conv_bias_activation_amd as ba
    import workloads as wl
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "i32": torch.int32}
    if isinstance(case, wl.GemmCase):
        if case.dist_r:
            return None                      # the residual entry points are not tuned
        inp = wl.gen_gemm(case, 0)
        A = to_device(inp["A"].reshape(case.M, case.K), case.in_dtype)
        B = to_device(inp["B"].reshape(case.K, case.N), case.in_dtype)
        bias = None if inp["bias"] is None else to_device(inp["bias"], case.bias_dtype)
        C = torch.empty((case.M, case.N), dtype=tdt[case.out_dtype], device="cuda")
        ws = torch.empty(ba.gemm_bias_act_workspace_size(case.M, case.N) // 4, dtype=torch.float32,
                         device="cuda")
        return ba.tune_gemm(A, B, bias, C, case.act, float(np.float32(case.alpha)), workspace=ws,
                            reps=reps)
    if case.dist_r:
        return None
    inp = wl.gen_conv(case, 0)
    x = to_device(inp["x"].reshape(case.N, case.C, case.H, case.W), case.in_dtype)
    w = to_device(inp["w"].reshape(case.Co, case.C, case.kh, case.kw), case.in_dtype)
    bias = None if inp["bias"] is None else to_device(inp["bias"], case.bias_dtype)
    Ho, Wo = case.out_hw()
    y = torch.empty((case.N, case.Co, Ho, Wo), dtype=tdt[case.out_dtype], device="cuda")
    n = ba.conv2d_bias_act_workspace_size(case.N, case.C, case.H, case.W, case.Co, case.kh, case.kw,
                                          case.strides, case.pads, case.dilations)
    ws = torch.empty(n // 4, dtype=torch.float32, device="cuda")
    return ba.tune_conv(x, w, bias, y, case.strides, case.pads, case.dilations, case.act,
                        workspace=ws, reps=reps)


def time_steps(step, steps, warmup):
    """Mean ms per step over `steps` back-to-back steps, measured with HIP
    events recorded on the stream the library launches on (torch's current
    stream), between two device synchronisations."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(s)
    for _ in range(steps):
        step()
    e1.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


def _rates(case, ms):
    tf = case.flops / (ms * 1e-3) / 1e12
    gbs = case.alg_bytes / (ms * 1e-3) / 1e9
    return {"tflops": round(tf, 2), "frac_mfma": round(tf / PEAK_TFLOPS[case.in_dtype], 4),
            "alg_GBs": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}


def graph_trials(step, eager_ms, trials=20, min_trial_ms=1.0):
    """Device throughput without the host's per-call cost: R steps captured in
    one HIP graph (R chosen so one replay lasts >= min_trial_ms), `trials`
    replays each timed with HIP events; per-step median and minimum."""
    import torch
    R = int(max(1, min(500, -(-min_trial_ms // max(eager_ms, 1e-4)))))
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for _ in range(R):
                step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g.replay()
    g.replay()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    times = []
    for _ in range(trials):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        g.replay()
        e1.record(s)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / R)
    del g
    return R, float(np.median(times)), float(np.min(times))


def cold_trials(step, trials=20, flush_bytes=512 << 20):
    """Single steps after writing a buffer larger than the 256 MB last-level
    cache (which also evicts the L2s): inputs come from HBM.  The flush kernel
    is still running while the host queues the step, so the events bracket the
    step's kernels only."""
    import torch
    scratch = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream()
    times = []
    for t in range(trials + 2):
        scratch.fill_(t & 0xFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        step()
        e1.record(s)
        torch.cuda.synchronize()
        if t >= 2:
            times.append(e0.elapsed_time(e1))
    del scratch
    return float(np.median(times)), float(np.min(times))


# workloads whose roofline is HBM (or launch latency): also timed from a cold cache
COLD_WORKLOADS = ("gemm_leaky_1024x640x256_f16", "conv3x3_tanh_8x64x56_f16")


def measure_case(case, path, min_ms=200.0):
    """Eager back-to-back steps (mean, host call cost included), then graph
    replays (median / min per step, device time), and for the HBM-bound
    workloads single cold-cache steps."""
    step, nk = make_step(case, 0, path)
    ms1, _ = time_steps(step, 5, 3)
    reps = int(max(10, min(2000, min_ms / max(ms1, 1e-3))))
    ms, _ = time_steps(step, reps, 5)
    import conv_bias_activation_amd as ba
    out = {"ms": round(ms, 5), **_rates(case, ms), "kernels": nk, "tile": ba.last_tile_config()}
    R, med, mn = graph_trials(step, ms)
    out["graph"] = {"steps_per_replay": R, "trials": 20, "median_ms": round(med, 5),
                    "min_ms": round(mn, 5), **_rates(case, med)}
    if case.name in COLD_WORKLOADS:
        cmed, cmn = cold_trials(step)
        out["cold"] = {"trials": 20, "median_ms": round(cmed, 5), "min_ms": round(cmn, 5),
                       **_rates(case, cmed)}
    return out


def launch_floor():
    """Per-call time of the smallest kernel torch launches (an in-place add on
    64 floats) on this stream, eager back-to-back and in graph replays: the
    launch and scheduling floor that a latency-bound call cannot go below."""
    import torch
    t = torch.zeros(64, dtype=torch.float32, device="cuda")
    step = lambda: t.add_(1.0)
    ms, _ = time_steps(step, 2000, 50)
    R, med, mn = graph_trials(step, ms)
    return {"kernel": "torch add_ on 64 floats", "eager_ms": round(ms, 5),
            "graph_median_ms": round(med, 5), "graph_min_ms": round(mn, 5), "steps_per_replay": R}


def path_rule_case():
    """The static fused-vs-two-kernel rule's case: the 4096^3 bf16 GEMM + ReLU
    with C two bytes off its allocation (not aligned for 4-element accesses).
    Device time per call (graph replays) of the fused call, the two-kernel
    call and the auto call (which applies the rule), with the kernel each
    launched."""
    import torch
    import conv_bias_activation_amd as ba
    import workloads as wl
    case = wl.CASES["gemm_relu_4096_bf16"]
    inp = wl.gen_gemm(case, 0)
    A = to_device(inp["A"].reshape(case.M, case.K), "bf16")
    B = to_device(inp["B"].reshape(case.K, case.N), "bf16")
    bias = to_device(inp["bias"], "f32")
    buf = torch.empty(case.M * case.N + 1, dtype=torch.bfloat16, device="cuda")
    C = buf[1:].view(case.M, case.N)
    ws = torch.empty(case.M * case.N, dtype=torch.float32, device="cuda")
    calls = {"fused": lambda: ba.gemm_bias_act(A, B, bias, C, "relu"),
             "2k": lambda: ba.gemm_bias_act_2k(A, B, bias, C, "relu", workspace=ws),
             "auto": lambda: ba.gemm_bias_act_auto(A, B, bias, C, "relu", workspace=ws)}
    # the tuner may have recorded a path for this problem (with an aligned C);
    # forget it so the auto call applies the static rule
    ba.set_gemm_path(case.M, case.N, case.K, ba.dtypes_code("bf16", "bf16", "f32", "bf16"), "relu", None)
    out = {"workload": case.name + ", C misaligned by 2 bytes",
           "static_path": ba.gemm_static_path(A, B, bias, C, "relu", workspace=ws)}
    for name, step in calls.items():
        ms, _ = time_steps(step, 20, 5)
        out[name] = {"tile": ba.last_tile_config()}
        R, med, mn = graph_trials(step, ms)
        out[name].update({"graph_median_ms": round(med, 5), "graph_min_ms": round(mn, 5),
                          **_rates(case, med)})
    del buf, ws
    return out


# workloads whose oracle is also timed on one thread (the small and conv
# configurations; the large GEMMs only with all threads)
ONE_THREAD_WORKLOADS = ("gemm_leaky_1024x640x256_f16", "conv3x3_tanh_8x64x56_f16",
                        "conv7x7s2_tanh_16x3x224_f32", "conv1x1s2_tanh_16x256x56_f32",
                        "conv3x3d2_tanh_32x128x28_bf16")


def _scaled(run, n, limit, target_s):
    """Grows the sample n (up to limit) until run(n) takes about target_s."""
    dt, fl = run(n)
    for _ in range(3):
        if dt >= 0.5 * target_s or n >= limit:
            break
        n = int(min(limit, max(n + 1, n * target_s / max(dt, 1e-6))))
        dt, fl = run(n)
    return n, dt, fl


def oracle_timing(case, target_s=0.5, threads=None):
    """The fp64 oracle (contraction + bias + activation) on a bounded sample of
    the workload: leading output rows (GEMM) or sampled output elements
    (conv), sized from a short calibration run to take about target_s."""
    import oracle as orc
    import workloads as wl
    O = orc.Oracle()
    full_threads = O.num_threads()
    nt = threads or full_threads
    O.set_num_threads(nt)
    try:
        if isinstance(case, wl.GemmCase):
            inp = wl.gen_gemm(case, 0)
            B = O.decode(inp["B"], case.in_dtype).reshape(case.K, case.N)
            bias = O.decode(inp["bias"], case.bias_dtype) if inp["bias"] is not None else None
            Aw = inp["A"].reshape(case.M, case.K)

            def run(rows):
                A = O.decode(Aw[:rows], case.in_dtype)
                t0 = time.perf_counter()
                O.gemm(A, B, bias, case.act, orc.f32(case.alpha))
                return time.perf_counter() - t0, 2.0 * rows * case.N * case.K

            rows, dt, fl = _scaled(run, max(1, nt), case.M, target_s)
            sample = f"{rows} of {case.M} output rows"
        else:
            inp = wl.gen_conv(case, 0)
            x = O.decode(inp["x"], case.in_dtype).reshape(case.N, case.C, case.H, case.W)
            w = O.decode(inp["w"], case.in_dtype).reshape(case.Co, case.C, case.kh, case.kw)
            bias = O.decode(inp["bias"], case.bias_dtype) if inp["bias"] is not None else None
            Ho, Wo = case.out_hw()
            total = case.N * case.Co * Ho * Wo
            kflops = 2.0 * case.C * case.kh * case.kw

            def run(n):
                idx = wl.sample_indices(total, n, 0)
                t0 = time.perf_counter()
                O.conv2d_elems(x, w, bias, case.strides, case.pads, case.dilations, idx, case.act)
                return time.perf_counter() - t0, kflops * idx.size

            n, dt, fl = _scaled(run, 256 * max(1, nt), total, target_s)
            sample = f"{n} of {total} output elements"
    finally:
        O.set_num_threads(full_threads)
    return {"threads": nt, "seconds": round(dt, 3), "gflops_fp64": round(fl / dt / 1e9, 3),
            "sample": sample + " (contraction, bias and activation; inputs decoded beforehand)"}


def cpu_baseline(case, target_s):
    """The oracle as it stands, on a subset of the workload's output rows."""
    import oracle as orc
    import workloads as wl
    O = orc.Oracle()
    if not isinstance(case, wl.GemmCase):
        return None
    inp = wl.gen_gemm(case, 0)
    A = O.decode(inp["A"], case.in_dtype).reshape(case.M, case.K)
    B = O.decode(inp["B"], case.in_dtype).reshape(case.K, case.N)
    bias = O.decode(inp["bias"], case.bias_dtype) if inp["bias"] is not None else None
    rows = max(1, O.num_threads())
    t0 = time.perf_counter()
    O.gemm(A[:rows], B, bias, case.act, orc.f32(case.alpha))
    t1 = time.perf_counter() - t0
    rows = int(min(case.M, max(rows, rows * target_s / max(t1, 1e-6))))
    rows -= rows % max(1, O.num_threads()) if rows > O.num_threads() else 0
    t0 = time.perf_counter()
    O.gemm(A[:rows], B, bias, case.act, orc.f32(case.alpha))
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * case.N * case.K
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": O.num_threads(),
            "kind": "oracle",
            "sample": f"{rows} of {case.M} output rows of {case.name} (full K and N), fp64, "
                      f"{dt:.1f} s wall; inputs decoded beforehand",
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model()}


def main():
    args = _parse()
    if args.fingerprint:
        print(kernel_fingerprint(args.fingerprint))
        return
    if args.gpus != 1:
        print(json.dumps({"error": f"--gpus {args.gpus}: this benchmark runs on exactly one GPU; "
                                   "the fused kernel shards by rows/columns with no exchange, so "
                                   "N GPUs would each run this same step on 1/N of the rows"}))
        sys.exit(2)
    import torch
    if args.calibrate_copy:
        n = 256 << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": n, "calibrate_copy_bytes_written": n,
                          "launches": args.steps}), flush=True)
        return
    if args.launch_floor:
        print(json.dumps({"launch_floor": launch_floor()}), flush=True)
        return
    import conv_bias_activation_amd as ba
    import workloads as wl

    case = wl.CASES[args.workload] if args.workload in wl.CASES else wl.FILTER_CASES[args.workload]
    if args.tile >= 0:
        ba.force_tile_config(args.tile)
    if args.halo_variant >= 0:
        ba.force_halo_variant(args.halo_variant)
    step, _ = make_step(case, 0, args.path)
    ms, wall = time_steps(step, args.steps, args.warmup)
    tflops = case.flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[case.in_dtype]
    if isinstance(case, wl.GemmCase):
        cfg = {"workload": case.name, "M": case.M, "N": case.N, "K": case.K,
               "in": case.in_dtype, "bias": case.bias_dtype, "out": case.out_dtype, "act": case.act}
    else:
        cfg = {"workload": case.name, "in": case.in_dtype, "out": case.out_dtype, "act": case.act}
    cfg["tile"] = ba.last_tile_config()
    if args.path != "fused":
        cfg["path"] = args.path
    if args.halo_variant >= 0:
        cfg["halo_variant"] = args.halo_variant
    line = {
        "metric": "TFLOP/s of fused act(A\u00b7B+bias) and conv2d+tanh; % of MI355X MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.in_dtype,
        "data": "synthetic (seeded PCG64 inputs of the workload's shape and distribution)",
        "config": cfg,
        "frac_of_peak": round(tflops / peak, 4),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4),
                     "traffic": measured_traffic(case.name, cfg["tile"], args.path),
                     "kernel": kernel_name(cfg["tile"]),
                     "per_launch_flops": case.flops,
                     "mean_launch_ms": round(ms, 5)},
        "wall_s_timed": round(wall, 3),
    }
    if not args.no_others:
        others = {}
        for name, c in wl.CASES.items():
            entry = {}
            for path in ("fused", "2k"):
                if path == "2k" and c.in_dtype == "i8":
                    entry[path] = {"skipped": "int8 GEMMs run the fused path only"}
                    continue
                try:
                    entry[path] = measure_case(c, path)
                except Exception as e:  # report, never hide
                    entry[path] = {"error": repr(e)}
            try:
                entry["tuned_path"] = tune_case(c)
            except Exception as e:  # report, never hide
                entry["tuned_path"] = {"error": repr(e)}
            if not args.no_cpu_baseline:
                try:
                    entry["cpu_oracle"] = oracle_timing(c)
                    if name in ONE_THREAD_WORKLOADS:
                        entry["cpu_oracle_1thread"] = oracle_timing(c, threads=1)
                except Exception as e:  # report, never hide
                    entry["cpu_oracle"] = {"error": repr(e)}
            others[name] = entry
            torch.cuda.empty_cache()
        line["others"] = others
        # 16-bit convs with 5x5 and 7x7 filters (not named workloads)
        larger = {}
        for name, c in wl.FILTER_CASES.items():
            try:
                larger[name] = measure_case(c, "fused")
            except Exception as e:  # report, never hide
                larger[name] = {"error": repr(e)}
        line["larger_filters"] = larger
        try:
            line["launch_floor"] = launch_floor()
        except Exception as e:  # report, never hide
            line["launch_floor"] = {"error": repr(e)}
        try:
            line["path_rule"] = path_rule_case()
        except Exception as e:  # report, never hide
            line["path_rule"] = {"error": repr(e)}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
