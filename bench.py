#!/usr/bin/env python3
"""Achieved HBM bandwidth of the fused memory-bound kernels on one MI355X.

One step = one pass of every kernel of the hot path over the large
workloads, each with inputs resident in HBM:
  C3   fused chain 0.5 * GELU(x + 1), fp32, 8,388,608 elements
  C4   row softmax bf16, 32768 x 4096 (single-pass, rows on chip)
  C5a  row softmax fp32, 1024 x 131072 (rows wider than one workgroup: slices
       exchanging partial max / sum, a caller workspace allocated untimed)
  C5b  tanh-GELU bf16, 2^30 elements
Algorithmic bytes = one read + one write of every element ("Lecture 6: GPU
Kernels and Triton", section 9.3: bandwidth utilisation = bytes moved /
time / peak). ``value`` = total algorithmic bytes of the K timed steps /
wall time between two device synchronisations, in GB/s (1e9 B/s).

Per-kernel durations come from HIP events recorded on the launch stream
around every launch of K further steps (not the timed ones: the events
would add to the step). Each kernel is also set against a plain copy of
its own bytes (``copy_same_bytes_ms``, ``frac_of_copy``), timed the same way
in K steps of copies: a copy's rate depends on its size. The CPU baseline
repeats the oracle over whole steps on the host's cores for at least 10 s.

Prints ONE JSON line. ``--gpus`` above 1 is refused: the build measures one
GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published
STEP = ("C3", "C4", "C5a", "C5b")
TRAFFIC_FILE = ROOT / "profiles" / "traffic.json"
KERNEL_SOURCES = ("device_common.hpp", "ew_kernels.hpp", "softmax_kernels.hpp", "elementwise.hip",
                  "softmax.hip")
# Kernel-name fragments (as rocprofv3 prints them) of each workload's kernel.
KERNEL_NAMES = {
    "C3": ("ew_vec_kernel<fk::IoF32", "AffActAffOp"),
    "C4": ("softmax_reg_kernel<fk::IoBF16",),
    "C5a": ("softmax_split_kernel<fk::IoF32",),
    "C5b": ("ew_vec_kernel<fk::IoBF16", "GeluOp"),
    "copy": ("copy_vec_kernel",),
    "layernorm_gelu": ("layernorm_reg_kernel<fk::IoBF16",),
    "gelu_backward": ("ew2_vec_kernel<fk::IoBF16", "GeluBwdOp"),
    "softmax_backward": ("softmax_bwd_reg_kernel<fk::IoBF16",),
    "online_c5a": ("softmax_rolling_kernel<fk::IoF32",),
}
# Next-row kernels in the counter run (bytes per launch: one read of each
# input, one write of the output; gamma and beta of the LayerNorm once).
EXTRA = ("layernorm_gelu", "gelu_backward", "softmax_backward", "online_c5a")
EXTRA_BYTES = {"layernorm_gelu": 2 * 32768 * 4096 * 2 + 2 * 4096 * 2,
               "gelu_backward": 3 * (1 << 30) * 2,
               "softmax_backward": 3 * 32768 * 4096 * 2,
               "online_c5a": 2 * 1024 * 131072 * 4}
CPU_BASELINE_MIN_SECONDS = 10.0
WARM_SECONDS = 0.1      # launches before each extras measurement (clocks up)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        h.update((ROOT / "memory_bound_elementwise_fk_amd" / "csrc" / name).read_bytes())
    return h.hexdigest()[:16]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (e.g. under a profiler)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the copy ceiling and the unfused-chain comparison")
    ap.add_argument("--counters-run", action="store_true",
                    help="launch each kernel of the step twice plus a 1 GiB calibration copy, "
                         "nothing else (for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE passes)")
    ap.add_argument("--profile-run", action="store_true",
                    help="launch each next-row kernel twice on the extras' shapes (Linear + GELU "
                         "bf16 8192x16384x4096, attention B4 H32 T4096 d128 full and causal, "
                         "LayerNorm + GELU bf16 32768x4096, C5a through the online path), "
                         "nothing else (for rocprofv3 --pmc passes of SQ counters)")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn the two rocprofv3 counter_collection.csv files of a "
                         "--counters-run into profiles/traffic.json and exit")
    return ap.parse_args()


def main() -> int:
    args = parse()
    if args.ingest_counters:
        return ingest_counters(*args.ingest_counters)
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(every kernel here runs on one GPU's share of the data).", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    from memory_bound_elementwise_fk_amd import LIB_PATH

    if not LIB_PATH.exists():
        import __graft_entry__

        __graft_entry__.build()
    import memory_bound_elementwise_fk_amd as fk
    from memory_bound_elementwise_fk_amd import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    # ---- inputs resident in HBM, outputs preallocated
    log("generating inputs")
    host = {name: wl.make_input(name) for name in STEP}
    xs = {name: wl.to_torch(a, "cuda:0") for name, a in host.items()}
    ys = {name: torch.empty_like(t) for name, t in xs.items()}
    torch.cuda.synchronize()

    # C5a rows are wider than one workgroup: the split path exchanges partial
    # statistics through a caller workspace (any contents), allocated here
    # once (untimed)
    ws_bytes = fk.fk_softmax_workspace_bytes(*xs["C5a"].shape, xs["C5a"].dtype)
    ws = torch.empty(max(ws_bytes, 8), dtype=torch.uint8, device=dev)
    launches = {
        "C3": lambda: fk.fk_elementwise_chain(xs["C3"], ys["C3"], wl.CHAIN_C3),
        "C4": lambda: fk.fk_softmax_rows(xs["C4"], ys["C4"]),
        "C5a": lambda: fk.fk_softmax_rows_ws(xs["C5a"], ys["C5a"], ws),
        "C5b": lambda: fk.fk_gelu_tanh(xs["C5b"], ys["C5b"]),
    }
    if args.counters_run:
        return counters_run(fk, torch, launches, xs, ys)
    if args.profile_run:
        return profile_run(fk, torch, xs, ys)
    kbytes = {name: wl.algorithmic_bytes(name) for name in STEP}
    step_bytes = sum(kbytes.values())

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        for name in STEP:
            launches[name]()
    torch.cuda.synchronize()

    # ---- timed region: K steps between two synchronisations, nothing else
    # enqueued (events around every launch would add ~5 % to the step)
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for name in STEP:
            launches[name]()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0

    # ---- per-kernel durations: K more steps with HIP events recorded on the
    # launch stream around every launch
    ev = {name: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(args.steps)] for name in STEP}
    for k in range(args.steps):
        for name in STEP:
            a, b = ev[name][k]
            a.record(stream)
            launches[name]()
            b.record(stream)
    torch.cuda.synchronize()
    launch_ms = {name: sorted(a.elapsed_time(b) for a, b in ev[name]) for name in STEP}
    per_kernel_ms = {name: sum(t) / args.steps for name, t in launch_ms.items()}
    value = step_bytes * args.steps / wall / 1e9
    log(f"step {wall / args.steps * 1e3:.3f} ms, {value:.1f} GB/s")

    kernels = {}
    for name in STEP:
        ms = per_kernel_ms[name]
        gbs = kbytes[name] / (ms * 1e-3) / 1e9
        t = launch_ms[name]
        med = t[len(t) // 2] if len(t) % 2 else 0.5 * (t[len(t) // 2 - 1] + t[len(t) // 2])
        kernels[name] = {"ms": round(ms, 5), "median_ms": round(med, 5), "min_ms": round(t[0], 5),
                         "bytes": kbytes[name], "GBps": round(gbs, 1),
                         "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4)}
    # a pair of events around one ~12 us launch adds a few microseconds of
    # its own; the dispatch timestamps of a kernel trace are the figure to
    # use for that kernel (and the equal-size copy below carries the same)
    kernels["C3"]["note"] = ("events add a few us to a launch this short: the kernel trace's dispatch "
                             "timestamps are authoritative for it (also see frac_of_copy, timed alike)")

    # ---- parity spot check of what was timed (full checks live in tests/)
    spot = spot_check(host, ys, wl)
    log(f"spot check: {spot}")

    # ---- each kernel's own ceiling: K more steps in which every kernel is
    # replaced by a plain 16-byte copy of its bytes (its input read once, the
    # same number of bytes written), timed the same way. A copy's rate depends
    # on its size (a short one pays its launch and pipeline fill), so each
    # kernel is set against the copy of equal size; this overwrites the
    # outputs, which is why it runs after the spot check
    copy_ms = copy_steps(fk, torch, xs, ys, stream, args.steps)
    for name in STEP:  # the step's outputs again (the extras reuse them)
        launches[name]()
    torch.cuda.synchronize()
    for name in STEP:
        kernels[name]["copy_same_bytes_ms"] = round(copy_ms[name], 5)
        kernels[name]["frac_of_copy"] = round(copy_ms[name] / per_kernel_ms[name], 4)

    extras = {}
    if not args.no_extras:
        extras = measure_extras(fk, wl, torch, xs, ys, stream)

    dominant = max(STEP, key=lambda n: per_kernel_ms[n])
    achieved = kbytes[dominant] / (per_kernel_ms[dominant] * 1e-3) / 1e9
    roofline = {"bound": "hbm", "kernel": dominant, "achieved": round(achieved, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": traffic_bytes(dominant)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(host, kbytes)

    result = {
        "metric": "achieved HBM GB/s (% of ~8 TB/s peak) for fused GELU/chain and row softmax",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded PCG64 chunks; sizes and distributions of the five workloads)",
        "config": {
            "workload": "one step = C3 chain fp32 8,388,608 + C4 softmax bf16 32768x4096 + "
                        "C5a softmax fp32 1024x131072 (split across workgroups) + C5b tanh-GELU bf16 2^30",
            "step_bytes": step_bytes,
            "frac_of_peak": round(value / PEAK_HBM_GBS, 4),
            "kernels": kernels,
            "spot_check": spot,
            **extras,
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)
    return 0 if spot["ok"] else 1


def copy_steps(fk, torch, xs, ys, stream, steps):
    """Average duration of a copy of each step kernel's input (x to y, all of
    x's bytes), over `steps` steps with HIP events around every launch."""
    ev = {name: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(steps)] for name in STEP}
    for k in range(-1, steps):  # step -1: warmup
        for name in STEP:
            x, y = xs[name], ys[name]
            if k >= 0:
                ev[name][k][0].record(stream)
            fk.fk_copy(x, y, x.numel() * x.element_size())
            if k >= 0:
                ev[name][k][1].record(stream)
    torch.cuda.synchronize()
    return {name: sum(a.elapsed_time(b) for a, b in ev[name]) / steps for name in STEP}


def spot_check(host, ys, wl):
    """Compare a sample of every timed output with the oracle."""
    import numpy as np

    import oracle

    rng = np.random.default_rng(1)
    ok = True
    worst = {}
    # elementwise: 65536 random positions
    for name in ("C3", "C5b"):
        x = host[name]
        idx = np.sort(rng.choice(x.size, 65536, replace=False))
        got = wl.from_torch(ys[name])[idx]
        if name == "C3":
            ref = oracle.chain(x[idx], wl.CHAIN_C3)
            rel = np.abs(got.astype(np.float64) - ref) / np.maximum(np.abs(ref), 1.2e-38)
            worst[name] = float(rel.max())
            ok &= worst[name] <= 1e-5
        else:
            ref = oracle.gelu_tanh(x[idx])
            d = np.abs(_ord16(got) - _ord16(ref))
            worst[name] = int(d.max())
            ok &= worst[name] <= 1
    # softmax: 16 random rows
    for name in ("C4", "C5a"):
        x = host[name]
        rows = np.sort(rng.choice(x.shape[0], 16, replace=False))
        got = wl.from_torch(ys[name][rows.tolist()])
        ref = oracle.softmax_rows(np.ascontiguousarray(x[rows]))
        if name == "C4":
            worst[name] = int(np.abs(_ord16(got) - _ord16(ref)).max())
            ok &= worst[name] <= 1
        else:
            worst[name] = float(np.abs(got.astype(np.float64) - ref).max())
            ok &= worst[name] <= 2e-6
    return {"ok": bool(ok), "worst": worst,
            "tolerance": {"C3": "1e-5 rel", "C5b": "1 bf16 ulp", "C4": "1 bf16 ulp",
                          "C5a": "2e-6 abs"}}


def _ord16(bits):
    import numpy as np

    b = bits.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def measure_extras(fk, wl, torch, xs, ys, stream):
    """Copy ceiling and fused-vs-unfused chain, outside the timed step."""
    out = {}

    def avg_ms(fn, reps):
        # warm up for ~0.1 s of launches first: each measurement here follows
        # host-side input generation, during which the GPU idles and its
        # clocks drop (a single warm-up launch left some kernels 5-10 % slow)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        for _ in range(2000):
            fn()
            torch.cuda.synchronize()
            if time.perf_counter() - t0 > WARM_SECONDS:
                break
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        b.synchronize()
        return a.elapsed_time(b) / reps

    # copy ceilings at 2 GiB per tensor: this library's 16-byte copy and the
    # runtime's own device-to-device copy (torch copy_ -> hipMemcpyAsync)
    nbytes = xs["C5b"].numel() * 2
    ms = avg_ms(lambda: fk.fk_copy(xs["C5b"], ys["C5b"], nbytes), 10)
    copy_gbs = 2 * nbytes / (ms * 1e-3) / 1e9
    rt_ms = avg_ms(lambda: ys["C5b"].copy_(xs["C5b"]), 10)
    rt_gbs = 2 * nbytes / (rt_ms * 1e-3) / 1e9
    out["copy_ceiling"] = {"bytes": 2 * nbytes, "ms": round(ms, 4), "GBps": round(copy_gbs, 1),
                           "frac_of_peak": round(copy_gbs / PEAK_HBM_GBS, 4),
                           "runtime_copy_ms": round(rt_ms, 4),
                           "runtime_copy_GBps": round(rt_gbs, 1),
                           "runtime_copy_frac_of_peak": round(rt_gbs / PEAK_HBM_GBS, 4),
                           "note": "fk_copy and the runtime's device-to-device copy "
                                   "(hipMemcpyAsync through torch copy_), 2 GiB each way"}

    # C3 fused vs the same three ops as three kernels (fp32 intermediates).
    # Each repetition first streams a 2 GiB copy so the 32 MiB operands are
    # not served from the 256 MB Infinity Cache.
    x = xs["C3"]
    t1, t2, t3 = torch.empty_like(x), torch.empty_like(x), torch.empty_like(x)
    ops = list(wl.CHAIN_C3)

    def timed(fn, reps=20):
        total = 0.0
        for _ in range(reps):
            fk.fk_copy(xs["C5b"], ys["C5b"], nbytes)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            total += a.elapsed_time(b)
        return total / reps

    fused_ms = timed(lambda: fk.fk_elementwise_chain(x, t3, ops))
    unfused_ms = timed(lambda: (fk.fk_elementwise_chain(x, t1, ops[:1]),
                                fk.fk_elementwise_chain(t1, t2, ops[1:2]),
                                fk.fk_elementwise_chain(t2, t3, ops[2:])))
    fb = wl.algorithmic_bytes("C3")
    ub = wl.algorithmic_bytes("C3", unfused=True)
    del t1, t2, t3

    # The small workloads (C1, C2, C3) fit in the 256 MB Infinity Cache:
    # each is launched back to back over rotating input/output pairs
    # totalling more than 1 GiB, next to both copies of the same bytes
    out["rotating_buffers"] = rotating_buffers(fk, wl, torch, stream)
    out["chain_rotating_buffers"] = out["rotating_buffers"]["C3"]

    # C5a through the online two-pass kernel (fk_softmax_rows without a
    # workspace takes it too), against the split path of the step
    out["softmax_online_c5a"] = online_c5a(fk, wl, torch, xs, ys, avg_ms)

    # LayerNorm (+ GELU epilogue) on the C4 row shape (bf16 32768 x 4096) and
    # the C2 row shape (fp32 4096 x 1000, rows shifted every 16th); the
    # algorithmic bytes are one read of x and one write of y (gamma and beta,
    # 2 * cols elements, are counted once)
    import numpy as np

    from memory_bound_elementwise_fk_amd import workloads as wl_

    ln = {}
    # x ~ 8 N(0, 1) (C4's shape and scale, without its masked entries),
    # gamma ~ 1 + 0.25 N(0, 1), beta ~ 0.5 N(0, 1)
    xb = wl_.to_torch(wl_.draw(32768 * 4096, seed=0, scale=8.0, dtype="bf16"),
                      "cuda:0").view(32768, 4096)
    prng = np.random.default_rng(8)
    gb = wl_.to_torch(wl_.f32_to_bf16_bits(
        (1.0 + 0.25 * prng.standard_normal(4096)).astype(np.float32)), "cuda:0")
    bb = wl_.to_torch(wl_.f32_to_bf16_bits(
        (0.5 * prng.standard_normal(4096)).astype(np.float32)), "cuda:0")
    yb = torch.empty_like(xb)
    ms = avg_ms(lambda: fk.fk_layernorm_rows(xb, yb, gb, bb, gelu=True), 20)
    nb = 2 * xb.numel() * 2 + 2 * xb.shape[1] * 2
    ln["bf16_32768x4096_gelu"] = {"ms": round(ms, 5), "bytes": nb,
                                  "GBps": round(nb / (ms * 1e-3) / 1e9, 1),
                                  "frac_of_peak": round(nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    del xb, yb
    xf = wl_.to_torch(wl_.make_input("C2"), "cuda:0")
    yf = torch.empty_like(xf)
    gf = torch.from_numpy((1.0 + 0.25 * prng.standard_normal(1000)).astype(np.float32)).to("cuda:0")
    bf = torch.from_numpy((0.5 * prng.standard_normal(1000)).astype(np.float32)).to("cuda:0")
    ms = avg_ms(lambda: fk.fk_layernorm_rows(xf, yf, gf, bf), 50)
    nb = 2 * xf.numel() * 4 + 2 * xf.shape[1] * 4
    ln["f32_4096x1000"] = {"ms": round(ms, 5), "bytes": nb,
                           "GBps": round(nb / (ms * 1e-3) / 1e9, 1),
                           "note": "32 MB of traffic: launch- and latency-bound like C3"}
    out["layernorm"] = ln
    del xf, yf

    # backward kernels: bf16 GELU backward over the C5b tensor (dy = the C5b
    # input again; two reads and one write, 6 bytes per element) and bf16
    # softmax backward on the C4 shape (y, dy = C4 input and its softmax)
    bw = {}
    x5 = xs["C5b"]        # x: the C5b input
    dy5 = ys["C5b"]       # dy: a distinct 2 GiB tensor (the GELU output of the step)
    dx5 = torch.empty_like(x5)
    ms = avg_ms(lambda: fk.fk_gelu_tanh_backward(x5, dy5, dx5), 10)
    nb = 3 * x5.numel() * 2
    bw["gelu_bf16_2^30"] = {"ms": round(ms, 5), "bytes": nb,
                            "GBps": round(nb / (ms * 1e-3) / 1e9, 1),
                            "frac_of_peak": round(nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    y4 = ys["C4"]
    dx4 = torch.empty_like(y4)
    ms = avg_ms(lambda: fk.fk_softmax_rows_backward(y4, xs["C4"], dx4), 20)
    nb = 3 * y4.numel() * 2
    bw["softmax_bf16_32768x4096"] = {"ms": round(ms, 5), "bytes": nb,
                                     "GBps": round(nb / (ms * 1e-3) / 1e9, 1),
                                     "frac_of_peak": round(nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    out["backward"] = bw
    del dx4, dx5

    # Linear + GELU on the matrix cores (MLP up-projection: 8192 tokens,
    # 4096 -> 16384 features, bf16), against torch's library matmul
    # (hipBLASLt) alone and followed by a separate GELU kernel
    M, N, K = 8192, 16384, 4096
    xl = wl_.to_torch(wl_.draw(M * K, seed=3, dtype="bf16"), "cuda:0").view(M, K)
    wlin = wl_.to_torch(wl_.draw(N * K, seed=4, scale=K ** -0.5, dtype="bf16"), "cuda:0").view(N, K)
    bl = wl_.to_torch(wl_.draw(N, seed=5, dtype="bf16"), "cuda:0")
    yl = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    flops = 2.0 * M * N * K
    fused = avg_ms(lambda: fk.fk_linear_gelu(xl, wlin, bl, yl), 10)
    lib_mm = avg_ms(lambda: torch.nn.functional.linear(xl, wlin, bl), 10)
    lib_unfused = avg_ms(lambda: torch.nn.functional.gelu(torch.nn.functional.linear(xl, wlin, bl),
                                                          approximate="tanh"), 10)
    out["linear_gelu"] = {
        "shape": [M, N, K], "fused_ms": round(fused, 4),
        "fused_TFLOPs": round(flops / (fused * 1e-3) / 1e12, 1),
        "frac_of_mfma_peak": round(flops / (fused * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "library_linear_ms": round(lib_mm, 4),
        "library_linear_then_gelu_ms": round(lib_unfused, 4),
        "note": "library = torch.nn.functional.linear (hipBLASLt) and its separate GELU"}
    # the same in fp16
    xh, wh, bh = xl.to(torch.float16), wlin.to(torch.float16), bl.to(torch.float16)
    yh = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
    fused16 = avg_ms(lambda: fk.fk_linear_gelu(xh, wh, bh, yh), 10)
    lib16 = avg_ms(lambda: torch.nn.functional.gelu(torch.nn.functional.linear(xh, wh, bh),
                                                    approximate="tanh"), 10)
    out["linear_gelu"]["fp16"] = {"fused_ms": round(fused16, 4),
                                  "fused_TFLOPs": round(flops / (fused16 * 1e-3) / 1e12, 1),
                                  "library_linear_then_gelu_ms": round(lib16, 4)}
    del xl, wlin, bl, yl, xh, wh, bh, yh

    # FlashAttention forward on the pages' benchmark grid (B = 4, H = 32,
    # d = 128, T = 128 ... 4096)
    att = {}
    for T in (128, 256, 512, 1024, 2048, 4096):
        qa, ka, va = (wl_.to_torch(wl_.draw(4 * 32 * T * 128, seed=6 + i, dtype="bf16"),
                                   "cuda:0").view(4, 32, T, 128) for i in range(3))
        oa = torch.empty_like(qa)
        for causal in (False, True):
            fl = 4.0 * 4 * 32 * T * T * 128 * (0.5 if causal else 1.0)
            reps = 20 if T <= 1024 else 5
            ms_fk = avg_ms(lambda: fk.fk_attention_fwd(qa, ka, va, oa, causal=causal), reps)
            att[f"T{T}_{'causal' if causal else 'full'}"] = {
                "ms": round(ms_fk, 4), "TFLOPs": round(fl / (ms_fk * 1e-3) / 1e12, 1),
                "frac_of_mfma_peak": round(fl / (ms_fk * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del qa, ka, va, oa
    # fp16, the dtype the pages benchmark
    for T in (1024, 4096):
        qa, ka, va = (wl_.to_torch(wl_.draw(4 * 32 * T * 128, seed=6 + i), "cuda:0")
                      .to(torch.float16).view(4, 32, T, 128) for i in range(3))
        oa = torch.empty_like(qa)
        for causal in (False, True):
            fl = 4.0 * 4 * 32 * T * T * 128 * (0.5 if causal else 1.0)
            reps = 20 if T <= 1024 else 5
            ms_fk = avg_ms(lambda: fk.fk_attention_fwd(qa, ka, va, oa, causal=causal), reps)
            att[f"fp16_T{T}_{'causal' if causal else 'full'}"] = {
                "ms": round(ms_fk, 4), "TFLOPs": round(fl / (ms_fk * 1e-3) / 1e12, 1),
                "frac_of_mfma_peak": round(fl / (ms_fk * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del qa, ka, va, oa
    out["attention_fwd"] = att
    out["chain_fused_vs_unfused"] = {
        "fused_ms": round(fused_ms, 5), "unfused_ms": round(unfused_ms, 5),
        "fused_bytes": fb, "unfused_bytes": ub,
        "fused_GBps": round(fb / (fused_ms * 1e-3) / 1e9, 1),
        "unfused_GBps": round(ub / (unfused_ms * 1e-3) / 1e9, 1),
        "speedup": round(unfused_ms / fused_ms, 3),
        "pages_traffic_ratio": 3.0,
        "note": "cold Infinity Cache before each measurement"}
    return out


def _median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


# Rotating-buffer configurations: workload, pairs (input + output per pair;
# all pairs together hold more than 1 GiB, four times the Infinity Cache)
ROTATING = (("C1", 160), ("C2", 40), ("C3", 20))
ROT_REPLAYS = 8   # replays of the graph of one launch per pair


def rotating_buffers(fk, wl, torch, stream):
    """C1, C2 and C3 launched back to back over rotating pairs, next to
    fk_copy and the runtime's copy of the same bytes, launched alike.

    One launch per pair is captured into a HIP graph (so the launches are
    not bound by the host's per-call cost: C1 takes ~4.5 us on the device,
    about what one call through the binding costs on the host); the graph
    is replayed ROT_REPLAYS times between events, and a replay's span /
    pairs is one launch's time. Median and minimum are over the replays
    (8 x pairs launches: 1280 for C1, 320 for C2, 160 for C3). If capture
    is unavailable the same launches run eagerly."""
    out = {}
    for name, npairs in ROTATING:
        x0 = wl.to_torch(wl.make_input(name), "cuda:0")
        pairs = [(x0.clone(), torch.empty_like(x0)) for _ in range(npairs)]
        nbytes = x0.numel() * x0.element_size()
        total = 2 * nbytes * npairs
        if name == "C1":
            launch = lambda a, b: fk.fk_gelu_tanh(a, b)  # noqa: E731
        elif name == "C2":
            launch = lambda a, b: fk.fk_softmax_rows(a, b)  # noqa: E731
        else:
            launch = lambda a, b: fk.fk_elementwise_chain(a, b, wl.CHAIN_C3)  # noqa: E731

        def per_launch_ms(fn):
            def all_pairs():
                for a, b in pairs:
                    fn(a, b)

            all_pairs()  # warm-up (and first-call setup) outside the capture
            torch.cuda.synchronize()
            replay, how = all_pairs, "eager"
            try:
                g = torch.cuda.CUDAGraph()
                side = torch.cuda.Stream()
                side.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(side):
                    with torch.cuda.graph(g, stream=side):
                        all_pairs()
                torch.cuda.current_stream().wait_stream(side)
                replay, how = g.replay, "graph"
                replay()
                torch.cuda.synchronize()
            except Exception as exc:  # noqa: BLE001
                log(f"{name}: graph capture unavailable ({exc}); eager launches")
                torch.cuda.synchronize()
            t0 = time.perf_counter()   # clocks up before the timed replays
            while time.perf_counter() - t0 < WARM_SECONDS:
                replay()
                torch.cuda.synchronize()
            per = []
            for _ in range(ROT_REPLAYS):
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record()
                replay()
                b.record()
                b.synchronize()
                per.append(a.elapsed_time(b) / npairs)
            return per, how

        t_k, how = per_launch_ms(launch)
        t_c, _ = per_launch_ms(lambda a, b: fk.fk_copy(a, b, nbytes))
        t_r, _ = per_launch_ms(lambda a, b: b.copy_(a))
        alg = wl.algorithmic_bytes(name)
        med = _median(t_k)
        gbs = alg / (med * 1e-3) / 1e9
        faster_copy = min(_median(t_c), _median(t_r))
        out[name] = {"median_ms": round(med, 5), "min_ms": round(min(t_k), 5),
                     "bytes": alg, "GBps": round(gbs, 1),
                     "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4),
                     "fk_copy_median_ms": round(_median(t_c), 5),
                     "runtime_copy_median_ms": round(_median(t_r), 5),
                     "frac_of_faster_copy": round(faster_copy / med, 4),
                     "launches": ROT_REPLAYS * npairs, "launched_as": how,
                     "pairs": npairs, "pair_bytes_total": total}
        del pairs, x0
    return out


def online_c5a(fk, wl, torch, xs, ys, avg_ms):
    """C5a (fp32 1024 x 131072) through the online two-pass kernel and
    through fk_softmax_rows (no workspace: the same online path)."""
    x, y = xs["C5a"], ys["C5a"]
    alg = wl.algorithmic_bytes("C5a")
    out = {"path_without_workspace": fk.fk_softmax_rows_path(x, y)}
    for key, fn in (("online", lambda: fk.fk_softmax_rows_online(x, y)),
                    ("fk_softmax_rows", lambda: fk.fk_softmax_rows(x, y))):
        ms = avg_ms(fn, 20)
        gbs = alg / (ms * 1e-3) / 1e9
        out[key] = {"ms": round(ms, 5), "bytes": alg, "GBps": round(gbs, 1),
                    "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4)}
    return out


def traffic_bytes(kernel: str):
    """HBM bytes per launch of the dominant kernel from committed counter runs.

    profiles/traffic.json holds FETCH_SIZE/WRITE_SIZE readings scaled by a
    plain copy of known size; it is used only while the kernel sources are
    unchanged since the counters were taken (same source hash).
    """
    if not TRAFFIC_FILE.exists():
        return None
    try:
        rec = json.loads(TRAFFIC_FILE.read_text())
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash():
        return None
    entry = rec.get("kernels", {}).get(kernel)
    return None if entry is None else entry.get("bytes_per_launch")


def cpu_baseline(host, kbytes):
    """The oracle over whole steps on the host cores, repeated for >= 10 s."""
    import oracle
    from memory_bound_elementwise_fk_amd import workloads as wl

    threads = oracle.default_threads()
    log(f"cpu baseline: oracle over whole steps on {threads} threads")
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.chain(host["C3"], wl.CHAIN_C3, threads=threads)
        oracle.softmax_rows(host["C4"], threads=threads)
        oracle.softmax_rows(host["C5a"], threads=threads)
        oracle.gelu_tanh(host["C5b"], threads=threads)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= CPU_BASELINE_MIN_SECONDS:
            break
    total = sum(kbytes.values()) * reps
    # one core on a bounded sample: the first 2^24 elements of C5b and the
    # first 4096 rows of C4 (4 bytes of algorithmic traffic per element each)
    n1 = 1 << 24
    t1 = time.perf_counter()
    oracle.gelu_tanh(host["C5b"][:n1], threads=1)
    g1 = n1 * 4 / (time.perf_counter() - t1) / 1e9
    rows1 = host["C4"][:4096]
    t1 = time.perf_counter()
    oracle.softmax_rows(rows1, threads=1)
    s1 = rows1.size * 4 / (time.perf_counter() - t1) / 1e9
    return {"value": round(total / dt / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "seconds": round(dt, 3), "steps": reps,
            "sample": f"{reps} full steps (C3 + C4 + C5a + C5b, every element) through the "
                      "double-precision C++ oracle, split over contiguous ranges/rows",
            "single_core": {"C5b_first_2^24_GBps": round(g1, 3),
                            "C4_first_4096_rows_GBps": round(s1, 3)}}


def counters_run(fk, torch, launches, xs, ys):
    """Each step kernel twice and one 1 GiB copy, for per-dispatch counters;
    then twice each of the LayerNorm + GELU, GELU backward, softmax backward
    and online-path C5a launches the extras time (same shapes)."""
    calib = 1 << 30
    a = torch.empty(calib, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    fk.fk_copy(a, b, calib)
    for _ in range(2):
        for name in STEP:
            launches[name]()
    torch.cuda.synchronize()
    del a, b
    extra = extra_launches(fk, torch, xs, ys)
    for _ in range(2):
        for name in EXTRA:
            extra[name]()
    torch.cuda.synchronize()
    log(f"counters run done: calibration copy {calib} B, then 2 x {', '.join(STEP)}, "
        f"then 2 x {', '.join(EXTRA)}")
    return 0


def profile_run(fk, torch, xs, ys):
    """Two launches each of the next-row kernels on the extras' shapes."""
    from memory_bound_elementwise_fk_amd import workloads as wl

    M, N, K = 8192, 16384, 4096
    xl = wl.to_torch(wl.draw(M * K, seed=3, dtype="bf16"), "cuda:0").view(M, K)
    wlin = wl.to_torch(wl.draw(N * K, seed=4, scale=K ** -0.5, dtype="bf16"), "cuda:0").view(N, K)
    bl = wl.to_torch(wl.draw(N, seed=5, dtype="bf16"), "cuda:0")
    yl = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    T = 4096
    qa, ka, va = (wl.to_torch(wl.draw(4 * 32 * T * 128, seed=6 + i, dtype="bf16"),
                              "cuda:0").view(4, 32, T, 128) for i in range(3))
    oa = torch.empty_like(qa)
    extra = extra_launches(fk, torch, xs, ys)
    runs = [("linear_gelu", lambda: fk.fk_linear_gelu(xl, wlin, bl, yl)),
            ("attention_full", lambda: fk.fk_attention_fwd(qa, ka, va, oa, causal=False)),
            ("attention_causal", lambda: fk.fk_attention_fwd(qa, ka, va, oa, causal=True)),
            ("layernorm_gelu", extra["layernorm_gelu"]),
            ("online_c5a", lambda: fk.fk_softmax_rows_online(xs["C5a"], ys["C5a"]))]
    for name, fn in runs:
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        log(f"profile run: 2 x {name}")
    return 0


def extra_launches(fk, torch, xs, ys):
    """The memory-bound next-row kernels on the extras' shapes: LayerNorm +
    GELU bf16 32768 x 4096 (random gamma, beta), GELU backward over the C5b
    tensor (dy: the step's GELU output), softmax backward on the C4 shape
    (y: the step's softmax output, dy: the C4 input)."""
    import numpy as np

    from memory_bound_elementwise_fk_amd import workloads as wl

    xb = wl.to_torch(wl.draw(32768 * 4096, seed=0, scale=8.0, dtype="bf16"),
                     "cuda:0").view(32768, 4096)
    prng = np.random.default_rng(8)
    gb = wl.to_torch(wl.f32_to_bf16_bits(
        (1.0 + 0.25 * prng.standard_normal(4096)).astype(np.float32)), "cuda:0")
    bb = wl.to_torch(wl.f32_to_bf16_bits(
        (0.5 * prng.standard_normal(4096)).astype(np.float32)), "cuda:0")
    yb = torch.empty_like(xb)
    dx5 = torch.empty_like(xs["C5b"])
    dx4 = torch.empty_like(ys["C4"])
    return {
        "layernorm_gelu": lambda: fk.fk_layernorm_rows(xb, yb, gb, bb, gelu=True),
        "gelu_backward": lambda: fk.fk_gelu_tanh_backward(xs["C5b"], ys["C5b"], dx5),
        "softmax_backward": lambda: fk.fk_softmax_rows_backward(ys["C4"], xs["C4"], dx4),
        "online_c5a": lambda: fk.fk_softmax_rows_online(xs["C5a"], ys["C5a"]),
    }


def _read_counter_csv(path):
    """{(dispatch_id, kernel_name): value} of the one counter a rocprofv3 CSV holds."""
    import csv

    out, names = {}, set()
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            names.add(row["Counter_Name"])
            key = (int(row["Dispatch_Id"]), row["Kernel_Name"])
            out[key] = out.get(key, 0.0) + float(row["Counter_Value"])
    if len(names) != 1:
        raise SystemExit(f"{path}: expected one counter, found {sorted(names)}")
    return names.pop(), out


def _match(kernel_name: str, frags) -> bool:
    return all(f in kernel_name for f in frags)


def ingest_counters(fetch_csv: str, write_csv: str) -> int:
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of a --counters-run -> traffic.json.

    Each counter is scaled by what it reads for the calibration copy, whose
    true traffic is known (1 GiB read and 1 GiB written), so the figures are
    HBM-side bytes per launch of each kernel.
    """
    from memory_bound_elementwise_fk_amd import workloads as wl

    fname, fetch = _read_counter_csv(fetch_csv)
    wname, write = _read_counter_csv(write_csv)
    if fname != "FETCH_SIZE" or wname != "WRITE_SIZE":
        raise SystemExit(f"expected FETCH_SIZE then WRITE_SIZE, got {fname}, {wname}")
    calib = float(1 << 30)

    def per_kernel(table, frags):
        vals = [v for (d, k), v in sorted(table.items()) if _match(k, frags)]
        return vals

    cf, cw = per_kernel(fetch, KERNEL_NAMES["copy"]), per_kernel(write, KERNEL_NAMES["copy"])
    if not cf or not cw:
        raise SystemExit("calibration copy not found in the counter files")
    f_scale = calib / (cf[0] * 1024.0)
    w_scale = calib / (cw[0] * 1024.0)
    rec = {"source_hash": kernel_source_hash(),
           "calibration": {"bytes_each_way": int(calib), "fetch_kib": cf[0], "write_kib": cw[0],
                           "fetch_scale": f_scale, "write_scale": w_scale},
           "kernels": {}}
    for name in STEP:
        fv = per_kernel(fetch, KERNEL_NAMES[name])
        wv = per_kernel(write, KERNEL_NAMES[name])
        if not fv or not wv:
            raise SystemExit(f"kernel of {name} not found in the counter files")
        fb = sum(fv) / len(fv) * 1024.0 * f_scale
        wb = sum(wv) / len(wv) * 1024.0 * w_scale
        alg = wl.algorithmic_bytes(name)
        rec["kernels"][name] = {"fetch_bytes": round(fb), "write_bytes": round(wb),
                                "bytes_per_launch": round(fb + wb), "algorithmic_bytes": alg,
                                "ratio_to_algorithmic": round((fb + wb) / alg, 4),
                                "dispatches": len(fv)}
    # the next-row kernels, when the run counted them
    for name in EXTRA:
        fv = per_kernel(fetch, KERNEL_NAMES[name])
        wv = per_kernel(write, KERNEL_NAMES[name])
        if not fv or not wv:
            continue
        fb = sum(fv) / len(fv) * 1024.0 * f_scale
        wb = sum(wv) / len(wv) * 1024.0 * w_scale
        alg = EXTRA_BYTES[name]
        rec.setdefault("next_rows", {})[name] = {
            "fetch_bytes": round(fb), "write_bytes": round(wb), "bytes_per_launch": round(fb + wb),
            "algorithmic_bytes": alg, "ratio_to_algorithmic": round((fb + wb) / alg, 4),
            "dispatches": len(fv)}
    TRAFFIC_FILE.parent.mkdir(exist_ok=True)
    TRAFFIC_FILE.write_text(json.dumps(rec, indent=2) + "\n")
    print(json.dumps(rec, indent=2))
    return 0


if __name__ == "__main__":
    sys.exit(main())
