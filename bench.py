#!/usr/bin/env python3
"""Throughput of the batched power-of-two C2C FFT on one MI355X.

Default workload: forward C2C FFT of 16384 rows of N = 4096 complex64 points
(re, im i.i.d. standard normal, seed 2; 512 MiB in, 512 MiB out), the one-kernel
LDS-resident path.  One step = one fft_exec_c2c call over the whole batch with
the input already resident in HBM.

Prints ONE JSON line with:
  value      GFLOP/s = batch * 5 N log2 N / t, t = ms_per_step: K steps launched
             back to back between ONE pair of HIP events on the launch stream
             (pseudo-flops, 10 per radix-2 butterfly)
  roofline   achieved HBM GB/s of the step's one kernel (input + output bytes /
             the same t: a step is one launch, so t is that kernel's average
             launch duration) against 8000 GB/s, plus `traffic`: HBM bytes per
             launch measured with rocprofv3 counters (FETCH_SIZE + WRITE_SIZE
             scaled by a copy kernel of known size), read from profiles/ and
             null once the kernel sources have changed
  cpu_baseline  the fp64 CPU oracle on a bounded sample of the same rows, with
             the thread count and the host CPU model; for row workloads also
             `parity`: the largest per-row relative RMS error of the timed
             output's first rows against the oracle's result for them, and
             the bound 1e-6 log2 N
  launch_us  a separate pass with a pair of events around every launch: mean /
             median / min / max of the per-launch durations
  copy_ceiling  the library's streaming copy (fft_stream_copy: every byte read
             once and written once, nontemporal 8-byte lanes as in the row
             kernels, the fastest copy measured) of the same byte
             count, timed like the steps, and the step's algorithmic rate as a
             fraction of the copy's (the practical ceiling of the access pattern)
  rotated    the same steps cycling over --rotate buffer sets (default 3), so
             that no step finds its input in the 256 MB MALL

Other workloads (--workload) time the 2^24-point multi-pass transform, the
2048x2048x8 2D transform, the 32 x 2^18 polynomial products and a 256^3 3D
transform the same way, and the R2C transform of 16384 real rows of 8192
points (value = batch * 2.5 N log2 N / t, half the complex count), and rows
of 1000 (mixed radix) and 1009 (Bluestein) points, the 2D R2C transform of
eight real 2048 x 2048 images, and 64 rows of 10^6 points (two mixed-radix
super-stage passes of radix 1000).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "C2C FFT GFLOP/s (5N·log2N/t) + achieved HBM TB/s, fp32 N=4096 batch 16384"
WORKLOADS = ("c2c_n4096_b16384", "c2c_n1024_b64", "c2c_n16777216_b1", "c2c2d_2048x2048_b8",
             "polymul_l262144_b32", "c2c3d_256x256x256_b1", "r2c_n8192_b16384", "c2c_n1000_b65536",
             "c2c_n1009_b65536", "r2c2d_2048x2048_b8", "c2c_n1000000_b64", "c2cpl_n4096_b16384")


# The sources each single-kernel workload's kernel is built from: a stored
# counter record applies while these files are unchanged.
KERNEL_SOURCES = {
    "c2c_n4096_b16384": ("rows.hip", "stockham.hpp", "radix_plan.hpp", "io.hpp", "tile_common.hpp"),
    "c2c_n1024_b64": ("rows.hip", "stockham.hpp", "radix_plan.hpp", "io.hpp", "tile_common.hpp"),
    "c2cpl_n4096_b16384": ("rows.hip", "stockham.hpp", "radix_plan.hpp", "io.hpp", "tile_common.hpp"),
    "r2c_n8192_b16384": ("real.hip", "stockham.hpp", "radix_plan.hpp", "tile_common.hpp"),
    "c2c_n1000_b65536": ("mixed.hip", "stockham.hpp", "radix_plan.hpp", "io.hpp", "tile_common.hpp"),
    "c2c_n1009_b65536": ("bluestein.hip", "stockham.hpp", "radix_plan.hpp", "io.hpp", "tile_common.hpp"),
}


def kernel_sources_digest(workload: str = WORKLOADS[0]) -> str:
    """sha256 over the HIP sources of the workload's kernel (all of csrc/ for
    multi-kernel workloads), to tell whether stored counters still apply."""
    csrc = os.path.join(ROOT, "fft_convolution_amd", "csrc")
    names = KERNEL_SOURCES.get(workload) or [n for n in os.listdir(csrc) if n.endswith((".hip", ".hpp", ".cpp"))]
    h = hashlib.sha256()
    for name in sorted(names):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()


def stored_traffic(workload: str):
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_sources_sha256") != kernel_sources_digest(workload):
        return None
    return rec.get("traffic_bytes_per_launch")


def ensure_built():
    import fft_convolution_amd as fm
    if not os.path.exists(fm.lib_path):
        from fft_convolution_amd import build
        build.build()
    fm.lib()
    return fm


def setup_workload(name, dev, fm, torch, sets=1):
    """Returns (step_fn, info): step(k) runs the hot path once on buffer set
    k mod `sets` (each set: its own input, output and workspace, all resident
    in HBM; set 0 holds the seeded workload input, the others copies)."""
    from fft_convolution_amd import workloads as wl
    spec = dict(wl.WORKLOADS[name])
    stream = torch.cuda.current_stream().cuda_stream

    def ws_of(nbytes):
        return torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None

    if name.startswith("c2c_n"):
        n, batch = spec["n"], spec["batch"]
        x_np = wl.workload_input(name)
        plan = fm.Plan(n, torch.complex64)
        wsb = fm.fft_workspace_size(plan.handle, batch)
        x0 = torch.from_numpy(x_np).to(dev)
        bufs = [(x0 if k == 0 else x0.clone(), torch.empty_like(x0), ws_of(wsb)) for k in range(sets)]

        def step(k=0):
            x, y, ws = bufs[k % sets]
            fm.fft_exec_c2c(plan.handle, fm.FFT_FORWARD, x, y, batch, ws, stream)
        desc = plan.describe()
        kernels = len(desc.split("radices=")[1].split()[0].split("x")) if ("path=multipass" in desc or "path=mixpass" in desc) \
            else (5 if "passes" in desc else 1)
        # the oracle's route for the length: the radix-2 FFT, the direct DFT,
        # or (rows too long for an O(N^2) pass in the time budget) a bounded
        # set of bins of the direct DFT, scaled to whole rows
        pow2 = n & (n - 1) == 0
        info = dict(n=n, batch=batch, dtype="f32", flops=batch * 5.0 * n * math.log2(n), bytes=2 * x0.numel() * 8,
                    plan=desc, kernels=kernels, sample_rows=lambda rows: x_np[:rows],
                    oracle_fn="fft" if pow2 else ("dft" if n <= 16384 else "dft_bins"),
                    oracle_unit=5.0 * n * math.log2(n), keep=(plan, bufs),
                    out_rows=lambda rows: bufs[0][1][:rows].cpu().numpy())
        return step, info
    if name.startswith("c2cpl_n"):
        # split planes: re and im of the same seeded complex rows
        import numpy as np
        n, batch = spec["n"], spec["batch"]
        x_np = wl.workload_input(name)
        plan = fm.Plan(n, torch.complex64)
        wsb = fm.fft_planar_workspace_size(plan.handle, batch)
        re0 = torch.from_numpy(np.ascontiguousarray(x_np.real)).to(dev)
        im0 = torch.from_numpy(np.ascontiguousarray(x_np.imag)).to(dev)
        bufs = [((re0, im0) if k == 0 else (re0.clone(), im0.clone())) + (torch.empty_like(re0), torch.empty_like(im0),
                                                                         ws_of(wsb)) for k in range(sets)]

        def step(k=0):
            xr, xi, yr, yi, ws = bufs[k % sets]
            fm.fft_exec_planar(plan.handle, fm.FFT_FORWARD, xr, xi, yr, yi, batch, ws, stream)
        info = dict(n=n, batch=batch, dtype="f32", flops=batch * 5.0 * n * math.log2(n), bytes=4 * re0.numel() * 4,
                    plan=plan.describe() + " layout=planar", kernels=1, sample_rows=lambda rows: x_np[:rows],
                    oracle_fn="fft", oracle_unit=5.0 * n * math.log2(n), keep=(plan, bufs),
                    out_rows=lambda rows: bufs[0][2][:rows].cpu().numpy() + 1j * bufs[0][3][:rows].cpu().numpy())
        return step, info
    if name.startswith("c2c2d") or name.startswith("c2c3d"):
        three = name.startswith("c2c3d")
        dims = (spec["d"], spec["h"], spec["w"]) if three else (spec["h"], spec["w"])
        batch = spec["batch"]
        x_np = wl.workload_input(name)
        plan = fm.Plan(dims, torch.complex64)
        x0 = torch.from_numpy(x_np).to(dev)
        bufs = [(x0 if k == 0 else x0.clone(), torch.empty_like(x0)) for k in range(sets)]
        fn = fm.fft_exec_3d if three else fm.fft_exec_2d

        def step(k=0):
            x, y = bufs[k % sets]
            fn(plan.handle, fm.FFT_FORWARD, x, y, batch, None, stream)
        n = int(math.prod(dims))
        info = dict(batch=batch, dtype="f32", flops=batch * 5.0 * n * math.log2(n), bytes=2 * x0.numel() * 8,
                    plan=plan.describe(), kernels=3 if three else 2, keep=(plan, bufs),
                    sample_rows=lambda rows: x_np[:rows], oracle_unit=5.0 * n * math.log2(n),
                    oracle_fn="fft3" if three else "fft2",
                    **dict(zip(("d", "h", "w") if three else ("h", "w"), dims)))
        return step, info
    if name.startswith("r2c2d"):
        h, w, batch = spec["h"], spec["w"], spec["batch"]
        x_np = wl.workload_input(name)
        plan = fm.RealPlan((h, w), torch.float32)
        wsb = fm.fft_workspace_size(plan.handle, batch)
        x0 = torch.from_numpy(x_np).to(dev)
        bufs = [(x0 if k == 0 else x0.clone(), torch.empty(batch, h, w // 2 + 1, dtype=torch.complex64, device=dev),
                 ws_of(wsb)) for k in range(sets)]

        def step(k=0):
            x, y, ws = bufs[k % sets]
            fm.fft_exec_r2c(plan.handle, x, y, batch, ws, stream)
        info = dict(h=h, w=w, batch=batch, dtype="f32", flops=batch * 2.5 * h * w * math.log2(h * w),
                    bytes=x0.numel() * 4 + bufs[0][1].numel() * 8, plan=plan.describe(), kernels=3,
                    sample_rows=lambda rows: x_np[:rows], oracle_unit=2.5 * h * w * math.log2(h * w),
                    oracle_fn="rfft2", keep=(plan, bufs))
        return step, info
    if name.startswith("r2c"):
        n, batch = spec["n"], spec["batch"]
        x_np = wl.workload_input(name)
        plan = fm.RealPlan(n, torch.float32)
        wsb = fm.fft_workspace_size(plan.handle, batch)
        x0 = torch.from_numpy(x_np).to(dev)
        bufs = [(x0 if k == 0 else x0.clone(),
                 torch.empty(batch, n // 2 + 1, dtype=torch.complex64, device=dev), ws_of(wsb)) for k in range(sets)]

        def step(k=0):
            x, y, ws = bufs[k % sets]
            fm.fft_exec_r2c(plan.handle, x, y, batch, ws, stream)
        info = dict(n=n, batch=batch, dtype="f32", flops=batch * 2.5 * n * math.log2(n),
                    bytes=x0.numel() * 4 + bufs[0][1].numel() * 8, plan=plan.describe(),
                    kernels=1 if wsb == 0 else 2, sample_rows=lambda rows: x_np[:rows],
                    oracle_unit=2.5 * n * math.log2(n), oracle_fn="rfft", keep=(plan, bufs))
        return step, info
    if name.startswith("polymul"):
        length, batch = spec["length"], spec["batch"]
        a_np, b_np = wl.workload_input(name)
        n = 1
        while n < 2 * length - 1:
            n *= 2
        plan = fm.Plan(n, torch.complex128)
        wsb = fm.fft_poly_mul_workspace_size(plan.handle, batch)
        a0 = torch.from_numpy(a_np).to(dev)
        b0 = torch.from_numpy(b_np).to(dev)
        bufs = [(a0 if k == 0 else a0.clone(), b0 if k == 0 else b0.clone(),
                 torch.empty(batch, 2 * length - 1, dtype=torch.int64, device=dev), ws_of(wsb),
                 torch.empty(1, dtype=torch.float64, device=dev)) for k in range(sets)]

        def step(k=0):
            a, b, c, ws, resid = bufs[k % sets]
            fm.fft_poly_mul(plan.handle, a, length, b, length, c, batch, ws, resid, stream)
        info = dict(n=n, length=length, batch=batch, dtype="f64", flops=batch * 3 * 5.0 * n * math.log2(n),
                    bytes=(a0.numel() + b0.numel() + bufs[0][2].numel()) * 8, plan=plan.describe(), kernels=4,
                    keep=(plan, bufs), sample_pairs=lambda p: (a_np[:p], b_np[:p]),
                    oracle_unit=3 * 5.0 * n * math.log2(n))
        return step, info
    raise SystemExit("unknown workload %s" % name)


def cpu_baseline(name, info, budget_s):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload."""
    import numpy as np
    import oracle
    threads = len(os.sched_getaffinity(0))
    oracle.set_threads(threads)
    parity = None
    if name.startswith("polymul"):
        total = info["batch"]
        a, b = info["sample_pairs"](1)
        t0 = time.perf_counter()
        oracle.polymul_fft(a, b, n=info["n"])
        per = time.perf_counter() - t0
        pairs = int(max(1, min(total, budget_s / max(per, 1e-9) * min(threads, total) / 2)))
        a, b = info["sample_pairs"](pairs)
        t0 = time.perf_counter()
        oracle.polymul_fft(a, b, n=info["n"])
        dt = time.perf_counter() - t0
        units, sample = pairs, "first %d of %d pairs" % (pairs, total)
    elif name.startswith("c2c2d") or name.startswith("c2c3d") or name.startswith("r2c2d"):
        # The first image, then as many of the batch as fit the budget, the
        # whole set transformed again until the budget is used.
        fn = getattr(oracle, info["oracle_fn"])
        x = info["sample_rows"](1)
        t0 = time.perf_counter()
        fn(x)
        per = time.perf_counter() - t0
        imgs = int(max(1, min(info["batch"], budget_s / max(per, 1e-9))))
        x = info["sample_rows"](imgs)
        reps, dt = 0, 0.0
        while reps == 0 or dt < budget_s:
            t0 = time.perf_counter()
            fn(x)
            dt += time.perf_counter() - t0
            reps += 1
        units = imgs * reps
        sample = "first %d of %d images, transformed %d time(s)" % (imgs, info["batch"], reps)
    elif info.get("oracle_fn") == "dft_bins":
        # One row of N points: bins 0, 1, ... of its direct DFT (O(N) each),
        # as many as fit the budget, scaled to whole rows (N bins a row).
        n = info["n"]
        x = info["sample_rows"](1)
        t0 = time.perf_counter()
        oracle.dft_sample(x, np.arange(16))
        per_bin = (time.perf_counter() - t0) / 16
        bins = int(max(16, min(n, budget_s / max(per_bin, 1e-12))))
        t0 = time.perf_counter()
        oracle.dft_sample(x, np.arange(bins))
        dt = time.perf_counter() - t0
        units = bins / n
        sample = "bins 0..%d of row 0 (direct DFT, %d of %d bins), scaled to whole rows" % (bins - 1, bins, n)
    else:
        # The first rows of the batch, as many as fit the budget; if the whole
        # batch takes less, it is transformed repeatedly until the budget is used.
        total = info["batch"]
        probe = min(total, 256)
        fn = getattr(oracle, info.get("oracle_fn", "fft"))
        x = info["sample_rows"](probe)
        t0 = time.perf_counter()
        fn(x)
        per_row = (time.perf_counter() - t0) / probe
        rows = int(max(1, min(total, budget_s / max(per_row, 1e-12))))
        x = info["sample_rows"](rows)
        reps, dt = 0, 0.0
        while reps == 0 or dt < budget_s:
            t0 = time.perf_counter()
            ref = fn(x)
            dt += time.perf_counter() - t0
            reps += 1
        units = rows * reps
        sample = "first %d of %d rows, transformed %d time(s)" % (rows, total, reps)
        if "out_rows" in info:
            # the timed output's rows against the oracle's, which this leg has
            # just computed: the largest per-row relative RMS error
            k = min(rows, 256)
            y = np.asarray(info["out_rows"](k), dtype=np.complex128)
            r = np.asarray(ref[:k], dtype=np.complex128)
            err = np.sqrt(np.sum(np.abs(y - r) ** 2, axis=1) / np.sum(np.abs(r) ** 2, axis=1))
            parity = {"rows": k, "max_rel_rms": float(err.max()), "bound": 1e-6 * math.log2(info["n"])}
    out = {"value": units * info["oracle_unit"] / dt / 1e9, "unit": "GFLOP/s", "cores": threads,
           "kind": "oracle", "sample": sample, "seconds": round(dt, 3), "cpu": cpu_model()}
    if parity is not None:
        out["parity"] = parity
    return out


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo ("unknown" where absent)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=WORKLOADS[0], choices=WORKLOADS)
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rotate", type=int, default=3,
                    help="buffer sets for the extra rotated-buffer timing (1 = none)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a device-to-device copy of the input's size (for counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    fm = ensure_built()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    sets = max(1, args.rotate)
    step, info = setup_workload(args.workload, dev, fm, torch, sets=sets)
    stream = torch.cuda.current_stream()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # The practical ceiling, measured first: the library's streaming copy of
    # the same byte count (half the algorithmic bytes each way), at least
    # 512 MiB each way so that it streams from HBM rather than the 256 MB MALL.
    copy_bytes = max(info["bytes"] // 2, 512 << 20)
    src = torch.empty(copy_bytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        fm.fft_stream_copy(src, dst, copy_bytes, stream.cuda_stream)
    torch.cuda.synchronize()
    c0, c1 = ev(), ev()
    c0.record()
    for _ in range(args.steps):
        fm.fft_stream_copy(src, dst, copy_bytes, stream.cuda_stream)
    c1.record()
    torch.cuda.synchronize()
    copy_ms = c0.elapsed_time(c1) / args.steps
    del src, dst

    for _ in range(args.warmup):
        step(0)
    torch.cuda.synchronize()

    def region(stride):
        """K steps launched back to back between one pair of events on the
        launch stream (step i on buffer set i * stride mod sets); ms per step."""
        start, end = ev(), ev()
        torch.cuda.synchronize()
        start.record()
        for i in range(args.steps):
            step(i * stride)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / args.steps

    # Timed region: the same buffers every step (the figure `value` is from).
    ms = region(0)

    # Separate pass, not part of `value`: each launch between its own pair of
    # events, for the spread of single-launch durations.
    marks = [(ev(), ev()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for a, b in marks:
        a.record()
        step(0)
        b.record()
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in marks)

    # Rotated: consecutive steps on different buffer sets, so that nothing a
    # step reads is still in the 256 MB MALL from the step before.
    rotated = None
    if sets > 1:
        for k in range(sets):
            step(k)
        rotated = {"sets": sets, "ms_per_step": round(region(1), 5)}

    if args.copy_calibration:
        # A plain elementwise kernel that reads and writes known byte counts
        # (the input's size each way), for scaling the HBM counters.
        src = torch.ones(info["bytes"] // 2 // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()

    gflops = info["flops"] / (ms * 1e-3) / 1e9
    tbs = info["bytes"] / (ms * 1e-3) / 1e12
    out = {
        "metric": METRIC if args.workload == WORKLOADS[0] else "%s GFLOP/s" % args.workload,
        "value": round(gflops, 1),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": info["dtype"],
        "data": "synthetic",
        "config": {"workload": args.workload, "plan": info["plan"],
                   **{k: info[k] for k in ("n", "d", "h", "w", "batch", "length") if k in info}},
        "hbm_tb_s": round(tbs, 3),
        "launch_us": {"mean": round(sum(per) / len(per) * 1e3, 2), "median": round(per[len(per) // 2] * 1e3, 2),
                      "min": round(per[0] * 1e3, 2), "max": round(per[-1] * 1e3, 2)},
        "copy_ceiling": {"what": "fft_stream_copy of the same bytes (half each way), launched back to back",
                         "gb_s": round(2 * copy_bytes / (copy_ms * 1e-3) / 1e9, 1),
                         "frac_of_copy": round((info["bytes"] / ms) / (2 * copy_bytes / copy_ms), 4)},
        "rotated": rotated,
        "gpu": torch.cuda.get_device_name(dev),
        "gpu_arch": getattr(torch.cuda.get_device_properties(dev), "gcnArchName", None),
        "hip": torch.version.hip,
    }
    if info["kernels"] == 1:
        # One kernel per step: algorithmic bytes (input read once + output
        # written once) over that kernel's average launch duration, which is
        # the timed region's ms per step (the same figure as `value`).
        achieved = info["bytes"] / (ms * 1e-3) / 1e9
        out["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                           "traffic": stored_traffic(args.workload),
                           "kernel_avg_us": round(ms * 1e3, 2)}
    else:
        out["roofline"] = None
        out["roofline_note"] = ("%d kernels per step; per-kernel durations are in the rocprofv3 "
                                "summaries under profiles/" % info["kernels"])
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.workload, info, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
