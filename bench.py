"""Benchmark of the layout-remapping copy on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic input: a
single lr_layout_copy of the fp16 8192 x 8192 transpose
(8192,8192):(8192,1) -> (8192,8192):(1,8192) -- plan, launch, kernel.  Inputs are
resident in HBM before the timed region.  Steps rotate over several source /
destination buffer pairs (>= 1 GiB together) so that no step finds its data in
the 256 MB Infinity Cache left there by the step before.

Prints one JSON line.  `value` is effective GB/s = (bytes read + bytes written) /
time, with algorithmic bytes 2 * N * elem_bytes per step.  The `roofline` object
reports the dominant kernel's average duration from HIP events recorded on the
launch stream over the timed region; `cpu_baseline` times the CPU oracle on a
bounded slice of the same workload.  `workloads` adds the other large layouts
(each timed the same way) for reference.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")


def _kernel_hash() -> str:
    """Hash of the code that decides what the kernels read and write (the kernels and
    the planner), with comments and whitespace removed: only a code change makes
    the stored HBM counters stale."""
    import re

    h = hashlib.sha256()
    for f in ("kernels.hip", "plan.cpp", "lr_internal.h"):
        with open(os.path.join(ROOT, "layout_remapping_copy_amd", "csrc", f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update("".join(text.split()).encode())
    return h.hexdigest()[:16]


def _traffic(workload_key: str):
    """HBM bytes per launch measured by rocprofv3 counters (scaled by a plain copy
    of known size), if taken on the current kernel sources; else None."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    e = t.get(workload_key)
    if not e or e.get("kernel_hash") != _kernel_hash():
        return None
    return e.get("bytes_per_launch")


def _time_copies(lr, torch, pairs, Ls, Ld, eb, steps, warmup, flags=0):
    """Back-to-back copies rotating over buffer pairs; returns (ms per step, ms per
    kernel from HIP events on the launch stream)."""
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        s, d = pairs[i % len(pairs)]
        lr.layout_copy(s, Ls, d, Ld, elem_bytes=eb, flags=flags, stream=stream)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(steps):
        s, d = pairs[i % len(pairs)]
        lr.layout_copy(s, Ls, d, Ld, elem_bytes=eb, flags=flags, stream=stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return wall, ev0.elapsed_time(ev1) / steps


def _per_launch(lr, torch, pairs, Ls, Ld, eb, launches, flags=0, rotate=True):
    """Kernel time of each launch (HIP events around it on the launch stream), in us:
    rotating over the buffer pairs (cold: nothing cached from the previous launch)
    or on the first pair only (warm: the last-level cache may hold the data)."""
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
    s, d = pairs[0]
    lr.layout_copy(s, Ls, d, Ld, elem_bytes=eb, flags=flags, stream=stream)
    torch.cuda.synchronize()
    for i, (e0, e1) in enumerate(evs):
        s, d = pairs[i % len(pairs)] if rotate else pairs[0]
        e0.record(stream)
        lr.layout_copy(s, Ls, d, Ld, elem_bytes=eb, flags=flags, stream=stream)
        e1.record(stream)
    torch.cuda.synchronize()
    return sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs)


def _pairs(torch, dev, nbytes_src, nbytes_dst, first_src=None, min_total=1 << 30):
    n = max(2, -(-min_total // (nbytes_src + nbytes_dst)))
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    out = []
    for i in range(n):
        if i == 0 and first_src is not None:
            s = first_src
        else:
            s = torch.randint(0, 256, (nbytes_src,), dtype=torch.uint8, device=dev, generator=g)
        d = torch.full((nbytes_dst,), 0xA5, dtype=torch.uint8, device=dev)
        out.append((s, d))
    return out


def _cpu_baseline(w, seconds: float):
    """The oracle's copy (as it stands) on the first rows of the same transpose,
    repeated until about `seconds` of CPU time; GB/s on algorithmic bytes."""
    import numpy as np

    import oracle
    import workloads as W

    n = 8192
    rows = 512
    src = W.make_src(w)
    dst = W.make_dst(w)
    Ls = oracle.parse(f"({rows},{n}):({n},1)")   # rows [0, 512) of the source, all columns
    Ld = oracle.parse(f"({rows},{n}):(1,{n})")   # their transposed destinations
    done, t0 = 0, time.perf_counter()
    while True:
        dst = oracle.copy(src, Ls, dst, Ld, w.elem_bytes)
        done += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    bytes_ = 2 * rows * n * w.elem_bytes * done
    out = {
        "value": round(bytes_ / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"oracle.copy of rows 0..{rows - 1} of the 8192x8192 fp16 transpose "
                  f"({rows}x{n} elements), {done} repetitions in {dt:.1f} s, single NumPy thread",
    }
    # the same sample on every host thread at once (each thread its own destination)
    import concurrent.futures as cf

    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    if threads > 1:
        dsts = [W.make_dst(w) for _ in range(threads)]

        def work(i):
            k, t1 = 0, time.perf_counter()
            while True:
                oracle.copy(src, Ls, dsts[i], Ld, w.elem_bytes)
                k += 1
                if time.perf_counter() - t1 >= seconds:
                    return k

        t0 = time.perf_counter()
        with cf.ThreadPoolExecutor(threads) as ex:
            counts = list(ex.map(work, range(threads)))
        dt = time.perf_counter() - t0
        out["parallel"] = {"value": round(2 * rows * n * w.elem_bytes * sum(counts) / dt / 1e9, 4), "cores": threads,
                           "sample": f"the same sample, {sum(counts)} repetitions over {threads} threads in {dt:.1f} s"}
    del np
    return out


def counters_run(lr, torch, W, reps: int = 3):
    """Launch sequence for rocprofv3 runs (kernel trace or --pmc): each large
    workload `reps` times after one warm-up, then a plain contiguous copy of
    256 MiB (the reference of known size that scales FETCH_SIZE / WRITE_SIZE)."""
    dev = torch.device("cuda:0")
    names = ("transpose", "retile", "interleave", "interleave_cm", "nhwc2nchw", "padtiles", "shard_pack", "rgb_nhwc2nchw")
    for name in names:
        w = W.full(name)
        s = torch.randint(0, 256, (w.src_elems * w.elem_bytes,), dtype=torch.uint8, device=dev)
        d = torch.empty(w.dst_elems * w.elem_bytes, dtype=torch.uint8, device=dev)
        for _ in range(reps + 1):
            lr.layout_copy(s, w.src_layout, d, w.dst_layout, elem_bytes=w.elem_bytes)
        torch.cuda.synchronize()
        print(f"counters: {name} grid={lr.copy_plan(w.src_layout, w.src_elems, w.dst_layout, w.dst_elems, w.elem_bytes)['grid']}",
              flush=True)
        del s, d
    n = 256 << 20
    s = torch.randint(0, 256, (n,), dtype=torch.uint8, device=dev)
    d = torch.empty(n, dtype=torch.uint8, device=dev)
    for _ in range(reps + 1):
        lr.layout_copy(s, f"{n // 16}:1", d, f"{n // 16}:1", elem_bytes=16)
    torch.cuda.synchronize()
    print(f"counters: plain copy {n} bytes grid={lr.copy_plan(f'{n // 16}:1', n // 16, f'{n // 16}:1', n // 16, 16)['grid']}",
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true")
    ap.add_argument("--path", default=None, help="force a copy path (for experiments)")
    ap.add_argument("--counters", action="store_true",
                    help="only launch each large workload a few times (for rocprofv3 runs)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the copy is measured on a single "
                                   "MI355X; --gpus must be 1"}), flush=True)
        sys.exit(2)

    import torch

    import layout_remapping_copy_amd as lr
    import workloads as W

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        sys.exit(1)
    lr.lib()  # fails loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    if args.counters:
        counters_run(lr, torch, W)
        return

    flags = 0
    if args.path:
        flags = lr.COPY_FORCE_PATH({v: k for k, v in lr.binding.PATH_NAMES.items()}[args.path])

    # ---- headline: fp16 8192 x 8192 transpose
    w = W.full("transpose")
    src0 = torch.from_numpy(W.make_src(w)).to(dev)
    pairs = _pairs(torch, dev, w.src_elems * 2, w.dst_elems * 2, first_src=src0)
    plan = lr.copy_plan(w.src_layout, w.src_elems, w.dst_layout, w.dst_elems, 2, flags)
    bytes_step = W.bytes_moved(w)
    torch.cuda.synchronize()
    wall_ms, kern_ms = _time_copies(lr, torch, pairs, w.src_layout, w.dst_layout, 2, args.steps, args.warmup, flags)
    value = bytes_step / (wall_ms * 1e-3) / 1e9
    achieved = bytes_step / (kern_ms * 1e-3) / 1e9
    # per-launch kernel times after the timed region: cold (rotating) and warm (one pair)
    cold = _per_launch(lr, torch, pairs, w.src_layout, w.dst_layout, 2, args.steps, flags)
    warm = _per_launch(lr, torch, pairs, w.src_layout, w.dst_layout, 2, args.steps, flags, rotate=False)

    # the library's own contiguous copy (16 bytes per lane) of equal bytes on the same
    # rotating buffers: what a copy without any remapping reaches at this size here
    n16 = bytes_step // 2 // 16
    _, copy_ms = _time_copies(lr, torch, pairs, f"{n16}:1", f"{n16}:1", 16, args.steps, args.warmup)
    copy_kernel = bytes_step / (copy_ms * 1e-3) / 1e9

    # same-box device-to-device copy of equal bytes, for context
    a, b = pairs[0][0], pairs[1][1]
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(20):
        pairs[(i + 1) % len(pairs)][1].copy_(pairs[i % len(pairs)][0])
    e1.record()
    torch.cuda.synchronize()
    d2d = bytes_step / (e0.elapsed_time(e1) / 20 * 1e-3) / 1e9
    del pairs, src0, a, b
    torch.cuda.empty_cache()

    out = {
        "metric": "layout_copy effective GB/s (read+write) and % of HBM peak on 1 MI355X",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u16",
        "data": "synthetic",
        "config": {
            "workload": "transpose fp16 8192x8192: (8192,8192):(8192,1) -> (8192,8192):(1,8192)",
            "path": plan["path"],
            "vec_elems": plan["vec_elems"],
            "bytes_per_step": bytes_step,
            "hbm_frac": round(value / HBM_PEAK_GBPS, 4),
            "d2d_copy_GBps": round(d2d, 1),
            "frac_of_d2d_copy": round(value / d2d, 4),
            "copy_kernel_GBps": round(copy_kernel, 1),
            "kernel_frac_of_copy_kernel": round(achieved / copy_kernel, 4),
            "buffers": "rotating pairs, >= 1 GiB in total",
            "kernel_us": {"median": round(cold[len(cold) // 2], 2), "best": round(cold[0], 2),
                          "warm_median": round(warm[len(warm) // 2], 2), "warm_best": round(warm[0], 2),
                          "warm": "one buffer pair repeated, the last-level cache may hold part of it"},
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": _traffic("transpose8192_fp16"),
        },
    }

    # ---- the other large remapping copies, timed the same way
    if not args.no_others:
        others = {}
        for name in ("retile", "interleave", "interleave_cm", "nhwc2nchw", "padtiles", "shard_pack", "rgb_nhwc2nchw"):
            wo = W.full(name)
            p = lr.copy_plan(wo.src_layout, wo.src_elems, wo.dst_layout, wo.dst_elems, wo.elem_bytes)
            prs = _pairs(torch, dev, wo.src_elems * wo.elem_bytes, wo.dst_elems * wo.elem_bytes)
            steps = max(10, args.steps)
            _, km = _time_copies(lr, torch, prs, wo.src_layout, wo.dst_layout, wo.elem_bytes, steps, args.warmup)
            gb = W.bytes_moved(wo) / (km * 1e-3) / 1e9
            warm = _per_launch(lr, torch, prs, wo.src_layout, wo.dst_layout, wo.elem_bytes, steps, rotate=False)
            wm = warm[len(warm) // 2]
            others[wo.name] = {"path": p["path"], "us": round(km * 1e3, 2), "GBps": round(gb, 1),
                               "hbm_frac": round(gb / HBM_PEAK_GBPS, 4), "us_warm_median": round(wm, 2),
                               "GBps_warm": round(W.bytes_moved(wo) / (wm * 1e-6) / 1e9, 1)}
            del prs
            torch.cuda.empty_cache()
        # latency-only cases: the aliased 8x8 tile copy and two 64-index evaluations
        # (per-launch HIP events, median of 50; these are launch-bound)
        w1 = W.tile8x8()
        s1 = torch.from_numpy(W.make_src(w1)).to(dev)
        d1 = torch.from_numpy(W.make_dst(w1)).to(dev)
        lat = _per_launch(lr, torch, [(s1, d1)], w1.src_layout, w1.dst_layout, 4, 50, lr.COPY_ORDERED_ALIAS, False)
        others["tile8x8_aliased"] = {"path": lr.copy_plan(w1.src_layout, w1.src_elems, w1.dst_layout, w1.dst_elems, 4,
                                                          lr.COPY_ORDERED_ALIAS)["path"],
                                     "us_median": round(lat[len(lat) // 2], 2), "us_best": round(lat[0], 2)}
        stream = torch.cuda.current_stream()
        for text in ("((4,8),2):((16,1),8)", "Sw<3,0,3> o (8,8):(8,1)"):
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(50)]
            lr.layout_eval(text, n=64)
            torch.cuda.synchronize()
            for e0, e1 in evs:
                e0.record(stream)
                lr.layout_eval(text, n=64)
                e1.record(stream)
            torch.cuda.synchronize()
            t = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs)
            others[f"eval64 {text}"] = {"us_median": round(t[len(t) // 2], 2), "us_best": round(t[0], 2)}
        # offset evaluation at scale: every index of a 2^27-element retile layout (the
        # 4096^2 retile's 128 x 64 tiles and Swizzle<3,3,3>, over a 16384 x 8192
        # matrix: four leaves, multiply-high division, the XOR swizzle), 8-byte
        # offsets written
        ev_layout = "Sw<3,3,3> o ((128,128),(64,128)):((64,1048576),(1,8192))"
        n_ev = 1 << 27
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
        ev_out = [lr.layout_eval(ev_layout, n=n_ev) for _ in range(2)]
        torch.cuda.synchronize()
        times = []
        for i, (e0, e1) in enumerate(evs):
            e0.record(stream)
            ev_out[i % 2] = lr.layout_eval(ev_layout, n=n_ev)
            e1.record(stream)
        torch.cuda.synchronize()
        t = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs)
        others["eval 2^27 of a 16384x8192 retile layout"] = {"us_median": round(t[len(t) // 2], 1),
                                             "Gindex_per_s": round(n_ev / (t[len(t) // 2] * 1e-6) / 1e9, 1),
                                             "GBps_written": round(8 * n_ev / (t[len(t) // 2] * 1e-6) / 1e9, 1)}
        del ev_out
        out["workloads"] = others

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = _cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
