"""Benchmark of the layout-remapping copy on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic input: a
single lr_layout_copy (plan, launch, kernel) of the largest configuration, the
bf16 head interleave (16,32,4096,128) contiguous -> head pairs adjacent at stride
1, 512 MiB read and 512 MiB written.  Inputs are resident in HBM before the timed
region.  Steps rotate over source / destination buffer pairs (>= 1 GiB together)
so that no step finds its data in the 256 MB Infinity Cache left there by the step
before.

Prints one JSON line.  `value` is effective GB/s = (bytes read + bytes written) /
wall time of K back-to-back steps, with algorithmic bytes 2 * N * elem_bytes per
step.  `roofline` reports the copy kernel's average duration from HIP events
recorded on the launch stream over the timed region; `cpu_baseline` times the CPU
oracle on a bounded slice of the same workload.  `workloads` gives every other
large layout the same treatment (its own roofline and its own same-size copy
ceiling: the library's contiguous copy of the same bytes on the same buffers).

Other modes (for rocprofv3 runs and their summaries under profiles/):
  --counters            launch each large workload a few times, then a plain
                        256 MiB copy whose counters scale FETCH_SIZE / WRITE_SIZE
  --summarize-counters DIR_FETCH DIR_WRITE [DIR_LDS]
                        read rocprofv3 --pmc CSV output and write profiles/traffic.json
  --summarize-trace DIR read rocprofv3 --kernel-trace CSV output and print a
                        markdown table of the library's kernels (per grid size)
  --launch NAME[:JSON]  (repeatable) workload NAME with the lr_copy_tuning
                        overrides in JSON, e.g. padtiles:{"gather_chunks":16}: one
                        untimed launch, then 12 cold launches (rotating buffers)
                        timed with HIP events; for before/after profiles
  --back-to-back K      with --launch: also K launches back to back, timed like
                        the benchmark's timed region
  --atom-sweep          head splits for head dims of 32-512 bytes: tiles of
                        atoms against the source order, beside a plain copy
  --layout-sweep        common layout transforms against a same-size copy
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")

HEADLINE = "interleave"
OTHERS = ("transpose", "retile", "interleave_cm", "nhwc2nchw", "padtiles", "shard_pack", "rgb_nhwc2nchw",
          "head_split")
# traffic.json keys: workload name + element type
DTYPE_NAME = {"transpose": "fp16", "retile": "bf16", "interleave": "bf16", "interleave_cm": "bf16",
              "nhwc2nchw": "fp16", "padtiles": "fp32", "shard_pack": "fp16", "rgb_nhwc2nchw": "fp16",
              "head_split": "bf16"}


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


def _traffic_key(name: str, w) -> str:
    return f"{w.name}_{DTYPE_NAME[name]}"


def _traffic(key: str):
    """HBM bytes per launch measured by rocprofv3 counters (scaled by a plain copy
    of known size), if taken on the current kernel sources; else None."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    e = t.get(key)
    if not e or e.get("kernel_hash") != _kernel_hash():
        return None
    return e.get("bytes_per_launch")


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


# ----------------------------------------------------------------------------
# timing helpers
# ----------------------------------------------------------------------------
def _time_copies(lr, torch, pairs, Ls, Ld, eb, steps, warmup, flags=0, tuning=None):
    """Back-to-back copies rotating over buffer pairs; returns (ms per step of wall
    time, ms per step from HIP events recorded on the launch stream)."""
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        s, d = pairs[i % len(pairs)]
        lr.layout_copy(s, Ls, d, Ld, elem_bytes=eb, flags=flags, stream=stream, tuning=tuning)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(steps):
        s, d = pairs[i % len(pairs)]
        lr.layout_copy(s, Ls, d, Ld, elem_bytes=eb, flags=flags, stream=stream, tuning=tuning)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return wall, ev0.elapsed_time(ev1) / steps


def _time_torch_copies(torch, pairs, steps, warmup):
    """torch's own device-to-device `dst.copy_(src)` of each pair's bytes, back to back
    over the rotating pairs, timed like _time_copies (HIP events on the current
    stream): the same-box copy the library's rates are also compared with."""
    for i in range(warmup):
        s, d = pairs[i % len(pairs)]
        d.copy_(s)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(steps):
        s, d = pairs[i % len(pairs)]
        d.copy_(s)
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps


def _per_launch(lr, torch, pairs, Ls, Ld, eb, launches, flags=0, rotate=True, tuning=None):
    """Kernel time of each launch (HIP events around it on the launch stream), in us,
    sorted: rotating over the buffer pairs (cold: nothing cached from the previous
    launch) or on the first pair only (warm: the last-level cache may hold data).
    One untimed launch comes first."""
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
    s, d = pairs[0]
    lr.layout_copy(s, Ls, d, Ld, elem_bytes=eb, flags=flags, stream=stream, tuning=tuning)
    torch.cuda.synchronize()
    for i, (e0, e1) in enumerate(evs):
        s, d = pairs[(i + 1) % len(pairs)] if rotate else pairs[0]
        e0.record(stream)
        lr.layout_copy(s, Ls, d, Ld, elem_bytes=eb, flags=flags, stream=stream, tuning=tuning)
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


def measure(lr, torch, dev, name, W, steps, warmup, flags=0, first_src=None):
    """Times one workload: the copy over rotating buffers (wall and HIP-event time
    per step), cold and warm per-launch times, and the library's contiguous copy of
    the same bytes on the same buffers (the ceiling a copy without any remapping
    reaches at this size)."""
    w = W.full(name)
    eb = w.elem_bytes
    plan = lr.copy_plan(w.src_layout, w.src_elems, w.dst_layout, w.dst_elems, eb, flags)
    pairs = _pairs(torch, dev, w.src_elems * eb, w.dst_elems * eb, first_src=first_src)
    nbytes = W.bytes_moved(w)
    wall_ms, kern_ms = _time_copies(lr, torch, pairs, w.src_layout, w.dst_layout, eb, steps, warmup, flags)
    cold = _per_launch(lr, torch, pairs, w.src_layout, w.dst_layout, eb, steps, flags)
    warm = _per_launch(lr, torch, pairs, w.src_layout, w.dst_layout, eb, steps, flags, rotate=False)
    n16 = nbytes // 2 // 16  # the same bytes each way, as 16-byte units
    _, copy_ms = _time_copies(lr, torch, pairs, f"{n16}:1", f"{n16}:1", 16, steps, warmup)
    whole = [(s_[:n16 * 16], d_[:n16 * 16]) for s_, d_ in pairs]
    torch_ms = _time_torch_copies(torch, whole, steps, warmup)
    del pairs, whole
    torch.cuda.empty_cache()
    gbps = nbytes / (kern_ms * 1e-3) / 1e9
    copy_gbps = nbytes / (copy_ms * 1e-3) / 1e9
    wm = warm[len(warm) // 2]
    return {
        "w": w, "plan": plan, "bytes": nbytes, "wall_ms": wall_ms, "kern_ms": kern_ms,
        "entry": {
            "path": plan["path"],
            "us": round(kern_ms * 1e3, 2),
            "GBps": round(gbps, 1),
            "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
            "copy_GBps": round(copy_gbps, 1),
            "frac_of_copy": round(gbps / copy_gbps, 4),
            "torch_copy_GBps": round(nbytes / (torch_ms * 1e-3) / 1e9, 1),
            "frac_of_torch_copy": round(gbps / (nbytes / (torch_ms * 1e-3) / 1e9), 4),
            "us_cold_median": round(cold[len(cold) // 2], 2),
            "us_cold_best": round(cold[0], 2),
            "us_warm_median": round(wm, 2),
            "GBps_warm": round(nbytes / (wm * 1e-6) / 1e9, 1),
            "roofline": {"bound": "hbm", "achieved": round(gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": _traffic(_traffic_key(name, w))},
        },
    }


# ----------------------------------------------------------------------------
# CPU baseline: the oracle as it stands
# ----------------------------------------------------------------------------
def _cpu_baseline(seconds: float):
    """The oracle's copy on a slice of the head interleave: batch 0, heads 0..3 (two
    head pairs), every (s, d) -- 2^21 elements, contiguous on both sides, so the
    slice is its own source and destination buffer.  Repeated until about `seconds`
    of work on one thread, then on every host thread at once (each thread its own
    destination, the same sample)."""
    import concurrent.futures as cf

    import numpy as np

    import oracle
    import workloads as W

    hs, s, d = 4, 4096, 128
    n = hs * s * d
    w = W.full(HEADLINE)
    src = W.gen_normal_bf16(n, w.seed)  # the first 2^21 elements of the full source
    Ls = oracle.parse(f"({hs},{s},{d}):({s * d},{d},1)")
    Ld = oracle.parse(f"((2,{hs // 2}),{s},{d}):((1,{2 * s * d}),{2 * d},2)")
    sample = (f"oracle.copy of batch 0, heads 0..3 of the (16,32,4096,128) bf16 head interleave "
              f"({n} elements, {2 * n * 2} bytes moved per repetition)")

    def run_for(dst, t_end):
        k = 0
        while True:
            oracle.copy(src, Ls, dst, Ld, 2)
            k += 1
            if time.perf_counter() >= t_end:
                return k

    dst0 = np.full(n * 2, 0xA5, np.uint8)
    t0 = time.perf_counter()
    reps1 = run_for(dst0, t0 + seconds)
    dt1 = time.perf_counter() - t0
    single = 2 * n * 2 * reps1 / dt1 / 1e9
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    out = {"value": round(single, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"{sample}; {reps1} repetitions in {dt1:.1f} s on one thread",
           "cpu_model": _cpu_model(), "host_threads_available": len(os.sched_getaffinity(0))}
    if threads > 1:
        dsts = [np.full(n * 2, 0xA5, np.uint8) for _ in range(threads)]
        t0 = time.perf_counter()
        with cf.ThreadPoolExecutor(threads) as ex:
            counts = list(ex.map(lambda i: run_for(dsts[i], t0 + seconds), range(threads)))
        dt = time.perf_counter() - t0
        par = 2 * n * 2 * sum(counts) / dt / 1e9
        out.update({"value": round(par, 4), "cores": threads,
                    "sample": f"{sample}; {sum(counts)} repetitions over {threads} threads in {dt:.1f} s "
                              "(NumPy releases the GIL in its indexing)",
                    "single_thread": {"value": round(single, 4), "cores": 1,
                                      "sample": f"{reps1} repetitions in {dt1:.1f} s"}})
    return out


# ----------------------------------------------------------------------------
# rocprofv3 helpers
# ----------------------------------------------------------------------------
def counters_run(lr, torch, W, reps: int = 3):
    """Launch sequence for rocprofv3 runs (kernel trace or --pmc): each large
    workload `reps` times after one warm-up, then a plain contiguous copy of
    256 MiB (the reference of known size that scales FETCH_SIZE / WRITE_SIZE)."""
    dev = torch.device("cuda:0")
    for name in (HEADLINE,) + OTHERS:
        w = W.full(name)
        s = torch.randint(0, 256, (w.src_elems * w.elem_bytes,), dtype=torch.uint8, device=dev)
        d = torch.empty(w.dst_elems * w.elem_bytes, dtype=torch.uint8, device=dev)
        for _ in range(reps + 1):
            lr.layout_copy(s, w.src_layout, d, w.dst_layout, elem_bytes=w.elem_bytes)
        torch.cuda.synchronize()
        grid = lr.copy_plan(w.src_layout, w.src_elems, w.dst_layout, w.dst_elems, w.elem_bytes)["grid"]
        print(f"counters: {_traffic_key(name, w)} grid={grid}", flush=True)
        del s, d
    n = 256 << 20
    s = torch.randint(0, 256, (n,), dtype=torch.uint8, device=dev)
    d = torch.empty(n, dtype=torch.uint8, device=dev)
    for _ in range(reps + 1):
        lr.layout_copy(s, f"{n // 16}:1", d, f"{n // 16}:1", elem_bytes=16)
    torch.cuda.synchronize()
    print(f"counters: plain_copy_256MiB grid={lr.copy_plan(f'{n // 16}:1', n // 16, f'{n // 16}:1', n // 16, 16)['grid']}",
          flush=True)


def launch_run(lr, torch, W, specs, reps: int = 12, back_to_back: int = 0):
    """Each NAME[:JSON] spec: its workload with that tuning, one untimed launch and
    then `reps` launches rotating over buffer pairs of >= 1 GiB in total (cold, as in
    the timed benchmark), each bracketed by HIP events.  With back_to_back = K, then
    also K launches back to back over the same buffers after 3 untimed ones, timed
    like the benchmark's timed region (HIP events around all K).  Prints one line per
    spec; under rocprofv3 each spec is one group of reps + 1 dispatches (reps + 4 + K
    with back_to_back)."""
    dev = torch.device("cuda:0")
    for spec in specs:
        name, _, js = spec.partition(":")
        tuning = json.loads(js) if js else None
        if name.startswith("sweep"):  # sweepK: the K-th transform of LAYOUT_SWEEP
            case, ts, td, eb_ = LAYOUT_SWEEP[int(name[5:])]
            Ls, Ld = lr.parse(ts), lr.parse(td)
            w = W.Workload(name=case, elem_bytes=eb_, src_layout=ts, dst_layout=td, src_elems=Ls.cosize,
                           dst_elems=Ld.cosize, seed=0, values="bits16", n_elems=Ls.size)
        else:
            w = W.full(name)
        eb = w.elem_bytes
        p = lr.copy_plan(w.src_layout, w.src_elems, w.dst_layout, w.dst_elems, eb, tuning=tuning)
        pairs = _pairs(torch, dev, w.src_elems * eb, w.dst_elems * eb)
        us = _per_launch(lr, torch, pairs, w.src_layout, w.dst_layout, eb, reps, tuning=tuning)
        med = us[len(us) // 2]
        b2b = ""
        if back_to_back:
            _, ms = _time_copies(lr, torch, pairs, w.src_layout, w.dst_layout, eb, back_to_back, 3, tuning=tuning)
            b2b = (f" us_back_to_back={ms * 1e3:.2f} "
                   f"GBps_back_to_back={W.bytes_moved(w) / (ms * 1e-3) / 1e9:.0f}")
        print(f"launch: {w.name} tuning={tuning} path={p['path']} grid={p['grid']} "
              f"tile={p['tile_a']}x{p['tile_b']} direct={p['direct']} pipeline_tiles={p['pipeline_tiles']} "
              f"gather_chunks={p['gather_chunks']} us_median={med:.2f} us_best={us[0]:.2f} "
              f"GBps_median={W.bytes_moved(w) / (med * 1e-6) / 1e9:.0f}{b2b}", flush=True)
        del pairs
        torch.cuda.empty_cache()


def atom_sweep(lr, torch, mode: str = "orders", steps: int = 20):
    """(16,s,h,d) -> (16,h,s,d) bf16 head splits for head dims of 32-512 bytes: tiles
    of atoms (vector order 3) against the source order (1) (mode "orders"), or tiles of
    atoms in 128- against 256-lane workgroups, with the 4096^2 retile too (mode
    "lanes"), back to back over rotating buffers, beside a contiguous copy of the same
    bytes.  One JSON line per head dim.  An order the planner cannot take falls back
    (its plan is printed)."""
    dev = torch.device("cuda:0")
    if mode == "lanes":
        import workloads as W
        r = W.full("retile")
        cases = [("retile", r.src_layout, r.dst_layout, r.src_elems)]
        for d, s, h in ((16, 4096, 32), (24, 4096, 32), (32, 4096, 32), (48, 4096, 32), (64, 4096, 32),
                        (96, 4096, 32), (128, 4096, 32), (192, 4096, 16), (256, 4096, 16)):
            cases.append((f"head dim {d}", f"(16,{s},{h},{d}):({s * h * d},{h * d},{d},1)",
                          f"(16,{s},{h},{d}):({h * s * d},{d},{s * d},1)", 16 * s * h * d))
        for name, ts, td, n in cases:
            pairs = _pairs(torch, dev, n * 2, n * 2)
            res = {}
            for rep in range(2):
                for lanes in (128, 256):
                    t = {"vector_order": 3, "workgroup_lanes": lanes}
                    p = lr.copy_plan(ts, n, td, n, 2, tuning=t)
                    _, ms = _time_copies(lr, torch, pairs, ts, td, 2, steps, 3, tuning=t)
                    res.setdefault(lanes, []).append(round(ms * 1e3, 2))
            n16 = n * 2 // 16
            _, cms = _time_copies(lr, torch, pairs, f"{n16}:1", f"{n16}:1", 16, steps, 3)
            print(json.dumps({"case": name, "atom_bytes": None if name == "retile" else 2 * int(name.split()[-1]),
                              "vector_order": p["vector_order"], "us_128": res[128], "us_256": res[256],
                              "copy_us": round(cms * 1e3, 2)}), flush=True)
            del pairs
            torch.cuda.empty_cache()
        return
    for d, s, h in ((16, 4096, 32), (24, 4096, 32), (40, 4096, 32), (48, 4096, 32), (64, 4096, 32), (80, 4096, 32),
                    (96, 4096, 32), (112, 4096, 32), (128, 4096, 32), (160, 4096, 16), (192, 4096, 16),
                    (256, 4096, 16)):
        b = 16
        ts = f"({b},{s},{h},{d}):({s * h * d},{h * d},{d},1)"
        td = f"({b},{s},{h},{d}):({h * s * d},{d},{s * d},1)"
        n = b * s * h * d
        pairs = _pairs(torch, dev, n * 2, n * 2)
        res = {}
        for vo in (3, 1):
            p = lr.copy_plan(ts, n, td, n, 2, tuning={"vector_order": vo})
            _, ms = _time_copies(lr, torch, pairs, ts, td, 2, steps, 3, tuning={"vector_order": vo})
            res[vo] = {"path": p["path"], "vector_order": p["vector_order"], "tile": p["tile_a"],
                       "us": round(ms * 1e3, 2), "GBps": round(4 * n / (ms * 1e-3) / 1e9)}
        # the staged path, which takes short common runs when the atom tiles do not
        staged = None
        try:
            fl = lr.COPY_FORCE_PATH(lr.PATH_STAGED)
            lr.copy_plan(ts, n, td, n, 2, fl)
            _, sms = _time_copies(lr, torch, pairs, ts, td, 2, steps, 3, flags=fl)
            staged = {"us": round(sms * 1e3, 2), "GBps": round(4 * n / (sms * 1e-3) / 1e9)}
        except lr.LayoutRemapError:
            pass
        n16 = n * 2 // 16
        _, cms = _time_copies(lr, torch, pairs, f"{n16}:1", f"{n16}:1", 16, steps, 3)
        default = lr.copy_plan(ts, n, td, n, 2)
        print(json.dumps({"head_dim": d, "atom_bytes": 2 * d, "planner": [default["path"], default["vector_order"]],
                          "order3": res[3], "order1": res[1], "staged": staged, "copy_us": round(cms * 1e3, 2)}),
              flush=True)
        del pairs
        torch.cuda.empty_cache()


# Common layout transforms beyond the workloads above: (name, source, destination,
# element bytes).
LAYOUT_SWEEP = (
    ("fp8 transpose 16384^2", "(16384,16384):(16384,1)", "(16384,16384):(1,16384)", 1),
    ("fp32 transpose 8192^2", "(8192,8192):(8192,1)", "(8192,8192):(1,8192)", 4),
    ("fp64 transpose 4096x8192", "(4096,8192):(8192,1)", "(4096,8192):(1,4096)", 8),
    ("odd-pitch fp16 transpose 8191^2", "(8191,8191):(8191,1)", "(8191,8191):(1,8191)", 2),
    ("batched fp16 64x64 transposes x 16384", "(64,64,16384):(64,1,4096)", "(64,64,16384):(1,64,4096)", 2),
    ("batched fp16 32x32 transposes x 65536", "(32,32,65536):(32,1,1024)", "(32,32,65536):(1,32,1024)", 2),
    ("batched fp16 16x16 transposes x 262144", "(16,16,262144):(16,1,256)", "(16,16,262144):(1,16,256)", 2),
    ("batched fp32 128x96 transposes x 4096", "(128,96,4096):(96,1,12288)", "(128,96,4096):(1,128,12288)", 4),
    ("NCHW->NHWC fp16 (128,256,56,56)", "(128,3136,256):(802816,1,3136)", "(128,3136,256):(802816,256,1)", 2),
    ("NCHW->NHWC fp16 (256,64,112,112)", "(256,12544,64):(802816,1,12544)", "(256,12544,64):(802816,64,1)", 2),
    ("NCHW->NHWC fp16 (256,32,112,112)", "(256,12544,32):(401408,1,12544)", "(256,12544,32):(401408,32,1)", 2),
    ("KV cache (b,s,h,d)->(b,h,d,s) bf16 (8,4096,32,128)", "(8,4096,32,128):(16777216,4096,128,1)",
     "(8,4096,32,128):(16777216,1,524288,4096)", 2),
    ("3-D reversal (a,b,c)->(c,b,a) fp32 512^3", "(512,512,512):(262144,512,1)", "(512,512,512):(1,512,262144)", 4),
    ("3-D permute (a,b,c)->(b,a,c) fp16 (64,1024,2048)", "(2048,1024,64):(1,2048,2097152)",
     "(2048,1024,64):(1,131072,2048)", 2),
    ("padded rows 4096 of 4160 -> compact, fp16 x 8192", "(4096,8192):(1,4160)", "(4096,8192):(1,4096)", 2),
    ("every second row -> compact, fp16 x 4096", "(4096,8192):(1,8192)", "(4096,8192):(1,4096)", 2),
)


def layout_sweep(lr, torch, steps: int = 20):
    """Each LAYOUT_SWEEP transform by the planner's choice, back to back over rotating
    buffers, beside a contiguous copy of the same bytes in 16-byte units (the last
    partial unit left out).  One JSON line each."""
    dev = torch.device("cuda:0")
    for name, ts, td, eb in LAYOUT_SWEEP:
        Ls = lr.parse(ts)
        n, ns, nd = Ls.size, Ls.cosize, lr.parse(td).cosize
        p = lr.copy_plan(ts, ns, td, nd, eb)
        pairs = _pairs(torch, dev, ns * eb, nd * eb)
        _, ms = _time_copies(lr, torch, pairs, ts, td, eb, steps, 3)
        cu = n * eb // 16
        whole = [(s_[:cu * 16], d_[:cu * 16]) for s_, d_ in pairs]  # whole 16-byte units
        _, cms = _time_copies(lr, torch, whole, f"{cu}:1", f"{cu}:1", 16, steps, 3)
        print(json.dumps({"case": name, "path": p["path"], "tile": [p["tile_a"], p["tile_b"]],
                          "vector_order": p["vector_order"], "us": round(ms * 1e3, 2),
                          "GBps": round(2 * n * eb / (ms * 1e-3) / 1e9), "copy_us": round(cms * 1e3, 2),
                          "frac_of_copy": round(cms / ms, 3)}), flush=True)
        del pairs
        torch.cuda.empty_cache()


# transposes for the tile-shape sweep: (name, rows, columns, element bytes) of a
# row-major source and its column-major destination, plus whole-block cases
SHAPE_SWEEP = [(f"{8 * eb}-bit transpose {r}x{c}", r, c, eb) for eb, r, c in (
    (1, 16384, 16384), (1, 8192, 16384), (2, 8192, 8192), (2, 16384, 16384), (2, 4096, 16384), (2, 16384, 4096),
    (4, 8192, 8192), (4, 4096, 8192), (8, 4096, 8192), (8, 4096, 4096), (8, 8192, 8192), (16, 4096, 4096),
    (16, 2048, 4096))]


def shape_sweep(lr, torch, matrices=None, steps: int = 20):
    """Transposes of 1- to 16-byte elements under every transpose tile shape but the
    8 x 8-chunk one (tile_shape 0-6 and 8), each twice in alternation, back to back over
    rotating buffers, beside a contiguous copy of the same bytes; then the layout
    sweep's NCHW -> NHWC and KV-cache transposes and the NHWC -> NCHW workload the same
    way.  `matrices` ("RxCxB": rows, columns, element bytes) replaces the whole list.
    One JSON line per transform, microseconds per shape."""
    import workloads as W
    dev = torch.device("cuda:0")
    if matrices:
        sweep = []
        for m in matrices:
            r, c, eb = (int(x) for x in m.split("x"))
            sweep.append((f"{8 * eb}-bit transpose {r}x{c}", r, c, eb))
        cases = [(name, f"({r},{c}):({c},1)", f"({r},{c}):(1,{r})", eb) for name, r, c, eb in sweep]
    else:
        cases = [(name, f"({r},{c}):({c},1)", f"({r},{c}):(1,{r})", eb) for name, r, c, eb in SHAPE_SWEEP]
        cases += [c for c in LAYOUT_SWEEP if c[0].startswith(("NCHW", "KV"))]
        w = W.full("nhwc2nchw")
        cases.append((w.name, w.src_layout, w.dst_layout, w.elem_bytes))
    for name, ts, td, eb in cases:
        Ls = lr.parse(ts)
        n, ns, nd = Ls.size, Ls.cosize, lr.parse(td).cosize
        pairs = _pairs(torch, dev, ns * eb, nd * eb)
        dflt = lr.copy_plan(ts, ns, td, nd, eb)
        shapes = {}
        for sh in (0, 1, 2, 3, 4, 5, 6, 8):
            p = lr.copy_plan(ts, ns, td, nd, eb, tuning={"tile_shape": sh})
            if p["path"] == "transpose" and (p["tile_a"], p["tile_b"]) not in [v[0] for v in shapes.values()]:
                shapes[sh] = ((p["tile_a"], p["tile_b"]), [])
        for rep in range(2):
            for sh, (_, res) in shapes.items():
                _, ms = _time_copies(lr, torch, pairs, ts, td, eb, steps, 3, tuning={"tile_shape": sh})
                res.append(round(ms * 1e3, 2))
        cu = n * eb // 16
        whole = [(s_[:cu * 16], d_[:cu * 16]) for s_, d_ in pairs]
        _, cms = _time_copies(lr, torch, whole, f"{cu}:1", f"{cu}:1", 16, steps, 3)
        print(json.dumps({"case": name, "eb": eb, "planner_tile": [dflt["tile_a"], dflt["tile_b"]],
                          "us": {str(sh): v[1] for sh, v in shapes.items()},
                          "tiles": {str(sh): list(v[0]) for sh, v in shapes.items()},
                          "copy_us": round(cms * 1e3, 2)}), flush=True)
        del pairs
        torch.cuda.empty_cache()


# transposes for the workgroup-order sweep (rows, columns, element bytes): pitches on,
# just short of and just past multiples of 16 KiB, and others
ORDER_SWEEP = ((8192, 8192, 2), (16384, 16384, 2), (8184, 8184, 2), (8200, 8200, 2), (8208, 8208, 2),
               (8224, 8224, 2), (16400, 16400, 2), (16416, 16416, 2), (4100, 4100, 4), (8200, 8200, 4),
               (4104, 8200, 4), (12296, 12296, 2), (10240, 10240, 2), (12280, 12280, 2))


def order_sweep(lr, torch, matrices=None, steps: int = 20):
    """Transposes under the planner's workgroup order and under orders 0, 1, 2 and 4
    (a-tiles fastest, b-tiles fastest, the two diagonals), each twice in alternation,
    back to back over rotating buffers, best of the two.  One JSON line per matrix."""
    dev = torch.device("cuda:0")
    mats = [tuple(int(x) for x in m.split("x")) for m in matrices] if matrices else ORDER_SWEEP
    for r, c, eb in mats:
        ts, td = f"({r},{c}):({c},1)", f"({r},{c}):(1,{r})"
        n = r * c
        p = lr.copy_plan(ts, n, td, n, eb)
        pairs = _pairs(torch, dev, n * eb, n * eb)
        res = {}
        for rep in range(2):
            for o in (None, 0, 1, 2, 4):
                t = None if o is None else {"tile_order": o}
                _, ms = _time_copies(lr, torch, pairs, ts, td, eb, steps, 3, tuning=t)
                res.setdefault("planner" if o is None else str(o), []).append(round(ms * 1e3, 2))
        print(json.dumps({"matrix": [r, c, eb], "pitch_bytes": [c * eb, r * eb], "tile": [p["tile_a"], p["tile_b"]],
                          "planner_order": p["order"], "us": {k: min(v) for k, v in res.items()}}), flush=True)
        del pairs
        torch.cuda.empty_cache()


def blocks_sweep(lr, torch, steps: int = 20):
    """Register-loaded LDS transposes with one against two V x V blocks per lane
    (transpose_blocks 1 and 2, the same tiles with half the lanes), each twice in
    alternation, back to back over rotating buffers, beside a contiguous copy of the
    same bytes: the transposes of the benchmark workloads and of LAYOUT_SWEEP, and
    fp16 16384^2.  One JSON line per transform."""
    import workloads as W
    dev = torch.device("cuda:0")
    cases = []
    for name in ("transpose", "interleave_cm", "nhwc2nchw", "shard_pack"):
        w = W.full(name)
        cases.append((w.name, w.src_layout, w.dst_layout, w.elem_bytes))
    cases.append(("fp16 transpose 16384^2", "(16384,16384):(16384,1)", "(16384,16384):(1,16384)", 2))
    cases += [c for c in LAYOUT_SWEEP]
    for name, ts, td, eb in cases:
        Ls = lr.parse(ts)
        n, ns, nd = Ls.size, Ls.cosize, lr.parse(td).cosize
        p1 = lr.copy_plan(ts, ns, td, nd, eb, tuning={"transpose_blocks": 1})
        p2 = lr.copy_plan(ts, ns, td, nd, eb, tuning={"transpose_blocks": 2})
        if p2["path"] != "transpose" or p2["block"] == p1["block"]:
            continue
        pairs = _pairs(torch, dev, ns * eb, nd * eb)
        res = {1: [], 2: []}
        for rep in range(2):
            for tb in (1, 2):
                _, ms = _time_copies(lr, torch, pairs, ts, td, eb, steps, 3, tuning={"transpose_blocks": tb})
                res[tb].append(round(ms * 1e3, 2))
        cu = n * eb // 16
        whole = [(s_[:cu * 16], d_[:cu * 16]) for s_, d_ in pairs]
        _, cms = _time_copies(lr, torch, whole, f"{cu}:1", f"{cu}:1", 16, steps, 3)
        print(json.dumps({"case": name, "tile": [p1["tile_a"], p1["tile_b"]], "lanes": [p1["block"], p2["block"]],
                          "us_1": res[1], "us_2": res[2], "copy_us": round(cms * 1e3, 2)}), flush=True)
        del pairs
        torch.cuda.empty_cache()


# 1-byte transposes: matrix shapes (rows x columns, row-major source, column-major
# destination) and the tunings compared on each
BYTE_SHAPES = ((16384, 16384), (8192, 8192), (8192, 16384), (16384, 8192), (4096, 4096), (6144, 6144),
               (12288, 12288), (2048, 32768), (32768, 2048))
BYTE_TUNINGS = (None, {"chunk_bytes": 16, "tile_shape": 0}, {"chunk_bytes": 16, "tile_shape": 1},
                {"chunk_bytes": 16, "tile_shape": 2}, {"chunk_bytes": 16, "tile_shape": 1, "direct_loads": 1},
                {"transpose_reads": 1, "direct_loads": 1, "tile_shape": 0},
                {"transpose_reads": 1, "direct_loads": 1, "tile_shape": 1},
                {"transpose_reads": 1, "direct_loads": 1, "tile_shape": 2},
                {"transpose_reads": 1, "pipeline_tiles": 2, "tile_shape": 0})


def byte_transpose_sweep(lr, torch, shapes, steps: int = 20):
    """1-byte (fp8 / u8) transposes: the planner's 8-byte chunks against 16-byte chunks
    through registers, with direct loads, and read back with the gfx950 1-byte
    transpose reads, back to back over rotating buffers, beside a contiguous copy of
    the same bytes.  One JSON line per shape and tuning."""
    dev = torch.device("cuda:0")
    for R, C in shapes:
        ts, td = f"({R},{C}):({C},1)", f"({R},{C}):(1,{R})"
        n = R * C
        pairs = _pairs(torch, dev, n, n)
        _, cms = _time_copies(lr, torch, pairs, f"{n // 16}:1", f"{n // 16}:1", 16, steps, 3)
        for t in BYTE_TUNINGS:
            p = lr.copy_plan(ts, n, td, n, 1, tuning=t)
            _, ms = _time_copies(lr, torch, pairs, ts, td, 1, steps, 3, tuning=t)
            print(json.dumps({"shape": [R, C], "tuning": t, "chunk_bytes": p["vec_elems"], "direct": p["direct"],
                              "transpose_reads": p["transpose_reads"], "pipeline_tiles": p["pipeline_tiles"],
                              "order": p["order"], "tile": [p["tile_a"], p["tile_b"]], "us": round(ms * 1e3, 2),
                              "GBps": round(2 * n / (ms * 1e-3) / 1e9), "copy_us": round(cms * 1e3, 2),
                              "frac_of_copy": round(cms / ms, 3)}), flush=True)
        del pairs
        torch.cuda.empty_cache()


# Batched small-matrix transposes (matrix A x B, source rows of A, destination rows
# of B, n matrices): element bytes, A, B, n -- 2^27 elements of 2 bytes, or 2^26 of 4
# and 2^25 of 8 (128 MiB each way)
BATCHED_SHAPES = ((2, 16, 16, 262144), (2, 32, 32, 65536), (2, 64, 64, 16384), (2, 24, 24, 116508),
                  (2, 16, 32, 131072), (4, 8, 8, 524288), (4, 16, 16, 131072), (4, 32, 32, 32768),
                  (4, 64, 32, 16384), (8, 16, 16, 65536), (8, 32, 32, 16384))


def batched_sweep(lr, torch, mode: str = "paths", steps: int = 20):
    """Batched small-matrix transposes: the planner's path against the batched,
    staged and transpose paths forced (mode "paths"), or the batched path under each
    of its 16 LDS swizzles and 2 block orders (mode "swizzles", 10 launches each),
    back to back over rotating buffers, beside a contiguous copy of the same bytes.
    One JSON line per shape and variant."""
    dev = torch.device("cuda:0")
    force = lr.COPY_FORCE_PATH(lr.PATH_BATCHED)
    for eb, A, B, n in BATCHED_SHAPES:
        ts, td = f"({B},{A},{n}):({A},1,{A * B})", f"({B},{A},{n}):(1,{B},{A * B})"
        Ls = lr.parse(ts)
        ns, nd, N = Ls.cosize, lr.parse(td).cosize, Ls.size
        pairs = _pairs(torch, dev, ns * eb, nd * eb)
        cu = N * eb // 16
        whole = [(s_[:cu * 16], d_[:cu * 16]) for s_, d_ in pairs]
        _, cms = _time_copies(lr, torch, whole, f"{cu}:1", f"{cu}:1", 16, steps, 3)
        if mode == "swizzles":
            for ci in range(16):
                for order in (0, 1):
                    t = {"batch_swizzle": ci, "batch_order": order}
                    p = lr.copy_plan(ts, ns, td, nd, eb, force, tuning=t)
                    _, ms = _time_copies(lr, torch, pairs, ts, td, eb, 10, 2, flags=force, tuning=t)
                    print(json.dumps({"matrix": [A, B], "elem_bytes": eb, "swizzle": ci, "order": order,
                                      "lds_swizzle": p["batch_swizzle"], "us": round(ms * 1e3, 2),
                                      "frac_of_copy": round(cms / ms, 3)}), flush=True)
            del pairs, whole
            torch.cuda.empty_cache()
            continue
        for label, flags in (("planner", 0), ("batched", force),
                             ("staged", lr.COPY_FORCE_PATH(lr.PATH_STAGED)),
                             ("transpose", lr.COPY_FORCE_PATH(lr.PATH_TRANSPOSE))):
            try:
                p = lr.copy_plan(ts, ns, td, nd, eb, flags)
            except lr.LayoutRemapError:
                print(json.dumps({"matrix": [A, B], "elem_bytes": eb, "count": n, "variant": label,
                                  "path": None}), flush=True)
                continue
            _, ms = _time_copies(lr, torch, pairs, ts, td, eb, steps, 3, flags=flags)
            print(json.dumps({"matrix": [A, B], "elem_bytes": eb, "count": n, "variant": label, "path": p["path"],
                              "us": round(ms * 1e3, 2), "GBps": round(2 * N * eb / (ms * 1e-3) / 1e9),
                              "copy_us": round(cms * 1e3, 2), "frac_of_copy": round(cms / ms, 3)}), flush=True)
        del pairs, whole
        torch.cuda.empty_cache()


def _csv_rows(directory: str, suffix: str):
    rows = []
    for path in sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True)):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def _pmc_per_dispatch(directory: str, counter: str):
    """{dispatch id: (kernel name, grid size, counter value)} from a --pmc run."""
    out = {}
    for r in _csv_rows(directory, "counter_collection.csv"):
        # the library's kernels only (not torch's fills and random draws between them)
        if r.get("Counter_Name") != counter or "lr::k_" not in r.get("Kernel_Name", ""):
            continue
        did = int(r["Dispatch_Id"])
        val = float(r["Counter_Value"])
        name = r.get("Kernel_Name", "")
        grid = int(r.get("Grid_Size", r.get("Grid_Size_X", 0)) or 0)
        k, g, v = out.get(did, (name, grid, 0.0))
        out[did] = (k, g, v + val)  # per-XCD / per-instance rows add up
    return out


def summarize_counters(d_fetch: str, d_write: str, d_lds: str = None) -> None:
    """Turns the counter runs of `bench.py --counters` into profiles/traffic.json:
    per workload, HBM bytes per launch = counter KiB x 1024 x (what the same counter
    reads for the plain 256 MiB copy, scaled to its known 256 MiB)."""
    fetch = _pmc_per_dispatch(d_fetch, "FETCH_SIZE")
    write = _pmc_per_dispatch(d_write, "WRITE_SIZE")
    lds = _pmc_per_dispatch(d_lds, "SQ_LDS_BANK_CONFLICT") if d_lds else {}
    lds_act = _pmc_per_dispatch(d_lds, "SQ_LDS_IDX_ACTIVE") if d_lds else {}
    order = [_traffic_key(n, __import__("workloads").full(n)) for n in (HEADLINE,) + OTHERS] + ["plain_copy_256MiB"]

    def groups(d):
        # dispatches in launch order, grouped 4 per workload (warm-up + 3)
        ids = sorted(d)
        per = len(ids) // len(order)
        return {order[i]: [d[x] for x in ids[i * per:(i + 1) * per]] for i in range(len(order))}

    gf, gw = groups(fetch), groups(write)
    gl, ga = (groups(lds), groups(lds_act)) if lds else ({}, {})
    ref = 256 << 20
    f_scale = ref / (sum(v for _, _, v in gf["plain_copy_256MiB"]) / len(gf["plain_copy_256MiB"]) * 1024)
    w_scale = ref / (sum(v for _, _, v in gw["plain_copy_256MiB"]) / len(gw["plain_copy_256MiB"]) * 1024)
    out = {"_scale": {"fetch": round(f_scale, 4), "write": round(w_scale, 4),
                      "reference": "plain contiguous copy of 256 MiB each way"}}
    for key in order:
        f = [v for _, _, v in gf[key]]
        wv = [v for _, _, v in gw[key]]
        rd = sum(f) / len(f) * 1024 * f_scale
        wr = sum(wv) / len(wv) * 1024 * w_scale
        e = {"bytes_per_launch": int(round(rd + wr)), "read": int(round(rd)), "write": int(round(wr)),
             "kernel_hash": _kernel_hash(), "kernel": gf[key][0][0], "fetch_kib": round(sum(f) / len(f)),
             "write_kib": round(sum(wv) / len(wv))}
        if gl:
            e["lds_bank_conflict_cycles"] = round(sum(v for _, _, v in gl[key]) / len(gl[key]))
            e["lds_active_cycles"] = round(sum(v for _, _, v in ga[key]) / len(ga[key]))
        out[key] = e
    with open(os.path.join(PROFILES, "traffic.json"), "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    # the markdown table of profiles/hbm_traffic_counters.md
    import workloads as W

    alg = {_traffic_key(n, W.full(n)): W.bytes_moved(W.full(n)) for n in (HEADLINE,) + OTHERS}
    alg["plain_copy_256MiB"] = 2 << 28
    print("| workload | kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read MB | HBM write MB | algorithmic MB |"
          " traffic / algorithmic | LDS bank-conflict cycles | LDS active cycles |")
    print("|---" * 10 + "|")
    for key in order:
        e = out[key]
        print(f"| {key} | `{_short(e['kernel'])}` | {e['fetch_kib']} | {e['write_kib']} | {e['read'] / 1e6:.1f} | "
              f"{e['write'] / 1e6:.1f} | {alg[key] / 1e6:.1f} | {e['bytes_per_launch'] / alg[key]:.4f} | "
              f"{e.get('lds_bank_conflict_cycles', '')} | {e.get('lds_active_cycles', '')} |")


def _short(name: str) -> str:
    return name.replace("void ", "").replace("lr::", "").split("(")[0]


def summarize_trace(directory: str, groups_of: int = 0) -> None:
    """Markdown table of the library's kernels from a rocprofv3 --kernel-trace run:
    per kernel and grid size, the number of dispatches and their durations.  With
    groups_of = N, the library's dispatches in launch order, N at a time (the
    --launch runs: one group per spec)."""
    import statistics

    disp = sorted((int(r["Dispatch_Id"]), r) for r in _csv_rows(directory, "kernel_trace.csv")
                  if "lr::k_" in r["Kernel_Name"])
    groups = {}
    for i, (_, r) in enumerate(disp):
        key = (_short(r["Kernel_Name"]), int(r["Grid_Size_X"]) * int(r.get("Grid_Size_Y", 1) or 1))
        if groups_of:
            key = (i // groups_of,) + key
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    head = "| launch group " if groups_of else ""
    print(head + "| kernel | grid (work-items) | dispatches | mean us | median us | min us | max us |")
    print("|---" * (8 if groups_of else 7) + "|")
    order = sorted(groups.items()) if groups_of else sorted(groups.items(), key=lambda x: -sum(x[1]))
    for key, v in order:
        g0 = f"| {key[0] + 1} " if groups_of else ""
        k, g = key[-2:]
        print(g0 + f"| `{k}` | {g} | {len(v)} | {statistics.mean(v):.2f} | {statistics.median(v):.2f} | "
              f"{min(v):.2f} | {max(v):.2f} |")


# ----------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true")
    ap.add_argument("--path", default=None, help="force a copy path (for experiments)")
    ap.add_argument("--counters", action="store_true",
                    help="only launch each large workload a few times (for rocprofv3 runs)")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR")
    ap.add_argument("--summarize-trace", metavar="DIR")
    ap.add_argument("--groups-of", type=int, default=0, help="with --summarize-trace: dispatches per launch group")
    ap.add_argument("--launch", action="append", metavar="NAME[:JSON]",
                    help="a workload by name, or sweepK for the K-th layout-sweep transform, with lr_copy_tuning "
                         "overrides as JSON")
    ap.add_argument("--atom-sweep", nargs="?", const="orders", choices=["orders", "lanes"],
                    help="head splits for head dims of 32-512 bytes: tiles of atoms against the source order, "
                         "or in 128- against 256-lane workgroups")
    ap.add_argument("--layout-sweep", action="store_true",
                    help="common layout transforms (transposes of every element size, batched small "
                         "matrices, NCHW <-> NHWC, 3-D permutes, row gathers) against a same-size copy")
    ap.add_argument("--byte-transpose-sweep", nargs="*", metavar="RxC",
                    help="1-byte transposes (all listed shapes, or these): 8- against 16-byte chunks, "
                         "direct loads and the 1-byte transpose reads")
    ap.add_argument("--batched-sweep", nargs="?", const="paths", choices=["paths", "swizzles"],
                    help="batched small-matrix transposes: the planner's path against the batched, staged and "
                         "transpose paths, or the batched path under each LDS swizzle and block order")
    ap.add_argument("--shape-sweep", nargs="*", metavar="RxCxB",
                    help="transposes of 1- to 16-byte elements under every transpose tile shape (all listed "
                         "matrices and layout transforms, or these rows x columns x element bytes)")
    ap.add_argument("--order-sweep", nargs="*", metavar="RxCxB",
                    help="transposes under the planner's workgroup order and orders 0, 1, 2 and 4")
    ap.add_argument("--blocks-sweep", action="store_true",
                    help="register-loaded LDS transposes with one against two register blocks per lane")
    ap.add_argument("--back-to-back", type=int, default=0, metavar="K",
                    help="with --launch: also time K back-to-back launches per spec")
    args = ap.parse_args()

    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.groups_of)
        return
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
    if args.launch:
        launch_run(lr, torch, W, args.launch, back_to_back=args.back_to_back)
        return
    if args.atom_sweep:
        atom_sweep(lr, torch, args.atom_sweep)
        return
    if args.layout_sweep:
        layout_sweep(lr, torch)
        return
    if args.blocks_sweep:
        blocks_sweep(lr, torch)
        return
    if args.order_sweep is not None:
        order_sweep(lr, torch, args.order_sweep)
        return
    if args.shape_sweep is not None:
        shape_sweep(lr, torch, args.shape_sweep)
        return
    if args.batched_sweep:
        batched_sweep(lr, torch, args.batched_sweep)
        return
    if args.byte_transpose_sweep is not None:
        shapes = [tuple(int(x) for x in s.split("x")) for s in args.byte_transpose_sweep] or BYTE_SHAPES
        byte_transpose_sweep(lr, torch, shapes)
        return

    flags = 0
    if args.path:
        flags = lr.COPY_FORCE_PATH({v: k for k, v in lr.binding.PATH_NAMES.items()}[args.path])

    # ---- headline: the (16,32,4096,128) bf16 head interleave
    src0 = torch.from_numpy(W.make_src(W.full(HEADLINE))).to(dev)
    h = measure(lr, torch, dev, HEADLINE, W, args.steps, args.warmup, flags, first_src=src0)
    del src0
    torch.cuda.empty_cache()
    w = h["w"]
    value = h["bytes"] / (h["wall_ms"] * 1e-3) / 1e9
    e = h["entry"]

    out = {
        "metric": "layout_copy effective GB/s (read+write) and % of HBM peak on 1 MI355X",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(h["wall_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u16",
        "data": "synthetic",
        "config": {
            "workload": "head interleave bf16 (16,32,4096,128): (16,32,4096,128):(16777216,524288,128,1) -> "
                        "(16,(2,16),4096,128):(16777216,(1,1048576),256,2)",
            "path": h["plan"]["path"],
            "vec_elems": h["plan"]["vec_elems"],
            "bytes_per_step": h["bytes"],
            "hbm_frac": round(value / HBM_PEAK_GBPS, 4),
            "copy_kernel_GBps": e["copy_GBps"],
            "kernel_frac_of_copy_kernel": e["frac_of_copy"],
            "torch_copy_GBps": e["torch_copy_GBps"],
            "kernel_frac_of_torch_copy": e["frac_of_torch_copy"],
            "buffers": "rotating pairs, >= 1 GiB in total",
            "kernel_us": {"timed_region_mean": e["us"], "cold_median": e["us_cold_median"],
                          "cold_best": e["us_cold_best"], "warm_median": e["us_warm_median"],
                          "warm": "one buffer pair repeated, the last-level cache may hold part of it"},
        },
        "roofline": e["roofline"],
    }

    # ---- every other large remapping copy, each with its own roofline and ceiling
    if not args.no_others:
        others = {}
        for name in OTHERS:
            r = measure(lr, torch, dev, name, W, max(20, args.steps), args.warmup)
            others[r["w"].name] = r["entry"]
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
        for i, (e0, e1) in enumerate(evs):
            e0.record(stream)
            ev_out[i % 2] = lr.layout_eval(ev_layout, n=n_ev)
            e1.record(stream)
        torch.cuda.synchronize()
        t = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs)
        others["eval 2^27 of a 16384x8192 retile layout"] = {
            "us_median": round(t[len(t) // 2], 1), "Gindex_per_s": round(n_ev / (t[len(t) // 2] * 1e-6) / 1e9, 1),
            "GBps_written": round(8 * n_ev / (t[len(t) // 2] * 1e-6) / 1e9, 1)}
        del ev_out
        out["workloads"] = others

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = _cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
