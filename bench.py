"""Benchmark of the fused attention forward pass on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME | --shape B,H,N,d,DTYPE] [--entry flash|naive]

One step is one call of the forward pass over the whole workload (every head,
every query tile): the complete hot path. Inputs are seeded synthetic tensors
already resident in device memory when timing starts. The default workload is
the 32K-token long-context case (B=1, H=16, N=32768, d=128, bf16, q and k
drawn with sigma 3). Prints one JSON line:

  value      attention TFLOP/s = 4*B*H*N^2*d / (wall time per step)
  roofline   the kernel's own average duration from HIP events on its stream,
             priced against the dense bf16/fp16 matrix-core peak (2516.6
             TFLOP/s: 256 CUs x 2.4 GHz x 4096 FLOP/clk) -- or the float32 one;
             `traffic` is the measured HBM bytes per launch from the committed
             rocprofv3 counter summary when it matches the current kernel source
  cpu_baseline  the float64 CPU oracle timed on this host on a bounded sample of
             the same workload (whole query rows, about 15 s of work)

  also       (default workload only) the kernel time and TFLOP/s of the
             4096-token case (B=1, H=8, d=128, bf16), the metric's other size

The default 1000 timed calls keep the GPU busy for about 8 s at 32K, long
enough for a utilisation sampler running beside the benchmark to see it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s and % of bf16 MFMA peak at N=4096/32768, d=128"
PEAK_TFLOPS = {"bf16": 2516.6, "fp16": 2516.6, "fp32": 157.3}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "io_aware_tiled_06_amd", "csrc")


# The sources each timed kernel is compiled from (its own file plus the shared
# device helpers): a counter record is only valid for the source it was taken on.
KERNEL_SOURCES = {"flash": ("flash_fwd.hip", "fa_device.h"), "naive": ("naive.hip", "fa_device.h")}


def kernel_source_hash(entry: str = "flash") -> str:
    """Hash of the sources a timed kernel is built from, and of any
    per-source code-generation flags of the build (they change the binary)."""
    from io_aware_tiled_06_amd.build import SOURCE_FLAGS

    h = hashlib.sha256()
    for name in sorted(KERNEL_SOURCES[entry]):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
        if SOURCE_FLAGS.get(name):
            h.update(b"\0flags\0" + " ".join(SOURCE_FLAGS[name]).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, entry: str):
    """HBM bytes per launch from the committed counter summary, or None if the
    summary is missing or was taken from a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    rec = data.get(f"{entry}:{workload}")
    if not rec or rec.get("source_hash") != kernel_source_hash(entry):
        return None
    return rec.get("hbm_bytes_per_launch")


def _counter_rows(path: str, counter: str):
    """(dispatch id, kernel name, grid size, value) of one counter in a
    rocprofv3 --pmc counter_collection.csv, in dispatch order."""
    import csv

    with open(path, newline="") as f:
        rows = [(int(r["Dispatch_Id"]), r["Kernel_Name"], r["Grid_Size"], float(r["Counter_Value"]))
                for r in csv.DictReader(f) if r["Counter_Name"] == counter]
    return sorted(rows)


# Kernels each entry point dispatches (name patterns in the profiler's records).
ENTRY_KERNELS = {"flash": r"flash_fwd_", "naive": r"naive_"}


def _short_name(name: str) -> str:
    return name.replace("void fa::(anonymous namespace)::", "").split("(")[0].replace("fa::", "").replace(" ", "")


def launch_counter(path: str, counter: str, entry: str, launches: int, warmup: int):
    """Per-launch total of one counter over every kernel an entry point
    dispatches: the dispatches matching ENTRY_KERNELS[entry], in order, fall
    into warmup + launches equal groups (one per call; a call may dispatch
    several kernels, e.g. the three passes of the naive path or the two
    launches of a split grid); the warm-up groups are left out and the rest
    averaged. Returns (kernel names, dispatches per launch, mean per launch)."""
    import re

    rows = [r for r in _counter_rows(path, counter) if re.search(ENTRY_KERNELS[entry], r[1])]
    total = warmup + launches
    if not rows or len(rows) % total:
        raise ValueError(f"{path}: {len(rows)} {entry} dispatches do not split into {total} launches")
    per = len(rows) // total
    timed = rows[warmup * per:]
    names = sorted({_short_name(n) for _, n, _, _ in timed})
    return names, per, sum(v for _, _, _, v in timed) / launches


def record_traffic(fetch_csv: str, write_csv: str, copy_fetch_csv: str, copy_write_csv: str,
                   workload: str = "n32768_d128_bf16", entry: str = "flash", launches: int = 2, warmup: int = 1,
                   copy_bytes: int = 1 << 30) -> dict:
    """Write the HBM-traffic record of (entry, workload) into profiles/traffic.json.

    Inputs: the counter files of four rocprofv3 --pmc runs: FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch) of `bench.py --workload W --entry E --steps
    <launches> --warmup <warmup> --no-cpu-baseline --no-also`, and the same two
    counters for `bench.py --copy-calibration 1073741824`. Every dispatch of
    the entry point's kernels counts; warm-up calls are left out and the rest
    averaged per call. Each counter is scaled so that the copy reads and
    writes exactly `copy_bytes`. The record carries the current kernel source
    hash, so bench.py uses it only for the binary it was taken on.
    """
    from io_aware_tiled_06_amd import traffic
    from io_aware_tiled_06_amd.workloads import WORKLOADS

    def copy_mean(path, counter):
        vals = [v for _, n, _, v in _counter_rows(path, counter) if "copyBuffer" in n]
        if not vals:
            raise ValueError(f"{path}: no copy dispatch")
        return sum(vals) / len(vals)

    names, per, fetch = launch_counter(fetch_csv, "FETCH_SIZE", entry, launches, warmup)
    _, _, write = launch_counter(write_csv, "WRITE_SIZE", entry, launches, warmup)
    cf, cw = copy_mean(copy_fetch_csv, "FETCH_SIZE"), copy_mean(copy_write_csv, "WRITE_SIZE")
    fs, ws = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    w = WORKLOADS[workload]
    rd, wr = round(fetch * 1024 * fs), round(write * 1024 * ws)
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        data = {}
    data[f"{entry}:{workload}"] = {
        "source_hash": kernel_source_hash(entry), "kernels": names, "dispatches_per_launch": per,
        "fetch_kib_per_launch": fetch, "write_kib_per_launch": write,
        "fetch_scale": round(fs, 6), "write_scale": round(ws, 6),
        "hbm_read_bytes_per_launch": rd, "hbm_write_bytes_per_launch": wr, "hbm_bytes_per_launch": rd + wr,
        "compulsory_bytes": traffic.compulsory_bytes(w.B, w.H, w.N, w.d, w.elem_bytes),
    }
    data["_calibration"] = {"copy_bytes": copy_bytes, "copy_fetch_kib": cf, "copy_write_kib": cw}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(data, f, indent=1)
    return data[f"{entry}:{workload}"]


class ClockSampler:
    """Samples the GPU's shader clock and board power while the timed loop runs.

    Reads the amdgpu kernel driver's sysfs files of the one GPU card present: the current
    shader-clock level (``pp_dpm_sclk``, the line marked ``*``) and the board
    power (hwmon ``power1_input``, microwatts) every ``period`` seconds from a
    host thread. The matrix-core peak assumes the full 2.4 GHz clock; under
    sustained dense work the card may run slower. The kernel driver's clock figure is
    the firmware's smoothed value, not a cycle count: it shows the trend, while
    the exact cycles of a launch come from the GRBM_COUNT counter under
    rocprofv3. Gives None where the files are absent or more than one card is
    present (the card could not be told apart).
    """

    def __init__(self, period: float = 0.005, root: str = "/sys/class/drm"):
        import glob
        import threading

        self.period = period
        self.sclk, self.power = [], []
        cards = [c for c in sorted(glob.glob(os.path.join(root, "card*", "device")))
                 if os.path.exists(os.path.join(c, "pp_dpm_sclk"))]
        self.card = cards[0] if len(cards) == 1 else None
        self.power_file = None
        self.cap_w = None
        if self.card:
            hw = sorted(glob.glob(os.path.join(self.card, "hwmon", "hwmon*")))
            if hw and os.path.exists(os.path.join(hw[0], "power1_input")):
                self.power_file = os.path.join(hw[0], "power1_input")
                try:
                    with open(os.path.join(hw[0], "power1_cap")) as f:
                        self.cap_w = int(f.read()) / 1e6
                except (OSError, ValueError):
                    pass
        self.levels_mhz = self._levels() if self.card else []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _levels(self) -> list:
        """The shader-clock levels the card lists (numbered lines of
        pp_dpm_sclk, MHz); the highest is its top clock."""
        import re

        out = []
        try:
            with open(os.path.join(self.card, "pp_dpm_sclk")) as f:
                for ln in f:
                    m = re.match(r"\s*\d+:\s*(\d+)\s*[Mm]hz", ln)
                    if m:
                        out.append(int(m.group(1)))
        except (OSError, ValueError):
            pass
        return out

    def _sample(self) -> None:
        import re

        try:
            with open(os.path.join(self.card, "pp_dpm_sclk")) as f:
                for ln in f:
                    m = re.search(r"(\d+)\s*[Mm]hz\s*\*", ln)
                    if m:
                        self.sclk.append(int(m.group(1)))
                        break
            if self.power_file:
                with open(self.power_file) as f:
                    self.power.append(int(f.read()) / 1e6)
        except (OSError, ValueError):
            pass

    def _run(self) -> None:
        while not self._stop.is_set():
            self._sample()
            self._stop.wait(self.period)

    def __enter__(self):
        if self.card:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self.card:
            self._stop.set()
            self._thread.join()
        return False

    def summary(self):
        if not self.sclk:
            return None
        import statistics

        out = {"sclk_mhz_median": statistics.median(self.sclk), "sclk_mhz_min": min(self.sclk),
               "sclk_mhz_max": max(self.sclk), "samples": len(self.sclk),
               "source": "sysfs pp_dpm_sclk (marked level) and hwmon power1_input, sampled during the timed loop"}
        if self.power:
            out["power_w_median"] = round(statistics.median(self.power), 1)
        if self.cap_w:
            out["power_cap_w"] = self.cap_w
        if self.levels_mhz:
            out["sclk_top_level_mhz"] = max(self.levels_mhz)
        return out


def time_entry(name: str, entry: str = "flash", steps: int = 20, warmup: int = 5) -> dict:
    """Kernel time of one entry point (fused or three-pass) on a named
    workload: HIP events on the launch stream around each call, the calls
    queued back to back behind a spin kernel. The metric names both the 4096-
    and the 32768-token cases; the comparison with the three-pass path uses
    the same timing."""
    import numpy as np
    import torch

    import io_aware_tiled_06_amd as fa
    from io_aware_tiled_06_amd import traffic
    from io_aware_tiled_06_amd.workloads import WORKLOADS, make_inputs

    w = WORKLOADS[name]
    dev = torch.device("cuda:0")
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[w.dtype]
    tq, tk, tv = (torch.from_numpy(x).to(tdt).to(dev) for x in make_inputs(w))
    o = torch.empty_like(tq)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    ws = None
    if entry == "naive":
        ws = torch.empty(fa.attn_naive_workspace_bytes(w.B, w.H, w.N, w.dtype), dtype=torch.uint8, device=dev)
        call = lambda: fa.attn_naive_fwd(tq, tk, tv, w.scale, out=o, workspace=ws)  # noqa: E731
    else:
        call = lambda: fa.flash_attn_fwd(tq, tk, tv, w.scale, out=o)  # noqa: E731
    for _ in range(warmup):
        call()
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize(dev)
    # A 0.07 ms launch is shorter than the host's time to issue an event and a
    # launch, so the device would idle inside some event pairs. A spin kernel
    # (about 10 ms) holds the stream while all launches and events are queued;
    # the pairs then bracket back-to-back launches only.
    torch.cuda._sleep(20_000_000)
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize(dev)
    ms = [a.elapsed_time(b) for a, b in ev]
    tflops = traffic.attention_flops(w.B, w.H, w.N, w.d) / (float(np.mean(ms)) * 1e-3) / 1e12
    out = {"workload": name, "entry": entry, "cache": cache_label(w), "kernel_ms": round(float(np.mean(ms)), 4),
           "kernel_ms_median": round(float(np.median(ms)), 4), "tflops": round(tflops, 3),
           "frac_of_peak": round(tflops / PEAK_TFLOPS[w.dtype], 4), "steps": steps,
           "workspace_bytes": int(ws.numel()) if ws is not None else 0}
    del ws
    torch.cuda.empty_cache()
    return out


INFINITY_CACHE_BYTES = 256 << 20  # MI355X's last-level (MALL) cache


def cache_label(w) -> str:
    """Whether a timed call can run from warm caches: back-to-back calls on
    inputs and outputs that fit the 256 MB Infinity Cache find them there
    (no cache flush between calls)."""
    from io_aware_tiled_06_amd import traffic

    c = traffic.compulsory_bytes(w.B, w.H, w.N, w.d, w.elem_bytes)
    if c <= INFINITY_CACHE_BYTES:
        return f"warm: Q, K, V, O and LSE ({c / 1e6:.1f} MB) fit the 256 MB Infinity Cache"
    return f"cold: Q, K, V, O and LSE ({c / 1e6:.1f} MB) exceed every cache"


def time_forward(name: str, steps: int = 20, warmup: int = 5) -> dict:
    """Kernel time of the fused forward pass on a named workload."""
    out = time_entry(name, "flash", steps, warmup)
    for k in ("entry", "workspace_bytes"):
        out.pop(k)
    return out


COMPARE_WORKLOADS = ("n4096_d128_bf16", "n10000_d128_fp16", "b32_n512_d64_bf16", "n32768_d128_bf16")


def phase_clock_summary(recs, event_us: float) -> dict:
    """Summary of one launch's phase-clock records (8 words each, see
    FA_DEBUG_CLOCK in flash_fwd.hip): per-workgroup phase times, how many
    workgroups each CU held and ran in their loops over the launch, the gap
    between a workgroup's end and the next start on its CU, when the first
    workgroups of each XCD started, and each XCD's clock and last end. A
    workgroup's phase boundaries are placed in real time with its own clock
    (its cycles over its s_memrealtime duration): clocks differ between
    XCDs and over time."""
    import collections

    import numpy as np

    a = np.asarray(recs, dtype=np.uint64).reshape(-1, 8)
    a = a[(a[:, 7] & 0xFF) == 1]
    r0 = a[:, 0].astype(np.int64)
    r1 = a[:, 1].astype(np.int64)
    cyc = a[:, 2:5].astype(np.float64)
    dur_ns = (r1 - r0) * 10.0  # s_memrealtime runs at 100 MHz
    ghz = float(cyc[:, 2].sum() / dur_ns.sum())
    ghz_wg = cyc[:, 2] / np.maximum(dur_ns, 1.0)  # each workgroup's own clock
    t0 = r0.min()
    start, end = (r0 - t0) * 10.0, (r1 - t0) * 10.0
    span = float(end.max())
    hw = a[:, 5].astype(np.int64)
    xcc = a[:, 6].astype(np.int64) & 0xF
    cu = xcc * 256 + ((hw >> 8) & 0xFF)
    pro, loop_end = cyc[:, 0] / ghz_wg, cyc[:, 1] / ghz_wg  # ns from the workgroup's start
    grid = np.arange(0.0, span + 20.0, 20.0)
    resident, in_loop = collections.Counter(), collections.Counter()
    gaps, last_end = [], []
    by_cu = collections.defaultdict(list)
    for i in range(len(a)):
        by_cu[int(cu[i])].append(i)
    for idx in by_cu.values():
        occ = np.zeros(len(grid), dtype=np.int32)
        lo = np.zeros(len(grid), dtype=np.int32)
        for i in idx:
            occ[(grid >= start[i]) & (grid < end[i])] += 1
            lo[(grid >= start[i] + pro[i]) & (grid < start[i] + loop_end[i])] += 1
        resident.update(occ.tolist())
        in_loop.update(lo.tolist())
        starts = np.sort(start[idx])
        for e in end[idx]:
            later = starts[starts >= e - 10.0]
            if len(later):
                gaps.append(float(later[0] - e))
        last_end.append(float(end[idx].max()))
    per_cu = collections.Counter(len(v) for v in by_cu.values())
    xcd_first = {int(x): round(float(start[xcc == x].min()) / 1e3, 3) for x in sorted(set(xcc.tolist()))}
    q = lambda v: [round(float(np.quantile(v, t)) / 1e3, 3) for t in (0.0, 0.5, 1.0)]  # noqa: E731
    xcd = {int(x): {"clock_ghz": round(float(cyc[xcc == x, 2].sum() / dur_ns[xcc == x].sum()), 3),
                    "workgroups": int((xcc == x).sum()), "last_end_us": round(float(end[xcc == x].max()) / 1e3, 2)}
           for x in sorted(set(xcc.tolist()))}
    tot = sum(resident.values())
    return {
        "event_us": round(event_us, 2), "span_us": round(span / 1e3, 2), "workgroups": int(len(a)),
        "cus": len(by_cu), "workgroups_per_cu": {int(k): v for k, v in sorted(per_cu.items())},
        "clock_ghz": round(ghz, 3),
        "prologue_us_min_median_max": q(pro), "loop_us_min_median_max": q(loop_end - pro),
        "epilogue_us_min_median_max": q(dur_ns - loop_end),
        "share_with_k_resident": {int(k): round(v / tot, 3) for k, v in sorted(resident.items())},
        "share_with_k_in_loop": {int(k): round(v / tot, 3) for k, v in sorted(in_loop.items())},
        "gap_end_to_next_start_us_median": round(float(np.median(gaps)) / 1e3, 3) if gaps else None,
        "cu_last_end_us_min_median_max": q(np.asarray(last_end)),
        "xcd_first_start_us": xcd_first,
        "per_xcd": xcd,
    }


def phase_clock(w, causal: bool, reps: int = 3, warmup: int = 30) -> None:
    """Run the workload through the phase-clock build and print one JSON line
    per launch (phase_clock_summary). The build's extra code keeps the
    kernels' registers and occupancy; its timings are those of the same
    launch with a few more instructions per workgroup."""
    import ctypes

    import torch

    import io_aware_tiled_06_amd as fa
    from io_aware_tiled_06_amd.workloads import make_inputs

    if not os.path.exists(fa.CLOCK_LIB_PATH):
        from io_aware_tiled_06_amd import build as _b

        _b.build(variant="clock")
    dev = torch.device("cuda:0")
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[w.dtype]
    tq, tk, tv = (torch.from_numpy(x).to(tdt).to(dev) for x in make_inputs(w))
    o = torch.empty_like(tq)
    n_max = 65536
    with fa.using_library(fa.CLOCK_LIB_PATH) as L:
        L.fa_clock_clear.restype = ctypes.c_int
        L.fa_clock_read.argtypes = [ctypes.POINTER(ctypes.c_ulonglong), ctypes.c_int]
        L.fa_clock_read.restype = ctypes.c_int
        for _ in range(warmup):
            fa.flash_attn_fwd(tq, tk, tv, w.scale, causal=causal, out=o)
        buf = (ctypes.c_ulonglong * (8 * n_max))()
        stream = torch.cuda.current_stream(dev)
        for rep in range(reps):
            for _ in range(5):  # the clock where a stream of calls holds it
                fa.flash_attn_fwd(tq, tk, tv, w.scale, causal=causal, out=o)
            torch.cuda.synchronize(dev)
            if L.fa_clock_clear() != 0:
                raise RuntimeError("fa_clock_clear failed")
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fa.flash_attn_fwd(tq, tk, tv, w.scale, causal=causal, out=o)
            e1.record(stream)
            torch.cuda.synchronize(dev)
            n = L.fa_clock_read(buf, n_max)
            if n < 0 or n > n_max:
                raise RuntimeError(f"fa_clock_read returned {n}")
            out = phase_clock_summary(list(buf)[:8 * n], e0.elapsed_time(e1) * 1e3)
            out = {"workload": w.name, "causal": causal, "rep": rep, **out}
            print(json.dumps(out), flush=True)


def compare_paths(steps: int = 20) -> None:
    """The fused and the three-pass path on each half-precision workload: one
    JSON line per (workload, path) with kernel time, TFLOP/s, fraction of the
    matrix-core peak, the three-pass workspace, and the measured HBM bytes
    per call with M/C (measured over compulsory bytes) when profiles/traffic.json
    holds a record taken on the current kernel source."""
    from io_aware_tiled_06_amd import traffic
    from io_aware_tiled_06_amd.workloads import WORKLOADS

    for name in COMPARE_WORKLOADS:
        w = WORKLOADS[name]
        for entry in ("flash", "naive"):
            n = steps if entry == "flash" or w.N < 32768 else max(3, steps // 5)
            rec = time_entry(name, entry, n, 2)
            hbm = measured_traffic(name, entry)
            c = traffic.compulsory_bytes(w.B, w.H, w.N, w.d, w.elem_bytes)
            rec["hbm_bytes_per_call"] = hbm
            rec["m_over_c"] = round(hbm / c, 3) if hbm else None
            rec["compulsory_bytes"] = c
            print(json.dumps(rec), flush=True)


def cpu_baseline(w, q, k, v, target_s: float = 15.0):
    """Time the float64 oracle for about target_s seconds on whole query rows of
    the workload (head by head)."""
    import numpy as np

    from oracle import attention_reference

    threads = None
    try:
        from threadpoolctl import threadpool_info

        threads = max((i.get("num_threads") or 0) for i in threadpool_info()) or None
    except Exception:  # noqa: BLE001 - informational only
        pass
    if threads is None:
        threads = len(os.sched_getaffinity(0))
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    rows0 = min(w.N, 512)
    t0 = time.perf_counter()
    attention_reference(q[0, 0][None, :rows0], k[0, 0][None], v[0, 0][None], w.scale)
    t_probe = time.perf_counter() - t0
    # whole heads first, then a row prefix of the next one, for ~target_s seconds
    want = int(rows0 * target_s / max(t_probe, 1e-6))
    n_heads = min(len(heads), want // w.N)
    rows_last = 0 if n_heads == len(heads) else max(0, min(w.N, want - n_heads * w.N))
    if n_heads == 0:
        rows_last = max(rows0, rows_last)
    t0 = time.perf_counter()
    for b, h in heads[:n_heads]:
        attention_reference(q[b, h][None], k[b, h][None], v[b, h][None], w.scale)
    if rows_last:
        b, h = heads[n_heads]
        attention_reference(q[b, h][None, :rows_last], k[b, h][None], v[b, h][None], w.scale)
    t = time.perf_counter() - t0
    rows = n_heads * w.N + rows_last
    flops = 4.0 * rows * w.N * w.d
    blas = None
    try:
        cfg = np.show_config(mode="dicts")
        blas = cfg["Build Dependencies"]["blas"]["name"]
    except Exception:  # noqa: BLE001 - informational only
        pass
    cpu = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    return {
        "value": round(flops / t / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "cpu_model": cpu,
        "blas": blas,
        "seconds": round(t, 2),
        "kind": "oracle",
        "sample": (f"{n_heads} whole head(s) + {rows_last} query rows of the next, each row against all "
                   f"{w.N} keys ({rows} rows of {w.B * w.H * w.N}), float64 numpy; {t:.2f} s"),
    }


def copy_calibration(nbytes: int, reps: int) -> None:
    """A plain device-to-device copy of `nbytes` (torch's copy kernel), to scale
    the FETCH_SIZE / WRITE_SIZE counters: it reads and writes exactly nbytes."""
    import torch

    x = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    y = torch.empty_like(x)
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}), flush=True)


SWEEP_N = (1024, 2048, 4096, 8192, 16384, 32768)


def traffic_sweep(entry: str) -> None:
    """Two launches (the first is a warm-up) of one entry point at each N in
    SWEEP_N, B=1, H=16, d=128, bf16, inputs N(0,1) drawn on the GPU from a
    fixed seed (traffic does not depend on the values). Run under
    `rocprofv3 --pmc FETCH_SIZE` / `WRITE_SIZE`: the dispatches appear in this
    order, one per flash launch and three per naive launch (all heads fit one
    workspace chunk)."""
    import torch

    import io_aware_tiled_06_amd as fa

    if not os.path.exists(fa.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(5)
    for n in SWEEP_N:
        shape = (1, 16, n, 128)
        q, k, v = (torch.randn(shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
                   for _ in range(3))
        torch.cuda.synchronize(dev)
        torch.cuda.reset_peak_memory_stats(dev)
        base = torch.cuda.memory_allocated(dev)
        o = torch.empty_like(q)
        ws = None
        if entry == "naive":
            ws = torch.empty(fa.attn_naive_workspace_bytes(1, 16, n, "bf16"), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize(dev)
        times = []
        for _ in range(2):
            t0 = time.perf_counter()
            if entry == "naive":
                fa.attn_naive_fwd(q, k, v, out=o, workspace=ws)
            else:
                fa.flash_attn_fwd(q, k, v, out=o)
            torch.cuda.synchronize(dev)
            times.append(time.perf_counter() - t0)
        print(json.dumps({"sweep": entry, "N": n, "B": 1, "H": 16, "d": 128, "dtype": "bf16",
                          "wall_ms": round(times[-1] * 1e3, 4),
                          "extra_device_bytes": int(torch.cuda.max_memory_allocated(dev) - base)}), flush=True)
        del q, k, v, o, ws
        torch.cuda.empty_cache()


CROSSOVER_N = (16, 32, 64, 128, 256, 512, 1024, 2048, 4096)


def crossover_sweep(reps: int = 10, d: int = 128, dtype: str = "bf16") -> None:
    """Fused versus three-pass path at a fixed amount of work: H = 16, head
    size d, element type dtype, B chosen so that B*H*N^2 = 16*4096^2 at every N. For each N and path:
    median kernel time over `reps` launches (HIP events on the current stream,
    after 2 warm-ups) and the device memory the call needs beyond Q, K, V
    (the outputs, plus the three-pass workspace), from torch's allocator peak.
    One JSON line per (path, N); a final line names the crossover, the largest
    N at which the three-pass path is faster (null if it never is)."""
    import numpy as np
    import torch

    import io_aware_tiled_06_amd as fa

    if not os.path.exists(fa.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(6)
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    work = 16 * 4096 * 4096
    faster_naive = []
    for n in CROSSOVER_N:
        b = max(1, work // (16 * n * n))
        shape = (b, 16, n, d)
        q, k, v = (torch.randn(shape, generator=gen, device=dev, dtype=torch.float32).to(tdt)
                   for _ in range(3))
        ms = {}
        for entry in ("flash", "naive"):
            torch.cuda.synchronize(dev)
            torch.cuda.reset_peak_memory_stats(dev)
            base = torch.cuda.memory_allocated(dev)
            o = torch.empty_like(q)
            lse = torch.empty((b, 16, n), dtype=torch.float32, device=dev)
            ws = None
            if entry == "naive":
                ws = torch.empty(fa.attn_naive_workspace_bytes(b, 16, n, dtype), dtype=torch.uint8, device=dev)
            call = (lambda: fa.attn_naive_fwd(q, k, v, out=o, workspace=ws)) if entry == "naive" else \
                (lambda: fa.flash_attn_fwd(q, k, v, out=o))
            for _ in range(2):
                call()
            st = torch.cuda.current_stream(dev)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
            ev[0].record(st)
            for i in range(reps):
                call()
                ev[i + 1].record(st)
            torch.cuda.synchronize(dev)
            t = float(np.median([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]))
            extra = torch.cuda.max_memory_allocated(dev) - base
            ms[entry] = t
            print(json.dumps({"crossover": entry, "N": n, "B": b, "H": 16, "d": d, "dtype": dtype,
                              "kernel_ms": round(t, 5),
                              "tflops": round(4.0 * b * 16 * n * n * d / (t * 1e-3) / 1e12, 2),
                              "extra_device_bytes": int(extra)}), flush=True)
            del o, lse, ws
            torch.cuda.empty_cache()
        if ms["naive"] < ms["flash"]:
            faster_naive.append(n)
        del q, k, v
        torch.cuda.empty_cache()
    print(json.dumps({"d": d, "dtype": dtype,
                      "crossover_naive_faster_up_to_N": max(faster_naive) if faster_naive else None,
                      "naive_faster_at": faster_naive}), flush=True)


def collect_counters(out_dir: str, workloads, entries, copy_bytes: int = 1 << 30) -> None:
    """Measure HBM bytes per call of each (entry, workload) and write the
    records into profiles/traffic.json.

    Runs, each as a child process under `rocprofv3 --pmc <counter> -f csv`
    (one counter per pass; this process itself never touches the GPU):
      bench.py --copy-calibration <copy_bytes>                  FETCH_SIZE, WRITE_SIZE
      bench.py --workload W --entry E --steps 2 --warmup 1
               --no-cpu-baseline --no-also                       FETCH_SIZE, WRITE_SIZE
    into out_dir/<name>/run_counter_collection.csv, then record_traffic on the
    four files of each pair. A pass that fails or outlives its time limit
    stops the collection."""
    import subprocess

    me = os.path.abspath(__file__)

    def pmc(name, counter, args, limit=300):
        d = os.path.join(out_dir, f"{name}_{counter}")
        cmd = ["timeout", "-s", "KILL", str(limit), "rocprofv3", "--pmc", counter, "-f", "csv", "-d", d, "-o", "run",
               "--", sys.executable, me, *args]
        print(f"[counters] {name} {counter}", file=sys.stderr, flush=True)
        with open(os.path.join(out_dir, f"{name}_{counter}.log"), "w") as log:
            r = subprocess.run(cmd, stdout=log, stderr=subprocess.STDOUT)
        csv_path = os.path.join(d, "run_counter_collection.csv")
        if r.returncode != 0 or not os.path.exists(csv_path):
            raise RuntimeError(f"{' '.join(cmd)} failed (status {r.returncode})")
        return csv_path

    os.makedirs(out_dir, exist_ok=True)
    copy = {c: pmc("copy", c, ["--copy-calibration", str(copy_bytes)]) for c in ("FETCH_SIZE", "WRITE_SIZE")}
    for wl in workloads:
        for entry in entries:
            args = ["--workload", wl, "--entry", entry, "--steps", "2", "--warmup", "1", "--no-cpu-baseline",
                    "--no-also"]
            f = pmc(f"{entry}_{wl}", "FETCH_SIZE", args)
            w = pmc(f"{entry}_{wl}", "WRITE_SIZE", args)
            rec = record_traffic(f, w, copy["FETCH_SIZE"], copy["WRITE_SIZE"], workload=wl, entry=entry,
                                 launches=2, warmup=1, copy_bytes=copy_bytes)
            print(json.dumps({"counters": f"{entry}:{wl}", **rec}), flush=True)


def bwd_compulsory_bytes(w) -> int:
    """Bytes a backward pass must move at least: Q, K, V, O and dO read, dQ, dK
    and dV written (element type), LSE read and the row statistic D written
    then read (float32)."""
    elems = w.B * w.H * w.N * w.d
    return 8 * elems * w.elem_bytes + 3 * 4 * w.B * w.H * w.N


def resolve_workload(name: str, shape: str | None):
    """The named workload, or (shape "B,H,N,d,DTYPE") a problem of that size
    with the workloads' input recipe, seed 9 and unit-variance q and k."""
    from io_aware_tiled_06_amd.workloads import WORKLOADS, Workload

    if not shape:
        return WORKLOADS[name]
    parts = shape.split(",")
    if len(parts) != 5:
        raise ValueError(f"--shape takes B,H,N,d,DTYPE, got {shape!r}")
    B, H, N, d = (int(x) for x in parts[:4])
    if min(B, H, N, d) < 1:
        raise ValueError(f"--shape sizes must be positive, got {shape!r}")
    return Workload(f"b{B}_h{H}_n{N}_d{d}_{parts[4]}", B, H, N, d, parts[4], 9)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000,
                    help="timed calls (with --record-traffic: the timed calls of the profiled run)")
    ap.add_argument("--warmup", type=int, default=20,
                    help="untimed calls first (with --record-traffic: those of the profiled run)")
    ap.add_argument("--workload", default="n32768_d128_bf16")
    ap.add_argument("--shape", default=None, metavar="B,H,N,d,DTYPE",
                    help="time this problem instead of a named workload (inputs drawn as the workloads' are, "
                         "seed 9, unit-variance q and k; no traffic record)")
    ap.add_argument("--entry", choices=["flash", "naive"], default="flash")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (dQ, dK, dV from the forward's O and LSE); FLOPs counted as "
                         "2.5x the forward's (the five N x N x d products of the gradient)")
    ap.add_argument("--causal", action="store_true",
                    help="time the causal entry point (query i sees keys 0..i); FLOPs count visible pairs only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration) and exit")
    ap.add_argument("--traffic-sweep", choices=["flash", "naive"], default=None,
                    help="only run the N sweep used for the traffic-versus-N counters and exit")
    ap.add_argument("--record-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write profiles/traffic.json from four rocprofv3 --pmc counter files and exit (no GPU)")
    ap.add_argument("--crossover-sweep", action="store_true",
                    help="only run the fused-versus-three-pass sweep at fixed work (time and memory) and exit")
    ap.add_argument("--crossover-d", type=int, default=128, choices=[64, 128],
                    help="head size of the crossover sweep")
    ap.add_argument("--phase-clock", action="store_true",
                    help="only run the phase-clock build (libflashattn_clock.so) on --workload/--shape: per-workgroup "
                         "phase times, per-CU residency and when each XCD's first workgroups started; then exit")
    ap.add_argument("--compare-paths", action="store_true",
                    help="only time the fused and the three-pass path on the four half-precision workloads and exit")
    ap.add_argument("--collect-counters", metavar="OUT_DIR", default=None,
                    help="only run the rocprofv3 FETCH_SIZE/WRITE_SIZE passes (child processes) of --workloads x "
                         "--entries and write profiles/traffic.json, then exit")
    ap.add_argument("--workloads", default="n32768_d128_bf16", help="comma list for --collect-counters")
    ap.add_argument("--entries", default="flash", help="comma list for --collect-counters")
    ap.add_argument("--no-also", action="store_true",
                    help="skip the extra 4096-token timing of the default workload (counter collection)")
    args = ap.parse_args()
    if args.record_traffic:
        print(json.dumps(record_traffic(*args.record_traffic, workload=args.workload, entry=args.entry,
                                        launches=args.steps, warmup=args.warmup)), flush=True)
        return 0
    if args.collect_counters:
        collect_counters(args.collect_counters, args.workloads.split(","), args.entries.split(","))
        return 0
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, 3)
        return 0
    if args.traffic_sweep:
        traffic_sweep(args.traffic_sweep)
        return 0
    if args.crossover_sweep:
        crossover_sweep(d=args.crossover_d)
        return 0
    if args.compare_paths:
        compare_paths()
        return 0
    if args.phase_clock:
        phase_clock(resolve_workload(args.workload, args.shape), args.causal)
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the library has no multi-GPU path",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import io_aware_tiled_06_amd as fa
    from io_aware_tiled_06_amd import traffic
    from io_aware_tiled_06_amd.workloads import make_inputs

    if not os.path.exists(fa.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    w = resolve_workload(args.workload, args.shape)
    dev = torch.device("cuda:0")
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[w.dtype]
    print(f"[bench] {args.entry} {w.name}: generating inputs", file=sys.stderr, flush=True)
    q, k, v = make_inputs(w)
    tq, tk, tv = (torch.from_numpy(x).to(tdt).to(dev) for x in (q, k, v))
    o = torch.empty_like(tq)
    ws = None
    if (args.causal or args.backward) and args.entry != "flash":
        print("--causal and --backward apply to the fused entry points only", file=sys.stderr)
        return 2
    if args.entry == "naive":
        nbytes = fa.attn_naive_workspace_bytes(w.B, w.H, w.N, w.dtype)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        step = lambda: fa.attn_naive_fwd(tq, tk, tv, w.scale, out=o, workspace=ws)  # noqa: E731
    elif args.backward:
        o, lse = fa.flash_attn_fwd(tq, tk, tv, w.scale, causal=args.causal)
        gen = torch.Generator(device=dev).manual_seed(w.seed + 100)
        dout = torch.randn(tq.shape, generator=gen, device=dev, dtype=torch.float32).to(tdt)
        grads = [torch.empty_like(tq) for _ in range(3)]
        delta = torch.empty((2,) + tuple(lse.shape), dtype=torch.float32, device=dev)
        step = lambda: fa.flash_attn_bwd(tq, tk, tv, o, lse, dout, w.scale, causal=args.causal,  # noqa: E731
                                         dq=grads[0], dk=grads[1], dv=grads[2], delta=delta)
    else:
        step = lambda: fa.flash_attn_fwd(tq, tk, tv, w.scale, causal=args.causal, out=o)  # noqa: E731

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)

    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize(dev)
    with ClockSampler() as clk:
        t0 = time.perf_counter()
        for i in range(args.steps):
            ev[i][0].record(stream)
            step()
            ev[i][1].record(stream)
        torch.cuda.synchronize(dev)
        wall = time.perf_counter() - t0
    ev_ms = [a.elapsed_time(b) for a, b in ev]

    flops = traffic.attention_flops(w.B, w.H, w.N, w.d)
    if args.causal:  # visible (query, key) pairs: N (N + 1) / 2 per head
        flops = 2.0 * w.B * w.H * w.N * (w.N + 1) * w.d
    if args.backward:
        flops *= 2.5
    ms_per_step = wall / args.steps * 1e3
    value = flops / (ms_per_step * 1e-3) / 1e12
    kern_ms = float(np.mean(ev_ms))
    achieved = flops / (kern_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    hbm = None if (args.causal or args.backward) else measured_traffic(w.name, args.entry)
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "entry": args.entry, "causal": bool(args.causal),
                   "pass": "backward" if args.backward else "forward", "B": w.B, "H": w.H,
                   "N": w.N, "d": w.d,
                   "qk_sigma": w.qk_sigma, "seed": w.seed, "scale": w.scale},
        "pct_of_peak": round(100.0 * value / peak, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": hbm,
            "kernel_ms": round(kern_ms, 4),
            "kernel_ms_min": round(float(np.min(ev_ms)), 4),
            "kernel_ms_median": round(float(np.median(ev_ms)), 4),
            "compulsory_bytes": (bwd_compulsory_bytes(w) if args.backward
                                 else traffic.compulsory_bytes(w.B, w.H, w.N, w.d, w.elem_bytes)),
        },
        "device": torch.cuda.get_device_name(dev),
        "device_cus": torch.cuda.get_device_properties(dev).multi_processor_count,
        "device_arch": torch.cuda.get_device_properties(dev).gcnArchName,
        "device_l2_bytes": torch.cuda.get_device_properties(dev).L2_cache_size,
        "cache": cache_label(w),
        "peak_formula": "256 CUs x 2.4 GHz x 4096 FLOP/clk/CU (dense bf16/fp16 matrix cores); fp32: 157.3 TFLOP/s",
    }
    clock = clk.summary()
    if clock:
        # kernel-driver telemetry only: the firmware's clock figure is a smoothed value;
        # the exact cycles of a launch come from the GRBM_COUNT counter
        line["clock"] = clock
    if args.backward:
        line["roofline"]["kernels"] = "bwd_delta + bwd_dq + bwd_dkdv (one backward pass)"
    if (args.entry == "flash" and not (args.causal or args.backward or args.no_also)
            and w.name == "n32768_d128_bf16"):
        print("[bench] the 4096-token forward (the metric's other case)", file=sys.stderr, flush=True)
        line["also"] = time_forward("n4096_d128_bf16")
    if not args.no_cpu_baseline and not args.backward:
        print("[bench] cpu baseline (float64 oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w, q, k, v)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
