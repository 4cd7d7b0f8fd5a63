"""Benchmark: MLA decode HBM GB/s on the 64K-row speculative-decode workload,
plus varlen-prefill TFLOP/s on the long-prefix prefill workload, one GPU.

One step is one ``mla_decode`` call on workload ``decode_b4_h16_q4_L64K``
(4 requests x 4 draft tokens x 16 heads against 65,536 cached latent rows
each), i.e. the whole decode path: split plan, page-table walk, staged
pages, both MFMA contractions, online softmax, partials and merge.  Inputs
are resident in HBM before timing; consecutive steps rotate through three
copies of the cache (906 MB > 3 x the 256 MB Infinity Cache), so each step
reads its rows from HBM.  ``value`` is algorithmic bytes per step / step
time: the cache rows every request holds, the query, the page-table entries
and lengths read, and the output and LSE written (no split-KV workspace
traffic, no re-reads).

The prefill leg times ``mla_prefill_varlen`` on
``prefill_b8_h16_P16K-96K_N200-2000`` and reports TFLOP/s of the absorbed
form as called (2 * 1088 flops per visible (query row, cached row) pair).

The append leg times ``mla_kv_append`` writing that prefill workload's 8,629
new rows into a bf16 and an INT8 cache (bytes: rows read plus rows and scales
written); at ~20 MB per call it is partly launch-bound.

The absorption leg times ``mla_q_absorb`` and ``mla_v_up`` on 8,629 tokens x
16 heads and reports both rooflines: they are memory-bound (85 flop per
byte), so GB/s of algorithmic bytes (inputs and weights read once, outputs
written once) against HBM is the one that bounds them.

The other decode workloads (``configs``: the 256-row latency case, the
ragged 16-request batch with 32 heads, the 256K-row INT8 batch) are timed
the same way, each after a fixed warm-up of its own (0.25 s of its calls,
whatever --warmup says), with two or three cache copies rotated (the
256-row case is deliberately cache-hot).  Beside them: 128 folded rows on the 64K
cache (``wide_rows_decode``) and a serving batch of 64 requests of 4K rows
(``batch_decode``).

The CPU baseline is the fp64 oracle on the host's cores (at most 16
threads), timed on the full decode workload (all 16 query tokens, all
heads), repeated until about 10 s of CPU work have run; it is a reported
baseline, not a target.  Each other decode workload carries its own (the
whole call, once); the prefill leg carries the oracle on 128 seeded new
tokens (all heads), in TFLOP/s of those tokens' flops.

Besides the headline means (events around the whole timed region), the
decode and prefill legs report the spread of block means: the timed region
split into blocks of back-to-back calls with events only at block edges
(events between single calls add a launch gap to every call).  Before its
W warm-up steps the headline leg runs a fixed 0.25 s of the same calls, so
that the shader clock has ramped up after the idle input generation.  The
JSON records the cards' current sclk / mclk levels (amdgpu sysfs) before
the GPU is touched and after the run.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-prefill]
                       [--no-cpu-baseline] [--prefill-steps P] [--calib-copy-mb M]
       python bench.py --record-traffic FETCH_DIR WRITE_DIR [--calib-copy-mb M]

The rooflines' ``traffic`` is the HBM bytes per call read from
profiles/mla_decode_b4_h16_q4_L64K_traffic.json and
profiles/mla_prefill_b8_h16_P16K-96K_N200-2000_traffic.json (written by --record-traffic
from two rocprofv3 counter runs); it is null when the kernel sources have changed since
those counters were taken.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode HBM GB/s (% peak) + varlen prefill TFLOP/s, 64K-prefix KV, 1 GPU"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FLOP_PER_PAIR = 2 * (576 + 512)


def decode_algorithmic_bytes(case) -> int:
    """Bytes the decode method itself must move (see module docstring)."""
    c = case.cache
    L = c.kv_lens.astype(np.int64)
    row_bytes = 576 * 2 if c.kv_dtype == "bf16" else 576 + 4
    T, H = case.total_q(), case.heads
    pages = int(((L + c.page_size - 1) // c.page_size).sum())  # page-table entries read
    return int(L.sum() * row_bytes + T * H * 576 * 2 + T * H * 512 * 2 + T * H * 4 + pages * 4
               + case.batch * 4)


def decode_flops(case) -> int:
    L = case.cache.kv_lens.astype(np.int64)
    vis = 0
    for b in range(case.batch):
        for i in range(case.q_len):
            vis += int(L[b]) - case.q_len + i + 1
    return vis * case.heads * FLOP_PER_PAIR


def prefill_flops(case) -> int:
    tot = 0
    for b in range(case.batch):
        P = int(case.prefix_lens[b])
        n = int(case.cu_seqlens_q[b + 1] - case.cu_seqlens_q[b])
        tot += n * P + n * (n + 1) // 2
    return tot * case.heads * FLOP_PER_PAIR


def prefill_algorithmic_bytes(case) -> int:
    c = case.cache
    L = c.kv_lens.astype(np.int64)
    T, H = case.total_q(), case.heads
    return int(L.sum() * 1152 + T * H * 576 * 2 + T * H * 512 * 2 + T * H * 4)


def block_spread(fn_list, stream, blocks: int, per_block: int) -> dict:
    """Spread of the per-call time: `blocks` blocks of `per_block` back-to-back calls
    (fn_list[i % len]), HIP events on `stream` only at block edges; min / median / max of
    the blocks' mean microseconds per call."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(blocks + 1)]
    k = 0
    with torch.cuda.stream(stream):
        ev[0].record(stream)
        for b in range(blocks):
            for _ in range(per_block):
                fn_list[k % len(fn_list)]()
                k += 1
            ev[b + 1].record(stream)
    torch.cuda.synchronize()
    us = np.array([ev[i].elapsed_time(ev[i + 1]) * 1e3 / per_block for i in range(blocks)])
    return {"min": round(float(us.min()), 2), "median": round(float(np.median(us)), 2),
            "max": round(float(us.max()), 2), "blocks": blocks, "calls_per_block": per_block}


def warm(fn_list, stream, seconds: float) -> int:
    """Run fn_list[i % len] back to back on `stream` for about `seconds` of wall time (the
    shader clock ramps up over the first tenths of a second of work after an idle stretch);
    returns the number of calls."""
    import torch
    t0 = time.time()
    n = 0
    batch = 4
    while True:
        with torch.cuda.stream(stream):
            for _ in range(batch):
                fn_list[n % len(fn_list)]()
                n += 1
        torch.cuda.synchronize()
        if time.time() - t0 >= seconds:
            return n
        batch = min(2 * batch, 256)


def gpu_clocks():
    """Current sclk / mclk level of each card from the amdgpu sysfs tables (pp_dpm_sclk,
    pp_dpm_mclk: the level marked '*'), or None when they are not readable.  Read from
    files, so that no child program is started from this (possibly profiled) process."""
    import glob
    import re
    out = {}
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        card = os.path.basename(os.path.dirname(dev))
        if not re.fullmatch(r"card\d+", card):
            continue
        rec = {}
        for name in ("pp_dpm_sclk", "pp_dpm_mclk"):
            try:
                with open(os.path.join(dev, name)) as f:
                    for line in f:
                        if line.rstrip().endswith("*") and ":" in line:
                            rec[name[len("pp_dpm_"):]] = line.split(":", 1)[1].replace("*", "").strip()
            except OSError:
                pass
        if rec:
            out[card] = rec
    return out or None


def time_calls(fn_list, stream, warmup: int, steps: int) -> float:
    """Run fn_list[i % len] warmup + steps times back to back on `stream`; returns the
    milliseconds of the timed steps, from HIP events recorded on `stream` around the
    whole timed region (no events between calls, which would add gaps)."""
    import torch
    with torch.cuda.stream(stream):
        for i in range(warmup):
            fn_list[i % len(fn_list)]()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        t0.record(stream)
        for i in range(steps):
            fn_list[(warmup + i) % len(fn_list)]()
        t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1)


# The sources that shape each leg's kernels and plan (its recorded HBM traffic is dropped
# when the code of any of them changes; comments do not count).
KERNEL_SOURCES = {
    "decode": ["mla_attention_paged_amd/csrc/mla_api.cpp", "mla_attention_paged_amd/csrc/mla_decode.hip",
               "mla_attention_paged_amd/csrc/mla_device.h", "mla_attention_paged_amd/csrc/mla_internal.h",
               "mla_attention_paged_amd/csrc/mla_ws.h"],
    "prefill": ["mla_attention_paged_amd/csrc/mla_api.cpp", "mla_attention_paged_amd/csrc/mla_prefill.hip",
                "mla_attention_paged_amd/csrc/mla_device.h", "mla_attention_paged_amd/csrc/mla_internal.h",
                "mla_attention_paged_amd/csrc/mla_ws.h"],
}
# kernels whose counter readings make up one call of each leg
LEG_KERNELS = {"decode": ("mla::decode_phase1_pipe", "mla::decode_merge"),
               "prefill": ("mla::prefill_worklist", "mla::prefill_persistent_ws(")}
COUNTER_RUN_FLAGS = ("--steps 5 --warmup 20 --prefill-steps 2 --no-configs --no-append --no-cpu-baseline "
                     "--no-absorb --no-pages --no-varlen --no-scaled --no-scaled-prefill")
TRAFFIC_FILES = {"decode": os.path.join(ROOT, "profiles", "mla_decode_b4_h16_q4_L64K_traffic.json"),
                 "prefill": os.path.join(ROOT, "profiles", "mla_prefill_b8_h16_P16K-96K_N200-2000_traffic.json")}
LEG_WORKLOAD = {"decode": 1, "prefill": 3}


def strip_comments(src: str) -> str:
    """C/C++ source without comments, each line's trailing blanks and blank lines:
    the code the digest covers (string and character literals kept as they are)."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    lines = [ln.rstrip() for ln in "".join(out).split("\n")]
    return "\n".join(ln for ln in lines if ln)


def sources_digest(leg: str = "decode") -> str:
    """SHA-256 of the code (comments stripped) of the sources that shape a leg's call."""
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[leg]:
        with open(os.path.join(ROOT, rel)) as f:
            h.update(strip_comments(f.read()).encode())
    return h.hexdigest()


def recorded_traffic(leg: str, workload: str):
    """HBM bytes per call of a leg from the committed counter runs (FETCH_SIZE + WRITE_SIZE,
    calibrated against a plain copy), or None when the kernels changed since they were taken."""
    try:
        with open(TRAFFIC_FILES[leg]) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != sources_digest(leg) or rec.get("workload") != workload:
        return None
    return rec.get("hbm_bytes_per_call")


def _counter_means(path: str):
    """{kernel name: mean counter value (KiB) per dispatch} from a rocprofv3 counter CSV,
    plus the largest copy-kernel reading (the calibration copy)."""
    import csv
    import glob
    files = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {path}")
    sums, counts, copy_max = {}, {}, 0.0
    for row in csv.DictReader(open(files[0])):
        name, val = row["Kernel_Name"], float(row["Counter_Value"])
        if "copyBuffer" in name:
            copy_max = max(copy_max, val)
            continue
        sums[name] = sums.get(name, 0.0) + val
        counts[name] = counts.get(name, 0) + 1
    return {k: sums[k] / counts[k] for k in sums}, copy_max


def record_traffic(fetch_dir: str, write_dir: str, calib_mb: int) -> int:
    """Turn the FETCH_SIZE and WRITE_SIZE runs of this script (with --calib-copy-mb) into the
    traffic records of the decode and prefill legs: HBM bytes per call, each counter scaled by
    the factor that maps its reading of the calibration copy onto the copy's true size."""
    import synth
    calib = calib_mb * (1 << 20)
    fetch, fcopy = _counter_means(fetch_dir)
    write, wcopy = _counter_means(write_dir)
    ffac = calib / (fcopy * 1024.0)
    wfac = calib / (wcopy * 1024.0)
    for leg, prefixes in LEG_KERNELS.items():
        per_kernel = {}
        total = 0.0
        for name in sorted(set(fetch) | set(write)):
            if not any(name.startswith(p) for p in prefixes):
                continue
            fb = fetch.get(name, 0.0) * 1024.0 * ffac
            wb = write.get(name, 0.0) * 1024.0 * wfac
            per_kernel[name] = {"fetch_bytes": round(fb), "write_bytes": round(wb)}
            total += fb + wb
        if not per_kernel:
            continue
        rec = {"workload": synth.WORKLOADS[LEG_WORKLOAD[leg]]["name"], "source_sha256": sources_digest(leg),
               "source_digest": f"SHA-256 of the {leg} sources' code, comments stripped (bench.strip_comments)",
               "hbm_bytes_per_call": round(total), "per_kernel": per_kernel,
               "fetch_scale": round(ffac, 4), "write_scale": round(wfac, 4),
               "calibration": f"plain device copy of {calib_mb} MiB (torch copy_), largest copy dispatch reading",
               "commands": [f"rocprofv3 --pmc FETCH_SIZE --kernel-trace -f csv -d {fetch_dir} -o fetch -- "
                            f"python3 bench.py {COUNTER_RUN_FLAGS} --calib-copy-mb {calib_mb}",
                            f"rocprofv3 --pmc WRITE_SIZE --kernel-trace -f csv -d {write_dir} -o write -- "
                            f"python3 bench.py {COUNTER_RUN_FLAGS} --calib-copy-mb {calib_mb}",
                            f"python3 bench.py --record-traffic {fetch_dir} {write_dir} --calib-copy-mb {calib_mb}"]}
        os.makedirs(os.path.dirname(TRAFFIC_FILES[leg]), exist_ok=True)
        with open(TRAFFIC_FILES[leg], "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(json.dumps(rec))
    return 0


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_threads() -> int:
    """Threads the oracle baseline runs with: the CPUs this process may use, at most 16
    (the host CPU share that goes with one GPU of an eight-GPU node)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def decode_leg(mla, torch, stream, case, copies: int, steps: int, warm_s: float, hot: bool = False) -> dict:
    """Time mla_decode on `case` (resident inputs; `copies` cache copies rotated unless hot),
    after `warm_s` seconds of warm-up calls; algorithmic GB/s, TFLOP/s and roofline fractions."""
    from mla_gpu import decode_inputs
    d = decode_inputs(case)
    kvs = [d["kv"]] + ([] if hot else [d["kv"].clone() for _ in range(max(0, copies - 1))])
    T, H = case.total_q(), case.heads
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    wsb = mla.mla_splitkv_workspace_size(case.batch, H, case.q_len, T, case.max_seq_len, d["kind"])
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    grid, _ = mla.mla_decode_plan(case.batch, H, case.q_len, case.max_seq_len, d["kind"])

    def make(kv):
        def call():
            mla.mla_decode(d["q"], kv, d["scale"], d["kind"], d["pt"], case.cache.max_pages, d["seq_lens"],
                           case.batch, case.q_len, H, case.cache.page_size, case.max_seq_len, case.softmax_scale,
                           out, lse, ws, ws.numel(), stream)
        return call

    calls = [make(kv) for kv in kvs]
    nwarm = warm(calls, stream, warm_s)
    ms = time_calls(calls, stream, 0, steps) / steps
    nbytes = decode_algorithmic_bytes(case)
    flops = decode_flops(case)
    gbs = nbytes / (ms * 1e-3) / 1e9
    tfl = flops / (ms * 1e-3) / 1e12
    res = {"workload": case.name, "batch": case.batch, "heads": H, "q_len": case.q_len,
           "kv_lens": "all " + str(int(case.seq_lens[0])) if len(set(case.seq_lens.tolist())) == 1
           else f"{int(case.seq_lens.min())}-{int(case.seq_lens.max())} (sum {int(case.seq_lens.sum())})",
           "kv_dtype": case.cache.kv_dtype, "us_per_call": round(ms * 1e3, 2), "GBps": round(gbs, 1),
           "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "tflops": round(tfl, 1),
           "frac_mfma": round(tfl / BF16_PEAK_TFLOPS, 4), "algorithmic_bytes_per_call": nbytes,
           "flops_per_call": flops, "phase1_workgroups": grid, "warmup_calls": nwarm, "steps": steps,
           "kv_copies_rotated": 1 if hot else len(kvs), "spread_us": block_spread(calls, stream, 5, max(4, steps // 5))}
    del kvs, d, ws, out, lse
    torch.cuda.empty_cache()
    return res


def oracle_decode_baseline(case, nbytes: int, min_s: float = 0.0) -> dict:
    """The fp64 oracle on the whole decode call (all query tokens, all heads), repeated until
    `min_s` seconds of CPU work have run (at least once)."""
    import oracle
    nt = oracle_threads()
    runs, cpu_s = 0, 0.0
    while runs == 0 or (cpu_s < min_s and cpu_s / runs * (runs + 1) <= 3 * min_s):
        t = time.time()
        oracle.decode(case, nthreads=nt)
        cpu_s += time.time() - t
        runs += 1
    return {"value": round(nbytes * runs / cpu_s / 1e9, 4), "unit": "GB/s", "cores": nt,
            "host_cpus": os.cpu_count(), "cpu_model": host_cpu_model(), "kind": "oracle",
            "seconds": round(cpu_s, 2), "runs": runs, "us_per_call": round(cpu_s / runs * 1e6, 1),
            "sample": f"the full {case.name} call (all {case.total_q()} query tokens x {case.heads} heads), "
                      f"fp64 C oracle, {runs} run(s), {nt} threads"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--prefill-steps", type=int, default=5)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other decode workloads (256-row, ragged 16 x 32 heads, 256K-row INT8)")
    ap.add_argument("--no-append", action="store_true")
    ap.add_argument("--no-absorb", action="store_true",
                    help="skip the query-absorption / value up-projection leg")
    ap.add_argument("--no-pages", action="store_true",
                    help="skip the page-size leg (the 64K decode with 128- and 1536-row pages)")
    ap.add_argument("--no-varlen", action="store_true",
                    help="skip the ragged-draft decode leg (1..4 drafts per request) on the 64K decode shape")
    ap.add_argument("--no-scaled", action="store_true",
                    help="skip the INT8 / FP8 cache decode leg on the 64K decode shape")
    ap.add_argument("--no-scaled-prefill", action="store_true",
                    help="skip the INT8 / FP8 cache prefill leg on the prefill workload's shape")
    ap.add_argument("--copies", type=int, default=3)
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="also run a plain device-to-device copy of this many MiB (3 times), whose "
                         "HBM counter readings calibrate the per-kernel FETCH_SIZE / WRITE_SIZE figures")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU work: write profiles/mla_decode_b4_h16_q4_L64K_traffic.json from the two rocprofv3 counter runs")
    args = ap.parse_args()
    if args.record_traffic:
        return record_traffic(args.record_traffic[0], args.record_traffic[1], args.calib_copy_mb or 1024)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library runs each call on a single GPU and has no "
              "multi-GPU path. Run with --gpus 1.", file=sys.stderr)
        return 2

    clocks_before = gpu_clocks()  # before this process touches the GPU
    import torch

    import mla_attention_paged_amd as mla
    import synth

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from mla_gpu import decode_inputs, prefill_inputs

    torch.cuda.set_device(0)
    mla.library()
    stream = torch.cuda.Stream()

    # ---------------- decode: the metric ----------------
    t_gen = time.time()
    case = synth.make_workload(1)
    gen_s = time.time() - t_gen
    base = decode_inputs(case)
    kv_copies = [base["kv"]] + [base["kv"].clone() for _ in range(max(0, args.copies - 1))]
    T, H = case.total_q(), case.heads
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ws_bytes = mla.mla_splitkv_workspace_size(case.batch, H, case.q_len, T, case.max_seq_len, base["kind"])
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    grid, _ = mla.mla_decode_plan(case.batch, H, case.q_len, case.max_seq_len, base["kind"])

    def make_call(kv):
        def call():
            mla.mla_decode(base["q"], kv, base["scale"], base["kind"], base["pt"], case.cache.max_pages,
                           base["seq_lens"], case.batch, case.q_len, H, 64, case.max_seq_len,
                           case.softmax_scale, out, lse, ws, ws.numel(), stream)
        return call

    calls = [make_call(kv) for kv in kv_copies]
    ramp_calls = warm(calls, stream, 0.25)  # shader clock ramp after the idle input generation
    total_ms = time_calls(calls, stream, args.warmup, args.steps)
    ms_per_step = total_ms / args.steps
    spread = block_spread(calls, stream, 10, 20)
    nbytes = decode_algorithmic_bytes(case)
    flops = decode_flops(case)
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    traffic = recorded_traffic("decode", case.name)
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": case.name, "batch": case.batch, "heads": H, "q_len": case.q_len,
                   "kv_len": int(case.seq_lens[0]), "page_size": 64, "kv_dtype": "bf16",
                   "kv_copies_rotated": len(kv_copies), "phase1_workgroups": grid,
                   "clock_ramp_calls_before_warmup": ramp_calls},
        # The decode call is the unit: its two kernels (phase one, about 88% of the time,
        # and the merge) run back to back on one stream and are timed together.
        "roofline": {"bound": "hbm", "achieved": round(value, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(value / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "mla_decode call (decode_phase1_pipe + decode_merge)",
                     "algorithmic_bytes_per_call": nbytes,
                     "us_per_call": round(ms_per_step * 1e3, 2)},
        "decode_tflops": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
        "spread_us": spread,
        "input_generation_s": round(gen_s, 1),
    }

    # ---------------- prefill leg ----------------
    if not args.no_prefill:
        pcase = synth.make_workload(3)
        pin = prefill_inputs(pcase)
        PT = pcase.total_q()
        pout = torch.empty((PT, pcase.heads, 512), dtype=torch.bfloat16, device="cuda")
        plse = torch.empty((PT, pcase.heads), dtype=torch.float32, device="cuda")
        pws_bytes = mla.mla_splitkv_workspace_size(pcase.batch, pcase.heads, pcase.max_q_len(), PT,
                                                   pcase.max_seq_len, pin["kind"])
        pws = torch.empty(max(pws_bytes, 1), dtype=torch.uint8, device="cuda")

        def pcall():
            mla.mla_prefill_varlen(pin["q"], pin["cu"], pin["prefix"], pin["kv"], pin["scale"], pin["kind"],
                                   pin["pt"], pcase.cache.max_pages, pcase.batch, PT, pcase.max_q_len(),
                                   pcase.max_seq_len, pcase.heads, 64, pcase.softmax_scale, pout, plse,
                                   pws, pws.numel(), stream)

        ptotal = time_calls([pcall], stream, 2, args.prefill_steps)
        pflops = prefill_flops(pcase)
        pms = ptotal / args.prefill_steps
        tflops = pflops / (pms * 1e-3) / 1e12
        p_spread = block_spread([pcall], stream, 4, 2)
        result["prefill"] = {
            "workload": pcase.name, "total_new_tokens": PT, "heads": pcase.heads,
            "prefix_lens": pcase.prefix_lens.tolist(),
            "new_lens": np.diff(pcase.cu_seqlens_q).tolist(),
            "ms_per_call": round(pms, 3), "tflops": round(tflops, 2), "flops_per_call": pflops,
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                         "traffic": recorded_traffic("prefill", pcase.name),
                         "algorithmic_bytes_per_call": prefill_algorithmic_bytes(pcase),
                         "kernel": "mla_prefill_varlen call (prefill_worklist + prefill_persistent_ws)"},
            "spread_ms": {k: (round(v / 1e3, 3) if k in ("min", "median", "max") else v)
                          for k, v in p_spread.items()},
        }
        if not args.no_cpu_baseline:
            # the oracle on a seeded sample of the new tokens (all heads), per flop
            import oracle
            cores = oracle_threads()
            sample = np.sort(np.random.default_rng(5).choice(PT, 128, replace=False)).astype(np.int32)
            cu = pcase.cu_seqlens_q
            req = np.searchsorted(cu, sample, side="right") - 1
            vis = pcase.prefix_lens[req] + (sample - cu[req]) + 1
            sflops = int(np.sum(vis.astype(np.int64)) * pcase.heads * 2 * 1088)
            t = time.time()
            oracle.prefill(pcase, tokens=sample, nthreads=cores)
            cs = time.time() - t
            result["prefill"]["cpu_baseline"] = {
                "value": round(sflops / cs / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
                "host_cpus": os.cpu_count(), "kind": "oracle", "seconds": round(cs, 2),
                "extrapolated_full_call_s": round(cs * pflops / sflops, 1),
                "sample": f"128 seeded new tokens of {PT} (all {pcase.heads} heads), fp64 C oracle; "
                          f"{sflops} flops of the call's {pflops}"}

    # ---------------- the other decode workloads ----------------
    if not args.no_configs:
        legs = {}
        for k, steps, hot in ((0, 400, True), (2, 60, False), (4, 40, False)):
            kcase = synth.make_workload(k)
            legs[kcase.name] = decode_leg(mla, torch, stream, kcase, 2, steps, 0.25, hot=hot)
            if k == 0:
                legs[kcase.name]["note"] = "cache-resident latency case (one cache copy, not rotated)"
            if not args.no_cpu_baseline:
                legs[kcase.name]["cpu_baseline"] = oracle_decode_baseline(
                    kcase, legs[kcase.name]["algorithmic_bytes_per_call"])
            del kcase
        result["configs"] = legs
        # 128 folded rows (two row blocks per share): the same 64K cache as the headline shape
        wcase = synth.make_decode_case(2, 4, 32, 4, seq_lens=[65536] * 4, name="decode_b4_h32_q4_L64K")
        result["wide_rows_decode"] = decode_leg(mla, torch, stream, wcase, 3, 100, 0.25)
        del wcase
        # a serving batch: 64 requests of 4K rows, 4 drafts (4 phase-one workgroups per
        # request, so the partials are merged by row blocks)
        bcase = synth.make_decode_case(11, 64, 16, 4, seq_lens=[4096] * 64, name="decode_b64_h16_q4_L4K")
        result["batch_decode"] = decode_leg(mla, torch, stream, bcase, 3, 100, 0.25)
        del bcase

    # ---------------- absorption and up-projection on the prefill workload's tokens ----------------
    if not args.no_absorb:
        AT, AH = 8629, 16
        g = torch.Generator(device="cuda").manual_seed(11)
        aq = torch.randn((AT, AH, 192), generator=g, device="cuda").to(torch.bfloat16)
        wuk = (torch.randn((AH, 512, 128), generator=g, device="cuda") * 0.05).to(torch.bfloat16)
        wuv = (torch.randn((AH, 128, 512), generator=g, device="cuda") * 0.05).to(torch.bfloat16)
        aout = torch.empty((AT, AH, 576), dtype=torch.bfloat16, device="cuda")
        ao = torch.randn((AT, AH, 512), generator=g, device="cuda").to(torch.bfloat16)
        vout = torch.empty((AT, AH, 128), dtype=torch.bfloat16, device="cuda")
        legs = {}
        # algorithmic bytes: inputs read once, outputs written once, the weights once
        w_bytes = AH * 512 * 128 * 2
        for name, fn, nbytes in (
                ("q_absorb", lambda: mla.mla_q_absorb(aq, wuk, aout, AT, AH, stream),
                 AT * AH * (192 + 576) * 2 + w_bytes),
                ("v_up", lambda: mla.mla_v_up(ao, wuv, vout, AT, AH, stream),
                 AT * AH * (512 + 128) * 2 + w_bytes)):
            n = 200
            warm([fn], stream, 0.25)
            ms = time_calls([fn], stream, 0, n) / n
            fl = 2 * AT * AH * 128 * 512
            legs[name] = {"us_per_call": round(ms * 1e3, 2), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                          "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                          "bytes_per_call": nbytes, "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                          "frac_mfma": round(fl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4), "flops_per_call": fl}
        result["absorb"] = {"workload": f"{AT} tokens x {AH} heads (the prefill workload's new tokens)",
                            "kernel": "nt_gemm (bf16 MFMA)", "bound": "hbm (85 flop/B)", **legs}
        del aq, wuk, wuv, aout, ao, vout
        torch.cuda.empty_cache()

    # ---------------- page sizes: the 64K decode with 128- and 1536-row pages ----------------
    if not args.no_pages:
        legs = {}
        for ps in (128, 1536):
            pcase2 = synth.make_decode_case(2, case.batch, H, case.q_len, seq_lens=case.seq_lens.tolist(), page_size=ps)
            pin2 = decode_inputs(pcase2)
            pkv = [pin2["kv"]] + [pin2["kv"].clone() for _ in range(max(0, args.copies - 1))]

            def make_pcall(kv, pin2=pin2, pcase2=pcase2, ps=ps):
                def call():
                    mla.mla_decode(pin2["q"], kv, None, 0, pin2["pt"], pcase2.cache.max_pages, pin2["seq_lens"],
                                   pcase2.batch, pcase2.q_len, H, ps, pcase2.max_seq_len, pcase2.softmax_scale,
                                   out, lse, ws, ws.numel(), stream)
                return call

            psteps = 100
            pcalls = [make_pcall(kv) for kv in pkv]
            warm(pcalls, stream, 0.25)
            pms = time_calls(pcalls, stream, 0, psteps) / psteps
            pbytes = decode_algorithmic_bytes(pcase2)
            legs[str(ps)] = {"us_per_call": round(pms * 1e3, 2),
                             "GBps": round(pbytes / (pms * 1e-3) / 1e9, 1),
                             "frac_hbm": round(pbytes / (pms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            del pkv, pin2
            torch.cuda.empty_cache()
        result["page_sizes"] = {"workload": f"{case.name} with pages of 128 and 1536 rows", **legs}

    # ---------------- ragged drafts: the 64K decode shape with 1, 2, 3, 4 drafts ----------------
    if not args.no_varlen:
        qls = np.array([1, 2, 3, 4], np.int32)
        vcase = synth.make_prefill_case(2, H, prefix_lens=case.seq_lens - qls, new_lens=qls)
        vin = prefill_inputs(vcase)
        vT = vcase.total_q()
        vlens = torch.from_numpy(vcase.cache.kv_lens.copy()).cuda()
        vkv = [vin["kv"]] + [vin["kv"].clone() for _ in range(max(0, args.copies - 1))]
        vws_b = mla.mla_splitkv_workspace_size(vcase.batch, H, 4, vT, vcase.max_seq_len, vin["kind"])
        vws = torch.empty(max(vws_b, 1), dtype=torch.uint8, device="cuda")
        vout = torch.empty((vT, H, 512), dtype=torch.bfloat16, device="cuda")
        vlse = torch.empty((vT, H), dtype=torch.float32, device="cuda")

        def make_vcall(kv):
            def call():
                mla.mla_decode_varlen(vin["q"], vin["cu"], kv, vin["scale"], vin["kind"], vin["pt"],
                                      vcase.cache.max_pages, vlens, vcase.batch, vT, 4, H, 64, vcase.max_seq_len,
                                      vcase.softmax_scale, vout, vlse, vws, vws.numel(), stream)
            return call

        vsteps = 100
        vcalls = [make_vcall(kv) for kv in vkv]
        warm(vcalls, stream, 0.25)
        vms = time_calls(vcalls, stream, 0, vsteps) / vsteps
        L = vcase.cache.kv_lens.astype(np.int64)
        vbytes = int(L.sum() * 1152 + vT * H * (576 * 2 + 512 * 2 + 4) + int(((L + 63) // 64).sum()) * 4
                     + vcase.batch * 8)
        result["varlen_decode"] = {"workload": "decode_b4_h16_L64K, drafts 1/2/3/4 per request (mla_decode_varlen)",
                                   "us_per_call": round(vms * 1e3, 2),
                                   "GBps": round(vbytes / (vms * 1e-3) / 1e9, 1),
                                   "frac_hbm": round(vbytes / (vms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                   "algorithmic_bytes_per_call": vbytes}
        del vkv, vin, vws
        torch.cuda.empty_cache()

    # ---------------- scaled caches: the 64K decode shape with INT8 and FP8 rows ----------------
    if not args.no_scaled:
        legs = {}
        for dt in ("int8", "fp8"):
            scase = synth.make_decode_case(2, case.batch, case.heads, case.q_len,  # workload 1 seed
                                           seq_lens=case.seq_lens.tolist(), kv_dtype=dt)
            sin = decode_inputs(scase)
            skv = [sin["kv"]] + [sin["kv"].clone() for _ in range(max(0, args.copies - 1))]
            sws_b = mla.mla_splitkv_workspace_size(scase.batch, H, scase.q_len, T, scase.max_seq_len, sin["kind"])
            sws = torch.empty(max(sws_b, 1), dtype=torch.uint8, device="cuda")

            def make_scall(kv, sin=sin, scase=scase, sws=sws):
                def call():
                    mla.mla_decode(sin["q"], kv, sin["scale"], sin["kind"], sin["pt"], scase.cache.max_pages,
                                   sin["seq_lens"], scase.batch, scase.q_len, H, 64, scase.max_seq_len,
                                   scase.softmax_scale, out, lse, sws, sws.numel(), stream)
                return call

            ssteps = 100
            scalls = [make_scall(kv) for kv in skv]
            warm(scalls, stream, 0.25)
            sms = time_calls(scalls, stream, 0, ssteps) / ssteps
            sbytes = decode_algorithmic_bytes(scase)
            gbs = sbytes / (sms * 1e-3) / 1e9
            legs[dt] = {"us_per_call": round(sms * 1e3, 2), "GBps": round(gbs, 1),
                        "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_call": sbytes,
                        "tflops": round(decode_flops(scase) / (sms * 1e-3) / 1e12, 1)}
            del skv, sin, sws
            torch.cuda.empty_cache()
        result["scaled_cache_decode"] = {"workload": f"{case.name} with INT8 / FP8 (E4M3) rows and fp32 row scales",
                                         "kernel": "mla_decode call (decode_ws_codes<INT8 | FP8> + decode_merge)",
                                         "bound": "hbm", **legs}

    # ---------------- scaled caches: the prefill workload's shape with INT8 and FP8 rows ----------------
    if not args.no_scaled_prefill and not args.no_prefill:
        legs = {}
        base3 = synth.make_workload(3)
        for dt in ("int8", "fp8"):
            qcase = synth.make_prefill_case(4, base3.heads, prefix_lens=base3.prefix_lens,
                                            new_lens=np.diff(base3.cu_seqlens_q), kv_dtype=dt,
                                            name=f"{base3.name}_{dt}")
            qin = prefill_inputs(qcase)
            QT = qcase.total_q()
            qout = torch.empty((QT, qcase.heads, 512), dtype=torch.bfloat16, device="cuda")
            qlse = torch.empty((QT, qcase.heads), dtype=torch.float32, device="cuda")
            qws_b = mla.mla_splitkv_workspace_size(qcase.batch, qcase.heads, qcase.max_q_len(), QT,
                                                   qcase.max_seq_len, qin["kind"])
            qws = torch.empty(max(qws_b, 1), dtype=torch.uint8, device="cuda")

            def qcall(qin=qin, qcase=qcase, QT=QT, qout=qout, qlse=qlse, qws=qws):
                mla.mla_prefill_varlen(qin["q"], qin["cu"], qin["prefix"], qin["kv"], qin["scale"], qin["kind"],
                                       qin["pt"], qcase.cache.max_pages, qcase.batch, QT, qcase.max_q_len(),
                                       qcase.max_seq_len, qcase.heads, 64, qcase.softmax_scale, qout, qlse,
                                       qws, qws.numel(), stream)

            qms = time_calls([qcall], stream, 2, 3) / 3
            qfl = prefill_flops(qcase)
            legs[dt] = {"ms_per_call": round(qms, 3), "tflops": round(qfl / (qms * 1e-3) / 1e12, 1),
                        "frac_mfma": round(qfl / (qms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
            del qin, qout, qlse, qws
            torch.cuda.empty_cache()
        result["scaled_cache_prefill"] = {
            "workload": f"{base3.name} with INT8 / FP8 (E4M3) rows and fp32 row scales",
            "kernel": "mla_prefill_varlen call (prefill_persistent_ws_codes: both wave kinds widen their share of the next tile's codes)",
            "bound": "mfma", **legs}

    # ---------------- append leg: the prefill workload's new rows into the cache ----------------
    if not args.no_append:
        acase = synth.make_workload(3)
        pt = acase.cache.page_table
        num_pages = int(pt.max()) + 1
        rows = int(acase.cu_seqlens_q[-1])
        g = torch.Generator(device="cuda").manual_seed(7)
        new = torch.randn((rows, 576), generator=g, device="cuda").to(torch.bfloat16)
        cu = torch.from_numpy(acase.cu_seqlens_q.astype(np.int32)).cuda()
        start = torch.from_numpy(acase.prefix_lens.astype(np.int32)).cuda()
        pt_d = torch.from_numpy(np.ascontiguousarray(pt, dtype=np.int32)).cuda()
        legs = {}
        for kind, name in ((mla.MLA_KV_BF16, "bf16"), (mla.MLA_KV_INT8, "int8"), (mla.MLA_KV_FP8, "fp8")):
            if kind == mla.MLA_KV_BF16:
                kv = torch.zeros((num_pages, 64, 576), dtype=torch.bfloat16, device="cuda")
                sc = None
                row_out = 1152
            else:
                kv = torch.zeros((num_pages, 64, 576), dtype=torch.int8 if name == "int8" else torch.uint8,
                                 device="cuda")
                sc = torch.ones((num_pages, 64), dtype=torch.float32, device="cuda")
                row_out = 576 + 4

            def acall(kv=kv, sc=sc, kind=kind):
                mla.mla_kv_append(new, cu, start, kv, sc, kind, pt_d, pt.shape[1], acase.batch, rows, 64, stream)

            asteps = 200
            warm([acall], stream, 0.25)  # the clocks ramp up again after the idle input generation
            ams = time_calls([acall], stream, 0, asteps) / asteps
            abytes = rows * (1152 + row_out)  # rows read + rows (and scales) written
            legs[name] = {"us_per_call": round(ams * 1e3, 2), "GBps": round(abytes / (ams * 1e-3) / 1e9, 1),
                          "frac_hbm": round(abytes / (ams * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                          "bytes_per_call": abytes}
            del kv, sc
        result["append"] = {"workload": f"{acase.name} new rows ({rows} rows of 576, at their prefix positions)",
                            "kernel": "mla_kv_append", "bound": "hbm", **legs}

    # ---------------- counter calibration: a plain copy of known size ----------------
    if args.calib_copy_mb > 0:
        n = args.calib_copy_mb * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["calib_copy_bytes"] = n
        del src, dst

    # ---------------- CPU baseline: the oracle ----------------
    if not args.no_cpu_baseline:
        # repeat the whole call until about 10 s of CPU work have run (at most 30 s)
        result["cpu_baseline"] = oracle_decode_baseline(case, nbytes, 10.0)
    result["gpu_clocks"] = {"before": clocks_before, "after": gpu_clocks()}
    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
