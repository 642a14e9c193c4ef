#!/usr/bin/env python3
"""Benchmark of the paged absorbed-MLA path on one MI355X.

A step is one pass of the whole path over one batch: the write phase (RoPE +
scatter of the new latent rows) followed by the attention phase (on-device
schedule, MFMA attention, split-KV combine); both run in one fused call
(pa_latent_forward, or pa_separate_forward for the grouped-query workloads),
whose first launch carries the write rows beside the schedule. The default workload is the
DeepSeek-V3-dims absorbed MLA decode batch: bf16, 64 sequences with one new
token each, past lengths uniform in [4096, 16384], 128 heads, latent 576,
value 512, rotary 64 at offset 512, block size 64, random block permutation,
values N(0,1)*0.5, scale 1/sqrt(192). Inputs are seeded synthetic data, resident
in HBM before timing starts.

Prints one JSON line. `value` is algorithmic TFLOP/s of the step (2 (hs+vhs)
flops per (token, head, visible key)) over K back-to-back steps, by default
captured into one HIP graph (`--launch eager` launches them from Python).
`roofline` reports the dominant kernel (the attention kernel) against the HBM
bound (this workload sits below the bf16 MFMA ridge): `frac` is the phase's
algorithmic bytes over the kernel's mean duration, measured live with HIP
events that the library records around that launch on its stream; beside it
the same figures for the whole attention call (`phase`) and the whole step
(`step`), mean/median/p10/p90, and per-step statistics after a MALL flush.
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
F16_PEAK_TFLOPS = 2500.0

WORKLOADS = {
    "c4": "dsv3_576_512_64_decode_bf16_b64_ctx4k-16k",
    "c2": "glm_192_128_64_decode_bf16_b32_ctx512-4k",
    "c3": "glm_192_128_64_chunked_prefill_f16_4x1024",
    "c5": "mixed_576_512_64_f16_window1024_softcap50",
    "c1": "tiny_64_32_16_prefill_decode_f16",
    # grouped-query (separate cache layout) workloads: 32 query heads over 8 key/value heads, 128/128
    "gqa_decode": "gqa_128_32q8kv_decode_bf16_b32_ctx512-4k",
    "gqa_prefill": "gqa_128_32q8kv_chunked_prefill_f16_4x1024",
    "gqa_tiny": "gqa_tiny_64_64_4q2kv_prefill_decode_f16",
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c4", choices=sorted(WORKLOADS))
    ap.add_argument("--launch", default="graph", choices=["graph", "eager"],
                    help="graph: the timed steps are captured into one HIP graph and launched once; "
                         "eager: launched one by one from Python")
    ap.add_argument("--flush-steps", type=int, default=20,
                    help="extra steps, each after a MALL flush, for per-step statistics (0: none)")
    ap.add_argument("--flush-mib", type=int, default=512, help="scratch written before each flushed step")
    ap.add_argument("--calls", default="fused", choices=["fused", "separate"],
                    help="a step as one fused call (pa_latent_forward / pa_separate_forward) or as the write "
                         "call followed by the attention call")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (reference for HBM byte counters)")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print the markdown summary of a rocprofv3 --kernel-trace --stats output directory")
    ap.add_argument("--summarize-counters", nargs=4, metavar=("FETCH", "WRITE", "CAL_FETCH", "CAL_WRITE"),
                    help="print the markdown summary of four rocprofv3 --pmc output directories: FETCH_SIZE "
                         "and WRITE_SIZE of the bench, then of --calibrate-copy")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="DIR",
                    help="print the markdown summary of rocprofv3 --pmc output directories (SQ/GRBM counters)")
    ap.add_argument("--cmd", default="", help="command line recorded in a summary")
    ap.add_argument("--power-seconds", type=float, default=0.0,
                    help="after the timed runs, replay the step graph for this many seconds while sampling the "
                         "socket power with amd-smi (reported under roofline.power; 0: skip)")
    return ap.parse_args()


def calibrate_copy(mib: int):
    """A plain copy of known size: reads and writes exactly mib MiB, so the HBM
    byte counters of its dispatch give the scale factor of those counters."""
    import torch
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": n, "reads": n, "writes": n}), flush=True)


# The attention kernel the roofline reports on, its source files (any change
# makes stored HBM counters stale) and the profile that holds its counters.
DOMINANT_KERNEL = "attn_mla_kernel"   # the benchmark workload's kernel (576/512 rows)


def attention_kernel_name(w: dict) -> str:
    """The attention kernel the library launches for this workload: the
    four-wave 576/512 kernel for rows wider than 192 channels, else the
    generic one."""
    a = w["attrs"]
    if a.get("kv_cache_layout") == "SEPARATE":
        return "attn_kernel"
    return DOMINANT_KERNEL if a["head_size"] > 192 or a["v_head_size"] > 128 else "attn_kernel"


KERNEL_SOURCES = ["paged_absorbed_mla_amd/csrc/pa_attn_mla.cuh", "paged_absorbed_mla_amd/csrc/pa_attn.cuh",
                  "paged_absorbed_mla_amd/csrc/pa_device.h", "paged_absorbed_mla_amd/csrc/inst/attnm_bf16_576_512.hip",
                  "paged_absorbed_mla_amd/build.py"]
COUNTERS_PROFILE = "profiles/attn_mla_kernel_dsv3_576_512_bf16_decode_b64_hbm_counters.md"


def kernel_sources_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str):
    """HBM bytes per dispatch of the dominant kernel from the committed counter
    summary, or None when it is missing, for another workload, or taken on
    other kernel sources."""
    path = os.path.join(ROOT, COUNTERS_PROFILE)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    i = text.find("```json")
    if i < 0:
        return None
    blob = json.loads(text[i + 7:text.index("```", i + 7)])
    if blob.get("sources") != kernel_sources_hash() or blob.get("workload") != workload:
        return None
    return int(round(blob["fetch_kib"] * 1024 * blob["fetch_scale"] + blob["write_kib"] * 1024 * blob["write_scale"]))


def _rocprof_rows(d: str, name: str):
    import csv
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith(name):
                with open(os.path.join(root, f)) as fh:
                    return list(csv.DictReader(fh))
    raise FileNotFoundError(f"no *{name} under {d}")


def _short(kname: str) -> str:
    return kname.split("(")[0].replace("void ", "")


def summarize_trace(d: str, cmd: str):
    rows = _rocprof_rows(d, "kernel_stats.csv")
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    print("| kernel | calls | avg us | min us | max us | share |\n|---|---|---|---|---|---|")
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        print(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
              f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
              f"{100 * float(r['TotalDurationNs']) / total:.1f}% |")
    if cmd:
        print(f"\nCommand: `{cmd}`")


def _counter_means(d: str, counter: str):
    import collections
    acc = collections.defaultdict(list)
    for r in _rocprof_rows(d, "counter_collection.csv"):
        if r["Counter_Name"] == counter:
            acc[_short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}, {k: len(v) for k, v in acc.items()}


def summarize_counters(fetch_d: str, write_d: str, cal_fetch_d: str, cal_write_d: str, cmd: str):
    fetch, nf = _counter_means(fetch_d, "FETCH_SIZE")
    write, _ = _counter_means(write_d, "WRITE_SIZE")
    cf, _ = _counter_means(cal_fetch_d, "FETCH_SIZE")
    cw, _ = _counter_means(cal_write_d, "WRITE_SIZE")
    copy = [k for k in cf if "copy" in k.lower()]
    assert copy, f"no copy kernel among {list(cf)}"
    mib = 1024
    kib_copied = mib * 1024
    fs = kib_copied / cf[copy[0]]
    ws = kib_copied / cw[copy[0]]
    print(f"Calibration: `{copy[0]}` copies {mib} MiB ({kib_copied:,} KiB read and written); its counters read "
          f"FETCH_SIZE {cf[copy[0]]:,.0f} KiB and WRITE_SIZE {cw[copy[0]]:,.0f} KiB per dispatch, so the scale "
          f"factors are {fs:.3f} (fetch) and {ws:.3f} (write).\n")
    print("| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | fetched MB (scaled) | written MB (scaled) |")
    print("|---|---|---|---|---|---|")
    for k in sorted(fetch, key=lambda k: -fetch[k]):
        wk = write.get(k, float("nan"))
        print(f"| `{k}` | {nf[k]} | {fetch[k]:,.1f} | {wk:,.1f} | {fetch[k] * 1024 * fs / 1e6:,.1f} | "
              f"{wk * 1024 * ws / 1e6:,.1f} |")
    dom = [k for k in fetch if DOMINANT_KERNEL in k]
    if dom:
        blob = {"kernel": dom[0], "fetch_kib": round(fetch[dom[0]], 1), "write_kib": round(write[dom[0]], 1),
                "fetch_scale": round(fs, 4), "write_scale": round(ws, 4), "workload": WORKLOADS["c4"],
                "sources": kernel_sources_hash()}
        print("\nMachine-readable figures for `bench.py` (`sources` names the kernel sources these counters "
              "belong to; bench.py reports `traffic` only while they are unchanged):\n")
        print("```json\n" + json.dumps(blob) + "\n```")
    if cmd:
        print(f"\nCommands: {cmd}")


def summarize_pmc(dirs, cmd: str):
    """Per-kernel means of every counter in the given --pmc runs (one dispatch
    per row of counter_collection.csv), with the kernel's mean duration from
    the same runs' kernel traces, and derived MFMA figures: MFMA-busy SIMD
    cycles (SQ_VALU_MFMA_BUSY_CYCLES) per SIMD over the kernel duration at the
    2.4 GHz peak clock, and over the waves' lifetime (SQ_WAVE_CYCLES counts
    quad-cycles; one wave per SIMD in the 576/512 kernel)."""
    import collections
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    durs = collections.defaultdict(list)
    for d in dirs:
        for r in _rocprof_rows(d, "counter_collection.csv"):
            vals[_short(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
            durs[_short(r["Kernel_Name"])].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    simds = 256 * 4
    for k in sorted(vals):
        if not k.startswith("pa::") and "pa::" not in k:
            continue
        c = {n: sum(v) / len(v) for n, v in vals[k].items()}
        print(f"\n`{k}` (mean over {max(len(v) for v in vals[k].values())} dispatches per counter; "
              f"duration {sum(durs[k]) / len(durs[k]):.1f} us mean)\n")
        print("| counter | per dispatch |\n|---|---|")
        for n in sorted(c):
            print(f"| {n} | {c[n]:,.0f} |")
        dur = sum(durs[k]) / len(durs[k])
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
            busy = c["SQ_VALU_MFMA_BUSY_CYCLES"] / simds
            print(f"\n- MFMA-busy cycles per SIMD: {busy:,.0f} = {100 * busy / (dur * 2400):.1f}% of the "
                  f"duration at the 2.4 GHz peak clock")
            if "SQ_WAVE_CYCLES" in c:
                life = 4 * c["SQ_WAVE_CYCLES"] / simds
                print(f"- wave lifetime per SIMD {life:,.0f} cycles (SQ_WAVE_CYCLES x 4): MFMA busy "
                      f"{100 * busy / life:.1f}% of it")
        for mops in ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F16"):
            if mops in c:
                print(f"- MFMA flops ({mops} x 512): {c[mops] * 512 / 1e9:,.1f} GFLOP per dispatch = "
                      f"{c[mops] * 512 / (dur * 1e-6) / 1e12:,.0f} TFLOP/s over the dispatch")
    if cmd:
        print(f"\nCommands: {cmd}")


def cpu_baseline(w, target_s: float, single: bool = True):
    """Time the CPU oracle (write phase + attention) on the first sequences of the
    workload until about target_s seconds of work, scaled to TFLOP/s."""
    import numpy as np
    from oracle import paged_latent as orc
    from oracle import paged_separate as sep

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    cum = w["cumulative_sequence_length"]
    a = w["attrs"]
    vhs = a["v_head_size"] or a["head_size"]
    B = len(cum) - 1
    done_flops = 0
    done_tokens = 0
    separate = a.get("kv_cache_layout") == "SEPARATE"
    t0 = time.perf_counter()
    caches = sep.write_phase(w) if separate else (orc.write_phase(w),)
    b = 0
    while b < B and time.perf_counter() - t0 < target_s:
        toks = np.arange(cum[b], cum[b + 1])
        if toks.size:
            (sep.attention if separate else orc.attention)(w, *caches, tokens=toks)
            for t in toks:
                pos = int(w["past_seqlens"][b]) + int(t - cum[b])
                lo = 0 if a["local_window_size"] < 0 else max(0, pos - a["local_window_size"])
                done_flops += 2 * (a["head_size"] + vhs) * a["num_heads"] * (pos - lo + 1)
            done_tokens += toks.size
        b += 1
    dt = time.perf_counter() - t0
    out = {"value": done_flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
           "sample": f"write phase for all {w['dims']['token_count']} tokens + attention for the first {b} "
                     f"of {B} sequences ({done_tokens} tokens), {dt:.1f} s, float64 NumPy",
           "cpu_model": cpu_model(), "os_cpu_count": os.cpu_count()}
    if single:
        # The same oracle with its BLAS pool limited to one thread, on a
        # shorter sample (attention of the first sequences only).
        try:
            from threadpoolctl import threadpool_limits
        except Exception:
            return out
        with threadpool_limits(limits=1):
            t1 = time.perf_counter()
            f1 = tok1 = 0
            b1 = 0
            while b1 < B and time.perf_counter() - t1 < target_s / 3:
                toks = np.arange(cum[b1], cum[b1 + 1])
                if toks.size:
                    (sep.attention if separate else orc.attention)(w, *caches, tokens=toks)
                    for t in toks:
                        pos = int(w["past_seqlens"][b1]) + int(t - cum[b1])
                        lo = 0 if a["local_window_size"] < 0 else max(0, pos - a["local_window_size"])
                        f1 += 2 * (a["head_size"] + vhs) * a["num_heads"] * (pos - lo + 1)
                    tok1 += toks.size
                b1 += 1
            d1 = time.perf_counter() - t1
        out["single_thread"] = {"value": f1 / d1 / 1e12, "unit": "TFLOP/s", "cores": 1,
                                "sample": f"attention for the first {b1} of {B} sequences ({tok1} tokens), "
                                          f"{d1:.1f} s, BLAS limited to one thread"}
    return out


def stats(xs):
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {"mean": round(float(a.mean()), 5), "median": round(float(np.median(a)), 5),
            "p10": round(float(np.percentile(a, 10)), 5), "p90": round(float(np.percentile(a, 90)), 5)}


def step_with_events(pa, dev, s, a, b, ka, kb):
    """One step with events a/b around its attention phase and ka/kb (recorded
    by the library on its launch stream) around the attention kernel. By
    default the step is the fused call (pa_latent_forward / pa_separate_forward:
    the write rows run in the attention phase's first launch), so a/b bracket
    the whole call; with --calls separate the write is its own call before a."""
    if not dev.fused:
        dev.write()
        a.record(s)
        pa.pa_latent_profile_next(ka, kb)
        dev.attention()
        b.record(s)
    else:
        a.record(s)
        pa.pa_latent_profile_next(ka, kb)
        dev.forward()
        b.record(s)


def timed_steps(torch, pa, dev, steps, graph):
    """K back-to-back steps (write + attention) bracketed by events, with events
    around each attention phase and, recorded by the library on its launch
    stream, around each attention kernel. graph=True captures the K steps into
    one HIP graph (after the eager warm-up, so every signature is warmed) and
    times one launch of it."""
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a_, b_ in ev + kev:                 # torch creates an event on its first record
        a_.record(stream)
        b_.record(stream)
    torch.cuda.synchronize()

    def body(s):
        # (inside a graph capture the events become graph nodes; only the
        # bracketing events outside the graph are read then)
        for k in range(steps):
            step_with_events(pa, dev, s, ev[k][0], ev[k][1], kev[k][0], kev[k][1])

    start_all = torch.cuda.Event(enable_timing=True)
    end_all = torch.cuda.Event(enable_timing=True)
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            body(torch.cuda.current_stream())
        torch.cuda.synchronize()
        g.replay()                          # one untimed launch of the graph
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start_all.record(stream)
        g.replay()
        end_all.record(stream)
        torch.cuda.synchronize()
    else:
        t0 = time.perf_counter()
        start_all.record(stream)
        body(stream)
        end_all.record(stream)
        torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return (start_all.elapsed_time(end_all), [a.elapsed_time(b) for a, b in ev],
            [a.elapsed_time(b) for a, b in kev], wall)


def flushed_steps(torch, pa, dev, steps, mib):
    """Steps with the 256 MB MALL (and the L2s) flushed before each: a write of
    `mib` MiB of scratch outside the timed events, then one step with events
    around the attention phase and its kernel. Per-step statistics."""
    stream = torch.cuda.current_stream()
    scratch = torch.empty(mib << 20, dtype=torch.uint8, device=dev.device)
    phase, kern = [], []
    for _ in range(steps):
        scratch.fill_(1)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ka, kb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ka.record(stream)
        kb.record(stream)
        step_with_events(pa, dev, stream, a, b, ka, kb)
        torch.cuda.synchronize()
        phase.append(a.elapsed_time(b))
        kern.append(ka.elapsed_time(kb))
    del scratch
    return {"flush_mib": mib, "steps": steps, "phase_ms": stats(phase), "kernel_ms": stats(kern)}


def _json_find(obj, pred):
    """Values of the keys of a parsed JSON tree for which pred(key) holds."""
    out = []
    if isinstance(obj, dict):
        for k, v in obj.items():
            if pred(str(k).lower()):
                out.append(v)
            out.extend(_json_find(v, pred))
    elif isinstance(obj, list):
        for v in obj:
            out.extend(_json_find(v, pred))
    return out


def _watts(v):
    """A power reading as amd-smi / rocm-smi print it (a number, a string, or
    {"value": ..., "unit": "W"}), in watts, or None."""
    if isinstance(v, dict):
        v = v.get("value")
    try:
        return float(str(v).split()[0])
    except (TypeError, ValueError, IndexError):
        return None


def _smi_json(args):
    import subprocess
    try:
        r = subprocess.run(args, capture_output=True, text=True, timeout=20)
        starts = [i for i in (r.stdout.find("["), r.stdout.find("{")) if i >= 0]
        return json.loads(r.stdout[min(starts):]) if starts else None
    except (OSError, ValueError, subprocess.SubprocessError):
        return None


def power_sample(torch, dev, steps: int, seconds: float):
    """Sustained load: a HIP graph of `steps` steps replayed back to back for
    `seconds` while a thread reads the socket power with amd-smi about twice a
    second. Reports the readings, the board's power cap and the sustained
    step time (the clock settles where the power meets the cap). The first
    second's readings are skipped."""
    import threading
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(steps):
            dev.step()
    torch.cuda.synchronize()
    readings, stop = [], threading.Event()

    def sampler():
        stop.wait(1.0)                      # readings once the load has settled
        while not stop.is_set():
            j = _smi_json(["amd-smi", "metric", "-p", "-g", "0", "--json"])
            vals = [_watts(v) for v in _json_find(j, lambda k: k == "socket_power")] if j is not None else []
            vals = [v for v in vals if v is not None]
            if vals:
                readings.append(vals[0])
            stop.wait(0.5)

    th = threading.Thread(target=sampler, daemon=True)
    g.replay()
    torch.cuda.synchronize()
    th.start()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    n = 0
    a.record()
    while time.perf_counter() - t0 < seconds:
        g.replay()
        n += 1
        torch.cuda.synchronize()
    b.record()
    torch.cuda.synchronize()
    stop.set()
    th.join(timeout=30)
    cap_j = _smi_json(["rocm-smi", "--showmaxpower", "--json"])
    caps = [_watts(v) for v in _json_find(cap_j, lambda k: "max" in k and "power" in k)] if cap_j is not None else []
    caps = [c for c in caps if c is not None]
    return {"what": f"socket power (amd-smi) while a graph of {steps} steps is replayed back to back",
            "seconds": round(seconds, 1), "samples": len(readings),
            "socket_w": stats(readings) if readings else None, "cap_w": caps[0] if caps else None,
            "sustained_ms_per_step": round(a.elapsed_time(b) / (n * steps), 5)}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.cmd)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, args.cmd)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc, args.cmd)
        return
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the path is single-device; "
              "no sharding or collectives are built.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import paged_absorbed_mla_amd as pa
    from paged_absorbed_mla_amd import workloads as wl
    from paged_absorbed_mla_amd.device import DeviceWorkload

    t_gen = time.perf_counter()
    w = wl.make(args.config)
    counts = wl.algorithmic_counts(w)
    print(f"[bench] workload {args.config} generated in {time.perf_counter() - t_gen:.1f} s: "
          f"T={w['dims']['token_count']} B={w['dims']['batch']} kv_rows={counts['kv_rows']}", file=sys.stderr, flush=True)
    dev = DeviceWorkload(w, "cuda:0")
    dev.fused = dev.fused and args.calls == "fused"
    for _ in range(args.warmup):
        dev.step()
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)

    # K eager steps: events around every attention call and, recorded by the
    # library on its launch stream, around every attention kernel (event
    # timestamps recorded inside a HIP graph are not usable). Then, with
    # --launch graph, the same K steps captured into one HIP graph and
    # launched once: the whole-job time `value` is taken from that run.
    ms_total_e, attn_ms, kern_ms, wall_e = timed_steps(torch, pa, dev, args.steps, False)
    ms_step_e = ms_total_e / args.steps
    attn_avg_ms = float(np.mean(attn_ms))
    kern_avg_ms = float(np.mean(kern_ms))
    print(f"[bench] {args.steps} steps (eager): {ms_step_e:.4f} ms/step (events), wall "
          f"{wall_e * 1e3 / args.steps:.4f} ms/step; attention phase avg {attn_avg_ms:.4f} ms, median "
          f"{np.median(attn_ms):.4f} ms; {attention_kernel_name(w)} avg {kern_avg_ms:.4f} ms, median "
          f"{np.median(kern_ms):.4f} ms", file=sys.stderr, flush=True)
    ms_step, wall = ms_step_e, wall_e
    if args.launch == "graph":
        ms_total_g, _, _, wall = timed_steps(torch, pa, dev, args.steps, True)
        ms_step = ms_total_g / args.steps
        print(f"[bench] {args.steps} steps (one HIP graph): {ms_step:.4f} ms/step (events), wall "
              f"{wall * 1e3 / args.steps:.4f} ms/step", file=sys.stderr, flush=True)
    flushed = None
    if args.flush_steps > 0:
        flushed = flushed_steps(torch, pa, dev, args.flush_steps, args.flush_mib)
        print(f"[bench] {args.flush_steps} steps after a {args.flush_mib} MiB MALL flush each: attention phase "
              f"median {flushed['phase_ms']['median']:.4f} ms, kernel median {flushed['kernel_ms']['median']:.4f} ms",
              file=sys.stderr, flush=True)

    flops = counts["flops"]
    byts = counts["bytes"]
    tflops_step = flops / (ms_step * 1e-3) / 1e12
    peak_tf = BF16_PEAK_TFLOPS if w["dtype"] == "bf16" else F16_PEAK_TFLOPS
    hbm_bound = (byts / (HBM_PEAK_GBS * 1e9)) >= (flops / (peak_tf * 1e12))
    # Roofline of the dominant kernel: the phase's algorithmic bytes (flops) per
    # launch over the kernel's own average duration.
    k_gbs = byts / (kern_avg_ms * 1e-3) / 1e9
    k_tflops = flops / (kern_avg_ms * 1e-3) / 1e12
    traffic = stored_traffic(WORKLOADS[args.config]) if args.config == "c4" else None
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": round(k_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(k_gbs / HBM_PEAK_GBS, 4), "traffic": traffic}
    else:
        roof = {"bound": "mfma", "achieved": round(k_tflops, 1), "peak": peak_tf, "unit": "TFLOP/s",
                "frac": round(k_tflops / peak_tf, 4), "traffic": traffic}
    def side(ms):
        gbs = byts / (ms * 1e-3) / 1e9
        tfl = flops / (ms * 1e-3) / 1e12
        return {"gbs": round(gbs, 1), "tflops": round(tfl, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                "mfma_frac": round(tfl / peak_tf, 4)}
    roof.update({
        "frac_basis": f"{attention_kernel_name(w)}: algorithmic bytes (flops) of the attention phase over the "
                      "kernel's mean duration, HIP events the library records around its launch on its stream",
        "kernel": f"{attention_kernel_name(w)} (HIP events on its launch stream)",
        "avg_ms": round(kern_avg_ms, 5),
        "kernel_ms": stats(kern_ms),
        "alg_bytes_per_launch": int(byts), "alg_flops_per_launch": int(flops),
        "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
        "phase": dict({"what": ("attention call: schedule launch + attention kernel + combine (events around "
                                "the call)") if not dev.fused else
                               ("fused call (pa_latent_forward / pa_separate_forward): schedule launch carrying the write rows + "
                                "attention kernel + combine (events around the call)"),
                       "avg_ms": round(attn_avg_ms, 5), "ms": stats(attn_ms)},
                      **side(attn_avg_ms)),
        "step": dict({"what": f"write + attention ({'one fused call' if dev.fused else 'two calls'}), whole-job "
                              f"time / steps ({args.launch} launch)",
                      "ms": round(ms_step, 5), "eager_ms": round(ms_step_e, 5)}, **side(ms_step)),
    })
    if flushed is not None:
        roof["phase_after_mall_flush"] = dict(flushed, **side(flushed["phase_ms"]["median"]))
    out = {
        "metric": "paged-MLA decode attention TFLOP/s + HBM GB/s (% of roofline), 576/512 bf16",
        "value": round(tflops_step, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w["dtype"],
        "data": "synthetic (seeded)",
        "launch": args.launch,
        "calls": "fused" if dev.fused else "separate",
        "config": {"workload": WORKLOADS[args.config], "tokens": w["dims"]["token_count"],
                   "batch": w["dims"]["batch"], "num_heads": w["attrs"]["num_heads"],
                   "head_size": w["attrs"]["head_size"], "v_head_size": w["attrs"]["v_head_size"],
                   "block_size": w["attrs"]["block_size"], "kv_rows": counts["kv_rows"],
                   **({"kv_num_heads": w["attrs"]["kv_num_heads"]} if "kv_num_heads" in w["attrs"] else {}),
                   "tokens_per_s": round(w["dims"]["token_count"] / (ms_step * 1e-3), 1)},
        "roofline": roof,
    }
    if args.power_seconds > 0:
        roof["power"] = power_sample(torch, dev, args.steps, args.power_seconds)
        print(f"[bench] power: {json.dumps(roof['power'])}", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
