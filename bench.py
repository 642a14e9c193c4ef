#!/usr/bin/env python3
"""Benchmark of the paged absorbed-MLA path on one MI355X.

A step is one pass of the whole path over one batch: the write phase (RoPE +
scatter of the new latent rows) followed by the attention phase (on-device
schedule, MFMA attention, split-KV combine). The default workload is the
DeepSeek-V3-dims absorbed MLA decode batch: bf16, 64 sequences with one new
token each, past lengths uniform in [4096, 16384], 128 heads, latent 576,
value 512, rotary 64 at offset 512, block size 64, random block permutation,
values N(0,1)*0.5, scale 1/sqrt(192). Inputs are seeded synthetic data, resident
in HBM before timing starts.

Prints one JSON line. `value` is algorithmic TFLOP/s of the step (2 (hs+vhs)
flops per (token, head, visible key)); `roofline` reports the attention phase
against the HBM bound (this workload sits below the bf16 MFMA ridge) with the
phase duration measured live with HIP events on the launch stream;
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
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c4", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (reference for HBM byte counters)")
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


def cpu_baseline(w, target_s: float):
    """Time the CPU oracle (write phase + attention) on the first sequences of the
    workload until about target_s seconds of work, scaled to TFLOP/s."""
    import numpy as np
    from oracle import paged_latent as orc
    from paged_absorbed_mla_amd import workloads as wl

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
    t0 = time.perf_counter()
    cache = orc.write_phase(w)
    b = 0
    while b < B and time.perf_counter() - t0 < target_s:
        toks = np.arange(cum[b], cum[b + 1])
        if toks.size:
            orc.attention(w, cache, tokens=toks)
            for t in toks:
                pos = int(w["past_seqlens"][b]) + int(t - cum[b])
                lo = 0 if a["local_window_size"] < 0 else max(0, pos - a["local_window_size"])
                done_flops += 2 * (a["head_size"] + vhs) * a["num_heads"] * (pos - lo + 1)
            done_tokens += toks.size
        b += 1
    dt = time.perf_counter() - t0
    return {"value": done_flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"write phase for all {w['dims']['token_count']} tokens + attention for the first {b} "
                      f"of {B} sequences ({done_tokens} tokens), {dt:.1f} s, float64 NumPy"}


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the path is single-device; "
              "multi-GPU sharding is described in DESIGN.md but not built.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from paged_absorbed_mla_amd import workloads as wl
    from paged_absorbed_mla_amd.device import DeviceWorkload

    t_gen = time.perf_counter()
    w = wl.make(args.config)
    counts = wl.algorithmic_counts(w)
    print(f"[bench] workload {args.config} generated in {time.perf_counter() - t_gen:.1f} s: "
          f"T={w['dims']['token_count']} B={w['dims']['batch']} kv_rows={counts['kv_rows']}", file=sys.stderr, flush=True)
    dev = DeviceWorkload(w, "cuda:0")
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        dev.step()
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start_all = torch.cuda.Event(enable_timing=True)
    end_all = torch.cuda.Event(enable_timing=True)
    start_all.record(stream)
    for k in range(args.steps):
        dev.write()
        ev[k][0].record(stream)
        dev.attention()
        ev[k][1].record(stream)
    end_all.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = start_all.elapsed_time(end_all)
    ms_step = ms_total / args.steps
    attn_ms = [a.elapsed_time(b) for a, b in ev]
    attn_avg_ms = float(np.mean(attn_ms))
    print(f"[bench] {args.steps} steps: {ms_step:.4f} ms/step (events), wall {wall * 1e3 / args.steps:.4f} ms/step; "
          f"attention phase avg {attn_avg_ms:.4f} ms, median {np.median(attn_ms):.4f} ms", file=sys.stderr, flush=True)

    flops = counts["flops"]
    byts = counts["bytes"]
    tflops_step = flops / (ms_step * 1e-3) / 1e12
    attn_gbs = byts / (attn_avg_ms * 1e-3) / 1e9
    attn_tflops = flops / (attn_avg_ms * 1e-3) / 1e12
    peak_tf = BF16_PEAK_TFLOPS if w["dtype"] == "bf16" else F16_PEAK_TFLOPS
    hbm_bound = (byts / (HBM_PEAK_GBS * 1e9)) >= (flops / (peak_tf * 1e12))
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(attn_gbs / HBM_PEAK_GBS, 4), "traffic": None}
    else:
        roof = {"bound": "mfma", "achieved": round(attn_tflops, 1), "peak": peak_tf, "unit": "TFLOP/s",
                "frac": round(attn_tflops / peak_tf, 4), "traffic": None}
    roof.update({
        "kernel": "attention phase: pa_latent_attention (schedule + attn_kernel + combine)",
        "avg_ms": round(attn_avg_ms, 5),
        "alg_bytes_per_launch": int(byts), "alg_flops_per_launch": int(flops),
        "also": {"tflops": round(attn_tflops, 1), "gbs": round(attn_gbs, 1),
                 "mfma_frac": round(attn_tflops / peak_tf, 4), "hbm_frac": round(attn_gbs / HBM_PEAK_GBS, 4)},
    })
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
        "config": {"workload": WORKLOADS[args.config], "tokens": w["dims"]["token_count"],
                   "batch": w["dims"]["batch"], "num_heads": w["attrs"]["num_heads"],
                   "head_size": w["attrs"]["head_size"], "v_head_size": w["attrs"]["v_head_size"],
                   "block_size": w["attrs"]["block_size"], "kv_rows": counts["kv_rows"],
                   "tokens_per_s": round(w["dims"]["token_count"] / (ms_step * 1e-3), 1)},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
