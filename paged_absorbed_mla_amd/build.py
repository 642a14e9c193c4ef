"""Ahead-of-time build of the gfx950 library libpa_latent.so (hipcc, no JIT).

Every .hip source under csrc/ (and csrc/inst/) is compiled to an object with
hipcc for gfx950 in parallel, then linked into a shared library next to this
file. Usage: python -m paged_absorbed_mla_amd.build [--jobs N] [--verbose]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libpa_latent.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
    # No packed-FP32 instructions in device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wno-unused-result",
]


# Extra flags by source-file prefix. The four-wave 576/512 kernel keeps its PV
# accumulators in AGPRs through inline assembly; its compiler-built MFMAs use
# the VGPR form so S, P and the query stay in VGPRs. The generic kernels use
# the VGPR form throughout: otherwise the one-wave instances park the scores
# and accumulators in AGPRs and copy them back for every softmax step.
_VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
FILE_FLAGS = {"attnm_": _VGPR_FORM, "attn_": _VGPR_FORM, "attns_": _VGPR_FORM}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def sources():
    out = []
    for d in (CSRC, os.path.join(CSRC, "inst")):
        for f in sorted(os.listdir(d)):
            if f.endswith(".hip"):
                out.append(os.path.join(d, f))
    return out


def _compile(src: str, verbose: bool, extra) -> str:
    rel = os.path.relpath(src, CSRC).replace(os.sep, "_")
    obj = os.path.join(BUILD, rel[:-4] + ".o")
    per_file = [f for pre, fl in FILE_FLAGS.items() if os.path.basename(src).startswith(pre) for f in fl]
    cmd = [hipcc(), *HIPCC_FLAGS, *per_file, *extra, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if verbose and msgs:
        print(msgs, flush=True)
    return obj


def build(jobs: int = 0, verbose: bool = False, extra=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, list(extra)), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--save-temps", action="store_true", help="keep device assembly under _build/")
    a = ap.parse_args(argv)
    extra = ["-save-temps=obj"] if a.save_temps else []
    path = build(a.jobs, a.verbose, extra)
    print(path)


if __name__ == "__main__":
    main(sys.argv[1:])
