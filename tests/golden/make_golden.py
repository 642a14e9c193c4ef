"""Writes tests/golden/tiny_oracle_samples.txt: oracle outputs of the tiny
prefill+decode workload (f16, 2 sequences, 4 heads, 64/32/16@48, block 16,
seed 0) at fixed (token, channel) positions, plus a checksum of the written
cache. Calls only the oracle and the seeded generator; run it again only when
a change of the oracle's arithmetic is justified by the pages.

    python tests/golden/make_golden.py
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

from oracle import paged_latent as orc  # noqa: E402
from paged_absorbed_mla_amd import workloads as wl  # noqa: E402

SAMPLES = [(0, 0), (0, 127), (19, 5), (20, 64), (27, 31), (35, 0), (35, 100), (35, 127)]


def main():
    w = wl.make("c1")
    cache, out = orc.run(w)
    lines = ["# token channel value (oracle output of the tiny workload, float64, repr)"]
    for t, c in SAMPLES:
        lines.append(f"{t} {c} {float(out[t, c])!r}")
    lines.append(f"# cache_sum {int(cache.astype(np.int64).sum())}")
    with open(os.path.join(HERE, "tiny_oracle_samples.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
