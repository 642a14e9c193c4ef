"""Golden fixtures (tests/golden/): values the pages print, and stored oracle
outputs of the tiny workload (written by tests/golden/make_golden.py, which
calls only the oracle and the seeded generator)."""
import json
import os
import re

import numpy as np

import paged_absorbed_mla_amd as pa
from oracle import paged_latent as orc
from paged_absorbed_mla_amd import workloads as wl

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
GOLD = os.path.join(HERE, "golden")


def test_attribute_defaults_match_the_pages():
    s = json.load(open(os.path.join(GOLD, "op_schema.json")))
    a = pa.make_attrs(num_heads=1, head_size=64)
    for name, value in s["attribute_defaults"].items():
        assert getattr(a, name) == value, name


def test_c_abi_takes_exactly_the_latent_inputs():
    """The two entry points together take every input the LATENT mode uses and
    none of the schema's other inputs (value, value_cache, head_sink, norms,
    scales, metadata are rejected by the op's routing on the pages)."""
    s = json.load(open(os.path.join(GOLD, "op_schema.json")))
    text = open(os.path.join(ROOT, "include", "pa_latent.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    taken = set()
    for fn in ("pa_latent_write", "pa_latent_attention"):
        sig = re.search(fn + r"\(([^;]*)\);", text, re.S).group(1)
        taken |= {n for n in re.findall(r"\b([a-z_]+)\s*(?=[,)])", sig + ")")}
    schema = set(s["inputs"])
    assert set(s["latent_inputs_used"]) <= taken
    assert (taken & schema) == set(s["latent_inputs_used"])


def test_oracle_tiny_outputs_match_stored_values():
    w = wl.make("c1")
    cache, out = orc.run(w)
    lines = [l.split() for l in open(os.path.join(GOLD, "tiny_oracle_samples.txt")) if not l.startswith("#")]
    for t, c, v in lines:
        assert out[int(t), int(c)] == float(v), (t, c)
    checksum = [l for l in open(os.path.join(GOLD, "tiny_oracle_samples.txt")) if "cache_sum" in l][0]
    assert int(cache.astype(np.int64).sum()) == int(checksum.split()[-1])
