"""The parity bar rejects wrong outputs (CPU only).

The GPU parity tests compare the HIP path with the oracle through
parity.check_output. These checks show that the bar is discriminative on the
workloads it is applied to: an all-zero output and an output with two heads
exchanged both fail it, as does an output off by a few units in the last place
of every element of one head. The outputs here are the oracle's own, so no GPU
is involved.
"""
import numpy as np
import pytest

import parity
from oracle import paged_latent as orc
from paged_absorbed_mla_amd import workloads as wl

CASES = [("c1", 1), ("c2", 16), ("c4", 16), ("c5", 16)]


@pytest.fixture(scope="module", params=CASES, ids=[f"{c}/{s}" for c, s in CASES])
def case(request):
    cfg, sd = request.param
    w = wl.make(cfg, scale_down=sd)
    _, out = orc.run(w)
    return w, out


def _round(w, x):
    return orc.round_to(x, w["dtype"])


def test_rounded_reference_passes(case):
    w, ref = case
    parity.check_output(w["dtype"], _round(w, ref), ref, heads=w["attrs"]["num_heads"])


def test_zero_output_fails(case):
    w, ref = case
    with pytest.raises(AssertionError):
        parity.check_output(w["dtype"], np.zeros_like(ref), ref)


def test_head_swapped_output_fails(case):
    w, ref = case
    bad = parity.swap_heads(_round(w, ref), w["attrs"]["num_heads"])
    with pytest.raises(AssertionError):
        parity.check_output(w["dtype"], bad, ref)


def test_token_swapped_output_fails(case):
    """Outputs of two tokens of different sequences exchanged."""
    w, ref = case
    cum = w["cumulative_sequence_length"]
    t0, t1 = int(cum[0]), int(cum[-1]) - 1
    bad = _round(w, ref)
    bad[[t0, t1]] = bad[[t1, t0]]
    with pytest.raises(AssertionError):
        parity.check_output(w["dtype"], bad, ref)


def test_nonfinite_output_fails(case):
    w, ref = case
    bad = _round(w, ref)
    bad[0, 0] = np.nan
    with pytest.raises(AssertionError):
        parity.check_output(w["dtype"], bad, ref)
