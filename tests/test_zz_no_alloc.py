"""pa_latent_attention_noalloc (the read phase on the library's static device
scratch, for callers that cannot allocate) against pa_latent_attention with a
caller workspace, through the C ABI: two calls in a row, the second on a
smaller input, each bit-identical to the existing entry point on the same
inputs (same kernels, same schedule) and within the oracle tolerance; and a
call whose workspace exceeds the static scratch is rejected before any launch.
"""
import numpy as np
import pytest

import parity
from paged_absorbed_mla_amd import _lib
from paged_absorbed_mla_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _both(w):
    torch = _torch()
    from paged_absorbed_mla_amd.device import DeviceWorkload
    print(f"\n[case] noalloc {w['name']} dtype={w['dtype']} dims={w['dims']}", flush=True)
    d = DeviceWorkload(w, "cuda:0")
    d.write()
    d.attention()
    out_static = torch.empty_like(d.output).fill_(float("nan"))
    _lib.pa_latent_attention_noalloc(d.attrs, d.dims, d.code, d.query, d.key_cache, d.cos, d.sin, d.cumseq,
                                     d.past, d.block_table, out_static)
    torch.cuda.synchronize()
    ref = d.output.view(torch.int16).cpu().numpy()
    got = out_static.view(torch.int16).cpu().numpy()
    assert np.array_equal(got, ref), "static-scratch output differs from the caller-workspace output"
    return d, out_static


def test_noalloc_two_calls_second_smaller():
    torch = _torch()
    big = wl.make("c4")                         # the benchmark's decode batch
    small = wl.make("c4", scale_down=8)
    assert small["dims"]["token_count"] < big["dims"]["token_count"]
    for w in (big, small):
        d, out = _both(w)
        if w is small:
            _, ref = parity.oracle(w)
            parity.check_output(w["dtype"], out.to(torch.float64).cpu().numpy(), ref, what="noalloc small",
                                heads=w["attrs"]["num_heads"])


def test_noalloc_rejects_a_workspace_beyond_the_scratch():
    torch = _torch()
    from paged_absorbed_mla_amd.device import DeviceWorkload
    w = wl.make("c5")                           # needs well over 64 MiB of workspace
    d = DeviceWorkload(w, "cuda:0", workspace=False)
    need = _lib.pa_latent_workspace_size(d.attrs, d.dims, d.code, 0)
    assert need > (64 << 20)
    st = _lib.pa_latent_attention_noalloc(d.attrs, d.dims, d.code, d.query, d.key_cache, d.cos, d.sin,
                                          d.cumseq, d.past, d.block_table, d.output, check=False)
    assert st == _lib.PA_ERR_WORKSPACE_TOO_SMALL
    assert "static scratch" in _lib.pa_last_error()
    torch.cuda.synchronize()
