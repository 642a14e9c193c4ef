"""HIP-graph capture of the path (write phase + attention) through the C ABI.

The op is capture/replay safe after a warmed call (docs.rs page,
PagedCaptureSignature, capture_support and the warm gate in execute; PR #1978
"Tests": capture + 3 replays bit-equal to eager). Here: a step is run
eagerly, captured into a graph, and replayed three times with eager work and
synchronisation between the replays (the written cache rows restored to their
old contents, the output poisoned); every replay must reproduce the eager
cache and output bit for bit. A capture of a signature that has not run
eagerly is refused before anything is enqueued.
"""
import numpy as np
import pytest

from paged_absorbed_mla_amd import _lib
from paged_absorbed_mla_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _dev(w):
    from paged_absorbed_mla_amd.device import DeviceWorkload
    print(f"\n[case] capture {w['name']} dtype={w['dtype']} dims={w['dims']}", flush=True)
    return DeviceWorkload(w, "cuda:0")


def _bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().copy()


@pytest.mark.parametrize("cfg,sd", [("c1", 1), ("c4", 4), ("c2", 4)])
def test_capture_three_replays_bit_equal_to_eager(cfg, sd):
    torch = _torch()
    w = wl.make(cfg, scale_down=sd)
    d = _dev(w)
    before = d.key_cache.clone()
    d.write()
    d.attention()
    torch.cuda.synchronize()
    assert _lib.pa_latent_capture_ready(d.attrs, d.dims, d.code) == (True, True)
    eager_out, eager_cache = _bits(d.output), _bits(d.key_cache)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        d.write()
        d.attention()
    for rep in range(3):
        d.key_cache.copy_(before)                     # eager work between replays
        d.output.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_bits(d.key_cache), eager_cache), f"replay {rep}: cache differs"
        assert np.array_equal(_bits(d.output), eager_out), f"replay {rep}: output differs"
    del g


@pytest.mark.parametrize("cfg,sd", [("c1", 1), ("c4", 4)])
def test_capture_forward_three_replays_bit_equal_to_eager(cfg, sd):
    """The fused call (pa_latent_forward) under the same gate and replay check."""
    torch = _torch()
    w = wl.make(cfg, scale_down=sd)
    d = _dev(w)
    before = d.key_cache.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):                         # not warmed yet: refused, nothing enqueued
        st = _lib.pa_latent_forward(d.attrs, d.dims, d.code, d.query, d.key, d.cos, d.sin, d.slot_mapping,
                                    d.cumseq, d.past, d.block_table, d.key_cache, d.output, d.workspace,
                                    d.ws_bytes, check=False)
    assert st == _lib.PA_ERR_CAPTURE_NOT_WARMED
    del g
    d.forward()
    torch.cuda.synchronize()
    eager_out, eager_cache = _bits(d.output), _bits(d.key_cache)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        d.forward()
    for rep in range(3):
        d.key_cache.copy_(before)                     # eager work between replays
        d.output.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_bits(d.key_cache), eager_cache), f"replay {rep}: cache differs"
        assert np.array_equal(_bits(d.output), eager_out), f"replay {rep}: output differs"
    del g


def test_capture_of_an_unwarmed_signature_is_refused():
    torch = _torch()
    spec = wl.Spec(name="unwarmed", dtype="bf16", past=[7, 31], new=[3, 1], num_heads=5, head_size=64,
                   v_head_size=32, rotary_dim=16, rotary_offset=48, block_size=16, scale=0.125, seed=5)
    d = _dev(wl.build(spec))
    assert _lib.pa_latent_capture_ready(d.attrs, d.dims, d.code) == (False, False)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st_w = _lib.pa_latent_write(
            d.attrs, d.dims, d.code, d.key, d.cos, d.sin, d.slot_mapping, d.cumseq, d.past, d.key_cache,
            check=False)
        st_a = _lib.pa_latent_attention(d.attrs, d.dims, d.code, d.query, d.key_cache, d.cos, d.sin, d.cumseq,
                                        d.past, d.block_table, d.output, d.workspace, d.ws_bytes, check=False)
    assert st_w == _lib.PA_ERR_CAPTURE_NOT_WARMED and st_a == _lib.PA_ERR_CAPTURE_NOT_WARMED
    assert "eagerly" in _lib.pa_last_error()
    del g
    # after an eager call the same signature is ready
    d.write()
    d.attention()
    torch.cuda.synchronize()
    assert _lib.pa_latent_capture_ready(d.attrs, d.dims, d.code) == (True, True)


def test_capture_separate_layout_three_replays_bit_equal_to_eager():
    """The separate (grouped-query) entry points under the same gate: after an
    eager step the capture replays bit-equal; a different kv_num_heads is a
    different signature and is refused."""
    torch = _torch()
    w = wl.make("gqa_decode", scale_down=4)
    d = _dev(w)
    before_k, before_v = d.key_cache.clone(), d.value_cache.clone()
    d.write()
    d.attention()
    torch.cuda.synchronize()
    eager = (_bits(d.output), _bits(d.key_cache), _bits(d.value_cache))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        d.write()
        d.attention()
    for rep in range(3):
        d.key_cache.copy_(before_k)
        d.value_cache.copy_(before_v)
        d.output.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (_bits(d.output), _bits(d.key_cache), _bits(d.value_cache))
        for name, a, b in zip(("output", "key cache", "value cache"), got, eager):
            assert np.array_equal(a, b), f"replay {rep}: {name} differs"
    del g
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2):
        st = _lib.pa_separate_attention(d.attrs, d.kvh // 2, d.dims, d.code, d.query, d.key_cache, d.value_cache,
                                        d.cos, d.sin, d.cumseq, d.past, d.block_table, d.output, d.workspace,
                                        d.ws_bytes, check=False)
    assert st == _lib.PA_ERR_CAPTURE_NOT_WARMED
    del g2


def test_capture_separate_forward_three_replays_bit_equal_to_two_calls():
    """The separate layout's fused call (pa_separate_forward), warmed eagerly,
    captured and replayed three times: every replay bit-equal to the eager
    write then attention."""
    torch = _torch()
    w = wl.make("gqa_decode", scale_down=4)
    d = _dev(w)
    before_k, before_v = d.key_cache.clone(), d.value_cache.clone()
    d.write()
    d.attention()
    torch.cuda.synchronize()
    eager = (_bits(d.output), _bits(d.key_cache), _bits(d.value_cache))
    d.key_cache.copy_(before_k)
    d.value_cache.copy_(before_v)
    d.output.fill_(float("nan"))
    d.forward()
    torch.cuda.synchronize()
    got = (_bits(d.output), _bits(d.key_cache), _bits(d.value_cache))
    for name, a, b in zip(("output", "key cache", "value cache"), got, eager):
        assert np.array_equal(a, b), f"eager fused call: {name} differs from the two calls"
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        d.forward()
    for rep in range(3):
        d.key_cache.copy_(before_k)
        d.value_cache.copy_(before_v)
        d.output.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (_bits(d.output), _bits(d.key_cache), _bits(d.value_cache))
        for name, a, b in zip(("output", "key cache", "value cache"), got, eager):
            assert np.array_equal(a, b), f"replay {rep}: {name} differs"
    del g
