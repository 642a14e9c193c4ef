"""GPU parity of the separate (grouped-query) layout: the HIP path through the
C ABI (pa_separate_write, pa_separate_attention) against the CPU oracle
oracle/paged_separate.py.

Each case prints its name and shape before touching the GPU. The workloads
are the generator's grouped-query ones (Llama-style 128-wide heads, 8 key/value
heads shared by 4 query heads each; a tiny 64-wide one), scaled down for
element-wise checks and at full size in the launch configuration of the
attention phase, plus edge cases of the head grouping and the padded sizes.
"""
import numpy as np
import pytest

from paged_absorbed_mla_amd import workloads as wl

import parity

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _run(w):
    torch = _torch()
    from paged_absorbed_mla_amd.device import DeviceWorkload
    a = w["attrs"]
    print(f"\n[case] {w.get('name')} dtype={w['dtype']} H={a['num_heads']} kvH={a['kv_num_heads']} "
          f"hs={a['head_size']} vhs={a['v_head_size']} dims={w['dims']}", flush=True)
    d = DeviceWorkload(w)
    before_k, before_v = w["key_cache"].copy(), w["value_cache"].copy()
    d.write()
    d.attention()
    torch.cuda.synchronize()
    return d, before_k, before_v


def _check(w, tokens=None, what=""):
    d, bk, bv = _run(w)
    rk, rv, ref = parity.oracle_separate(w, tokens=tokens)
    parity.check_write_separate(w, d.cache_bits(), d.value_cache_bits(), rk, rv, bk, bv)
    rows = None if tokens is None else np.asarray(tokens)
    mx, rel = parity.check_output(w["dtype"], d.output_f64(), ref, rows=rows, what=what or w["name"],
                                  heads=w["attrs"]["num_heads"])
    print(f"[result] {what or w['name']}: max-abs {mx:.3e} rel {rel:.3e}", flush=True)
    return d, ref


SMALL = [("gqa_tiny", 1), ("gqa_decode", 4), ("gqa_prefill", 16)]


@pytest.mark.parametrize("cfg,sd", SMALL, ids=[f"{c}/{s}" for c, s in SMALL])
def test_separate_parity_elementwise(cfg, sd):
    _check(wl.make(cfg, scale_down=sd), what=f"{cfg}/{sd}")


@pytest.mark.parametrize("cfg", ["gqa_decode", "gqa_prefill"])
def test_separate_parity_full_size(cfg):
    """Full size, every token and head compared with the oracle."""
    _check(wl.make(cfg), what=f"{cfg} full")


def _spec(**kw):
    """A mixed batch (prefill chunks and decodes) of the separate layout; the
    key/value heads are shared by groups of num_heads / kv_num_heads heads."""
    base = dict(name="edge_gqa", dtype="f16", past=[0, 37, 5, 300], new=[40, 3, 70, 1], num_heads=8,
                head_size=128, v_head_size=128, rotary_dim=128, rotary_offset=0, block_size=16,
                scale=1.0 / np.sqrt(128.0), seed=21, layout="SEPARATE", kv_num_heads=2)
    base.update(kw)
    return wl.Spec(**base)


EDGES = {
    "mha_kv_equals_heads": dict(num_heads=8, kv_num_heads=8),
    "mqa_one_kv_head": dict(num_heads=16, kv_num_heads=1),
    "first_token": dict(past=[0], new=[1]),
    "window_37": dict(local_window_size=37),
    "softcap_30": dict(softcap=30.0),
    "no_rotary": dict(do_rotary=0),
    "interleaved_partial_rope": dict(rotary_interleaved=1, rotary_dim=64, rotary_offset=32),
    "block_size_64": dict(block_size=64),
    "block_size_256": dict(block_size=256, past=[300, 2], new=[9, 60]),
    "v_narrower_than_k": dict(v_head_size=64),
    "head_size_96_padded": dict(head_size=96, v_head_size=96, rotary_dim=32, scale=0.0, has_scale=0),
    "head_size_64_bucket": dict(head_size=64, v_head_size=64, rotary_dim=64, scale=0.0, has_scale=0),
    "head_size_64_v_32": dict(head_size=64, v_head_size=32, rotary_dim=32, scale=0.125),
    "slot_drops": dict(slot_drop_frac=0.1),
    "bf16_decode_only": dict(dtype="bf16", past=[900, 17, 4000, 1], new=[1, 1, 1, 1], num_heads=32,
                             kv_num_heads=8),
    "bf16_decode_64_wide": dict(dtype="bf16", past=[900, 17, 2500], new=[1, 1, 1], head_size=64,
                                v_head_size=64, rotary_dim=32, scale=0.0, has_scale=0),
    "empty_middle_seq": dict(past=[4, 50, 7], new=[3, 0, 5]),
    # longer prefill chunks, both storage types
    "prefill_f16": dict(past=[0, 300], new=[200, 150], num_heads=32, kv_num_heads=8),
    "prefill_bf16": dict(dtype="bf16", past=[0, 300], new=[200, 150], num_heads=32, kv_num_heads=8),
}


@pytest.mark.parametrize("name", sorted(EDGES))
def test_separate_edge_case(name):
    _check(wl.build(_spec(name=name, **EDGES[name])), what=name)


def test_separate_poisoned_unreachable_rows_do_not_leak():
    _check(wl.build(_spec(name="poisoned"), poison=True), what="poisoned")


def test_separate_block_permutation_bit_identical():
    torch = _torch()
    w = wl.make("gqa_decode", scale_down=4)
    d1, _, _ = _run(w)
    o1 = d1.output_f64()
    NB = w["key_cache"].shape[0]
    perm = np.random.default_rng(44).permutation(NB)
    kc = np.empty_like(w["key_cache"]); kc[perm] = w["key_cache"]
    vc = np.empty_like(w["value_cache"]); vc[perm] = w["value_cache"]
    bt = w["block_table"].copy(); bt[bt >= 0] = perm[bt[bt >= 0]]
    bs = w["attrs"]["block_size"]
    sl = w["slot_mapping"].copy(); ok = sl >= 0
    sl[ok] = perm[sl[ok] // bs] * bs + sl[ok] % bs
    w2 = dict(w, key_cache=kc, value_cache=vc, block_table=bt, slot_mapping=sl, name="permuted")
    d2, _, _ = _run(w2)
    torch.cuda.synchronize()
    assert np.array_equal(d2.output_f64(), o1)


# Seeded random geometries of the grouped-query layout: key/value head counts
# and group sizes, head sizes in both compiled buckets (padded ones included),
# value sizes up to the head size, block sizes, ragged batches, windows,
# softcaps, rotary modes and dropped slots, element by element.
def _random_spec(seed):
    import math
    r = np.random.default_rng(9100 + seed)
    kvh = int(r.choice([1, 2, 4, 8]))
    group = int(r.choice([1, 2, 4, 8]))
    hs = int(r.choice([16, 32, 48, 64, 80, 96, 112, 128]))
    vhs = 8 * int(r.integers(1, hs // 8 + 1))
    do_rotary = int(r.random() < 0.7)
    rd = ro = 0
    if do_rotary:
        rd = 16 * int(r.integers(1, hs // 16 + 1))
        ro = 8 * int(r.integers(0, (hs - rd) // 8 + 1))
    B = int(r.integers(1, 5))
    past = [int(x) for x in r.integers(0, 260, size=B)]
    new = [int(x) for x in r.integers(0, 40, size=B)]
    if sum(new) == 0:
        new[0] = 1
    return wl.Spec(name=f"gqa_random{seed}_{hs}_{vhs}_{kvh}x{group}", dtype=str(r.choice(["f16", "bf16"])),
                   past=past, new=new, num_heads=kvh * group, head_size=hs, v_head_size=vhs, rotary_dim=rd,
                   rotary_offset=ro, do_rotary=do_rotary, rotary_interleaved=int(r.random() < 0.5),
                   block_size=int(r.choice([16, 32, 64, 128])), scale=float(r.uniform(0.5, 1.5) / math.sqrt(hs)),
                   softcap=float(r.uniform(1.0, 30.0)) if r.random() < 0.3 else 0.0,
                   local_window_size=int(r.integers(0, 64)) if r.random() < 0.4 else -1,
                   slot_drop_frac=0.1 if r.random() < 0.3 else 0.0, seed=300 + seed,
                   layout="SEPARATE", kv_num_heads=kvh)


@pytest.mark.parametrize("seed", range(12))
def test_separate_random_geometry(seed):
    spec = _random_spec(seed)
    _check(wl.build(spec), what=spec.name)


@pytest.mark.parametrize("cfg,sd", SMALL, ids=[f"{c}/{s}" for c, s in SMALL])
def test_separate_forward_bit_identical_to_write_then_attention(cfg, sd):
    """pa_separate_forward (key and value rows in the attention phase's first
    launch) against pa_separate_write + pa_separate_attention."""
    torch = _torch()
    from paged_absorbed_mla_amd.device import DeviceWorkload
    w = wl.make(cfg, scale_down=sd)
    print(f"\n[case] separate forward {cfg}/{sd} dims={w['dims']}", flush=True)
    a, b = DeviceWorkload(w), DeviceWorkload(w)
    a.write()
    a.attention()
    b.forward()
    torch.cuda.synchronize()
    assert np.array_equal(a.cache_bits(), b.cache_bits()), "key cache differs"
    assert np.array_equal(a.value_cache_bits(), b.value_cache_bits()), "value cache differs"
    assert np.array_equal(a.output.view(torch.int16).cpu().numpy(), b.output.view(torch.int16).cpu().numpy())
