"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Each case prints its name and shape before touching the GPU. Element-wise
parity runs at sizes the oracle finishes in seconds (several tiles, ragged
tails); the five full-size workloads run in the launch configuration the
benchmark times and are compared on sampled tokens.
"""
import math
import sys

import numpy as np
import pytest

from oracle import paged_latent as orc
from paged_absorbed_mla_amd import workloads as wl

import parity

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _dev(w, **kw):
    from paged_absorbed_mla_amd.device import DeviceWorkload
    print(f"\n[case] {w.get('name')} dtype={w['dtype']} dims={w['dims']}", flush=True)
    return DeviceWorkload(w, **kw)


def _run(w, split_kv=None):
    torch = _torch()
    d = _dev(w)
    before = w["key_cache"].copy()
    d.write()
    d.attention(split_kv=split_kv)
    torch.cuda.synchronize()
    return d, before


# ---------------------------------------------------------------------------
# The five workloads, scaled so the oracle checks every element
# ---------------------------------------------------------------------------

SMALL = [("c1", 1), ("c2", 4), ("c3", 8), ("c4", 8), ("c5", 4)]


@pytest.mark.parametrize("cfg,sd", SMALL, ids=[f"{c}/{s}" for c, s in SMALL])
def test_parity_elementwise(cfg, sd):
    w = wl.make(cfg, scale_down=sd)
    d, before = _run(w)
    ref_cache, ref_out = parity.oracle(w)
    parity.check_write(w, d.cache_bits(), ref_cache, before)
    mx, rel = parity.check_output(w["dtype"], d.output_f64(), ref_out, what=cfg, heads=w["attrs"]["num_heads"])
    print(f"[result] {cfg}/{sd}: max-abs {mx:.3e} rel {rel:.3e}", flush=True)


# Full-size workloads in the benchmark's launch configuration, every token
# and head compared with the oracle (it takes a few seconds per workload).
@pytest.mark.parametrize("cfg", ["c2", "c3", "c4", "c5"])
def test_parity_full_size(cfg):
    w = wl.make(cfg)
    d, before = _run(w)
    ref_cache, ref_out = parity.oracle(w)
    parity.check_write(w, d.cache_bits(), ref_cache, before)
    mx, rel = parity.check_output(w["dtype"], d.output_f64(), ref_out, what=cfg, heads=w["attrs"]["num_heads"])
    print(f"[result] {cfg} full, {w['dims']['token_count']} tokens: max-abs {mx:.3e} rel {rel:.3e}", flush=True)


# The fused call (pa_latent_forward: write rows inside the attention phase's
# first launch) against the two calls in order: bit-identical cache and output.
@pytest.mark.parametrize("cfg,sd", SMALL + [("c4", 1)], ids=[f"{c}/{s}" for c, s in SMALL + [("c4", 1)]])
def test_forward_bit_identical_to_write_then_attention(cfg, sd):
    torch = _torch()
    w = wl.make(cfg, scale_down=sd)
    a = _dev(w)
    b = _dev(w)
    a.write()
    a.attention()
    b.forward()
    torch.cuda.synchronize()
    assert np.array_equal(a.cache_bits(), b.cache_bits()), f"{cfg}/{sd}: cache differs"
    ao = a.output.view(torch.int16).cpu().numpy()
    bo = b.output.view(torch.int16).cpu().numpy()
    assert np.array_equal(ao, bo), f"{cfg}/{sd}: output differs"
    print(f"[result] {cfg}/{sd}: forward bit-identical to write + attention", flush=True)


def test_forward_full_size_against_oracle():
    """The benchmark's step (the fused call) on the full DeepSeek-V3 decode batch."""
    torch = _torch()
    w = wl.make("c4")
    d = _dev(w)
    before = w["key_cache"].copy()
    d.forward()
    torch.cuda.synchronize()
    ref_cache, ref_out = parity.oracle(w)
    parity.check_write(w, d.cache_bits(), ref_cache, before)
    mx, rel = parity.check_output(w["dtype"], d.output_f64(), ref_out, what="c4 forward",
                                  heads=w["attrs"]["num_heads"])
    print(f"[result] c4 forward: max-abs {mx:.3e} rel {rel:.3e}", flush=True)


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cfg,sd", [("c4", 8), ("c5", 4), ("c3", 8), ("c2", 4)])
def test_split_partition_invariance(cfg, sd):
    """Automatic split-KV partition vs one workgroup per query tile. Both must
    match the oracle; between them only the rounding of the probabilities to the
    MFMA input type differs (different running-max references per piece), so
    they agree to well inside the parity tolerance."""
    torch = _torch()
    w = wl.make(cfg, scale_down=sd)
    d = _dev(w)
    d.write()
    d.attention(split_kv=True)
    torch.cuda.synchronize()
    a = d.output_f64().copy()
    d.attention(split_kv=False)
    torch.cuda.synchronize()
    b = d.output_f64().copy()
    _, ref = parity.oracle(w)
    parity.check_output(w["dtype"], a, ref, what=f"{cfg} split")
    parity.check_output(w["dtype"], b, ref, what=f"{cfg} whole")
    rel = np.linalg.norm(a - b) / np.linalg.norm(ref)
    assert rel <= parity.REL_FRO[w["dtype"]] / 2, rel


def _permute(w, seed):
    rng = np.random.default_rng(seed)
    NB, bs = w["key_cache"].shape[0], w["key_cache"].shape[1]
    perm = rng.permutation(NB)
    w2 = dict(w)
    c = np.empty_like(w["key_cache"])
    c[perm] = w["key_cache"]
    w2["key_cache"] = c
    bt = w["block_table"].copy()
    bt[bt >= 0] = perm[bt[bt >= 0]]
    w2["block_table"] = bt
    s = w["slot_mapping"].copy()
    ok = s >= 0
    s[ok] = perm[s[ok] // bs] * bs + s[ok] % bs
    w2["slot_mapping"] = s
    return w2


@pytest.mark.parametrize("cfg,sd", [("c1", 1), ("c5", 4), ("c4", 8)])
def test_block_permutation_bit_identical(cfg, sd):
    w = wl.make(cfg, scale_down=sd)
    torch = _torch()
    d1, _ = _run(w)
    d2, _ = _run(_permute(w, 7))
    o1 = d1.output.view(torch.int16).cpu().numpy()
    o2 = d2.output.view(torch.int16).cpu().numpy()
    assert np.array_equal(o1, o2)


@pytest.mark.parametrize("cfg,sd", [("c1", 1), ("c5", 4), ("c2", 4)])
def test_poisoned_unreachable_rows_do_not_leak(cfg, sd):
    """Rows no visible key can reach hold NaN; outputs must be unchanged and finite."""
    w = wl.make(cfg, scale_down=sd)
    wp = wl.make(cfg, scale_down=sd, poison=True)
    d1, _ = _run(w)
    d2, _ = _run(wp)
    o2 = d2.output_f64()
    assert np.all(np.isfinite(o2))
    assert np.array_equal(d1.output_f64(), o2)


def test_repeat_is_deterministic():
    torch = _torch()
    w = wl.make("c5", scale_down=4)
    d = _dev(w)
    d.write()
    d.attention()
    torch.cuda.synchronize()
    a = d.output_f64()
    for _ in range(3):
        d.write()          # idempotent: rewrites the same rows
        d.attention()
    torch.cuda.synchronize()
    assert np.array_equal(a, d.output_f64())


# ---------------------------------------------------------------------------
# Edge cases of the method
# ---------------------------------------------------------------------------

def _spec(**kw):
    base = dict(name="edge", dtype="bf16", past=[0, 37, 5], new=[1, 3, 70], num_heads=4, head_size=64,
                v_head_size=32, rotary_dim=16, rotary_offset=48, block_size=16, scale=0.125, seed=11)
    base.update(kw)
    return wl.Spec(**base)


def _edge(spec, split_kv=None):
    w = wl.build(spec)
    d, before = _run(w, split_kv=split_kv)
    ref_cache, ref_out = parity.oracle(w)
    parity.check_write(w, d.cache_bits(), ref_cache, before)
    parity.check_output(w["dtype"], d.output_f64(), ref_out, what=spec.name, heads=spec.num_heads)
    return w, d, ref_cache, ref_out


EDGES = {
    "first_token": dict(past=[0], new=[1]),
    "window0": dict(local_window_size=0),
    "window5": dict(local_window_size=5, past=[40, 3], new=[9, 30]),
    "no_rotary": dict(do_rotary=0),
    "interleaved": dict(rotary_interleaved=1),
    "bs32": dict(block_size=32),
    "bs128": dict(block_size=128, past=[200, 3], new=[2, 140]),
    "bs256": dict(block_size=256, past=[300], new=[20]),
    "one_head": dict(num_heads=1),
    "three_heads": dict(num_heads=3, past=[9, 0], new=[12, 23]),
    "softcap": dict(softcap=0.5, dtype="f16"),
    "f16": dict(dtype="f16"),
    "v_not_mult4": dict(v_head_size=30),
    "v_eq_hs": dict(v_head_size=64, scale=1 / 8),
    "hs80_padded": dict(head_size=80, v_head_size=48, rotary_offset=16, rotary_dim=64),
    "glm_dims_128heads": dict(num_heads=128, head_size=192, v_head_size=128, rotary_dim=64,
                              rotary_offset=128, block_size=64, past=[100, 700], new=[1, 1]),
    # long bfloat16 prefill on GLM dims (four-wave instance, two workgroups per CU)
    "glm_dims_prefill_bf16": dict(num_heads=16, head_size=192, v_head_size=128, rotary_dim=64,
                                  rotary_offset=128, block_size=16, past=[0, 300], new=[200, 150]),
    "dsv3_dims_multi_token": dict(num_heads=16, head_size=576, v_head_size=512, rotary_dim=64,
                                  rotary_offset=512, block_size=16, past=[33, 0], new=[9, 17]),
    "empty_middle_seq": dict(past=[4, 50, 7], new=[3, 0, 5]),
    "long_context": dict(past=[20000], new=[1], block_size=64),
    "slot_drop": dict(slot_drop_frac=0.3, past=[10, 20], new=[20, 10]),
    # no explicit scale, v_head_size == head_size: the default 1/sqrt(head_size)
    "default_scale_64": dict(v_head_size=64, has_scale=0, scale=0.0),
    "default_scale_192": dict(head_size=192, v_head_size=192, rotary_offset=128, rotary_dim=64,
                              has_scale=0, scale=0.0, past=[40, 3], new=[2, 21]),
}


@pytest.mark.parametrize("name", list(EDGES))
def test_edge_case(name):
    _edge(_spec(name=name, **EDGES[name]))


# The same method cases at DeepSeek-V3 latent dimensions (576 / 512), which run
# the wide-row kernel: score-scale sign and zero, softcap, window, float16,
# decode rows whose keys end inside a tile, and keys that straddle pieces.
_DSV3 = dict(num_heads=16, head_size=576, v_head_size=512, rotary_dim=64, rotary_offset=512, block_size=16,
             past=[33, 0, 70], new=[9, 17, 1], scale=0.06)
DSV3_EDGES = {
    "dsv3_neg_scale": dict(scale=-0.06),
    "dsv3_zero_scale": dict(scale=0.0),
    "dsv3_softcap": dict(softcap=2.0, dtype="f16"),
    "dsv3_window": dict(local_window_size=20),
    "dsv3_f16": dict(dtype="f16"),
    "dsv3_bs64_decode": dict(block_size=64, past=[300, 95, 1], new=[1, 1, 1]),
    "dsv3_interleaved": dict(rotary_interleaved=1),
    "dsv3_no_rotary": dict(do_rotary=0),
    "dsv3_interleaved_bf16_decode": dict(rotary_interleaved=1, block_size=64, past=[300, 95], new=[1, 1],
                                         num_heads=128),
}


@pytest.mark.parametrize("name", list(DSV3_EDGES))
def test_edge_case_dsv3(name):
    kw = dict(_DSV3)
    kw.update(DSV3_EDGES[name])
    _edge(_spec(name=name, **kw))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_second_pass_on_score_jump(dtype):
    """Fixed-reference softmax, second pass: an old key whose score exceeds
    its piece's first-tile reference by more than the probability type can
    represent (planted key = q / 4: jump ~ |q|^2 / 4 * scale * log2(e) ~ 180
    log2 units, against first-tile maxima near 20; cache and key values have
    standard deviation 1/4, so outputs stay within 1 and the absolute
    tolerance is not eaten by the output's own rounding) forces the workgroup
    to redo the piece with exact maxima; without that pass the probability is
    infinite. The jumps are planted for rows that are not the first of their
    wave (heads 37 and 5 of 64), and 64 heads leave two waves of every decode
    tile without a valid row. Keys are planted below the past length, where
    the write phase does not touch them."""
    kw = dict(_DSV3)
    kw.update(num_heads=64, past=[300, 700], new=[1, 1], block_size=16, scale=1.0, dtype=dtype,
              cache_std=0.25, key_std=0.25)
    w = wl.build(_spec(name=f"score_jump_{dtype}", **kw))
    H, hs, nr = 64, 576, 512
    q = orc.widen(w["query"], dtype).reshape(-1, H, hs)
    cache = w["key_cache"]
    flat = cache.reshape(-1, hs)
    bs = cache.shape[1]
    cum, bt = w["cumulative_sequence_length"], w["block_table"]
    for b, (h, j) in enumerate([(37, 250), (5, 611)]):
        assert j < w["past_seqlens"][b]
        slot = int(bt[b, j // bs]) * bs + j % bs
        flat[slot, :nr] = wl.to_storage_bits((0.25 * q[cum[b], h, :nr]).astype(np.float32), dtype)
    w["key_cache"] = flat.reshape(cache.shape)
    ref_cache, ref_out = parity.oracle(w)
    # One workgroup per query tile puts each planted key in a later tile of
    # its piece (the case that needs the second pass); the automatic split
    # spreads these few tiles one per piece and checks the combine with them.
    for split_kv in (False, True):
        d, before = _run(w, split_kv=split_kv)
        parity.check_write(w, d.cache_bits(), ref_cache, before)
        parity.check_output(dtype, d.output_f64(), ref_out, what=f"score_jump_{dtype} split_kv={split_kv}")


def test_schedule_in_global_scratch():
    """A batch whose schedule arrays exceed the scheduler's LDS array (1,500
    decode sequences of 4 heads: ~1,700 query tiles), so the schedule is
    built in the workspace instead; both partitions against the oracle."""
    rng = np.random.default_rng(12)
    n = 1500
    past = [int(x) for x in rng.integers(0, 96, size=n)]
    spec = _spec(name="many_sequences", past=past, new=[1] * n, block_size=16)
    w = wl.build(spec)
    # The scheduler's working arrays hold at least 3 B + 9 M int32 values for
    # B sequences and M query tiles of 32 rows; its LDS array holds 12,288.
    T, H = w["dims"]["token_count"], spec.num_heads
    assert 3 * n + 9 * ((T * H + 31) // 32 + min(n, T)) > 12288
    ref_cache, ref_out = parity.oracle(w)
    for split_kv in (True, False):
        d, _ = _run(w, split_kv=split_kv)
        parity.check_output(w["dtype"], d.output_f64(), ref_out, what=f"many_sequences split_kv={split_kv}",
                            heads=spec.num_heads)
    # The fused call: 1,500 write rows ride in the same launch as the
    # workspace-built schedule.
    d = _dev(w)
    before = w["key_cache"].copy()
    d.forward()
    _torch().cuda.synchronize()
    parity.check_write(w, d.cache_bits(), ref_cache, before)
    parity.check_output(w["dtype"], d.output_f64(), ref_out, what="many_sequences fused", heads=spec.num_heads)


@pytest.mark.parametrize("geom", ["64_32", "192_128", "576_512"])
def test_out_of_range_block_ids_stay_in_bounds(geom):
    """A block_table entry outside [0, num_blocks) inside a sequence's context
    (a violated precondition) is clamped into the cache: the call completes and
    every output is finite. Regression test for the generic kernel's boundary
    tiles, which read the table without the clamp."""
    kw = {"64_32": dict(),
          "192_128": dict(head_size=192, v_head_size=128, rotary_offset=128, rotary_dim=64, block_size=16),
          "576_512": dict(_DSV3)}[geom]
    kw = dict(kw)
    kw.update(past=[70, 40], new=[1, 9], name=f"bad_block_{geom}")
    w = wl.build(_spec(**kw))
    bt = w["block_table"]
    bt[0, 1] = w["dims"]["num_blocks"] + 1000      # past the cache
    bt[1, 2] = -7                                   # negative
    d, _ = _run(w)
    assert np.all(np.isfinite(d.output_f64()))


def test_first_token_and_window0_exact():
    """A token that sees only itself outputs its own value row, bit for bit."""
    torch = _torch()
    for kw in (dict(past=[0], new=[1]), dict(local_window_size=0)):
        w, d, ref_cache, _ = _edge(_spec(name="exact", **kw))
        hs, vhs, H = 64, 32, 4
        got = d.output.view(torch.int16).cpu().numpy().view(np.uint16)
        flat = ref_cache.reshape(-1, hs)
        for t in range(w["dims"]["token_count"]):
            s = w["slot_mapping"][t]
            for h in range(H):
                assert np.array_equal(got[t, h * vhs:(h + 1) * vhs], flat[s, :vhs])


def test_zero_tokens_no_launch():
    torch = _torch()
    w = wl.build(_spec(name="zero", past=[5], new=[1]))
    w["dims"]["token_count"] = 0
    d = _dev(w, workspace=False)
    assert d.write() == 0
    assert d.attention() == 0
    torch.cuda.synchronize()


def test_workspace_too_small():
    _torch()
    from paged_absorbed_mla_amd import _lib
    w = wl.make("c1")
    d = _dev(w)
    st = _lib.pa_latent_attention(d.attrs, d.dims, d.code, d.query, d.key_cache, d.cos, d.sin, d.cumseq,
                                  d.past, d.block_table, d.output, d.workspace, d.ws_bytes - 256,
                                  check=False)
    assert st == _lib.PA_ERR_WORKSPACE_TOO_SMALL


# ---------------------------------------------------------------------------
# Seeded random geometries: head sizes inside every compiled bucket (padded
# instances included), head counts, block sizes, ragged batches with empty
# sequences, windows, softcaps, rotary modes and dropped slots, each checked
# element by element against the oracle through the fused call.
# ---------------------------------------------------------------------------

def _random_spec(seed):
    r = np.random.default_rng(7000 + seed)
    bucket = seed % 3
    if bucket == 0:
        hs = int(r.choice([16, 32, 48, 64]))
        vhs = int(r.integers(1, min(hs, 32) + 1))
        heads = int(r.integers(1, 21))
        past_hi, new_hi = 300, 40
    elif bucket == 1:
        hs = int(r.choice([80, 96, 128, 144, 176, 192]))
        vhs = int(r.integers(1, min(hs, 128) + 1))
        heads = int(r.choice([1, 3, 8, 16, 20, 64]))
        past_hi, new_hi = 300, 40
    else:
        hs = int(r.choice([208, 256, 384, 512, 576]))
        vhs = int(r.integers(1, min(hs, 512) + 1))
        heads = int(r.choice([1, 5, 16, 128]))
        past_hi, new_hi = 200, 24 if heads < 128 else 2
    do_rotary = int(r.random() < 0.7)
    rd = ro = 0
    if do_rotary:
        rd = 16 * int(r.integers(1, min(hs, 128) // 16 + 1))
        ro = 8 * int(r.integers(0, (hs - rd) // 8 + 1))
    B = int(r.integers(1, 6))
    past = [int(x) for x in r.integers(0, past_hi + 1, size=B)]
    new = [int(x) for x in r.integers(0, new_hi + 1, size=B)]
    if sum(new) == 0:
        new[0] = 1
    return wl.Spec(name=f"random{seed}_{hs}_{vhs}_h{heads}", dtype=str(r.choice(["f16", "bf16"])), past=past,
                   new=new, num_heads=heads, head_size=hs, v_head_size=vhs, rotary_dim=rd, rotary_offset=ro,
                   do_rotary=do_rotary, rotary_interleaved=int(r.random() < 0.5),
                   block_size=int(r.choice([16, 32, 64, 128])),
                   scale=float(r.uniform(0.5, 1.5) / math.sqrt(hs)),
                   softcap=float(r.uniform(1.0, 30.0)) if r.random() < 0.3 else 0.0,
                   local_window_size=int(r.integers(0, 64)) if r.random() < 0.4 else -1,
                   slot_drop_frac=0.1 if r.random() < 0.3 else 0.0, seed=100 + seed)


@pytest.mark.parametrize("seed", range(24))
def test_random_geometry(seed):
    torch = _torch()
    spec = _random_spec(seed)
    w = wl.build(spec)
    d = _dev(w)
    before = w["key_cache"].copy()
    d.forward()
    torch.cuda.synchronize()
    ref_cache, ref_out = parity.oracle(w)
    parity.check_write(w, d.cache_bits(), ref_cache, before)
    mx, rel = parity.check_output(w["dtype"], d.output_f64(), ref_out, what=spec.name, heads=spec.num_heads)
    print(f"[result] {spec.name}: max-abs {mx:.3e} rel {rel:.3e}", flush=True)
