"""Pins for the CPU oracle: each test checks it against something other than itself.

Sources of truth used here: library routines for special cases (numpy's
float16 conversion, torch's float32->bfloat16 conversion, torch's
scaled_dot_product_attention on contiguous tensors), closed forms, invariants
the pages state (PR #1940 "PagedAttention v1 audit and MLA oracle": absorbed
LATENT equals decomposed multi-head latent attention, block-table permutation
invariance, slot -1 write suppression, equality with naive contiguous dense
attention; PR #1978 review verdict: first GLM token has exactly zero error),
and brute force on tiny inputs.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import paged_latent as orc
from paged_absorbed_mla_amd import workloads as wl


# ----------------------------------------------------------------------------
# 16-bit rounding
# ----------------------------------------------------------------------------

def _edge_values(rng, n):
    mags = np.concatenate([
        rng.standard_normal(n),
        rng.standard_normal(n) * 1e-5,            # f16 subnormal range
        rng.standard_normal(n) * 6e4,             # near f16 max
        rng.standard_normal(n) * 1e-39,           # bf16 subnormal range
        rng.standard_normal(n) * 1e38,
    ])
    return mags


def test_round_f16_matches_numpy():
    rng = np.random.default_rng(0)
    x = _edge_values(rng, 4000)
    # exact midpoints between neighbouring float16 values (ties)
    lo = rng.standard_normal(2000).astype(np.float16)
    hi = np.nextafter(lo, np.float16(np.inf))
    mid = (lo.astype(np.float64) + hi.astype(np.float64)) / 2
    x = np.concatenate([x, mid, [65504.0, 65519.99, 65520.0, 2.0**-25, 2.0**-24 * 1.5]])
    got = orc.to_bits(x, "f16")
    want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(1)
    x = _edge_values(rng, 4000).astype(np.float32)
    # float32 values that are exact bf16 midpoints
    base = rng.standard_normal(2000).astype(np.float32)
    bits = base.view(np.uint32) & np.uint32(0xFFFF0000) | np.uint32(0x8000)
    x = np.concatenate([x, bits.view(np.float32)])
    got = orc.to_bits(x.astype(np.float64), "bf16")
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_round_ties_to_even_by_hand():
    # 1 + 2^-8 lies halfway between bf16 neighbours 1 and 1 + 2^-7: ties go to the even one (1).
    assert orc.round_to(np.array([1 + 2.0**-8]), "bf16")[0] == 1.0
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even).
    assert orc.round_to(np.array([1 + 3 * 2.0**-8]), "bf16")[0] == 1 + 2.0**-6
    # float16: 2049 is halfway between 2048 and 2050 -> 2048.
    assert orc.round_to(np.array([2049.0]), "f16")[0] == 2048.0
    assert orc.round_to(np.array([2051.0]), "f16")[0] == 2052.0


def test_widen_is_exact():
    bits = np.arange(2**16, dtype=np.uint32).astype(np.uint16)
    for dt in ("f16", "bf16"):
        vals = orc.widen(bits, dt)
        finite = np.isfinite(vals)
        assert np.array_equal(orc.to_bits(vals[finite], dt), bits[finite])
    # float16 -0 and the bfloat16 encoding of 1.0
    assert orc.widen(np.array([0x3F80], dtype=np.uint16), "bf16")[0] == 1.0
    assert orc.widen(np.array([0x3C00], dtype=np.uint16), "f16")[0] == 1.0


# ----------------------------------------------------------------------------
# Token resolution
# ----------------------------------------------------------------------------

def test_resolve_tokens_brute_force():
    # Tiny config: pasts 0 and 21, new 20 and 16 (tiny workload of the pages' geometry).
    b, pos = orc.resolve_tokens(np.array([0, 20, 36]), np.array([0, 21]))
    assert list(b) == [0] * 20 + [1] * 16
    assert list(pos) == list(range(20)) + list(range(21, 37))
    # empty sequences in the middle are skipped
    b, pos = orc.resolve_tokens(np.array([0, 2, 2, 3]), np.array([5, 7, 9]))
    assert list(b) == [0, 0, 2] and list(pos) == [5, 6, 9]


# ----------------------------------------------------------------------------
# RoPE
# ----------------------------------------------------------------------------

def _exact_tables(P, rd, theta=10000.0):
    half = rd // 2
    inv = theta ** (-(2.0 * np.arange(half)) / rd)
    ang = np.arange(P)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


@pytest.mark.parametrize("interleaved", [False, True])
def test_rope_matches_complex_rotation(interleaved):
    rng = np.random.default_rng(3)
    hs, ro, rd, P = 64, 48, 16, 40
    cos, sin = _exact_tables(P, rd)
    x = rng.standard_normal(hs)
    for pos in (0, 1, 17, 39):
        y = orc.rope(x, pos, cos, sin, ro, rd, interleaved)
        half = rd // 2
        if interleaved:
            z = x[ro:ro + rd:2] + 1j * x[ro + 1:ro + rd:2]
        else:
            z = x[ro:ro + half] + 1j * x[ro + half:ro + rd]
        zr = z * np.exp(1j * np.arange(P)[pos] * (10000.0 ** (-(2.0 * np.arange(half)) / rd)))
        if interleaved:
            want_re, want_im = y[ro:ro + rd:2], y[ro + 1:ro + rd:2]
        else:
            want_re, want_im = y[ro:ro + half], y[ro + half:ro + rd]
        np.testing.assert_allclose(want_re, zr.real, rtol=0, atol=1e-12)
        np.testing.assert_allclose(want_im, zr.imag, rtol=0, atol=1e-12)
        # channels outside the rotary range pass through
        assert np.array_equal(y[:ro], x[:ro]) and np.array_equal(y[ro + rd:], x[ro + rd:])


def test_rope_pos0_is_identity_and_relative_position():
    rng = np.random.default_rng(4)
    hs, ro, rd, P = 192, 128, 64, 300
    cos, sin = _exact_tables(P, rd)
    q, k = rng.standard_normal(hs), rng.standard_normal(hs)
    assert np.array_equal(orc.rope(q, 0, cos, sin, ro, rd, False), q)
    d0 = orc.rope(q, 50, cos, sin, ro, rd, False) @ orc.rope(k, 20, cos, sin, ro, rd, False)
    d1 = orc.rope(q, 250, cos, sin, ro, rd, False) @ orc.rope(k, 220, cos, sin, ro, rd, False)
    assert abs(d0 - d1) < 1e-10
    # norms of rotated pairs are preserved
    y = orc.rope(q, 123, cos, sin, ro, rd, False)
    h = rd // 2
    np.testing.assert_allclose(y[ro:ro + h] ** 2 + y[ro + h:ro + rd] ** 2,
                               q[ro:ro + h] ** 2 + q[ro + h:ro + rd] ** 2, rtol=1e-12)


# ----------------------------------------------------------------------------
# Dense contiguous reference built without paging
# ----------------------------------------------------------------------------

def _complex_rope(x, pos, ro, rd, theta=10000.0, tables=None):
    """Independent RoPE: rotate pairs (d, d + rd/2) as complex numbers, using the given
    (cos, sin) tables at row pos."""
    y = np.array(x, dtype=np.float64, copy=True)
    h = rd // 2
    c, s = tables[0][pos], tables[1][pos]
    z = x[..., ro:ro + h] + 1j * x[..., ro + h:ro + rd]
    zr = z * (c + 1j * s)
    y[..., ro:ro + h] = zr.real
    y[..., ro + h:ro + rd] = zr.imag
    return y


def _paged_from_contiguous(seqs_rows, new_counts, bs, rng, hs, spare=3):
    """Scatter per-sequence contiguous rows (16-bit patterns, position order)
    into a permuted block cache; returns cache, block_table, slot_mapping for
    the new tokens (the last new_counts[b] positions of each sequence)."""
    B = len(seqs_rows)
    nblk = [(len(r) + bs - 1) // bs for r in seqs_rows]
    MB = max(nblk)
    NB = sum(nblk) + spare
    phys = rng.permutation(NB)
    cache = rng.integers(0, 2**16, size=(NB * bs, hs), dtype=np.uint16)
    cache = (cache & 0x3BFF)   # finite junk
    bt = np.full((B, MB), -1, dtype=np.int32)
    slots = []
    k = 0
    for b, rows in enumerate(seqs_rows):
        for lb in range(nblk[b]):
            bt[b, lb] = phys[k]
            k += 1
        for j, row in enumerate(rows):
            cache[bt[b, j // bs] * bs + j % bs] = row
        ctx = len(rows)
        for j in range(ctx - new_counts[b], ctx):
            slots.append(bt[b, j // bs] * bs + j % bs)
    return cache.reshape(NB, bs, 1, hs), bt, np.array(slots, dtype=np.int32)


def _dense_case(rng, *, pasts, news, H, hs, vhs, rd, ro, bs, window=-1, do_rotary=True, has_scale=True):
    """Build a workload plus its dense contiguous expectation via torch SDPA.
    has_scale=False leaves the scale attribute absent and lets SDPA apply its
    own default (1/sqrt of the query width)."""
    dt = "f16"
    P = max(p + n for p, n in zip(pasts, news))
    tables = _exact_tables(P, rd) if do_rotary else None
    cos_bits = wl.f32_to_f16_bits(tables[0].astype(np.float32)) if do_rotary else np.zeros((0, 0), np.uint16)
    sin_bits = wl.f32_to_f16_bits(tables[1].astype(np.float32)) if do_rotary else np.zeros((0, 0), np.uint16)
    tabs16 = (orc.widen(cos_bits, dt), orc.widen(sin_bits, dt)) if do_rotary else None
    seqs_rows, keys, queries, expect = [], [], [], []
    for p, n in zip(pasts, news):
        past_rows = wl.f32_to_f16_bits(rng.standard_normal((p, hs)).astype(np.float32))
        new_keys = wl.f32_to_f16_bits(rng.standard_normal((n, hs)).astype(np.float32))
        q = wl.f32_to_f16_bits(rng.standard_normal((n, H * hs)).astype(np.float32))
        # rotated new rows, as the write phase must place them
        rot_rows = []
        for i in range(n):
            kv = orc.widen(new_keys[i], dt)
            if do_rotary:
                kv = _complex_rope(kv, p + i, ro, rd, tables=tabs16)
            rot_rows.append(kv.astype(np.float16).view(np.uint16))
        rows = np.concatenate([past_rows, np.array(rot_rows).reshape(n, hs)], axis=0)
        seqs_rows.append(rows)
        keys.append(new_keys)
        queries.append(q)
        # dense attention over contiguous rows
        K = torch.from_numpy(orc.widen(rows, dt))                       # [ctx, hs]
        qf = orc.widen(q, dt).reshape(n, H, hs)
        if do_rotary:
            qf = np.stack([_complex_rope(qf[i], p + i, ro, rd, tables=tabs16) for i in range(n)])
        Q = torch.from_numpy(qf).permute(1, 0, 2).unsqueeze(0)          # [1, H, n, hs]
        ctx = p + n
        qpos = torch.arange(p, p + n)[:, None]
        kpos = torch.arange(ctx)[None, :]
        mask = kpos <= qpos
        if window >= 0:
            mask &= (qpos - kpos) <= window
        o = F.scaled_dot_product_attention(Q, K[None, None].expand(1, H, ctx, hs),
                                           K[None, None, :, :vhs].expand(1, H, ctx, vhs),
                                           attn_mask=mask, scale=float(np.float32(0.125)) if has_scale else None)
        expect.append(o[0].permute(1, 0, 2).reshape(n, H * vhs).numpy())
    cache, bt, slots = _paged_from_contiguous(
        [np.concatenate([r[:p], np.zeros((n, hs), np.uint16)]) for r, p, n in zip(seqs_rows, pasts, news)],
        news, bs, rng, hs)
    T = sum(news)
    cum = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    w = dict(dtype=dt, attrs=dict(num_heads=H, head_size=hs, v_head_size=vhs, block_size=bs,
                                  do_rotary=int(do_rotary), rotary_interleaved=0,
                                  rotary_dim=rd if do_rotary else 0, rotary_offset=ro if do_rotary else 0,
                                  local_window_size=window, softcap=0.0, has_scale=int(has_scale),
                                  scale=0.125 if has_scale else 0.0),
             query=np.concatenate(queries).reshape(T, H * hs), key=np.concatenate(keys).reshape(T, hs),
             key_cache=cache, cos_cache=cos_bits, sin_cache=sin_bits,
             cumulative_sequence_length=cum, past_seqlens=np.array(pasts, np.int32),
             block_table=bt, slot_mapping=slots)
    return w, np.concatenate(expect), seqs_rows


@pytest.mark.parametrize("do_rotary", [True, False])
@pytest.mark.parametrize("window", [-1, 0, 5, 40])
def test_oracle_equals_dense_contiguous_attention(do_rotary, window):
    rng = np.random.default_rng(10 + window + 7 * do_rotary)
    w, expect, seqs_rows = _dense_case(rng, pasts=[0, 21, 3], news=[20, 16, 1], H=4, hs=64, vhs=32,
                                       rd=16, ro=48, bs=16, window=window, do_rotary=do_rotary)
    cache, out = orc.run(w)
    np.testing.assert_allclose(out, expect, rtol=0, atol=1e-10)
    # the written rows land where the dense layout says, bit for bit
    flat = cache.reshape(-1, 64)
    bt = w["block_table"]
    for b, rows in enumerate(seqs_rows):
        for j in range(len(rows)):
            assert np.array_equal(flat[bt[b, j // 16] * 16 + j % 16], rows[j])


@pytest.mark.parametrize("hs,atol", [(64, 1e-10), (48, 1e-6)])
def test_default_scale_equals_sdpa_default(hs, atol):
    """No explicit scale and v_head_size == head_size: the op's default
    1/sqrt(head_size) (docs.rs page, execute, scale rule) equals SDPA's own
    default scale. With head_size 64 both are exactly 1/8; with 48 the op forms
    the scale in float32, so the outputs agree to float32 rounding of the scale."""
    rng = np.random.default_rng(60 + hs)
    w, expect, _ = _dense_case(rng, pasts=[0, 21], news=[20, 5], H=3, hs=hs, vhs=hs, rd=16, ro=hs - 16,
                               bs=16, has_scale=False)
    assert orc.effective_scale(w["attrs"]) == float(np.float32(1.0) / np.sqrt(np.float32(hs)))
    _, out = orc.run(w)
    np.testing.assert_allclose(out, expect, rtol=0, atol=atol)


def test_default_scale_absent_with_narrow_values_is_rejected():
    a = dict(num_heads=1, head_size=64, v_head_size=32, has_scale=0, scale=0.0)
    with pytest.raises(ValueError):
        orc.effective_scale(a)
    # v_head_size 0 means head_size: the default applies
    assert orc.effective_scale(dict(a, v_head_size=0)) == 0.125


def test_first_token_output_is_its_own_value_row():
    """A fresh sequence's first token sees only itself: output = RN(V row) exactly
    (the review verdict of PR #1978 reports exactly zero error for the first GLM token)."""
    w = wl.make("c1")
    cache, out = orc.run(w)
    vhs, hs = w["attrs"]["v_head_size"], w["attrs"]["head_size"]
    slot0 = w["slot_mapping"][0]
    vrow = orc.widen(cache.reshape(-1, hs)[slot0, :vhs], "f16")
    for h in range(w["attrs"]["num_heads"]):
        assert np.array_equal(out[0, h * vhs:(h + 1) * vhs], vrow)


# ----------------------------------------------------------------------------
# Closed forms
# ----------------------------------------------------------------------------

def _small(rng, window=-1, softcap=0.0, scale=0.125, past=(5, 30), new=(3, 2)):
    spec = wl.Spec(name="t", dtype="f16", past=list(past), new=list(new), num_heads=3, head_size=32,
                   v_head_size=16, rotary_dim=16, rotary_offset=16, block_size=16, scale=scale,
                   softcap=softcap, local_window_size=window, seed=int(rng.integers(1 << 30)))
    return wl.build(spec)


def test_zero_query_gives_mean_of_visible_values():
    rng = np.random.default_rng(20)
    for window in (-1, 4):
        w = _small(rng, window=window)
        w["query"][:] = 0
        cache, out = orc.run(w)
        flat = orc.widen(cache.reshape(-1, 32), "f16")
        b_of, pos_of = orc.resolve_tokens(w["cumulative_sequence_length"], w["past_seqlens"])
        for t in range(out.shape[0]):
            b, pos = b_of[t], pos_of[t]
            js = [j for j in range(pos + 1) if window < 0 or pos - j <= window]
            rows = [w["block_table"][b, j // 16] * 16 + j % 16 for j in js]
            mean = flat[rows, :16].mean(axis=0)
            for h in range(3):
                np.testing.assert_allclose(out[t, h * 16:(h + 1) * 16], mean, rtol=0, atol=1e-12)


def test_window_zero_gives_own_row_and_large_window_is_no_window():
    rng = np.random.default_rng(21)
    w = _small(rng, window=0)
    cache, out = orc.run(w)
    flat = orc.widen(cache.reshape(-1, 32), "f16")
    for t in range(out.shape[0]):
        own = flat[w["slot_mapping"][t], :16]
        for h in range(3):
            assert np.array_equal(out[t, h * 16:(h + 1) * 16], own)
    w_big = _small(np.random.default_rng(22), window=10**6)
    w_off = _small(np.random.default_rng(22), window=-1)
    assert np.array_equal(orc.run(w_big)[1], orc.run(w_off)[1])


def test_softcap_saturated_closed_form_and_large_cap_is_off():
    # softcap -> infinity leaves scores unchanged (up to rounding)
    a = orc.run(_small(np.random.default_rng(23), softcap=1e9))[1]
    b = orc.run(_small(np.random.default_rng(23), softcap=0.0))[1]
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    # huge scale saturates tanh: s_j = +-c, so weights are e^{+c} / e^{-c} by sign of q.k
    c = 2.0
    w = _small(np.random.default_rng(24), softcap=c, scale=1e6)
    cache, out = orc.run(w)
    flat = orc.widen(cache.reshape(-1, 32), "f16")
    b_of, pos_of = orc.resolve_tokens(w["cumulative_sequence_length"], w["past_seqlens"])
    cos, sin = orc.widen(w["cos_cache"], "f16"), orc.widen(w["sin_cache"], "f16")
    for t in range(out.shape[0]):
        b, pos = b_of[t], pos_of[t]
        rows = flat[[w["block_table"][b, j // 16] * 16 + j % 16 for j in range(pos + 1)]]
        for h in range(3):
            q = _complex_rope(orc.widen(w["query"][t, h * 32:(h + 1) * 32], "f16"), pos, 16, 16, tables=(cos, sin))
            sgn = np.sign(rows @ q)
            if np.any(np.abs(rows @ q) * 1e6 < 40):
                continue     # tanh not saturated in float64 for this key
            wts = np.exp(c * sgn)
            want = (wts[:, None] * rows[:, :16]).sum(0) / wts.sum()
            np.testing.assert_allclose(out[t, h * 16:(h + 1) * 16], want, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# Invariants the pages state
# ----------------------------------------------------------------------------

def _permute_blocks(w, rng):
    """Move every physical block to a new place and rewrite block_table and
    slot_mapping consistently."""
    NB, bs = w["key_cache"].shape[0], w["key_cache"].shape[1]
    perm = rng.permutation(NB)
    w2 = dict(w)
    cache2 = np.empty_like(w["key_cache"])
    cache2[perm] = w["key_cache"]
    w2["key_cache"] = cache2
    bt = w["block_table"].copy()
    valid = bt >= 0
    bt[valid] = perm[bt[valid]]
    w2["block_table"] = bt
    s = w["slot_mapping"].copy()
    ok = s >= 0
    s[ok] = perm[s[ok] // bs] * bs + s[ok] % bs
    w2["slot_mapping"] = s
    return w2, perm


@pytest.mark.parametrize("cfg", ["c1", "c5small"])
def test_block_permutation_invariance_bit_identical(cfg):
    if cfg == "c1":
        w = wl.make("c1")
    else:
        w = wl.make("c5", scale_down=16)
    w2, perm = _permute_blocks(w, np.random.default_rng(30))
    c1, o1 = orc.run(w)
    c2, o2 = orc.run(w2)
    assert np.array_equal(o1, o2)
    assert np.array_equal(c2[perm], c1)


def test_slot_minus_one_suppresses_the_write():
    w = wl.make("c5", scale_down=16)
    before = w["key_cache"].reshape(-1, w["attrs"]["head_size"]).copy()
    after = orc.write_phase(w).reshape(before.shape)
    written = set(int(s) for s in w["slot_mapping"] if s >= 0)
    assert (w["slot_mapping"] < 0).sum() > 0
    changed = np.nonzero(np.any(after != before, axis=1))[0]
    assert set(changed.tolist()) <= written
    untouched = np.setdiff1d(np.arange(before.shape[0]), np.array(sorted(written)))
    assert np.array_equal(after[untouched], before[untouched])
    # the dropped tokens' own positions still hold the stale rows
    b_of, pos_of = orc.resolve_tokens(w["cumulative_sequence_length"], w["past_seqlens"])
    bs = w["attrs"]["block_size"]
    for t in np.nonzero(w["slot_mapping"] < 0)[0]:
        row = w["block_table"][b_of[t], pos_of[t] // bs] * bs + pos_of[t] % bs
        assert np.array_equal(after[row], before[row])


@pytest.mark.parametrize("dims", [(64, 16, 8, 16, 4), (576, 128, 128, 64, 4)])
def test_absorbed_latent_equals_decomposed_mla(dims):
    """Absorbed LATENT attention == decomposed multi-head latent attention.

    Latent row = [c (hs - rd); k_r (rd)], q_h = [q_n (d_n); q_r (rd)]. Decomposed
    head h: key [W_UK_h c; RoPE(k_r)], value W_UV_h c[:vhs], query [q_n; RoPE(q_r)].
    Absorbed: q_abs = [W_UK_h^T q_n; q_r] against the latent row, output
    W_UV_h out_h. Uses the DeepSeek-V3 latent split (512 + 64) at full width."""
    hs, d_n, d_v, rd, H = dims
    lat = hs - rd
    vhs = lat
    rng = np.random.default_rng(40)
    pasts, news = [7, 0], [3, 4]
    P = max(p + n for p, n in zip(pasts, news))
    cos, sin = _exact_tables(P, rd)
    W_UK = rng.standard_normal((H, d_n, lat)) / math.sqrt(lat)
    W_UV = rng.standard_normal((H, d_v, vhs)) / math.sqrt(vhs)
    scale = float(np.float32(1.0 / math.sqrt(d_n + rd)))   # the scale attribute is a float32
    # contiguous latent rows (already "written") and queries, in float64 via f16 patterns
    outs_dec, outs_abs = [], []
    for p, n in zip(pasts, news):
        ctx = p + n
        lat_rows = rng.standard_normal((ctx, hs))
        qn = rng.standard_normal((n, H, d_n))
        qr = rng.standard_normal((n, H, rd))
        # decomposed
        for i in range(n):
            pos = p + i
            o_dec = np.zeros((H, d_v))
            o_abs = np.zeros((H, d_v))
            for h in range(H):
                keys = np.concatenate([lat_rows[:pos + 1, :lat] @ W_UK[h].T,
                                       np.stack([_complex_rope(lat_rows[j], j, lat, rd, tables=(cos, sin))[lat:]
                                                 for j in range(pos + 1)])], axis=1)
                qrot = _complex_rope(np.concatenate([np.zeros(lat), qr[i, h]]), pos, lat, rd,
                                     tables=(cos, sin))[lat:]
                qd = np.concatenate([qn[i, h], qrot])
                s = scale * keys @ qd
                wts = np.exp(s - s.max()); wts /= wts.sum()
                vals = lat_rows[:pos + 1, :vhs] @ W_UV[h].T
                o_dec[h] = wts @ vals
            # absorbed, through the oracle: one latent cache row per position, RoPE'd
            wts_rows = np.stack([orc.rope(lat_rows[j], j, cos, sin, lat, rd, False) for j in range(pos + 1)])
            q_abs = np.concatenate([np.einsum("hdl,hd->hl", W_UK, qn[i]), qr[i]], axis=1)    # [H, hs]
            w = _single_token_workload(q_abs, wts_rows, pos, H, hs, vhs, rd, lat, scale, cos, sin)
            out = orc.attention(w, w["key_cache"])[0].reshape(H, vhs)
            for h in range(H):
                o_abs[h] = W_UV[h] @ out[h]
            outs_dec.append(o_dec)
            outs_abs.append(o_abs)
    np.testing.assert_allclose(np.array(outs_abs), np.array(outs_dec), rtol=1e-9, atol=1e-11)


def _single_token_workload(q_abs, rows_rotated, pos, H, hs, vhs, rd, ro, scale, cos, sin):
    """A one-token workload whose values are float64 (bypasses 16-bit storage by
    monkeypatching widen through a float64 'dtype')."""
    ctx = pos + 1
    bs = 16
    nblk = (ctx + bs - 1) // bs
    cache = np.zeros((nblk * bs, hs))
    cache[:ctx] = rows_rotated
    return dict(dtype="f64", attrs=dict(num_heads=H, head_size=hs, v_head_size=vhs, block_size=bs,
                                        do_rotary=1, rotary_interleaved=0, rotary_dim=rd, rotary_offset=ro,
                                        local_window_size=-1, softcap=0.0, has_scale=1, scale=scale),
                query=q_abs.reshape(1, H * hs), key=None, key_cache=cache,
                cos_cache=cos, sin_cache=sin, cumulative_sequence_length=np.array([0, 1]),
                past_seqlens=np.array([pos]), block_table=np.arange(nblk).reshape(1, nblk), slot_mapping=None)


# ----------------------------------------------------------------------------
# Split-KV merge
# ----------------------------------------------------------------------------

def test_combine_partials_equals_single_softmax():
    rng = np.random.default_rng(50)
    s = rng.standard_normal(100) * 3
    v = rng.standard_normal((100, 7))
    wts = np.exp(s - s.max())
    want = wts @ v / wts.sum()
    cuts = [0, 13, 14, 60, 100]
    ms, ls, accs = [], [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        m = s[a:b].max()
        e = np.exp(s[a:b] - m)
        ms.append(m); ls.append(e.sum()); accs.append(e @ v[a:b])
    ms.append(-np.inf); ls.append(0.0); accs.append(np.zeros(7))    # an empty split
    np.testing.assert_allclose(orc.combine_partials(np.array(ms), np.array(ls), np.array(accs)), want,
                               rtol=1e-12, atol=1e-14)


def test_generator_is_deterministic_and_consistent():
    a = wl.make("c5", scale_down=16)
    b = wl.make("c5", scale_down=16)
    for k in ("query", "key", "key_cache", "block_table", "slot_mapping", "cos_cache"):
        assert np.array_equal(a[k], b[k])
    # slots are unique among non-negative entries
    s = a["slot_mapping"][a["slot_mapping"] >= 0]
    assert len(np.unique(s)) == len(s)
