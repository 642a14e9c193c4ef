"""Pins for the SEPARATE-layout (grouped-query) CPU oracle.

Each test checks the oracle against something other than itself: torch's
scaled_dot_product_attention with grouped heads (enable_gqa) on contiguous
rows, the LATENT oracle (pinned on its own in test_oracle.py) where the two
layouts coincide, a closed form of the head-group mapping, invariants PR #1940
states for its SEPARATE oracle (equality with naive contiguous dense attention
with partial RoPE, block-table permutation invariance, slot -1 write
suppression) and the kv-head ratio rule of its third commit.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import paged_latent as orc
from oracle import paged_separate as sep
from paged_absorbed_mla_amd import workloads as wl


def _tables(P, rd, theta=10000.0):
    half = rd // 2
    inv = theta ** (-(2.0 * np.arange(half)) / rd)
    ang = np.arange(P)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def _complex_rope(x, pos, ro, rd, tables):
    """RoPE of pairs (d, d + rd/2) as a complex multiplication (independent of the oracle's rope)."""
    y = np.array(x, dtype=np.float64, copy=True)
    h = rd // 2
    c, s = tables[0][pos], tables[1][pos]
    z = x[..., ro:ro + h] + 1j * x[..., ro + h:ro + rd]
    zr = z * (c + 1j * s)
    y[..., ro:ro + h] = zr.real
    y[..., ro + h:ro + rd] = zr.imag
    return y


def _f16(x):
    return wl.f32_to_f16_bits(np.asarray(x, dtype=np.float32))


def _gqa_case(rng, *, pasts, news, H, kvh, hs, vhs, rd, ro, bs, window=-1, softcap=0.0, do_rotary=True):
    """A paged SEPARATE workload and its dense expectation (torch SDPA with
    enable_gqa on contiguous rows gathered in position order)."""
    dt = "f16"
    P = max(p + n for p, n in zip(pasts, news))
    tab = _tables(P, rd)
    cos_bits, sin_bits = _f16(tab[0]), _f16(tab[1])
    tabs16 = (orc.widen(cos_bits, dt), orc.widen(sin_bits, dt))
    scale = 0.125
    krows_all, vrows_all, keys, values, queries, expect = [], [], [], [], [], []
    for p, n in zip(pasts, news):
        kpast = _f16(rng.standard_normal((p, kvh, hs)))
        vpast = _f16(rng.standard_normal((p, kvh, vhs)))
        knew = _f16(rng.standard_normal((n, kvh, hs)))
        vnew = _f16(rng.standard_normal((n, kvh, vhs)))
        q = _f16(rng.standard_normal((n, H * hs)))
        krot = np.empty_like(knew)
        for i in range(n):
            kv = orc.widen(knew[i], dt)
            if do_rotary:
                kv = _complex_rope(kv, p + i, ro, rd, tabs16)
            krot[i] = kv.astype(np.float16).view(np.uint16)
        krows = np.concatenate([kpast, krot])            # [ctx, kvh, hs] as the cache must hold them
        vrows = np.concatenate([vpast, vnew])
        krows_all.append(krows)
        vrows_all.append(vrows)
        keys.append(knew.reshape(n, kvh * hs))
        values.append(vnew.reshape(n, kvh * vhs))
        queries.append(q)
        qf = orc.widen(q, dt).reshape(n, H, hs)
        if do_rotary:
            qf = np.stack([_complex_rope(qf[i], p + i, ro, rd, tabs16) for i in range(n)])
        Q = torch.from_numpy(qf).permute(1, 0, 2).unsqueeze(0)                       # [1, H, n, hs]
        K = torch.from_numpy(orc.widen(krows, dt)).permute(1, 0, 2).unsqueeze(0)     # [1, kvh, ctx, hs]
        V = torch.from_numpy(orc.widen(vrows, dt)).permute(1, 0, 2).unsqueeze(0)
        ctx = p + n
        qpos = torch.arange(p, p + n)[:, None]
        kpos = torch.arange(ctx)[None, :]
        mask = kpos <= qpos
        if window >= 0:
            mask &= (qpos - kpos) <= window
        if softcap > 0:
            # softcap changes the scores before the softmax: form them explicitly
            Kx = K.repeat_interleave(H // kvh, dim=1)
            Vx = V.repeat_interleave(H // kvh, dim=1)
            s = (Q @ Kx.transpose(-1, -2)) * scale
            s = softcap * torch.tanh(s / softcap)
            s = s.masked_fill(~mask, float("-inf"))
            o = torch.softmax(s, dim=-1) @ Vx
        else:
            o = F.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=scale, enable_gqa=True)
        expect.append(o[0].permute(1, 0, 2).reshape(n, H * vhs).numpy())
    # Paged caches: permuted blocks, junk in every row the new tokens overwrite
    B = len(pasts)
    nblk = [(p + n + bs - 1) // bs for p, n in zip(pasts, news)]
    MB, NB = max(nblk), sum(nblk) + 3
    phys = rng.permutation(NB)
    kc = (rng.integers(0, 2**16, size=(NB * bs, kvh, hs), dtype=np.uint16) & 0x3BFF).astype(np.uint16)
    vc = (rng.integers(0, 2**16, size=(NB * bs, kvh, vhs), dtype=np.uint16) & 0x3BFF).astype(np.uint16)
    bt = np.full((B, MB), -1, dtype=np.int32)
    slots = []
    k = 0
    for b, (p, n) in enumerate(zip(pasts, news)):
        for lb in range(nblk[b]):
            bt[b, lb] = phys[k]
            k += 1
        for j in range(p):
            kc[bt[b, j // bs] * bs + j % bs] = krows_all[b][j]
            vc[bt[b, j // bs] * bs + j % bs] = vrows_all[b][j]
        for j in range(p, p + n):
            slots.append(bt[b, j // bs] * bs + j % bs)
    T = sum(news)
    cum = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    w = dict(dtype=dt,
             attrs=dict(num_heads=H, head_size=hs, v_head_size=vhs, block_size=bs, do_rotary=int(do_rotary),
                        rotary_interleaved=0, rotary_dim=rd if do_rotary else 0,
                        rotary_offset=ro if do_rotary else 0, local_window_size=window, softcap=softcap,
                        has_scale=1, scale=scale, kv_cache_layout="SEPARATE", kv_num_heads=kvh),
             query=np.concatenate(queries).reshape(T, H * hs), key=np.concatenate(keys),
             value=np.concatenate(values), key_cache=kc.reshape(NB, bs, kvh, hs),
             value_cache=vc.reshape(NB, bs, kvh, vhs), cos_cache=cos_bits, sin_cache=sin_bits,
             cumulative_sequence_length=cum, past_seqlens=np.array(pasts, np.int32),
             block_table=bt, slot_mapping=np.array(slots, dtype=np.int32))
    return w, np.concatenate(expect), krows_all, vrows_all


@pytest.mark.parametrize("H,kvh", [(4, 2), (4, 4), (6, 1), (8, 2)])
@pytest.mark.parametrize("window,do_rotary", [(-1, True), (5, True), (-1, False)])
def test_separate_equals_dense_gqa_sdpa(H, kvh, window, do_rotary):
    rng = np.random.default_rng(100 + 7 * H + kvh + window)
    w, expect, krows, vrows = _gqa_case(rng, pasts=[0, 21, 3], news=[20, 16, 1], H=H, kvh=kvh, hs=64,
                                        vhs=48, rd=32, ro=16, bs=16, window=window, do_rotary=do_rotary)
    kc, vc, out = sep.run(w)
    np.testing.assert_allclose(out, expect, rtol=0, atol=1e-10)
    # every row of every sequence sits where the dense layout says, bit for bit
    kflat, vflat = kc.reshape(-1, kvh, 64), vc.reshape(-1, kvh, 48)
    bt = w["block_table"]
    for b in range(len(krows)):
        for j in range(len(krows[b])):
            r = bt[b, j // 16] * 16 + j % 16
            assert np.array_equal(kflat[r], krows[b][j])
            assert np.array_equal(vflat[r], vrows[b][j])


def test_separate_softcap_equals_dense_gqa():
    rng = np.random.default_rng(140)
    w, expect, _, _ = _gqa_case(rng, pasts=[5, 30], news=[9, 2], H=4, kvh=2, hs=64, vhs=64, rd=16, ro=0,
                                bs=16, softcap=0.5)
    _, _, out = sep.run(w)
    np.testing.assert_allclose(out, expect, rtol=0, atol=1e-10)


def test_one_kv_head_equals_latent_when_values_are_the_unrotated_lead():
    """kv_num_heads = 1, value rows = the leading v_head_size channels of the key
    rows and a rotary range that starts at or after v_head_size: the SEPARATE
    result equals the LATENT result on the same cache (whose V is that lead)."""
    w = wl.make("c1")
    a = w["attrs"]
    hs, vhs = a["head_size"], a["v_head_size"]
    assert a["rotary_offset"] >= vhs
    ws = dict(w, attrs=dict(a, kv_cache_layout="SEPARATE", kv_num_heads=1),
              value=np.ascontiguousarray(w["key"][:, :vhs]),
              value_cache=np.ascontiguousarray(w["key_cache"][..., :vhs]))
    kc_l, out_l = orc.run(w)
    kc_s, vc_s, out_s = sep.run(ws)
    assert np.array_equal(kc_s, kc_l)
    assert np.array_equal(vc_s, kc_l[..., :vhs])
    np.testing.assert_allclose(out_s, out_l, rtol=0, atol=1e-12)


def test_head_groups_read_their_own_kv_head():
    """Closed form: with value head g's rows all equal to g + 1, query head h
    outputs 1 + h // (H / kvH) whatever the scores (up to float64 rounding of
    the weighted sum)."""
    w = wl.make("gqa_tiny")
    a = w["attrs"]
    H, kvh, vhs = a["num_heads"], a["kv_num_heads"], a["v_head_size"]
    vc = np.empty_like(w["value_cache"])
    val = np.empty_like(w["value"]).reshape(-1, kvh, vhs)
    for g in range(kvh):
        vc[:, :, g, :] = _f16(np.full(1, g + 1.0))[0]
        val[:, g, :] = _f16(np.full(1, g + 1.0))[0]
    w = dict(w, value_cache=vc, value=val.reshape(w["value"].shape))
    _, _, out = sep.run(w)
    out = out.reshape(out.shape[0], H, vhs)
    for h in range(H):
        np.testing.assert_allclose(out[:, h, :], 1.0 + h // (H // kvh), rtol=0, atol=1e-13)


@pytest.mark.parametrize("H,kvh,ok", [(4, 3, False), (4, 2, True), (4, 4, True), (4, 0, False), (4, 8, False)])
def test_kv_head_ratio_rule(H, kvh, ok):
    if ok:
        assert sep.check_heads(H, kvh) == H // kvh
    else:
        with pytest.raises(ValueError):
            sep.check_heads(H, kvh)


def _permute(w, rng):
    NB = w["key_cache"].shape[0]
    perm = rng.permutation(NB)           # new id of old block
    kc = np.empty_like(w["key_cache"])
    vc = np.empty_like(w["value_cache"])
    kc[perm] = w["key_cache"]
    vc[perm] = w["value_cache"]
    bt = w["block_table"].copy()
    used = bt >= 0
    bt[used] = perm[bt[used]]
    bs = w["attrs"]["block_size"]
    sl = w["slot_mapping"].copy()
    ok = sl >= 0
    sl[ok] = perm[sl[ok] // bs] * bs + sl[ok] % bs
    return dict(w, key_cache=kc, value_cache=vc, block_table=bt, slot_mapping=sl), perm


def test_block_permutation_invariance_bit_identical():
    w = wl.make("gqa_prefill", scale_down=32)
    w2, perm = _permute(w, np.random.default_rng(31))
    kc1, vc1, o1 = sep.run(w)
    kc2, vc2, o2 = sep.run(w2)
    assert np.array_equal(o1, o2)
    assert np.array_equal(kc2[perm], kc1)
    assert np.array_equal(vc2[perm], vc1)


def test_slot_minus_one_suppresses_both_writes_and_values_are_copied():
    w = wl.make("gqa_tiny")
    drop = np.array([3, 17, 30])
    w["slot_mapping"][drop] = -1
    a = w["attrs"]
    kvh, hs, vhs = a["kv_num_heads"], a["head_size"], a["v_head_size"]
    kb = w["key_cache"].reshape(-1, kvh, hs).copy()
    vb = w["value_cache"].reshape(-1, kvh, vhs).copy()
    kc, vc = sep.write_phase(w)
    kc, vc = kc.reshape(kb.shape), vc.reshape(vb.shape)
    written = [int(s) for s in w["slot_mapping"] if s >= 0]
    untouched = np.setdiff1d(np.arange(kb.shape[0]), written)
    assert np.array_equal(kc[untouched], kb[untouched])
    assert np.array_equal(vc[untouched], vb[untouched])
    # value rows land unrotated, bit for bit; key channels outside the rotary range too
    val = w["value"].reshape(-1, kvh, vhs)
    key = w["key"].reshape(-1, kvh, hs)
    ro, rd = a["rotary_offset"], a["rotary_dim"]
    for t, s in enumerate(w["slot_mapping"]):
        if s < 0:
            continue
        assert np.array_equal(vc[s], val[t])
        assert np.array_equal(kc[s][:, ro + rd:], key[t][:, ro + rd:])
        assert np.array_equal(kc[s][:, :ro], key[t][:, :ro])
