"""CPU oracle for PagedAttention in the SEPARATE cache layout (grouped-query attention).

TEST INFRASTRUCTURE. Only the tests, the smoke entry point and the benchmark's
CPU-baseline leg may import this module. The product path (the HIP library and
its Python binding) never calls it and shares no code with it.

What it computes is read off the pages:
  * PR #1940 "PagedAttention v1 audit and MLA oracle", second commit message:
    the oracle covers two dense modes over one block cache addressed by
    block_table / slot_mapping -- LATENT (the other module of this package)
    and SEPARATE: grouped-query attention with RoPE, softcap and a local
    window, a key cache and a separate value cache; it equals naive
    contiguous dense attention with partial RoPE and is invariant under a
    permuted block table, and slot -1 suppresses the write.
  * The same PR, third commit message: num_heads must be a multiple of
    kv_num_heads, otherwise a query head would address a key/value head that
    does not exist (rejection case 4/3, accepted cases 4/2 and 4/4).
  * PR #1978 "native PagedAttention LATENT kernel ...", review "Gates
    verified": schema input order query, key, value, key_cache, value_cache,
    ... -- SEPARATE is the layout that uses the value inputs.

Readings where the pages are silent (stated once here, applied below):
  * Query head h reads key/value head h // (num_heads / kv_num_heads): the
    num_heads / kv_num_heads query heads of a group are consecutive.
  * The same partial RoPE as the LATENT layout (channels [rotary_offset,
    rotary_offset + rotary_dim) of every query head and every key head, at
    the token's absolute position); value rows are stored unrotated.
  * Scale, softcap, window and the l = 0 rule are those of the LATENT layout.

Tensor shapes (16-bit patterns): query [T, H*hs], key [T, kvH*hs], value
[T, kvH*vhs], key_cache [NB, bs, kvH, hs], value_cache [NB, bs, kvH, vhs].

Precision as in the LATENT oracle: exact widening, float64 arithmetic,
round-to-nearest-even into the storage type.

Pins (tests/test_oracle_separate.py): torch scaled_dot_product_attention with
grouped heads (enable_gqa) on contiguous rows, the LATENT oracle at one KV head
with the value cache equal to the unrotated leading channels of the key cache,
a closed form of the head-group mapping, block-permutation invariance, slot -1
suppression of both writes, bit-exact value rows, and the ratio rule. No
function here is parity-unpinned.
"""
from __future__ import annotations

import numpy as np

from .paged_latent import effective_scale, resolve_tokens, rope, to_bits, widen


def check_heads(num_heads: int, kv_num_heads: int) -> int:
    """Query heads per key/value head; raises ValueError unless kv_num_heads >= 1
    divides num_heads (PR #1940, third commit)."""
    if kv_num_heads < 1 or num_heads < 1 or num_heads % kv_num_heads != 0:
        raise ValueError(f"num_heads ({num_heads}) must be a multiple of kv_num_heads ({kv_num_heads})")
    return num_heads // kv_num_heads


def write_phase(w: dict):
    """Return (key_cache, value_cache) bit patterns after the write phase.

    For each token t with slot_mapping[t] >= 0, in increasing t: every key head
    g of key[t] is rotated at pos(t) and stored at key_cache[slot, g]; every
    value head of value[t] is stored unchanged at value_cache[slot, g]."""
    a, dt = w["attrs"], w["dtype"]
    hs = a["head_size"]
    vhs = a["v_head_size"] or hs
    kvh = a["kv_num_heads"]
    check_heads(a["num_heads"], kvh)
    kc = np.array(w["key_cache"], dtype=np.uint16, copy=True)
    vc = np.array(w["value_cache"], dtype=np.uint16, copy=True)
    kflat = kc.reshape(-1, kvh, hs)
    vflat = vc.reshape(-1, kvh, vhs)
    _, pos_of = resolve_tokens(w["cumulative_sequence_length"], w["past_seqlens"])
    key = np.asarray(w["key"], dtype=np.uint16).reshape(-1, kvh, hs)
    value = np.asarray(w["value"], dtype=np.uint16).reshape(-1, kvh, vhs)
    rd = a["rotary_dim"] if a["do_rotary"] else 0
    ro = a["rotary_offset"]
    if rd:
        cos = widen(w["cos_cache"], dt)
        sin = widen(w["sin_cache"], dt)
        keep = np.ones(hs, dtype=bool)
        keep[ro:ro + rd] = False
    for t in range(key.shape[0]):
        slot = int(w["slot_mapping"][t])
        if slot < 0:
            continue
        for g in range(kvh):
            if rd:
                row = rope(widen(key[t, g], dt), int(pos_of[t]), cos, sin, ro, rd, bool(a["rotary_interleaved"]))
                bits = to_bits(row, dt)
                bits[keep] = key[t, g][keep]          # channels outside the rotary range: bit copies
                kflat[slot, g] = bits
            else:
                kflat[slot, g] = key[t, g]
            vflat[slot, g] = value[t, g]
    return kc, vc


def attention(w: dict, key_cache: np.ndarray, value_cache: np.ndarray, tokens=None) -> np.ndarray:
    """Attention output in float64, shape [T, num_heads * v_head_size].

    For token t and query head h in group g = h // (H / kvH): q = RoPE(query[t, h])
    at pos(t); visible keys j satisfy 0 <= j <= pos and (window < 0 or
    pos - j <= window); the cache row of j is block_table[b, j // bs] * bs + j % bs;
    s_j = scale * <q, key_cache[row_j, g]>, then softcap * tanh(s_j / softcap)
    when softcap > 0; weights exp(s_j - max s) / sum; output = sum of weights
    times value_cache[row_j, g]. `tokens` restricts the computation to a subset
    of token indices (rows not computed are NaN)."""
    a, dt = w["attrs"], w["dtype"]
    H, hs, bs = a["num_heads"], a["head_size"], a["block_size"]
    vhs = a["v_head_size"] or hs
    kvh = a["kv_num_heads"]
    grp = check_heads(H, kvh)
    win = a["local_window_size"]
    softcap = float(np.float32(a["softcap"]))
    scale = effective_scale(a)
    rd = a["rotary_dim"] if a["do_rotary"] else 0
    cos = widen(w["cos_cache"], dt) if rd else None
    sin = widen(w["sin_cache"], dt) if rd else None
    cumseq = np.asarray(w["cumulative_sequence_length"], dtype=np.int64)
    past = np.asarray(w["past_seqlens"], dtype=np.int64)
    bt = np.asarray(w["block_table"], dtype=np.int64)
    kflat = np.asarray(key_cache).reshape(-1, kvh, hs)
    vflat = np.asarray(value_cache).reshape(-1, kvh, vhs)
    query = np.asarray(w["query"])
    T = query.shape[0]
    out = np.full((T, H * vhs), np.nan, dtype=np.float64)
    want = np.ones(T, dtype=bool) if tokens is None else np.isin(np.arange(T), np.asarray(tokens))
    _, pos_of = resolve_tokens(cumseq, past)
    for b in range(past.size):
        t0, t1 = int(cumseq[b]), int(cumseq[b + 1])
        if t0 == t1 or not want[t0:t1].any():
            continue
        ctx = int(pos_of[t1 - 1]) + 1
        j = np.arange(ctx)
        rows = bt[b, j // bs] * bs + j % bs
        K = widen(kflat[rows], dt)                    # [ctx, kvH, hs], position order
        V = widen(vflat[rows], dt)                    # [ctx, kvH, vhs]
        for t in range(t0, t1):
            if not want[t]:
                continue
            pos = int(pos_of[t])
            lo = 0 if win < 0 else max(0, pos - win)
            q = widen(query[t].reshape(H, hs), dt)
            if rd:
                q = rope(q, pos, cos, sin, a["rotary_offset"], rd, bool(a["rotary_interleaved"]))
            o = np.empty((H, vhs), dtype=np.float64)
            for g in range(kvh):
                Kg = K[lo:pos + 1, g]                 # [n, hs]
                Vg = V[lo:pos + 1, g]                 # [n, vhs]
                s = scale * (q[g * grp:(g + 1) * grp] @ Kg.T)     # [grp, n]
                if softcap > 0:
                    s = softcap * np.tanh(s / softcap)
                m = s.max(axis=1, keepdims=True)      # pass 1: max
                e = np.exp(s - m)                     # pass 2: weights and sum
                l = e.sum(axis=1, keepdims=True)
                og = (e @ Vg) / l
                og[l[:, 0] == 0] = 0.0
                o[g * grp:(g + 1) * grp] = og
            out[t] = o.reshape(-1)
    return out


def run(w: dict, tokens=None):
    """Write phase, then read phase on the written caches.

    Returns (key cache bits, value cache bits, attention output float64)."""
    kc, vc = write_phase(w)
    return kc, vc, attention(w, kc, vc, tokens=tokens)
