"""CPU oracle for PagedAttention in the LATENT (absorbed multi-head latent attention) layout.

TEST INFRASTRUCTURE. Only the tests, the smoke entry point and the benchmark's
CPU-baseline leg may import this module. The product path (the HIP library and
its Python binding) never calls it and shares no code with it.

What it computes is read off the pages:
  * "onnx-runtime-ep-cuda src/kernels/paged_attention.rs" (docs.rs), module
    comment "LATENT semantics" and its device functions locate_token /
    rope_channel / write_impl / attn_impl: token -> (batch, position)
    resolution, partial RoPE on the [rotary_offset, rotary_offset+rotary_dim)
    suffix, scatter of the rotated key row to slot_mapping[t] (-1 skips),
    causal attention over the block_table-addressed prefix with
    local_window_size, scale then softcap, V = leading v_head_size channels of
    the same cached row, output 0 when the softmax denominator is 0.
  * PR #1940 "PagedAttention v1 audit and MLA oracle", second commit message:
    the oracle is dense attention over the block cache with a two-pass
    softmax; PR #1978 review verdict, "Gates verified": the kernel's online
    softmax is algebraically identical to that two-pass form.

Precision. Inputs arrive as raw 16-bit patterns (float16 or bfloat16). They
are widened exactly, and every step here runs in float64 (the pages' own
oracle is float32; float64 is used so the reference carries no rounding of its
own). Results stored in the 16-bit type are rounded to nearest, ties to even,
directly from float64 (the pages' kernel rounds with __float2half_rn /
__float2bfloat16_rn).

Pins (tests/test_oracle.py): each function here is checked against facts the
pages or mathematics fix -- library float16 rounding, a dense causal attention
built without paging through torch's scaled_dot_product_attention, the
absorbed == decomposed MLA identity, RoPE's rotation/relative-position
identities, block-permutation invariance, slot -1 suppression, closed forms
for q = 0, window 0 and softcap. No function here is parity-unpinned.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# 16-bit storage types
# ---------------------------------------------------------------------------

# (significand bits incl. the leading one, min normal exponent, max finite value)
_FORMATS = {
    "f16": (11, -14, 65504.0),
    "bf16": (8, -126, float(np.float32(3.3895313892515355e38))),
}


def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of 16-bit patterns to float64 ("f64": values already float64,
    used by the mathematical pins)."""
    if dtype == "f64":
        return np.asarray(bits, dtype=np.float64)
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the 16-bit type, nearest with ties to even.

    Returns the rounded values as float64 (exactly representable in `dtype`).
    Written from the definition: the quantum at x is 2^(e - p) where 2^e <= |x|
    < 2^(e+1) (clamped at the subnormal range), p+1 the significand width."""
    p, emin, fmax = _FORMATS[dtype]
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    finite = np.isfinite(x)
    out[~finite] = x[~finite]
    xf = x[finite]
    mag = np.abs(xf)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(mag > 0, mag, 1.0)))
    # log2 can be off by one at exact powers of two boundaries: fix up exactly.
    e = np.where(np.ldexp(1.0, e.astype(np.int64)) > mag, e - 1, e)
    e = np.where(np.ldexp(1.0, (e + 1).astype(np.int64)) <= mag, e + 1, e)
    e = np.maximum(e, emin)
    q = np.ldexp(1.0, (e - (p - 1)).astype(np.int64))
    r = np.rint(xf / q) * q            # np.rint rounds half to even; xf/q is exact
    half_ulp_top = fmax + np.ldexp(1.0, int(np.floor(np.log2(fmax))) - p)
    r = np.where(np.abs(xf) >= half_ulp_top, np.copysign(np.inf, xf), r)
    out[finite] = r
    return out


def to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 to the 16-bit type and return its bit patterns."""
    r = round_to(x, dtype)
    if dtype == "f16":
        return r.astype(np.float16).view(np.uint16)      # exact: r is representable
    f32 = r.astype(np.float32)                           # exact: r is representable
    return (f32.view(np.uint32) >> 16).astype(np.uint16)


# ---------------------------------------------------------------------------
# Token resolution (locate_token on the docs.rs page)
# ---------------------------------------------------------------------------

def resolve_tokens(cumseq: np.ndarray, past: np.ndarray):
    """For each new token t: batch b(t) = first i with t < cumseq[i+1], and
    absolute position pos(t) = past[b] + t - cumseq[b]."""
    cumseq = np.asarray(cumseq, dtype=np.int64)
    past = np.asarray(past, dtype=np.int64)
    T = int(cumseq[-1])
    assert cumseq[0] == 0 and np.all(np.diff(cumseq) >= 0), "cumseq must start at 0 and be monotone"
    b_of = np.empty(T, dtype=np.int64)
    pos_of = np.empty(T, dtype=np.int64)
    for t in range(T):
        b = 0
        for i in range(past.size):
            if t < cumseq[i + 1]:
                b = i
                break
        b_of[t] = b
        pos_of[t] = past[b] + t - cumseq[b]
    return b_of, pos_of


# ---------------------------------------------------------------------------
# Partial RoPE (rope_channel on the docs.rs page)
# ---------------------------------------------------------------------------

def rope(x: np.ndarray, pos: int, cos: np.ndarray, sin: np.ndarray, rotary_offset: int,
         rotary_dim: int, interleaved: bool) -> np.ndarray:
    """Rotate channels [rotary_offset, rotary_offset + rotary_dim) of the last
    axis of `x` (float64) at absolute position `pos`; other channels pass
    through. cos/sin are float64 tables of shape [P, rotary_dim/2].

    Non-interleaved: channel d with r = d - offset < half pairs with d + half
    and takes x[d] c_r - x[d+half] s_r; with r >= half it pairs with d - half
    and takes x[d] c_{r-half} + x[d-half] s_{r-half}. Interleaved: i = r // 2,
    even r takes x[d] c_i - x[d+1] s_i, odd r takes x[d] c_i + x[d-1] s_i.
    Every output reads the unrotated input."""
    y = np.array(x, dtype=np.float64, copy=True)
    if rotary_dim == 0:
        return y
    half = rotary_dim // 2
    c = cos[pos]
    s = sin[pos]
    o = rotary_offset
    src = np.asarray(x, dtype=np.float64)
    if interleaved:
        ev = src[..., o:o + rotary_dim:2]
        od = src[..., o + 1:o + rotary_dim:2]
        y[..., o:o + rotary_dim:2] = ev * c - od * s
        y[..., o + 1:o + rotary_dim:2] = od * c + ev * s
    else:
        lo = src[..., o:o + half]
        hi = src[..., o + half:o + rotary_dim]
        y[..., o:o + half] = lo * c - hi * s
        y[..., o + half:o + rotary_dim] = hi * c + lo * s
    return y


# ---------------------------------------------------------------------------
# Write phase (write_impl on the docs.rs page)
# ---------------------------------------------------------------------------

def write_phase(w: dict) -> np.ndarray:
    """Return the key cache (16-bit patterns) after the write phase.

    Tokens are applied in increasing order; slot -1 skips the write. With
    do_rotary = 0 the row is copied unchanged."""
    a, dt = w["attrs"], w["dtype"]
    hs = a["head_size"]
    cache = np.array(w["key_cache"], dtype=np.uint16, copy=True)
    flat = cache.reshape(-1, hs)
    b_of, pos_of = resolve_tokens(w["cumulative_sequence_length"], w["past_seqlens"])
    key = np.asarray(w["key"], dtype=np.uint16)
    rd = a["rotary_dim"] if a["do_rotary"] else 0
    if rd:
        cos = widen(w["cos_cache"], dt)
        sin = widen(w["sin_cache"], dt)
    for t in range(key.shape[0]):
        slot = int(w["slot_mapping"][t])
        if slot < 0:
            continue
        if rd:
            row = rope(widen(key[t], dt), int(pos_of[t]), cos, sin, a["rotary_offset"], rd,
                       bool(a["rotary_interleaved"]))
            bits = to_bits(row, dt)
            # Channels outside the rotary range are copied, bit for bit.
            keep = np.ones(hs, dtype=bool)
            keep[a["rotary_offset"]:a["rotary_offset"] + rd] = False
            bits[keep] = key[t][keep]
            flat[slot] = bits
        else:
            flat[slot] = key[t]
    return cache


# ---------------------------------------------------------------------------
# Read phase (attn_impl on the docs.rs page; two-pass softmax per PR #1940)
# ---------------------------------------------------------------------------

def effective_scale(a: dict) -> float:
    """Explicit scale, else 1/sqrt(head_size) when v_head_size == head_size."""
    hs = a["head_size"]
    vhs = a["v_head_size"] or hs
    if a.get("has_scale"):
        return float(np.float32(a["scale"]))
    if vhs != hs:
        raise ValueError("explicit scale required when v_head_size != head_size")
    return float(np.float32(1.0) / np.sqrt(np.float32(hs)))


def attention(w: dict, cache_bits: np.ndarray, tokens=None) -> np.ndarray:
    """Attention output in float64, shape [T, num_heads * v_head_size].

    For each token t and head h: q = RoPE(query[t, h]) at pos(t); visible keys
    j satisfy 0 <= j <= pos and (window < 0 or pos - j <= window); row_j is
    cache row block_table[b, j // bs] * bs + j % bs; s_j = scale * <q, row_j>,
    then softcap * tanh(s_j / softcap) when softcap > 0; weights
    exp(s_j - max s) / sum; output = sum of weights times row_j[:v_head_size].
    `tokens` restricts the computation to a subset of token indices (rows not
    computed are NaN)."""
    a, dt = w["attrs"], w["dtype"]
    H, hs, bs = a["num_heads"], a["head_size"], a["block_size"]
    vhs = a["v_head_size"] or hs
    win = a["local_window_size"]
    softcap = float(np.float32(a["softcap"]))
    scale = effective_scale(a)
    rd = a["rotary_dim"] if a["do_rotary"] else 0
    cos = widen(w["cos_cache"], dt) if rd else None
    sin = widen(w["sin_cache"], dt) if rd else None
    cumseq = np.asarray(w["cumulative_sequence_length"], dtype=np.int64)
    past = np.asarray(w["past_seqlens"], dtype=np.int64)
    bt = np.asarray(w["block_table"], dtype=np.int64)
    flat = np.asarray(cache_bits).reshape(-1, hs)
    query = np.asarray(w["query"])
    T = query.shape[0]
    out = np.full((T, H * vhs), np.nan, dtype=np.float64)
    want = np.ones(T, dtype=bool) if tokens is None else np.isin(np.arange(T), np.asarray(tokens))
    b_of, pos_of = resolve_tokens(cumseq, past)
    for b in range(past.size):
        t0, t1 = int(cumseq[b]), int(cumseq[b + 1])
        if t0 == t1 or not want[t0:t1].any():
            continue
        ctx = int(pos_of[t1 - 1]) + 1
        j = np.arange(ctx)
        rows = bt[b, j // bs] * bs + j % bs
        K = widen(flat[rows], dt)                     # [ctx, hs], position order
        for t in range(t0, t1):
            if not want[t]:
                continue
            pos = int(pos_of[t])
            lo = 0 if win < 0 else max(0, pos - win)
            Kv = K[lo:pos + 1]
            q = widen(query[t].reshape(H, hs), dt)
            if rd:
                q = rope(q, pos, cos, sin, a["rotary_offset"], rd, bool(a["rotary_interleaved"]))
            s = scale * (q @ Kv.T)                    # [H, n]
            if softcap > 0:
                s = softcap * np.tanh(s / softcap)
            m = s.max(axis=1, keepdims=True)          # pass 1: max
            e = np.exp(s - m)                         # pass 2: weights and sum
            l = e.sum(axis=1, keepdims=True)
            o = (e @ Kv[:, :vhs]) / l
            o[l[:, 0] == 0] = 0.0
            out[t] = o.reshape(-1)
    return out


def run(w: dict, tokens=None):
    """Write phase, then read phase on the written cache.

    Returns (cache bits after the write, attention output float64)."""
    cache = write_phase(w)
    return cache, attention(w, cache, tokens=tokens)


# ---------------------------------------------------------------------------
# Split-KV partial combination (log-sum-exp merge)
# ---------------------------------------------------------------------------

def combine_partials(ms: np.ndarray, ls: np.ndarray, accs: np.ndarray) -> np.ndarray:
    """Merge softmax partials over disjoint key sets.

    Partial i holds m_i = max score, l_i = sum exp(s - m_i) and
    acc_i = sum exp(s - m_i) v (unnormalised). With m = max m_i and
    w_i = exp(m_i - m) (0 for an empty partial, m_i = -inf), the result is
    sum w_i acc_i / sum w_i l_i -- the same value a single softmax over the
    union of the key sets gives."""
    ms = np.asarray(ms, dtype=np.float64)
    m = ms.max()
    wts = np.where(np.isneginf(ms), 0.0, np.exp(ms - m))
    den = (wts * np.asarray(ls, dtype=np.float64)).sum()
    num = (wts[:, None] * np.asarray(accs, dtype=np.float64)).sum(axis=0)
    return num / den if den > 0 else np.zeros_like(num)
