"""Seeded synthetic inputs for paged absorbed-MLA attention.

This module builds the inputs of one PagedAttention call in the LATENT cache
layout: query, new latent key rows, the paged block cache, the cos/sin tables
and the int32 index tensors (cumulative_sequence_length, past_seqlens,
block_table, slot_mapping). It holds none of the method's arithmetic: no RoPE,
no attention, no cache write. Both the HIP path and the CPU oracle consume what
it returns, as raw 16-bit patterns, so they see the same bytes.

Index tensors follow the KV-authority emission described on the page
"token-major/LATENT PagedAttention index emission (slice 3A.1)" (section "What
it adds"): block_table holds the physical block id per logical block, padded;
slot_mapping[t] = block_id * block_size + offset for the token's absolute
position; past_seqlens counts only the past (context minus new tokens). The
pad value of block_table is not printed there; -1 is used.

Values are drawn in float32 with numpy's default_rng and rounded to the storage
type with round-to-nearest-even. The cos/sin tables use the standard RoPE
frequencies theta^(-2i/rotary_dim), computed in float64, rounded to float32 and
then to the storage type.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, asdict
from typing import List, Optional

import numpy as np

F16_NAN_BITS = 0x7E00
BF16_NAN_BITS = 0x7FC0


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (ties to even); returns uint16 patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    if nan.any():
        out[nan] = BF16_NAN_BITS
    return out


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def to_storage_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f16":
        return f32_to_f16_bits(x)
    raise ValueError(f"unknown storage dtype {dtype!r}")


@dataclass
class Spec:
    """Geometry and value recipe of one workload."""
    name: str
    dtype: str                      # "f16" or "bf16"
    past: List[int]                 # past length per sequence
    new: List[int]                  # new tokens per sequence
    num_heads: int
    head_size: int
    v_head_size: int
    rotary_dim: int
    rotary_offset: int
    block_size: int
    scale: float
    has_scale: int = 1              # 0: no explicit scale (the op's default applies)
    softcap: float = 0.0
    local_window_size: int = -1
    do_rotary: int = 1
    rotary_interleaved: int = 0
    q_std: float = 1.0
    key_std: float = 1.0
    cache_std: float = 1.0
    theta: float = 10000.0
    slot_drop_frac: float = 0.0     # fraction of slot_mapping entries set to -1
    spare_blocks: int = 8
    permute_blocks: bool = True
    seed: int = 0
    layout: str = "LATENT"          # "LATENT" (one latent row per slot) or "SEPARATE" (GQA)
    kv_num_heads: int = 1           # SEPARATE: key/value heads (num_heads is a multiple)


# The five workloads. Sequence lengths that are drawn at random are drawn by
# `draw_lengths` from the seed, so a Spec built here holds placeholders.
def _tiny(seed: int = 0) -> Spec:
    return Spec(name="tiny_64_32_16_prefill_decode", dtype="f16", past=[0, 21], new=[20, 16],
                num_heads=4, head_size=64, v_head_size=32, rotary_dim=16, rotary_offset=48,
                block_size=16, scale=1.0 / 8.0, seed=seed)


def _glm_decode(seed: int = 1) -> Spec:
    return Spec(name="glm_192_128_64_decode", dtype="bf16", past=[], new=[],
                num_heads=16, head_size=192, v_head_size=128, rotary_dim=64, rotary_offset=128,
                block_size=64, scale=1.0 / math.sqrt(192.0), seed=seed)


def _glm_prefill(seed: int = 2) -> Spec:
    return Spec(name="glm_192_128_64_chunked_prefill", dtype="f16", past=[0, 512, 1024, 2048],
                new=[1024] * 4, num_heads=16, head_size=192, v_head_size=128, rotary_dim=64,
                rotary_offset=128, block_size=16, scale=1.0 / math.sqrt(192.0), seed=seed)


def _dsv3_decode(seed: int = 3) -> Spec:
    return Spec(name="dsv3_576_512_64_decode", dtype="bf16", past=[], new=[],
                num_heads=128, head_size=576, v_head_size=512, rotary_dim=64, rotary_offset=512,
                block_size=64, scale=1.0 / math.sqrt(192.0), q_std=0.5, key_std=0.5,
                cache_std=0.5, seed=seed)


def _mixed(seed: int = 4) -> Spec:
    return Spec(name="mixed_576_512_64_window_softcap", dtype="f16", past=[], new=[],
                num_heads=16, head_size=576, v_head_size=512, rotary_dim=64, rotary_offset=512,
                block_size=16, scale=1.0 / math.sqrt(192.0), softcap=50.0,
                local_window_size=1024, slot_drop_frac=0.05, seed=seed)


# Grouped-query (SEPARATE layout) workloads: per-head key and value caches,
# kv_num_heads key/value heads shared by groups of num_heads / kv_num_heads
# query heads, full-width RoPE at offset 0. Llama-style 128-wide heads.
def _gqa_tiny(seed: int = 5) -> Spec:
    return Spec(name="gqa_tiny_64_64_32_prefill_decode", dtype="f16", past=[0, 21], new=[20, 16],
                num_heads=4, head_size=64, v_head_size=64, rotary_dim=32, rotary_offset=0,
                block_size=16, scale=0.0, has_scale=0, seed=seed, layout="SEPARATE", kv_num_heads=2)


def _gqa_decode(seed: int = 6) -> Spec:
    return Spec(name="gqa_128_decode", dtype="bf16", past=[], new=[],
                num_heads=32, head_size=128, v_head_size=128, rotary_dim=128, rotary_offset=0,
                block_size=16, scale=1.0 / math.sqrt(128.0), seed=seed, layout="SEPARATE", kv_num_heads=8)


def _gqa_prefill(seed: int = 7) -> Spec:
    return Spec(name="gqa_128_chunked_prefill", dtype="f16", past=[0, 512, 1024, 2048], new=[1024] * 4,
                num_heads=32, head_size=128, v_head_size=128, rotary_dim=128, rotary_offset=0,
                block_size=16, scale=1.0 / math.sqrt(128.0), seed=seed, layout="SEPARATE", kv_num_heads=8)


CONFIGS = {
    "c1": _tiny,
    "c2": _glm_decode,
    "c3": _glm_prefill,
    "c4": _dsv3_decode,
    "c5": _mixed,
    "gqa_tiny": _gqa_tiny,
    "gqa_decode": _gqa_decode,
    "gqa_prefill": _gqa_prefill,
}


def draw_lengths(cfg: str, spec: Spec, rng: np.random.Generator, scale_down: int = 1) -> None:
    """Fill spec.past/new for the configs whose lengths are random.

    `scale_down` > 1 divides the drawn lengths and the sequence count, giving a
    smaller input with the same structure (used where the CPU oracle must
    finish in seconds)."""
    if cfg in ("c2", "gqa_decode"):
        n = max(1, 32 // scale_down)
        spec.past = [int(x) for x in rng.integers(512 // scale_down, 4096 // scale_down, size=n, endpoint=True)]
        spec.new = [1] * n
    elif cfg == "c4":
        n = max(1, 64 // scale_down)
        spec.past = [int(x) for x in rng.integers(4096 // scale_down, 16384 // scale_down, size=n, endpoint=True)]
        spec.new = [1] * n
    elif cfg == "c5":
        npre = max(1, 8 // scale_down)
        ndec = max(1, 56 // scale_down)
        pre = [int(x) for x in rng.integers(0, 2048 // scale_down, size=npre, endpoint=True)]
        dec = [int(x) for x in rng.integers(1024 // scale_down, 8192 // scale_down, size=ndec, endpoint=True)]
        spec.past = pre + dec
        spec.new = [max(1, 256 // scale_down)] * npre + [1] * ndec
    elif cfg in ("c3", "gqa_prefill") and scale_down > 1:
        spec.past = [p // scale_down for p in spec.past]
        spec.new = [max(1, n // scale_down) for n in spec.new]
    elif cfg == "c1" and scale_down > 1:
        pass


def spec_for(cfg: str, scale_down: int = 1, seed: Optional[int] = None) -> Spec:
    spec = CONFIGS[cfg]()
    if seed is not None:
        spec.seed = seed
    return spec


def build(spec: Spec, cfg: Optional[str] = None, scale_down: int = 1, poison: bool = False,
          lengths_drawn: bool = False) -> dict:
    """Materialise a workload. Draw order: lengths, block permutation, cache,
    query, key, slot drop mask."""
    rng = np.random.default_rng(spec.seed)
    if cfg is not None and not lengths_drawn:
        draw_lengths(cfg, spec, rng, scale_down)
    past = np.asarray(spec.past, dtype=np.int64)
    new = np.asarray(spec.new, dtype=np.int64)
    assert past.shape == new.shape and past.size >= 1
    B = past.size
    T = int(new.sum())
    H, hs, bs = spec.num_heads, spec.head_size, spec.block_size
    ctx = past + new
    blocks_per_seq = (ctx + bs - 1) // bs
    MB = int(max(1, blocks_per_seq.max()))
    NB = int(blocks_per_seq.sum()) + spec.spare_blocks

    phys = rng.permutation(NB).astype(np.int64) if spec.permute_blocks else np.arange(NB, dtype=np.int64)
    block_table = np.full((B, MB), -1, dtype=np.int32)
    k = 0
    for b in range(B):
        nblk = int(blocks_per_seq[b])
        block_table[b, :nblk] = phys[k:k + nblk]
        k += nblk

    sep = spec.layout == "SEPARATE"
    assert spec.layout in ("LATENT", "SEPARATE")
    kvh = spec.kv_num_heads if sep else 1
    vhs = spec.v_head_size or hs

    def filled(width):
        # Whole cache pre-filled, block by block, so memory stays bounded.
        c = np.empty((NB, bs, kvh, width), dtype=np.uint16)
        chunk = max(1, (1 << 22) // (bs * kvh * width))
        for s in range(0, NB, chunk):
            e = min(NB, s + chunk)
            vals = rng.standard_normal((e - s, bs, kvh, width), dtype=np.float32) * np.float32(spec.cache_std)
            c[s:e] = to_storage_bits(vals, spec.dtype)
        return c

    cache = filled(hs)
    vcache = filled(vhs) if sep else None
    query = to_storage_bits(rng.standard_normal((T, H * hs), dtype=np.float32) * np.float32(spec.q_std), spec.dtype)
    key = to_storage_bits(rng.standard_normal((T, kvh * hs), dtype=np.float32) * np.float32(spec.key_std),
                          spec.dtype)
    value = (to_storage_bits(rng.standard_normal((T, kvh * vhs), dtype=np.float32) * np.float32(spec.key_std),
                             spec.dtype) if sep else None)

    cumseq = np.zeros(B + 1, dtype=np.int32)
    cumseq[1:] = np.cumsum(new)
    slot = np.empty(T, dtype=np.int32)
    for b in range(B):
        for i in range(int(new[b])):
            pos = int(past[b]) + i
            slot[cumseq[b] + i] = int(block_table[b, pos // bs]) * bs + pos % bs
    if spec.slot_drop_frac > 0:
        ndrop = int(round(spec.slot_drop_frac * T))
        drop = rng.choice(T, size=ndrop, replace=False)
        slot[drop] = -1

    rd = spec.rotary_dim if spec.do_rotary else 0
    P = int(ctx.max())
    if rd > 0:
        half = rd // 2
        inv_freq = spec.theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / rd)
        ang = np.arange(P, dtype=np.float64)[:, None] * inv_freq[None, :]
        cos_bits = to_storage_bits(np.cos(ang).astype(np.float32), spec.dtype)
        sin_bits = to_storage_bits(np.sin(ang).astype(np.float32), spec.dtype)
    else:
        cos_bits = np.zeros((0, 0), dtype=np.uint16)
        sin_bits = np.zeros((0, 0), dtype=np.uint16)

    if poison:
        reachable = np.zeros(NB * bs, dtype=bool)
        for b in range(B):
            j = np.arange(int(ctx[b]))
            rows = block_table[b, j // bs].astype(np.int64) * bs + j % bs
            reachable[rows] = True
        nan_bits = BF16_NAN_BITS if spec.dtype == "bf16" else F16_NAN_BITS
        for c in (cache, vcache):
            if c is not None:
                c.reshape(NB * bs, -1)[~reachable] = nan_bits

    attrs = dict(
        num_heads=H, head_size=hs, v_head_size=spec.v_head_size, block_size=bs,
        do_rotary=int(spec.do_rotary), rotary_interleaved=int(spec.rotary_interleaved),
        rotary_dim=rd, rotary_offset=spec.rotary_offset if rd > 0 else 0,
        local_window_size=int(spec.local_window_size), softcap=float(spec.softcap),
        has_scale=int(spec.has_scale), scale=float(spec.scale) if spec.has_scale else 0.0,
    )
    dims = dict(token_count=T, batch=B, max_blocks_per_seq=MB, num_blocks=NB, rotary_rows=P if rd > 0 else 0)
    out = dict(
        name=spec.name, dtype=spec.dtype, attrs=attrs, dims=dims,
        query=query, key=key, key_cache=cache, cos_cache=cos_bits, sin_cache=sin_bits,
        cumulative_sequence_length=cumseq, past_seqlens=past.astype(np.int32),
        block_table=block_table, slot_mapping=slot, spec=asdict(spec),
    )
    if sep:
        attrs.update(kv_cache_layout="SEPARATE", kv_num_heads=kvh)
        out.update(value=value, value_cache=vcache)
    return out


def make(cfg: str, scale_down: int = 1, poison: bool = False, seed: Optional[int] = None) -> dict:
    """Build one of the five named workloads (c1..c5); `scale_down` shrinks it."""
    spec = spec_for(cfg, scale_down, seed)
    return build(spec, cfg=cfg, scale_down=scale_down, poison=poison)


def algorithmic_counts(w: dict) -> dict:
    """Bytes and MFMA flops the attention phase must move/compute (no overheads).

    bytes = visible KV rows x hs x |D| + q + out + cos/sin rows + block-table
    entries touched; flops = 2 (hs + vhs) per (token, head, visible key)."""
    a, d = w["attrs"], w["dims"]
    H, hs, vhs, bs = a["num_heads"], a["head_size"], a["v_head_size"] or a["head_size"], a["block_size"]
    win = a["local_window_size"]
    cum, past = w["cumulative_sequence_length"], w["past_seqlens"]
    kv_rows = 0
    pairs = 0
    blocks = 0
    for b in range(d["batch"]):
        n = int(cum[b + 1] - cum[b])
        p0 = int(past[b])
        pos = p0 + np.arange(n, dtype=np.int64)
        lo = np.zeros_like(pos) if win < 0 else np.maximum(0, pos - win)
        pairs += int((pos - lo + 1).sum())
        if n:
            first = int(lo.min())
            last = int(pos.max())
            kv_rows += last - first + 1
            blocks += last // bs - first // bs + 1
    T = d["token_count"]
    esz = 2
    kvh = a.get("kv_num_heads", 1)
    # LATENT: one latent row of hs channels per key (V is its leading part);
    # SEPARATE: kv_num_heads key rows of hs and value rows of vhs channels.
    row_bytes = (kvh * (hs + vhs) if a.get("kv_cache_layout") == "SEPARATE" else hs) * esz
    new_row_bytes = row_bytes
    byts = kv_rows * row_bytes + T * H * hs * esz + T * H * vhs * esz + T * a["rotary_dim"] * esz + blocks * 4
    flops = 2 * (hs + vhs) * H * pairs
    return dict(bytes=int(byts), flops=int(flops), kv_rows=int(kv_rows), visible_pairs=int(pairs) * H,
                write_bytes=int(2 * T * new_row_bytes))
