"""Comparison helpers for the GPU parity tests (HIP path vs the CPU oracle).

Tolerances: outputs within max-abs 2e-3 (float16) / 1.6e-2 (bfloat16) of the
oracle, and, because max-abs alone is weak where outputs are small, relative
Frobenius error <= 2e-3 (float16) / 1e-2 (bfloat16). Written cache rows: bit
exact outside the rotary channels, within 1 ulp of the storage type inside
them (the kernel rotates in float32, the oracle in float64; both round to
nearest even). Untouched cache rows: bit exact.
"""
import numpy as np

from oracle import paged_latent as orc

MAX_ABS = {"f16": 2e-3, "bf16": 1.6e-2}
REL_FRO = {"f16": 2e-3, "bf16": 1e-2}


def ordered(bits: np.ndarray) -> np.ndarray:
    """Map 16-bit float patterns to integers whose order and spacing follow the
    floats' (sign-magnitude to two's complement); +0 and -0 both map to 0."""
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def ulp_distance(a_bits, b_bits) -> np.ndarray:
    return np.abs(ordered(np.asarray(a_bits)) - ordered(np.asarray(b_bits)))


def check_write(w: dict, gpu_cache: np.ndarray, ref_cache: np.ndarray, before: np.ndarray):
    hs = w["attrs"]["head_size"]
    g = gpu_cache.reshape(-1, hs)
    r = ref_cache.reshape(-1, hs)
    b0 = before.reshape(-1, hs)
    slots = w["slot_mapping"]
    written = np.unique(slots[slots >= 0])
    untouched = np.setdiff1d(np.arange(g.shape[0]), written)
    assert np.array_equal(g[untouched], b0[untouched]), "rows without a slot changed"
    a = w["attrs"]
    rot = np.zeros(hs, dtype=bool)
    if a["do_rotary"]:
        rot[a["rotary_offset"]:a["rotary_offset"] + a["rotary_dim"]] = True
    gw, rw = g[written], r[written]
    assert np.array_equal(gw[:, ~rot], rw[:, ~rot]), "non-rotary channels of written rows differ"
    if rot.any():
        d = ulp_distance(gw[:, rot], rw[:, rot])
        assert d.max() <= 1, f"rotary channels differ by {d.max()} ulp"


def errors(got: np.ndarray, ref: np.ndarray):
    """(max-abs error, relative Frobenius error) of got against ref."""
    err = np.abs(got - ref)
    max_abs = float(err.max()) if err.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref)) / den if den > 0 else float(np.linalg.norm(got))
    return max_abs, rel


def check_output(dtype: str, got: np.ndarray, ref: np.ndarray, rows=None, what="", heads: int = 0):
    """Assert got matches ref within the tolerances. With heads > 1 it also
    asserts that the comparison discriminates on this data: unless the first
    two heads' reference outputs are identical (a token that sees only its own
    row, a zero scale), the reference with their columns exchanged must fail
    the same bar (so a head-permuted result could not pass)."""
    if rows is not None:
        got, ref = got[rows], ref[rows]
    assert np.all(np.isfinite(got)), f"{what}: non-finite outputs"
    max_abs, rel = errors(got, ref)
    assert max_abs <= MAX_ABS[dtype], f"{what}: max-abs {max_abs:.3e} > {MAX_ABS[dtype]}"
    assert rel <= REL_FRO[dtype], f"{what}: relative Frobenius {rel:.3e} > {REL_FRO[dtype]}"
    if heads > 1:
        _, rel_swapped = errors(swap_heads(ref, heads), ref)
        assert rel_swapped == 0.0 or rel_swapped > REL_FRO[dtype], \
            f"{what}: a head-swapped output would pass ({rel_swapped:.3e})"
    return max_abs, rel


def swap_heads(out: np.ndarray, heads: int, a: int = 0, b: int = 1) -> np.ndarray:
    """Copy of out [T, heads * v] with the columns of heads a and b exchanged."""
    v = out.shape[1] // heads
    o = out.copy()
    o[:, a * v:(a + 1) * v], o[:, b * v:(b + 1) * v] = out[:, b * v:(b + 1) * v], out[:, a * v:(a + 1) * v]
    return o


def oracle(w: dict, tokens=None):
    cache = orc.write_phase(w)
    return cache, orc.attention(w, cache, tokens=tokens)


def check_write_separate(w: dict, gpu_k: np.ndarray, gpu_v: np.ndarray, ref_k: np.ndarray, ref_v: np.ndarray,
                         before_k: np.ndarray, before_v: np.ndarray):
    """Separate layout: both caches, per slot (all key/value heads of a slot).
    Key rows as in check_write (bit exact outside the rotary channels, 1 ulp
    inside); value rows bit exact; slots no token writes unchanged."""
    a = w["attrs"]
    kvh, hs = a["kv_num_heads"], a["head_size"]
    vhs = a["v_head_size"] or hs
    gk, rk, bk = (x.reshape(-1, kvh, hs) for x in (gpu_k, ref_k, before_k))
    gv, rv, bv = (x.reshape(-1, kvh, vhs) for x in (gpu_v, ref_v, before_v))
    slots = w["slot_mapping"]
    written = np.unique(slots[slots >= 0])
    untouched = np.setdiff1d(np.arange(gk.shape[0]), written)
    assert np.array_equal(gk[untouched], bk[untouched]), "key slots without a token changed"
    assert np.array_equal(gv[untouched], bv[untouched]), "value slots without a token changed"
    assert np.array_equal(gv[written], rv[written]), "written value rows differ"
    rot = np.zeros(hs, dtype=bool)
    if a["do_rotary"]:
        rot[a["rotary_offset"]:a["rotary_offset"] + a["rotary_dim"]] = True
    kw, kr = gk[written], rk[written]
    assert np.array_equal(kw[..., ~rot], kr[..., ~rot]), "non-rotary channels of written key rows differ"
    if rot.any():
        d = ulp_distance(kw[..., rot], kr[..., rot])
        assert d.max() <= 1, f"rotary channels differ by {d.max()} ulp"


def oracle_separate(w: dict, tokens=None):
    from oracle import paged_separate as sep
    return sep.run(w, tokens=tokens)
