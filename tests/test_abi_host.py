"""C-ABI checks that need no GPU: the library loads, exports every entry point the
header declares, and rejects invalid requests before touching the device.

The rejection matrix mirrors the op's rules as the docs.rs page
"onnx-runtime-ep-cuda src/kernels/paged_attention.rs" states them
(unsupported_reason, PagedAttentionFactory::create, execute; unit tests
rejects_non_half_dtype and the execute-time geometry checks) and the rotary-cache
rules of PR #1940 ("PagedAttention v1 audit and MLA oracle", third commit) and
PR #1955's review (rotary_offset % 8, head_size % 8). Every call here fails (or
is a no-op) before any HIP call, so device pointers are dummies.
"""
import os
import re

import pytest

import paged_absorbed_mla_amd as pa
from paged_absorbed_mla_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DUMMY = 0x10000        # 16-byte aligned, never dereferenced


def header_functions():
    text = open(os.path.join(ROOT, "include", "pa_latent.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = pa.load()
    declared = header_functions()
    assert set(declared) == set(_lib.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name
    assert pa.pa_latent_abi_version() == 3


def glm_attrs(**kw):
    base = dict(num_heads=16, head_size=192, v_head_size=128, block_size=64, do_rotary=1,
                rotary_interleaved=0, rotary_dim=64, rotary_offset=128, local_window_size=-1,
                softcap=0.0, has_scale=1, scale=0.0721)
    base.update(kw)
    return pa.make_attrs(**base)


def dims(T=32, B=32, MB=65, NB=2100, P=4097):
    return pa.make_dims(T, B, MB, NB, P)


def attn(a, d=None, dtype=pa.PA_BF16, ptrs=None, ws=DUMMY, ws_bytes=1 << 30):
    p = dict(query=DUMMY, key_cache=DUMMY, cos=DUMMY, sin=DUMMY, cumseq=DUMMY, past=DUMMY, bt=DUMMY, out=DUMMY)
    p.update(ptrs or {})
    return pa.pa_latent_attention(a, d or dims(), dtype, p["query"], p["key_cache"], p["cos"], p["sin"],
                                  p["cumseq"], p["past"], p["bt"], p["out"], ws, ws_bytes, stream=0,
                                  check=False)


def write(a, d=None, dtype=pa.PA_BF16, ptrs=None):
    p = dict(key=DUMMY, cos=DUMMY, sin=DUMMY, slot=DUMMY, cumseq=DUMMY, past=DUMMY, cache=DUMMY)
    p.update(ptrs or {})
    return pa.pa_latent_write(a, d or dims(), dtype, p["key"], p["cos"], p["sin"], p["slot"], p["cumseq"],
                              p["past"], p["cache"], stream=0, check=False)


def forward(a, d=None, dtype=pa.PA_BF16, ptrs=None, ws=DUMMY, ws_bytes=1 << 30):
    p = dict(query=DUMMY, key=DUMMY, cos=DUMMY, sin=DUMMY, slot=DUMMY, cumseq=DUMMY, past=DUMMY, bt=DUMMY,
             cache=DUMMY, out=DUMMY)
    p.update(ptrs or {})
    return pa.pa_latent_forward(a, d or dims(), dtype, p["query"], p["key"], p["cos"], p["sin"], p["slot"],
                                p["cumseq"], p["past"], p["bt"], p["cache"], p["out"], ws, ws_bytes, stream=0,
                                check=False)


CASES = [
    # (description, attrs overrides, dims overrides, dtype, expected status, message fragment)
    ("float32 query", {}, {}, 1, pa.PA_ERR_NOT_IMPLEMENTED, "float16"),
    ("int8 storage", {}, {}, 3, pa.PA_ERR_NOT_IMPLEMENTED, "bfloat16"),
    ("zero heads", dict(num_heads=0), {}, pa.PA_BF16, pa.PA_ERR_INVALID_ARGUMENT, "num_heads"),
    ("head_size % 8", dict(head_size=190), {}, pa.PA_BF16, pa.PA_ERR_INVALID_ARGUMENT, "multiple of 8"),
    ("v_head_size > head_size", dict(v_head_size=200), {}, pa.PA_BF16, pa.PA_ERR_INVALID_ARGUMENT, "1..=head_size"),
    ("negative v_head_size", dict(v_head_size=-1), {}, pa.PA_BF16, pa.PA_ERR_INVALID_ARGUMENT, "1..=head_size"),
    ("block_size 8", dict(block_size=8), {}, pa.PA_BF16, pa.PA_ERR_INVALID_ARGUMENT, "power of two >= 16"),
    ("block_size 48", dict(block_size=48), {}, pa.PA_BF16, pa.PA_ERR_INVALID_ARGUMENT, "power of two >= 16"),
    ("rotary past head", dict(rotary_offset=160), {}, pa.PA_BF16, pa.PA_ERR_INVALID_ARGUMENT, "exceeds head_size"),
    ("rotary_dim % 16", dict(rotary_dim=24), {}, pa.PA_BF16, pa.PA_ERR_INVALID_ARGUMENT, "multiple of 16"),
    ("rotary_offset % 8", dict(rotary_offset=124), {}, pa.PA_BF16, pa.PA_ERR_INVALID_ARGUMENT, "multiple of 8"),
    ("head_size % 16 with rotary", dict(head_size=200, v_head_size=128, rotary_offset=128),
     {}, pa.PA_BF16, pa.PA_ERR_INVALID_ARGUMENT, "multiple of 16"),
    ("missing scale when v != hs", dict(has_scale=0), {}, pa.PA_BF16, pa.PA_ERR_INVALID_ARGUMENT, "explicit 'scale'"),
    ("zero batch", {}, dict(B=0), pa.PA_BF16, pa.PA_ERR_INVALID_ARGUMENT, "batch"),
    ("zero max blocks", {}, dict(MB=0), pa.PA_BF16, pa.PA_ERR_INVALID_ARGUMENT, "max_blocks_per_seq"),
    ("negative tokens", {}, dict(T=-1), pa.PA_BF16, pa.PA_ERR_INVALID_ARGUMENT, "token_count"),
    ("grid limit", {}, dict(T=1 << 30), pa.PA_BF16, pa.PA_ERR_INVALID_ARGUMENT, "grid limit"),
    ("no rotary rows", {}, dict(P=0), pa.PA_BF16, pa.PA_ERR_INVALID_ARGUMENT, "rotary_rows"),
]


@pytest.mark.parametrize("desc,akw,dkw,dtype,status,frag", CASES, ids=[c[0] for c in CASES])
def test_rejections_before_launch(desc, akw, dkw, dtype, status, frag):
    a = glm_attrs(**akw)
    d = dims(**dkw)
    for fn in (attn, write, forward):
        st = fn(a, d, dtype)
        assert st == status, (desc, fn.__name__, pa.pa_last_error())
        assert frag in pa.pa_last_error(), pa.pa_last_error()


@pytest.mark.parametrize("which", ["query", "key_cache", "cumseq", "past", "bt", "out", "cos", "sin"])
def test_attention_rejects_null_required_input(which):
    st = attn(glm_attrs(), ptrs={which: None})
    assert st == pa.PA_ERR_INVALID_ARGUMENT
    assert "NULL" in pa.pa_last_error()


@pytest.mark.parametrize("which", ["key", "slot", "cumseq", "past", "cache", "cos", "sin"])
def test_write_rejects_null_required_input(which):
    st = write(glm_attrs(), ptrs={which: None})
    assert st == pa.PA_ERR_INVALID_ARGUMENT
    assert "NULL" in pa.pa_last_error()


@pytest.mark.parametrize("which", ["query", "key", "slot", "cumseq", "past", "bt", "cache", "out", "cos", "sin"])
def test_forward_rejects_null_required_input(which):
    """The fused call checks the inputs of both phases before anything is enqueued."""
    st = forward(glm_attrs(), ptrs={which: None})
    assert st == pa.PA_ERR_INVALID_ARGUMENT
    assert "NULL" in pa.pa_last_error()


def test_cos_sin_optional_without_rotary():
    a = glm_attrs(do_rotary=0)
    # NULL cos/sin is accepted; the call then fails later only on the (NULL) workspace.
    assert attn(a, ptrs={"cos": None, "sin": None}, ws=None) == pa.PA_ERR_INVALID_ARGUMENT
    assert "workspace" in pa.pa_last_error()


def test_misaligned_pointer_rejected():
    assert attn(glm_attrs(), ptrs={"query": DUMMY + 2}) == pa.PA_ERR_INVALID_ARGUMENT
    assert "aligned" in pa.pa_last_error()
    assert attn(glm_attrs(), ws=DUMMY + 64) == pa.PA_ERR_INVALID_ARGUMENT
    assert "256-byte" in pa.pa_last_error()


def test_head_size_without_instance_is_not_implemented():
    a = glm_attrs(head_size=640, v_head_size=640, rotary_offset=512, has_scale=0)
    assert attn(a) == pa.PA_ERR_NOT_IMPLEMENTED
    assert "no attention instance" in pa.pa_last_error()
    # the write phase has no head-size limit beyond the schema rules: it only
    # fails here on the NULL key
    assert write(a, ptrs={"key": None}) == pa.PA_ERR_INVALID_ARGUMENT


def test_default_scale_when_v_equals_head_size():
    a = glm_attrs(v_head_size=0, has_scale=0)      # v = hs, scale = 1/sqrt(hs)
    assert attn(a, ws=None) == pa.PA_ERR_INVALID_ARGUMENT   # passes validation, stops at the workspace
    assert "workspace" in pa.pa_last_error()


def test_zero_tokens_is_a_no_op():
    d = dims(T=0)
    assert attn(glm_attrs(), d, ptrs={k: None for k in ("query", "out")}, ws=None) == pa.PA_OK
    assert write(glm_attrs(), d, ptrs={"key": None, "slot": None}) == pa.PA_OK
    assert pa.pa_last_error() == ""


def test_null_attrs_and_dims():
    lib = pa.load()
    assert lib.pa_latent_attention(None, None, 16, *([DUMMY] * 9), 0, None) == pa.PA_ERR_INVALID_ARGUMENT
    assert "attrs" in pa.pa_last_error()
    assert lib.pa_latent_write(None, None, 16, *([DUMMY] * 7), None) == pa.PA_ERR_INVALID_ARGUMENT


def test_binding_raises_with_message():
    with pytest.raises(pa.PaError, match="power of two"):
        pa.pa_latent_write(glm_attrs(block_size=24), dims(), pa.PA_BF16, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY,
                           DUMMY, DUMMY, stream=0)


# ----------------------------------------------------------------------------
# Separate (grouped-query) layout: the head-ratio rule of PR #1940's third
# commit (num_heads % kv_num_heads, rejection case 4/3), the value inputs, and
# the head sizes built for it.
# ----------------------------------------------------------------------------

def gqa_attrs(**kw):
    base = dict(num_heads=32, head_size=128, v_head_size=128, block_size=16, do_rotary=1,
                rotary_interleaved=0, rotary_dim=128, rotary_offset=0, local_window_size=-1,
                softcap=0.0, has_scale=0, scale=0.0)
    base.update(kw)
    return pa.make_attrs(**base)


def sep_attn(a, kvh, d=None, ptrs=None, ws=DUMMY, ws_bytes=1 << 30):
    p = dict(query=DUMMY, key_cache=DUMMY, value_cache=DUMMY, cos=DUMMY, sin=DUMMY, cumseq=DUMMY, past=DUMMY,
             bt=DUMMY, out=DUMMY)
    p.update(ptrs or {})
    return pa.pa_separate_attention(a, kvh, d or dims(), pa.PA_BF16, p["query"], p["key_cache"], p["value_cache"],
                                    p["cos"], p["sin"], p["cumseq"], p["past"], p["bt"], p["out"], ws, ws_bytes,
                                    stream=0, check=False)


def sep_write(a, kvh, d=None, ptrs=None):
    p = dict(key=DUMMY, value=DUMMY, cos=DUMMY, sin=DUMMY, slot=DUMMY, cumseq=DUMMY, past=DUMMY, cache=DUMMY,
             vcache=DUMMY)
    p.update(ptrs or {})
    return pa.pa_separate_write(a, kvh, d or dims(), pa.PA_BF16, p["key"], p["value"], p["cos"], p["sin"],
                                p["slot"], p["cumseq"], p["past"], p["cache"], p["vcache"], stream=0, check=False)


SEP_CASES = [
    ("ratio 4/3", dict(num_heads=4), 3, pa.PA_ERR_INVALID_ARGUMENT, "multiple of kv_num_heads"),
    ("ratio 32/5", {}, 5, pa.PA_ERR_INVALID_ARGUMENT, "multiple of kv_num_heads"),
    ("zero kv heads", {}, 0, pa.PA_ERR_INVALID_ARGUMENT, "kv_num_heads"),
    ("more kv heads than heads", dict(num_heads=4), 8, pa.PA_ERR_INVALID_ARGUMENT, "multiple of kv_num_heads"),
    ("v_head_size % 8", dict(v_head_size=100, has_scale=1, scale=0.1), 8, pa.PA_ERR_NOT_IMPLEMENTED,
     "multiple of 8"),
    ("block_size 8", dict(block_size=8), 8, pa.PA_ERR_INVALID_ARGUMENT, "power of two >= 16"),
]


@pytest.mark.parametrize("desc,akw,kvh,status,frag", SEP_CASES, ids=[c[0] for c in SEP_CASES])
def test_separate_rejections_before_launch(desc, akw, kvh, status, frag):
    a = gqa_attrs(**akw)
    for fn in (sep_attn, sep_write):
        st = fn(a, kvh)
        assert st == status, (desc, fn.__name__, pa.pa_last_error())
        assert frag in pa.pa_last_error(), pa.pa_last_error()


@pytest.mark.parametrize("H,kvh", [(4, 2), (4, 4), (32, 8), (32, 1)])
def test_separate_accepts_valid_ratios(H, kvh):
    # valid ratios pass every check and stop only at the (NULL) workspace
    assert sep_attn(gqa_attrs(num_heads=H), kvh, ws=None) == pa.PA_ERR_INVALID_ARGUMENT
    assert "workspace" in pa.pa_last_error()


def test_separate_forward_rejects_null_value_and_bad_ratio():
    a = glm_attrs(num_heads=8, head_size=128, v_head_size=128, rotary_offset=64, has_scale=0)
    D = DUMMY
    st = pa.pa_separate_forward(a, 2, dims(), pa.PA_BF16, D, D, None, D, D, D, D, D, D, D, D, D, D, 1 << 30,
                                stream=0, check=False)
    assert st == pa.PA_ERR_INVALID_ARGUMENT and "value" in pa.pa_last_error()
    st = pa.pa_separate_forward(a, 3, dims(), pa.PA_BF16, D, D, D, D, D, D, D, D, D, D, D, D, D, 1 << 30,
                                stream=0, check=False)
    assert st == pa.PA_ERR_INVALID_ARGUMENT


def test_separate_needs_value_inputs():
    assert sep_attn(gqa_attrs(), 8, ptrs={"value_cache": None}) == pa.PA_ERR_INVALID_ARGUMENT
    assert "value_cache" in pa.pa_last_error()
    assert sep_write(gqa_attrs(), 8, ptrs={"value": None}) == pa.PA_ERR_INVALID_ARGUMENT
    assert "'value'" in pa.pa_last_error()
    assert sep_write(gqa_attrs(), 8, ptrs={"vcache": None}) == pa.PA_ERR_INVALID_ARGUMENT
    assert "value_cache" in pa.pa_last_error()


def test_separate_head_size_without_instance_is_not_implemented():
    a = gqa_attrs(head_size=192, v_head_size=128, rotary_dim=64, has_scale=1, scale=0.07)
    assert sep_attn(a, 8) == pa.PA_ERR_NOT_IMPLEMENTED
    assert "separate layout" in pa.pa_last_error()
