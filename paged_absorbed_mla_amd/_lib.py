"""ctypes binding of libpa_latent.so (declared in include/pa_latent.h).

Argument marshalling only: every step of the write and attention phases runs in
the library's HIP kernels. The functions keep the C names. Pointer arguments
accept either raw integers (device addresses) or torch tensors, whose
data_ptr() is passed; `stream` defaults to torch's current stream on the
tensors' device. There is no fallback: if the library is missing, loading fails
with an error naming the build command.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpa_latent.so")

PA_OK = 0
PA_ERR_INVALID_ARGUMENT = 1
PA_ERR_NOT_IMPLEMENTED = 2
PA_ERR_WORKSPACE_TOO_SMALL = 3
PA_ERR_DEVICE = 4
PA_ERR_CAPTURE_NOT_WARMED = 5
PA_F16 = 10
PA_BF16 = 16

EXPORTED = ("pa_latent_write", "pa_latent_workspace_size", "pa_latent_attention", "pa_latent_forward",
            "pa_latent_attention_splits", "pa_latent_attention_noalloc", "pa_latent_capture_ready",
            "pa_separate_write", "pa_separate_workspace_size", "pa_separate_attention", "pa_separate_forward",
            "pa_latent_profile_next", "pa_last_error", "pa_latent_abi_version")


class pa_latent_attrs(ctypes.Structure):
    _fields_ = [
        ("num_heads", ctypes.c_int32),
        ("head_size", ctypes.c_int32),
        ("v_head_size", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("do_rotary", ctypes.c_int32),
        ("rotary_interleaved", ctypes.c_int32),
        ("rotary_dim", ctypes.c_int32),
        ("rotary_offset", ctypes.c_int32),
        ("local_window_size", ctypes.c_int32),
        ("softcap", ctypes.c_float),
        ("has_scale", ctypes.c_int32),
        ("scale", ctypes.c_float),
    ]


class pa_latent_dims(ctypes.Structure):
    _fields_ = [
        ("token_count", ctypes.c_int64),
        ("batch", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_blocks", ctypes.c_int64),
        ("rotary_rows", ctypes.c_int64),
    ]


class PaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"pa_latent status {status}: {message}")
        self.status = status


_lib = None


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the library once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    # PA_LATENT_LIB: path of another build of the same library (A/B timing of
    # compile-time variants); the in-tree build otherwise.
    path = path or os.environ.get("PA_LATENT_LIB") or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m paged_absorbed_mla_amd.build`")
    lib = ctypes.CDLL(path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    A, D = ctypes.POINTER(pa_latent_attrs), ctypes.POINTER(pa_latent_dims)
    lib.pa_latent_write.argtypes = [A, D, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.pa_latent_write.restype = ctypes.c_int
    lib.pa_latent_workspace_size.argtypes = [A, D, ctypes.c_int, ctypes.c_int, ctypes.POINTER(sz)]
    lib.pa_latent_workspace_size.restype = ctypes.c_int
    lib.pa_latent_attention.argtypes = [A, D, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.pa_latent_attention.restype = ctypes.c_int
    lib.pa_latent_forward.argtypes = [A, D, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.pa_latent_forward.restype = ctypes.c_int
    lib.pa_latent_attention_splits.argtypes = [A, D, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                               ctypes.c_int32, vp]
    lib.pa_latent_attention_splits.restype = ctypes.c_int
    lib.pa_latent_attention_noalloc.argtypes = [A, D, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.pa_latent_attention_noalloc.restype = ctypes.c_int
    lib.pa_latent_capture_ready.argtypes = [A, D, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_int32),
                                            ctypes.POINTER(ctypes.c_int32)]
    lib.pa_latent_capture_ready.restype = ctypes.c_int
    i32 = ctypes.c_int32
    lib.pa_separate_write.argtypes = [A, i32, D, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.pa_separate_write.restype = ctypes.c_int
    lib.pa_separate_workspace_size.argtypes = [A, i32, D, ctypes.c_int, ctypes.c_int, ctypes.POINTER(sz)]
    lib.pa_separate_workspace_size.restype = ctypes.c_int
    lib.pa_separate_attention.argtypes = [A, i32, D, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.pa_separate_attention.restype = ctypes.c_int
    lib.pa_separate_forward.argtypes = [A, i32, D, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                        vp, sz, vp]
    lib.pa_separate_forward.restype = ctypes.c_int
    lib.pa_latent_profile_next.argtypes = [vp, vp]
    lib.pa_latent_profile_next.restype = ctypes.c_int
    lib.pa_last_error.argtypes = []
    lib.pa_last_error.restype = ctypes.c_char_p
    lib.pa_latent_abi_version.argtypes = []
    lib.pa_latent_abi_version.restype = ctypes.c_int32
    _lib = lib
    return lib


def make_attrs(num_heads, head_size, v_head_size=0, block_size=16, do_rotary=0, rotary_interleaved=0,
               rotary_dim=0, rotary_offset=0, local_window_size=-1, softcap=0.0, has_scale=0,
               scale=0.0) -> pa_latent_attrs:
    return pa_latent_attrs(num_heads, head_size, v_head_size, block_size, do_rotary, rotary_interleaved,
                           rotary_dim, rotary_offset, local_window_size, float(softcap), has_scale,
                           float(scale))


def make_dims(token_count, batch, max_blocks_per_seq, num_blocks, rotary_rows=0) -> pa_latent_dims:
    return pa_latent_dims(int(token_count), int(batch), int(max_blocks_per_seq), int(num_blocks),
                          int(rotary_rows))


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()          # torch tensor


def _stream(stream, *tensors):
    if stream is not None:
        return stream if isinstance(stream, int) else getattr(stream, "cuda_stream", stream)
    import torch
    for t in tensors:
        if t is not None and not isinstance(t, int) and t.is_cuda:
            return torch.cuda.current_stream(t.device).cuda_stream
    return None


def _check(status: int) -> int:
    if status != PA_OK:
        raise PaError(status, load().pa_last_error().decode())
    return status


def pa_latent_write(attrs, dims, dtype, key, cos_cache, sin_cache, slot_mapping,
                    cumulative_sequence_length, past_seqlens, key_cache, stream=None, check=True):
    lib = load()
    st = lib.pa_latent_write(ctypes.byref(attrs), ctypes.byref(dims), int(dtype), _ptr(key), _ptr(cos_cache),
                             _ptr(sin_cache), _ptr(slot_mapping), _ptr(cumulative_sequence_length),
                             _ptr(past_seqlens), _ptr(key_cache), _stream(stream, key_cache, key))
    return _check(st) if check else st


def pa_latent_workspace_size(attrs, dims, dtype, device=0, check=True) -> int:
    lib = load()
    out = ctypes.c_size_t(0)
    st = lib.pa_latent_workspace_size(ctypes.byref(attrs), ctypes.byref(dims), int(dtype), int(device),
                                      ctypes.byref(out))
    if check:
        _check(st)
    return out.value if st == PA_OK else -st


def pa_latent_attention(attrs, dims, dtype, query, key_cache, cos_cache, sin_cache,
                        cumulative_sequence_length, past_seqlens, block_table, output, workspace,
                        workspace_bytes, stream=None, check=True):
    lib = load()
    st = lib.pa_latent_attention(ctypes.byref(attrs), ctypes.byref(dims), int(dtype), _ptr(query),
                                 _ptr(key_cache), _ptr(cos_cache), _ptr(sin_cache),
                                 _ptr(cumulative_sequence_length), _ptr(past_seqlens), _ptr(block_table),
                                 _ptr(output), _ptr(workspace), int(workspace_bytes),
                                 _stream(stream, output, query))
    return _check(st) if check else st


def pa_latent_forward(attrs, dims, dtype, query, key, cos_cache, sin_cache, slot_mapping,
                      cumulative_sequence_length, past_seqlens, block_table, key_cache, output, workspace,
                      workspace_bytes, stream=None, check=True):
    lib = load()
    st = lib.pa_latent_forward(ctypes.byref(attrs), ctypes.byref(dims), int(dtype), _ptr(query), _ptr(key),
                               _ptr(cos_cache), _ptr(sin_cache), _ptr(slot_mapping),
                               _ptr(cumulative_sequence_length), _ptr(past_seqlens), _ptr(block_table),
                               _ptr(key_cache), _ptr(output), _ptr(workspace), int(workspace_bytes),
                               _stream(stream, output, query))
    return _check(st) if check else st


def pa_latent_attention_splits(attrs, dims, dtype, query, key_cache, cos_cache, sin_cache,
                               cumulative_sequence_length, past_seqlens, block_table, output, workspace,
                               workspace_bytes, split_kv, stream=None, check=True):
    lib = load()
    st = lib.pa_latent_attention_splits(ctypes.byref(attrs), ctypes.byref(dims), int(dtype), _ptr(query),
                                        _ptr(key_cache), _ptr(cos_cache), _ptr(sin_cache),
                                        _ptr(cumulative_sequence_length), _ptr(past_seqlens),
                                        _ptr(block_table), _ptr(output), _ptr(workspace), int(workspace_bytes),
                                        int(split_kv), _stream(stream, output, query))
    return _check(st) if check else st


def pa_latent_attention_noalloc(attrs, dims, dtype, query, key_cache, cos_cache, sin_cache,
                                cumulative_sequence_length, past_seqlens, block_table, output, stream=None,
                                check=True):
    lib = load()
    st = lib.pa_latent_attention_noalloc(ctypes.byref(attrs), ctypes.byref(dims), int(dtype), _ptr(query),
                                         _ptr(key_cache), _ptr(cos_cache), _ptr(sin_cache),
                                         _ptr(cumulative_sequence_length), _ptr(past_seqlens), _ptr(block_table),
                                         _ptr(output), _stream(stream, output, query))
    return _check(st) if check else st


def pa_separate_write(attrs, kv_num_heads, dims, dtype, key, value, cos_cache, sin_cache, slot_mapping,
                      cumulative_sequence_length, past_seqlens, key_cache, value_cache, stream=None, check=True):
    lib = load()
    st = lib.pa_separate_write(ctypes.byref(attrs), int(kv_num_heads), ctypes.byref(dims), int(dtype), _ptr(key),
                               _ptr(value), _ptr(cos_cache), _ptr(sin_cache), _ptr(slot_mapping),
                               _ptr(cumulative_sequence_length), _ptr(past_seqlens), _ptr(key_cache),
                               _ptr(value_cache), _stream(stream, key_cache, key))
    return _check(st) if check else st


def pa_separate_workspace_size(attrs, kv_num_heads, dims, dtype, device=0, check=True) -> int:
    lib = load()
    out = ctypes.c_size_t(0)
    st = lib.pa_separate_workspace_size(ctypes.byref(attrs), int(kv_num_heads), ctypes.byref(dims), int(dtype),
                                        int(device), ctypes.byref(out))
    if check:
        _check(st)
    return out.value if st == PA_OK else -st


def pa_separate_forward(attrs, kv_num_heads, dims, dtype, query, key, value, cos_cache, sin_cache, slot_mapping,
                        cumulative_sequence_length, past_seqlens, block_table, key_cache, value_cache, output,
                        workspace, workspace_bytes, stream=None, check=True):
    lib = load()
    st = lib.pa_separate_forward(ctypes.byref(attrs), int(kv_num_heads), ctypes.byref(dims), int(dtype), _ptr(query),
                                 _ptr(key), _ptr(value), _ptr(cos_cache), _ptr(sin_cache), _ptr(slot_mapping),
                                 _ptr(cumulative_sequence_length), _ptr(past_seqlens), _ptr(block_table),
                                 _ptr(key_cache), _ptr(value_cache), _ptr(output), _ptr(workspace),
                                 int(workspace_bytes), _stream(stream, output, query))
    return _check(st) if check else st


def pa_separate_attention(attrs, kv_num_heads, dims, dtype, query, key_cache, value_cache, cos_cache, sin_cache,
                          cumulative_sequence_length, past_seqlens, block_table, output, workspace,
                          workspace_bytes, stream=None, check=True):
    lib = load()
    st = lib.pa_separate_attention(ctypes.byref(attrs), int(kv_num_heads), ctypes.byref(dims), int(dtype),
                                   _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(cos_cache),
                                   _ptr(sin_cache), _ptr(cumulative_sequence_length), _ptr(past_seqlens),
                                   _ptr(block_table), _ptr(output), _ptr(workspace), int(workspace_bytes),
                                   _stream(stream, output, query))
    return _check(st) if check else st


def pa_latent_capture_ready(attrs, dims, dtype, device=0):
    """(write_ready, attention_ready) of this signature on `device`."""
    w, a = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(load().pa_latent_capture_ready(ctypes.byref(attrs), ctypes.byref(dims), int(dtype), int(device),
                                          ctypes.byref(w), ctypes.byref(a)))
    return bool(w.value), bool(a.value)


def pa_latent_profile_next(before, after):
    """Register two events (torch.cuda.Event after one record(), or raw hipEvent_t
    handles as ints; None for none) to be recorded around the attention kernel of
    this thread's next pa_latent_attention call."""
    def handle(ev):
        if ev is None:
            return None
        return ctypes.c_void_p(int(ev.cuda_event) if hasattr(ev, "cuda_event") else int(ev))
    return _check(load().pa_latent_profile_next(handle(before), handle(after)))


def pa_last_error() -> str:
    return load().pa_last_error().decode()


def pa_latent_abi_version() -> int:
    return int(load().pa_latent_abi_version())
