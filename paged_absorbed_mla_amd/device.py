"""Device plumbing: put a workload's tensors in GPU memory with torch and call the
library through the binding. torch supplies memory and streams only; no torch
operator runs on the write or attention path.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import _lib


def dtype_code(dtype: str) -> int:
    return {"f16": _lib.PA_F16, "bf16": _lib.PA_BF16}[dtype]


def attrs_of(w: dict) -> "_lib.pa_latent_attrs":
    a = {k: v for k, v in w["attrs"].items() if k not in ("kv_cache_layout", "kv_num_heads")}
    return _lib.make_attrs(**a)


def kv_heads_of(w: dict) -> int:
    """Key/value heads of a separate-layout workload, 0 for the latent layout."""
    a = w["attrs"]
    return int(a["kv_num_heads"]) if a.get("kv_cache_layout") == "SEPARATE" else 0


def dims_of(w: dict) -> "_lib.pa_latent_dims":
    return _lib.make_dims(**w["dims"])


class DeviceWorkload:
    """The tensors of one call, resident in HBM, plus a workspace."""

    def __init__(self, w: dict, device: str = "cuda:0", workspace: bool = True):
        import torch
        self.w = w
        self.device = torch.device(device)
        tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[w["dtype"]]
        self.torch_dtype = tdt

        def u16(a):
            a = np.ascontiguousarray(a, dtype=np.uint16)
            return torch.from_numpy(a.view(np.int16)).to(self.device).view(tdt)

        def i32(a):
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(self.device)

        self.kvh = kv_heads_of(w)
        self.query = u16(w["query"])
        self.key = u16(w["key"])
        self.key_cache = u16(w["key_cache"])
        self.value = u16(w["value"]) if self.kvh else None
        self.value_cache = u16(w["value_cache"]) if self.kvh else None
        rd = w["attrs"]["rotary_dim"]
        self.cos = u16(w["cos_cache"]) if rd else None
        self.sin = u16(w["sin_cache"]) if rd else None
        self.cumseq = i32(w["cumulative_sequence_length"])
        self.past = i32(w["past_seqlens"])
        self.block_table = i32(w["block_table"])
        self.slot_mapping = i32(w["slot_mapping"])
        a = w["attrs"]
        vhs = a["v_head_size"] or a["head_size"]
        T = w["dims"]["token_count"]
        self.output = torch.zeros((T, a["num_heads"] * vhs), dtype=tdt, device=self.device)
        # step() runs both phases as one fused call
        self.fused = True
        self.attrs = attrs_of(w)
        self.dims = dims_of(w)
        self.code = dtype_code(w["dtype"])
        self.ws_bytes = 0
        self.workspace = None
        if workspace:
            if self.kvh:
                self.ws_bytes = _lib.pa_separate_workspace_size(self.attrs, self.kvh, self.dims, self.code,
                                                                self.device.index or 0)
            else:
                self.ws_bytes = _lib.pa_latent_workspace_size(self.attrs, self.dims, self.code,
                                                              self.device.index or 0)
            self.workspace = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=self.device)

    def write(self, stream=None):
        if self.kvh:
            return _lib.pa_separate_write(self.attrs, self.kvh, self.dims, self.code, self.key, self.value,
                                          self.cos, self.sin, self.slot_mapping, self.cumseq, self.past,
                                          self.key_cache, self.value_cache, stream)
        return _lib.pa_latent_write(self.attrs, self.dims, self.code, self.key, self.cos, self.sin,
                                    self.slot_mapping, self.cumseq, self.past, self.key_cache, stream)

    def attention(self, stream=None, split_kv: Optional[bool] = None):
        if self.kvh:
            if split_kv is not None:
                raise ValueError("the separate layout has no forced split-KV entry point")
            return _lib.pa_separate_attention(self.attrs, self.kvh, self.dims, self.code, self.query,
                                              self.key_cache, self.value_cache, self.cos, self.sin, self.cumseq,
                                              self.past, self.block_table, self.output, self.workspace,
                                              self.ws_bytes, stream)
        if split_kv is None:
            return _lib.pa_latent_attention(self.attrs, self.dims, self.code, self.query, self.key_cache,
                                            self.cos, self.sin, self.cumseq, self.past, self.block_table,
                                            self.output, self.workspace, self.ws_bytes, stream)
        return _lib.pa_latent_attention_splits(self.attrs, self.dims, self.code, self.query, self.key_cache,
                                               self.cos, self.sin, self.cumseq, self.past, self.block_table,
                                               self.output, self.workspace, self.ws_bytes, int(split_kv),
                                               stream)

    def forward(self, stream=None):
        """Write phase and attention in one call (pa_latent_forward / pa_separate_forward)."""
        if self.kvh:
            return _lib.pa_separate_forward(self.attrs, self.kvh, self.dims, self.code, self.query, self.key,
                                            self.value, self.cos, self.sin, self.slot_mapping, self.cumseq,
                                            self.past, self.block_table, self.key_cache, self.value_cache,
                                            self.output, self.workspace, self.ws_bytes, stream)
        return _lib.pa_latent_forward(self.attrs, self.dims, self.code, self.query, self.key, self.cos, self.sin,
                                      self.slot_mapping, self.cumseq, self.past, self.block_table,
                                      self.key_cache, self.output, self.workspace, self.ws_bytes, stream)

    def step(self, stream=None):
        """One pass of the whole path: write phase, then attention (one fused
        call, or the two calls when `fused` is off)."""
        if self.fused:
            self.forward(stream)
        else:
            self.write(stream)
            self.attention(stream)

    def cache_bits(self) -> np.ndarray:
        import torch
        return self.key_cache.view(torch.int16).cpu().numpy().view(np.uint16)

    def value_cache_bits(self) -> np.ndarray:
        import torch
        return self.value_cache.view(torch.int16).cpu().numpy().view(np.uint16)

    def output_f64(self) -> np.ndarray:
        import torch
        return self.output.to(torch.float64).cpu().numpy()
