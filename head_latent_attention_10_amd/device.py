"""Device-memory plumbing around the C ABI (torch is used for allocation and
streams only).

`DeviceInputs` holds one decode step's tensors on a GPU in their storage
types; `Decoder` owns a workspace and an output buffer and calls the library.
Inputs are duck-typed: any object with the fields `q, c_kv, c_kv_scale,
k_rope, block_table, seq_lens, W_UK, W_UV` (numpy arrays of the storage types)
and a `cfg` carrying shapes and dtype tags.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _lib

_TORCH_STORAGE = {np.dtype(np.float32): torch.float32, np.dtype(np.uint16): torch.int16,
                  np.dtype(np.uint8): torch.uint8, np.dtype(np.int32): torch.int32}


def to_device_array(a: np.ndarray, device) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


class DeviceInputs:
    FIELDS = ("q", "c_kv", "c_kv_scale", "k_rope", "block_table", "seq_lens", "W_UK", "W_UV")

    def __init__(self, inp, device="cuda"):
        self.cfg = inp.cfg
        self.device = torch.device(device)
        for f in self.FIELDS:
            v = getattr(inp, f)
            setattr(self, f, None if v is None else to_device_array(v, self.device))
        self.num_blocks = int(inp.c_kv.shape[0])
        self.max_blocks_per_seq = int(inp.block_table.shape[1])

    def params(self, num_splits: int = 0, batch: int | None = None) -> _lib.MlaDecodeParams:
        c = self.cfg
        return _lib.make_params(
            batch=c.batch if batch is None else batch, num_heads=c.heads, d_nope=c.d_nope,
            d_rope=c.d_rope, d_latent=c.d_latent, d_v=c.d_v, page_size=c.page_size,
            max_blocks_per_seq=self.max_blocks_per_seq, num_blocks=self.num_blocks,
            q_dtype=c.q_dtype, cache_dtype=c.cache_dtype, rope_dtype=c.rope_dtype,
            weight_dtype=c.weight_dtype, out_dtype=c.out_dtype, sm_scale=c.sm_scale,
            num_splits=num_splits)


def out_torch_dtype(tag: str):
    return torch.float32 if tag == "f32" else torch.int16   # bf16 bits


def bf16_bits_to_float(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.bfloat16).float()


class Decoder:
    """Workspace + output for repeated mla_decode calls on one set of inputs."""

    def __init__(self, dev: DeviceInputs, num_splits: int = 0):
        self.dev = dev
        self.p = dev.params(num_splits=num_splits)
        self.ws_bytes = _lib.mla_decode_workspace_size(self.p)
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev.device)
        c = dev.cfg
        self.out = torch.empty((c.batch, c.heads, c.d_v), dtype=out_torch_dtype(c.out_dtype),
                               device=dev.device)

    def __call__(self, stream=None, c_kv=None, k_rope=None, c_kv_scale=None):
        d = self.dev
        _lib.mla_decode(self.p, d.q, d.c_kv if c_kv is None else c_kv,
                        d.c_kv_scale if c_kv_scale is None else c_kv_scale,
                        d.k_rope if k_rope is None else k_rope, d.block_table, d.seq_lens,
                        d.W_UK, d.W_UV, self.out, self.workspace, self.ws_bytes, stream)
        return self.out

    def out_float(self) -> torch.Tensor:
        if self.dev.cfg.out_dtype == "f32":
            return self.out
        return bf16_bits_to_float(self.out)
