"""Seeded generation of one decode step's inputs.

Recipe (all draws from ``numpy.random.default_rng(seed)``, PCG64, in this order):
  1. ragged lengths: ``rng.integers(lo, hi, endpoint=True)`` per sequence;
  2. physical block assignment: ``rng.permutation(num_blocks)`` (identity when
     the workload is not permuted);
  3. q ~ N(0, 1), shape [B, h, d_nope + d_rope];
  4. W_UK ~ N(0, std = 1/sqrt(d_latent)), shape [h, d_nope, d_latent];
  5. W_UV ~ N(0, std = 1/sqrt(d_latent)), shape [h, d_v, d_latent];
  6. c_KV ~ N(0, 1) per cached token, drawn page by page in logical order;
  7. k_rope ~ N(0, 1) per cached token, drawn the same way.
fp32 draws are rounded to the storage type with round-to-nearest-even (torch's
bfloat16 / float8_e4m3fn casts).  An fp8 latent row stores bytes
``e4m3(clamp(x / s, +-448))`` with the per-token scale ``s = max|x| / 448``
(fp32), the OCP E4M3FN encoding.

Every pool slot that holds no cached token (spare blocks, the unused tail of a
sequence's last block) is filled with NaN, and block-table entries past a
sequence's last block point at a NaN block, so a stray read shows up in the
output instead of going unnoticed.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np
import torch

from .configs import MLAConfig

# storage encodings: raw numpy dtype of each tag
STORAGE = {"f32": np.float32, "bf16": np.uint16, "e4m3": np.uint8}
NAN_BITS = {"f32": np.float32(np.nan), "bf16": np.uint16(0x7FC0), "e4m3": np.uint8(0x7F)}
E4M3_MAX = 448.0
_PAGES_PER_DRAW = 64


@dataclass
class MLAInputs:
    cfg: MLAConfig
    seq_lens: np.ndarray      # [B] int32
    block_table: np.ndarray   # [B, max_blocks_per_seq] int32
    q: np.ndarray             # [B, h, d_nope + d_rope] storage of cfg.q_dtype
    c_kv: np.ndarray          # [num_blocks, P, d_latent] storage of cfg.cache_dtype
    c_kv_scale: Optional[np.ndarray]  # [num_blocks, P] float32 (e4m3 only)
    k_rope: np.ndarray        # [num_blocks, P, d_rope] storage of cfg.rope_dtype
    W_UK: np.ndarray          # [h, d_nope, d_latent] storage of cfg.weight_dtype
    W_UV: np.ndarray          # [h, d_v, d_latent]
    poison_block: int         # a NaN-filled block that table padding points at

    @property
    def sm_scale(self) -> float:
        return self.cfg.sm_scale

    @property
    def num_blocks(self) -> int:
        return self.c_kv.shape[0]

    @property
    def max_blocks_per_seq(self) -> int:
        return self.block_table.shape[1]

    def cache_bytes(self) -> int:
        """Bytes of latent cache one decode step reads (c_KV, k_rope, scales)."""
        cfg = self.cfg
        per_tok = cfg.d_latent * _itemsize(cfg.cache_dtype) + cfg.d_rope * _itemsize(cfg.rope_dtype)
        if cfg.cache_dtype == "e4m3":
            per_tok += 4
        return int(self.seq_lens.astype(np.int64).sum()) * per_tok


def _itemsize(tag: str) -> int:
    return np.dtype(STORAGE[tag]).itemsize


def round_to(tag: str, x: np.ndarray) -> np.ndarray:
    """fp32 -> storage bits of ``tag`` (round to nearest even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if tag == "f32":
        return x
    if tag == "bf16":
        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    raise ValueError(tag)


def quantize_e4m3_rows(x: np.ndarray):
    """Per-row fp8 encoding of an fp32 array [..., d] -> (bytes [..., d], scale [...])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    y = (x / safe[..., None]).astype(np.float32)
    y = np.where(scale[..., None] > 0, y, np.float32(0.0))
    y = np.clip(y, -E4M3_MAX, E4M3_MAX).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def generate(cfg: MLAConfig, seq_lens: Optional[Sequence[int]] = None,
             seed: Optional[int] = None) -> MLAInputs:
    """Draw one decode step's inputs for ``cfg`` (optionally with given lengths)."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    B, h, P = cfg.batch, cfg.heads, cfg.page_size
    if seq_lens is not None:
        lens = np.asarray(seq_lens, dtype=np.int64)
        if lens.shape != (B,):
            raise ValueError("seq_lens must have one entry per sequence")
    elif cfg.seq_len is not None:
        lens = np.full(B, cfg.seq_len, dtype=np.int64)
    else:
        lo, hi = cfg.seq_len_range
        lens = rng.integers(lo, hi, size=B, endpoint=True).astype(np.int64)

    pages = (lens + P - 1) // P
    used = int(pages.sum())
    spare = max(1, cfg.spare_blocks)
    num_blocks = used + spare
    if cfg.permuted:
        order = rng.permutation(num_blocks)
    else:
        order = np.arange(num_blocks)
    phys = order[:used]
    poison = int(order[used])          # first spare block

    max_blocks = int(pages.max()) + 1 if B > 0 else 1
    table = np.full((B, max_blocks), poison, dtype=np.int32)
    start = np.concatenate([[0], np.cumsum(pages)])
    for b in range(B):
        table[b, : pages[b]] = phys[start[b]: start[b + 1]]

    dq = cfg.d_nope + cfg.d_rope
    q = round_to(cfg.q_dtype, rng.standard_normal((B, h, dq), dtype=np.float32))
    wstd = np.float32(1.0 / np.sqrt(cfg.d_latent))
    W_UK = round_to(cfg.weight_dtype,
                    rng.standard_normal((h, cfg.d_nope, cfg.d_latent), dtype=np.float32) * wstd)
    W_UV = round_to(cfg.weight_dtype,
                    rng.standard_normal((h, cfg.d_v, cfg.d_latent), dtype=np.float32) * wstd)

    c_kv = np.full((num_blocks, P, cfg.d_latent), NAN_BITS[cfg.cache_dtype],
                   dtype=STORAGE[cfg.cache_dtype])
    scale = None
    if cfg.cache_dtype == "e4m3":
        scale = np.full((num_blocks, P), np.nan, dtype=np.float32)
    k_rope = np.full((num_blocks, P, cfg.d_rope), NAN_BITS[cfg.rope_dtype],
                     dtype=STORAGE[cfg.rope_dtype])

    for p0 in range(0, used, _PAGES_PER_DRAW):
        n = min(_PAGES_PER_DRAW, used - p0)
        x = rng.standard_normal((n, P, cfg.d_latent), dtype=np.float32)
        if cfg.cache_dtype == "e4m3":
            codes, s = quantize_e4m3_rows(x)
            c_kv[phys[p0: p0 + n]] = codes
            scale[phys[p0: p0 + n]] = s
        else:
            c_kv[phys[p0: p0 + n]] = round_to(cfg.cache_dtype, x)
    for p0 in range(0, used, _PAGES_PER_DRAW):
        n = min(_PAGES_PER_DRAW, used - p0)
        x = rng.standard_normal((n, P, cfg.d_rope), dtype=np.float32)
        k_rope[phys[p0: p0 + n]] = round_to(cfg.rope_dtype, x)

    # poison the unused tail of every sequence's last block
    for b in range(B):
        tail = int(lens[b] % P)
        if pages[b] > 0 and tail:
            blk = table[b, pages[b] - 1]
            c_kv[blk, tail:] = NAN_BITS[cfg.cache_dtype]
            k_rope[blk, tail:] = NAN_BITS[cfg.rope_dtype]
            if scale is not None:
                scale[blk, tail:] = np.nan

    return MLAInputs(cfg=cfg, seq_lens=lens.astype(np.int32), block_table=table, q=q,
                     c_kv=c_kv, c_kv_scale=scale, k_rope=k_rope, W_UK=W_UK, W_UV=W_UV,
                     poison_block=poison)


def make_inputs(name_or_cfg, **kw) -> MLAInputs:
    from .configs import CONFIGS
    cfg = CONFIGS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    return generate(cfg, **kw)


def repermute(inp: MLAInputs, seed: int) -> MLAInputs:
    """The same logical cache under a different physical block assignment."""
    rng = np.random.default_rng(seed)
    nb = inp.num_blocks
    new_of_old = rng.permutation(nb)          # old physical id -> new physical id
    c_kv = np.empty_like(inp.c_kv)
    c_kv[new_of_old] = inp.c_kv
    k_rope = np.empty_like(inp.k_rope)
    k_rope[new_of_old] = inp.k_rope
    scale = None
    if inp.c_kv_scale is not None:
        scale = np.empty_like(inp.c_kv_scale)
        scale[new_of_old] = inp.c_kv_scale
    table = new_of_old[inp.block_table].astype(np.int32)
    return MLAInputs(cfg=inp.cfg, seq_lens=inp.seq_lens.copy(), block_table=table, q=inp.q,
                     c_kv=c_kv, c_kv_scale=scale, k_rope=k_rope, W_UK=inp.W_UK, W_UV=inp.W_UV,
                     poison_block=int(new_of_old[inp.poison_block]))
