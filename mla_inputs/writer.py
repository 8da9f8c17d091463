"""Seeded inputs of the latent-cache writer (one new token per sequence).

Shapes: the DeepSeek-V3 attention layer (hidden size 7168, latent 512, rope
64) and the TransMLA-converted LLaMA-2-7B layer (hidden size 4096, latent 512,
rope 64), plus a tiny fp32 case.  Recipe (``numpy.random.default_rng(seed)``,
in this order):
  1. positions ~ U[0, max_pos) per sequence (or given);
  2. physical blocks: ``rng.permutation(num_blocks)``; sequence b's target page
     gets block perm[b], the rest of its table row points at a spare block;
  3. x ~ N(0, 1) [B, d_model];
  4. W_DKV ~ N(0, std = 1/sqrt(d_model)) [d_latent, d_model];
  5. gamma = 1 + 0.1 N(0, 1) [d_latent];
  6. W_KR ~ N(0, std = 1/sqrt(d_model)) [d_rope, d_model].
fp32 draws are rounded to the storage type (round to nearest even).  The pools
start NaN-filled, so every slot the writer must not touch keeps its bits.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

from .generate import NAN_BITS, STORAGE, round_to


@dataclass(frozen=True)
class WriterConfig:
    name: str
    batch: int
    d_model: int
    d_latent: int
    d_rope: int
    page_size: int
    max_pos: int
    x_dtype: str = "bf16"
    weight_dtype: str = "bf16"
    cache_dtype: str = "bf16"
    rope_dtype: str = "bf16"
    rms_eps: float = 1e-6
    rope_base: float = 10000.0
    spare_blocks: int = 2
    seed: int = 2000

    def replace(self, **kw) -> "WriterConfig":
        d = dict(self.__dict__)
        d.update(kw)
        return WriterConfig(**d)


_DSV3 = dict(d_model=7168, d_latent=512, d_rope=64, page_size=64, max_pos=32768)

WRITER_CONFIGS = {
    "writer_tiny_f32": WriterConfig("writer_tiny_f32", batch=3, d_model=64, d_latent=32, d_rope=8,
                                    page_size=16, max_pos=200, x_dtype="f32", weight_dtype="f32",
                                    cache_dtype="f32", rope_dtype="f32", seed=2001),
    "writer_transmla_b16": WriterConfig("writer_transmla_b16", batch=16, d_model=4096, d_latent=512,
                                        d_rope=64, page_size=64, max_pos=8192, seed=2002),
    "writer_dsv3_b8": WriterConfig("writer_dsv3_b8", batch=8, seed=2003, **_DSV3),
    "writer_dsv3_b64": WriterConfig("writer_dsv3_b64", batch=64, seed=2004, **_DSV3),
    "writer_dsv3_fp8_b32": WriterConfig("writer_dsv3_fp8_b32", batch=32, cache_dtype="e4m3",
                                        seed=2005, **_DSV3),
}


@dataclass
class WriterInputs:
    cfg: WriterConfig
    positions: np.ndarray      # [B] int32
    block_table: np.ndarray    # [B, max_blocks] int32
    num_blocks: int
    x: np.ndarray              # [B, d_model] storage of x_dtype
    W_DKV: np.ndarray          # [d_latent, d_model]
    gamma: np.ndarray          # [d_latent]
    W_KR: np.ndarray           # [d_rope, d_model]
    c_kv: np.ndarray           # [num_blocks, P, d_latent] storage, NaN-filled
    c_kv_scale: Optional[np.ndarray]  # [num_blocks, P] float32 (e4m3 only), NaN-filled
    k_rope: np.ndarray         # [num_blocks, P, d_rope] storage, NaN-filled


def generate_writer(cfg: WriterConfig, positions: Optional[Sequence[int]] = None,
                    seed: Optional[int] = None) -> WriterInputs:
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    B, P = cfg.batch, cfg.page_size
    if positions is None:
        pos = rng.integers(0, cfg.max_pos, size=B).astype(np.int32)
    else:
        pos = np.asarray(positions, dtype=np.int32)
        if pos.shape != (B,):
            raise ValueError("one position per sequence")
    num_blocks = B + max(1, cfg.spare_blocks)
    perm = rng.permutation(num_blocks)
    spare = int(perm[B])
    max_blocks = max(1, int(np.max(np.maximum(pos, 0)) // P) + 1) if B else 1
    table = np.full((B, max_blocks), spare, dtype=np.int32)
    for b in range(B):
        if pos[b] >= 0 and pos[b] // P < max_blocks:
            table[b, pos[b] // P] = perm[b]
    sd = np.float32(1.0 / np.sqrt(cfg.d_model))
    x = round_to(cfg.x_dtype, rng.standard_normal((B, cfg.d_model), dtype=np.float32))
    W_DKV = round_to(cfg.weight_dtype,
                     rng.standard_normal((cfg.d_latent, cfg.d_model), dtype=np.float32) * sd)
    gamma = round_to(cfg.weight_dtype,
                     1.0 + 0.1 * rng.standard_normal(cfg.d_latent, dtype=np.float32))
    W_KR = round_to(cfg.weight_dtype,
                    rng.standard_normal((cfg.d_rope, cfg.d_model), dtype=np.float32) * sd)
    c_kv = np.full((num_blocks, P, cfg.d_latent), NAN_BITS[cfg.cache_dtype],
                   dtype=STORAGE[cfg.cache_dtype])
    scale = (np.full((num_blocks, P), np.nan, dtype=np.float32)
             if cfg.cache_dtype == "e4m3" else None)
    k_rope = np.full((num_blocks, P, cfg.d_rope), NAN_BITS[cfg.rope_dtype],
                     dtype=STORAGE[cfg.rope_dtype])
    return WriterInputs(cfg, pos, table, num_blocks, x, W_DKV, gamma, W_KR, c_kv, scale, k_rope)


def make_writer_inputs(name_or_cfg, **kw) -> WriterInputs:
    cfg = WRITER_CONFIGS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    return generate_writer(cfg, **kw)
