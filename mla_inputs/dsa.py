"""Seeded inputs of the DSA (sparse) decode step: the dense decode step's
inputs plus the lightning indexer's query, head weights and key cache.

Shapes: the DeepSeek-V3.2 indexer (64 heads of width 128, top-2048) on the
DeepSeek-V3 attention shape, from "TransMLA & Sparse Latent Attention",
Chapter 6 ("The lightning indexer", "Fine-grained token selection") and
Chapter 7 (the indexer key kept per cached position).

Recipe: the dense inputs first (``generate``, same seed), then from
``numpy.random.default_rng(seed + 7919)``, in this order:
  1. q_I ~ N(0, 1) [B, H_I, d_I], stored as E4M3FN codes with one fp32 scale
     per (sequence, head) (the latent cache's per-row rule);
  2. w_I ~ N(0, 1/H_I) [B, H_I] fp32 (either sign);
  3. k_I ~ N(0, 1) per cached token, drawn page by page in each sequence's
     logical order, stored as E4M3FN codes with one fp32 scale per token in a
     pool [num_blocks, P, d_I] beside the latent pool (same block table).
Pool slots that hold no token keep NaN codes (0x7F) and NaN scales.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

from .configs import CONFIGS, MLAConfig
from .generate import MLAInputs, generate, quantize_e4m3_rows

_ROWS_PER_DRAW = 1 << 16


@dataclass(frozen=True)
class DSAConfig:
    name: str
    base: MLAConfig
    index_heads: int = 64
    index_dim: int = 128
    topk: int = 2048
    seq_lens: Optional[tuple] = None  # explicit lengths (else the base config's)

    @property
    def cfg(self) -> MLAConfig:
        return self.base

    def replace(self, **kw) -> "DSAConfig":
        d = dict(self.__dict__)
        d.update(kw)
        return DSAConfig(**d)


_DSV3 = dict(heads=128, d_nope=128, d_latent=512, d_rope=64, d_v=128, page_size=64)

DSA_CONFIGS = {
    # small: one sequence shorter than k, one exactly k, one longer; 8 indexer heads
    "dsa_tiny": DSAConfig(
        "dsa_tiny",
        MLAConfig(name="dsa_tiny", batch=3, heads=4, d_nope=16, d_latent=32, d_rope=8, d_v=16,
                  page_size=16, seq_len_range=(1, 2), cache_dtype="f32", q_dtype="f32",
                  rope_dtype="f32", weight_dtype="f32", seed=3000),
        index_heads=8, index_dim=32, topk=40, seq_lens=(17, 40, 333)),
    # DeepSeek-V3 shape, lengths around k = 2048 (below, at, above, several pages past)
    "dsa_dsv3_small": DSAConfig(
        "dsa_dsv3_small",
        MLAConfig(name="dsa_dsv3_small", batch=4, seq_len_range=(1, 2), seed=3001, **_DSV3),
        seq_lens=(700, 2048, 2049, 9000)),
    # the headline's ragged 1K..32K lengths with the DSA selection
    "dsa_dsv3_ragged_32k": DSAConfig(
        "dsa_dsv3_ragged_32k", CONFIGS["dsv3_ragged_32k"].replace(name="dsa_dsv3_ragged_32k")),
    # the pages' design point: 128K context, top-2048
    "dsa_dsv3_b4_128k": DSAConfig(
        "dsa_dsv3_b4_128k",
        MLAConfig(name="dsa_dsv3_b4_128k", batch=4, seq_len=131072, seed=3003, **_DSV3)),
    # fp8 latent cache with the DSA selection
    "dsa_dsv3_fp8_16k": DSAConfig(
        "dsa_dsv3_fp8_16k",
        MLAConfig(name="dsa_dsv3_fp8_16k", batch=8, seq_len=16384, cache_dtype="e4m3",
                  seed=3004, **_DSV3)),
}


@dataclass
class DSAInputs:
    dcfg: DSAConfig
    dense: MLAInputs
    q_I: np.ndarray         # [B, H_I, d_I] uint8 E4M3FN codes
    q_I_scale: np.ndarray   # [B, H_I] float32
    w_I: np.ndarray         # [B, H_I] float32
    k_I: np.ndarray         # [num_blocks, P, d_I] uint8 E4M3FN codes
    k_I_scale: np.ndarray   # [num_blocks, P] float32

    # the dense inputs' fields, so the oracle and the tests can use either
    def __getattr__(self, name):
        return getattr(self.__dict__["dense"], name)

    @property
    def topk(self) -> int:
        return self.dcfg.topk


def generate_dsa(dcfg: DSAConfig, seq_lens: Optional[Sequence[int]] = None) -> DSAInputs:
    lens = seq_lens if seq_lens is not None else dcfg.seq_lens
    dense = generate(dcfg.base, seq_lens=lens)
    cfg = dcfg.base
    B, P = cfg.batch, cfg.page_size
    H, d = dcfg.index_heads, dcfg.index_dim
    rng = np.random.default_rng(cfg.seed + 7919)
    q_codes, q_scale = quantize_e4m3_rows(rng.standard_normal((B, H, d), dtype=np.float32))
    w = (rng.standard_normal((B, H), dtype=np.float32) * np.float32(1.0 / np.sqrt(H))).astype(
        np.float32)
    nb = dense.num_blocks
    k_codes = np.full((nb, P, d), 0x7F, dtype=np.uint8)
    k_scale = np.full((nb, P), np.nan, dtype=np.float32)
    # logical rows of every sequence, page by page
    rows = []
    for b in range(B):
        T = int(dense.seq_lens[b])
        for j in range((T + P - 1) // P):
            rows.append((int(dense.block_table[b, j]), min(P, T - j * P)))
    total = sum(n for _, n in rows)
    done = 0
    it = iter(rows)
    pending = None
    while done < total:
        n_draw = min(_ROWS_PER_DRAW, total - done)
        x = rng.standard_normal((n_draw, d), dtype=np.float32)
        codes, sc = quantize_e4m3_rows(x)
        o = 0
        while o < n_draw:
            if pending is None:
                blk, n = next(it)
                pending = [blk, 0, n]
            blk, s0, n = pending
            take = min(n - s0, n_draw - o)
            k_codes[blk, s0: s0 + take] = codes[o: o + take]
            k_scale[blk, s0: s0 + take] = sc[o: o + take]
            o += take
            pending = None if s0 + take == n else [blk, s0 + take, n]
        done += n_draw
    return DSAInputs(dcfg, dense, q_codes, q_scale.astype(np.float32), w, k_codes, k_scale)


def make_dsa_inputs(name_or_cfg, **kw) -> DSAInputs:
    dcfg = DSA_CONFIGS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    return generate_dsa(dcfg, **kw)
