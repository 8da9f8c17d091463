"""Seeded inputs of the grouped-MLA decode step: the dense step's inputs (same
seed) with the latent pool repeated per group, groups 1.. drawn afresh.

Recipe: ``generate(cfg)`` gives the dense inputs and group 0's pool; then from
``numpy.random.default_rng(cfg.seed + 104729)`` each further group's latent rows
~ N(0, 1) per cached token (fp8: quantised per row, the dense recipe), written
through the same block table; every slot without a token keeps NaN.  Pools are
stacked group-major: [G, num_blocks, P, d_latent] (and [G, num_blocks, P]
scales for fp8).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .generate import NAN_BITS, STORAGE, MLAInputs, generate, quantize_e4m3_rows, round_to


@dataclass
class GroupedInputs:
    dense: MLAInputs
    groups: int
    c_pools: np.ndarray                 # [G, num_blocks, P, d_latent] storage
    scale_pools: Optional[np.ndarray]   # [G, num_blocks, P] float32 (e4m3 only)

    def __getattr__(self, name):
        return getattr(self.__dict__["dense"], name)


def generate_grouped(cfg, groups: int, seq_lens=None) -> GroupedInputs:
    dense = generate(cfg, seq_lens=seq_lens)
    rng = np.random.default_rng(cfg.seed + 104729)
    P = cfg.page_size
    pools = [dense.c_kv]
    scales = [dense.c_kv_scale]
    for _ in range(groups - 1):
        pool = np.full_like(dense.c_kv, NAN_BITS[cfg.cache_dtype])
        sc = None if dense.c_kv_scale is None else np.full_like(dense.c_kv_scale, np.nan)
        for b in range(cfg.batch):
            T = int(dense.seq_lens[b])
            for j in range((T + P - 1) // P):
                blk, n = int(dense.block_table[b, j]), min(P, T - j * P)
                x = rng.standard_normal((n, cfg.d_latent), dtype=np.float32)
                if cfg.cache_dtype == "e4m3":
                    codes, s = quantize_e4m3_rows(x)
                    pool[blk, :n], sc[blk, :n] = codes, s
                else:
                    pool[blk, :n] = round_to(cfg.cache_dtype, x)
        pools.append(pool)
        scales.append(sc)
    c_pools = np.ascontiguousarray(np.stack(pools)).astype(STORAGE[cfg.cache_dtype], copy=False)
    scale_pools = None if dense.c_kv_scale is None else np.ascontiguousarray(np.stack(scales))
    return GroupedInputs(dense, groups, c_pools, scale_pools)
