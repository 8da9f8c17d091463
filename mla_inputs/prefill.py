"""Seeded inputs of an MHA-mode prefill chunk: the decode step's inputs (same
seed: cache, block table, weights, sequence lengths T_b) plus a chunk of new
query tokens per sequence.

Recipe: ``generate(cfg)`` gives the cache of T_b tokens per sequence (the new
tokens already written); then from ``numpy.random.default_rng(cfg.seed + 7919)``
q ~ N(0, 1) of shape [B, max_q_len, h, d_nope + d_rope], rounded to the query
storage type, and, unless given, L_b = min(max_q_len, T_b) new tokens per
sequence.  The query rows past L_b are drawn too (a kernel must not read them
into any output row it writes).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

from .generate import MLAInputs, generate, round_to


@dataclass
class PrefillInputs:
    dense: MLAInputs
    q: np.ndarray          # [B, max_q_len, h, d_nope + d_rope] storage
    q_lens: np.ndarray     # [B] int32
    max_q_len: int

    def __getattr__(self, name):
        return getattr(self.__dict__["dense"], name)


def generate_prefill(cfg, max_q_len: int, seq_lens: Optional[Sequence[int]] = None,
                     q_lens: Optional[Sequence[int]] = None) -> PrefillInputs:
    dense = generate(cfg, seq_lens=seq_lens)
    rng = np.random.default_rng(cfg.seed + 7919)
    shape = (cfg.batch, max_q_len, cfg.heads, cfg.d_nope + cfg.d_rope)
    q = round_to(cfg.q_dtype, rng.standard_normal(shape, dtype=np.float32))
    if q_lens is None:
        q_lens = np.minimum(dense.seq_lens, max_q_len)
    return PrefillInputs(dense, np.ascontiguousarray(q), np.asarray(q_lens, dtype=np.int32),
                         int(max_q_len))
