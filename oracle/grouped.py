"""Plain CPU oracle of grouped MLA decode: the latent held as several
independent groups, the heads split evenly over them, one shared rope key.

TEST INFRASTRUCTURE ONLY.  Imported by the tests and the benchmark's checks;
never by the HIP library, with which it shares no code.  Arithmetic is fp64.

Source: the TransMLA OpenReview discussion, reply A2 (to the question of
serving TransMLA's other head counts and kv_ranks with FlashMLA): the KV cache
is partitioned into groups of 576 values each served as an ordinary MLA cache,
e.g. a kv_rank of 1088 as two 512-dimensional groups plus a 64-dimensional part
carrying the positional information; and the later reply to reviewer KGKd
(grouped TransMLA is a different model from the joint one: PCA per group).

Readings taken where the discussion is silent:
  * G1: head i belongs to group i // (h / G), as a query head belongs to its
    key group in GQA ([LESSON] Chapter 1); each group's latent is decoded with
    the dense decode step's formula, the 64 rope values shared by all groups;
  * G2: the cache stores the groups as separate page pools with one block
    table (group-major), so each group is a 576-wide MLA cache on its own.

Pins (tests/test_oracle_grouped_pins.py, CPU only): one group is the dense
oracle; equal pools give the dense result; a head reads only its own group;
GQA with G key groups is grouped MLA with selector up-projections (the
lesson's Chapter 2 construction applied per group, against the pinned GQA
oracle); the discussion's 1088 = 2 x 512 + 64.  No function here is parity
unpinned.
"""
from __future__ import annotations

import numpy as np

from .mla_oracle import _head_explicit, decode_storage, gather_sequence


def values_per_token(groups: int, d_latent: int, d_rope: int) -> int:
    """Cached values per token: every group's latent plus one rope key."""
    return groups * d_latent + d_rope


def group_of_head(i: int, heads: int, groups: int) -> int:
    """Reading G1."""
    if heads % groups:
        raise ValueError("heads must divide into the groups")
    return i // (heads // groups)


def grouped_decode(q, c_pools, scale_pools, k_rope, block_table, seq_lens, W_UK, W_UV, sm_scale,
                   page_size, q_tag="f32", cache_tag="f32", rope_tag="f32", weight_tag="f32",
                   batches=None, heads=None):
    """out[b, i, :]: head i decoded against latent pool c_pools[group_of_head(i)]
    ([G, num_blocks, P, d_c]; fp8 scales scale_pools [G, num_blocks, P]) and the
    shared k_rope.  Entries not computed are NaN."""
    G = c_pools.shape[0]
    B, h, _ = q.shape
    d_nope = W_UK.shape[1]
    Qf = decode_storage(q, q_tag)
    WK = decode_storage(W_UK, weight_tag)
    WV = decode_storage(W_UV, weight_tag)
    batches = range(B) if batches is None else batches
    heads = range(h) if heads is None else heads
    out = np.full((B, h, W_UV.shape[1]), np.nan, dtype=np.float64)
    for b in batches:
        rows = [gather_sequence(c_pools[g], k_rope, None if scale_pools is None else scale_pools[g],
                                block_table, seq_lens[b], b, page_size, cache_tag, rope_tag)
                for g in range(G)]
        for i in heads:
            C, R = rows[group_of_head(i, h, G)]
            out[b, i] = _head_explicit(Qf[b, i, :d_nope], Qf[b, i, d_nope:], C, R, WK[i], WV[i],
                                       float(sm_scale))
    return out
