"""Plain CPU oracle of MLA prefill in MHA mode: a chunk of new query tokens,
each attending causally to the cached tokens up to its own position, with the
keys and values reconstructed explicitly from the latent cache.

TEST INFRASTRUCTURE ONLY.  Imported by the tests and the benchmark's checks;
never by the HIP library, with which it shares no code.  Arithmetic is fp64.

Sources (cited by page title and section):
  [LESSON] "TransMLA & Sparse Latent Attention", Chapter 7 ("Bridging back to
           Session 03: DSA runs in MLA's MQA mode"): training and prefill run
           MLA in its MHA-like mode, reconstructing full-width keys and values,
           decode in the absorbed MQA-like mode; Chapter 6 ("Worked
           arithmetic"): the query at position t sees positions up to t.
  [TPLA]   "TPLA: Tensor Parallel Latent Attention ...", section 3.4 (Eq. 4,
           the unabsorbed form: k = W_UK c plus the decoupled rope key, v =
           W_UV c, scale 1 / sqrt(d_h + d_r)).

Readings: query l of sequence b (of L_b new tokens, T_b cached in all,
including the new ones) sits at position T_b - L_b + l and attends to positions
0 .. T_b - L_b + l; its rope part arrives rotated, as in decode.

Pins (tests/test_oracle_prefill_pins.py, CPU only): every query row equals the
decode oracle run on the prefix it may see; the last row equals the decode
oracle on the whole sequence; tokens after a row's position do not change it.
No function here is parity unpinned.
"""
from __future__ import annotations

import numpy as np

from .mla_oracle import _head_explicit, decode_storage, gather_sequence


def query_position(seq_len: int, q_len: int, l: int) -> int:
    """Position of query l of a chunk of q_len new tokens in a sequence of
    seq_len cached tokens (reading above)."""
    return seq_len - q_len + l


def mha_prefill(q, q_lens, c_kv, c_kv_scale, k_rope, block_table, seq_lens, W_UK, W_UV,
                sm_scale, page_size, q_tag="f32", cache_tag="f32", rope_tag="f32",
                weight_tag="f32", batches=None, heads=None, rows=None):
    """out[b, l, i, :] for q [B, L, h, d_nope + d_rope]; rows l >= q_lens[b] and
    entries not computed are NaN.  `rows` optionally restricts the rows."""
    B, L, h, _ = q.shape
    d_nope = W_UK.shape[1]
    d_v = W_UV.shape[1]
    Qf = decode_storage(q, q_tag)
    WK = decode_storage(W_UK, weight_tag)
    WV = decode_storage(W_UV, weight_tag)
    batches = range(B) if batches is None else batches
    heads = range(h) if heads is None else heads
    out = np.full((B, L, h, d_v), np.nan, dtype=np.float64)
    for b in batches:
        T, Lb = int(seq_lens[b]), int(q_lens[b])
        C, R = gather_sequence(c_kv, k_rope, c_kv_scale, block_table, T, b, page_size, cache_tag,
                               rope_tag)
        for l in (range(Lb) if rows is None else [r for r in rows if r < Lb]):
            p = query_position(T, Lb, l)
            for i in heads:
                out[b, l, i] = _head_explicit(Qf[b, l, i, :d_nope], Qf[b, l, i, d_nope:],
                                              C[: p + 1], R[: p + 1], WK[i], WV[i],
                                              float(sm_scale))
    return out
