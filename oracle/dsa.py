"""Plain CPU oracle of DeepSeek Sparse Attention (DSA) at decode time: the
lightning indexer, the top-k token selection, and MLA decode over the
selected tokens.

TEST INFRASTRUCTURE ONLY.  Imported by the tests and the benchmark's checks;
never by the HIP library, with which it shares no code.  Arithmetic is fp64.

Source (cited by page title and section):
  [LESSON] "TransMLA & Sparse Latent Attention", Chapter 6 "DeepSeek's Second
           Wall":
             - "The lightning indexer": the index score of a candidate position
               s for the current token is a weighted sum over the H_I indexer
               heads of ReLU(q_j . k_s); no softmax, no row-wide pass (the
               section's `indexer_score` listing computes exactly this).
               H_I = 64, d_I = 128, run in FP8.
             - "Fine-grained token selection": keep the k highest-scoring
               positions (k = 2048) and run attention over only those.
             - "Worked arithmetic" and "A sanity check ... by hand": a query
               at step t sees min(t, k) candidates; the pair counts 55 / 27
               (L = 10, k = 3) and 266,339,328 (L = 131,072, k = 2,048); a
               sequence no longer than k selects everything, identically to
               dense attention.
           Chapter 7, "Bridging back to Session 03: DSA runs in MLA's MQA
           mode": one selection per token, shared by every query head, on the
           absorbed decode path; each cached position keeps a d_I = 128 wide
           indexer key beside its latent.

Readings taken where the pages are silent:
  * D1: the indexer query and key are E4M3FN codes with an fp32 scale, one
    per (sequence, indexer head) for the query and one per cached token for
    the key (the same per-row rule as the latent cache); the oracle computes
    on the decoded values.  The head weights w are fp32 and may be negative.
  * D2: equal scores are ordered by position, the earlier position first; the
    selected positions are returned in increasing order.
  * D3: the candidates are the sequence's cached positions 0 .. T-1 (the new
    token is already cached, as for the dense decode step).
  * D4: the attention over the selection is the dense decode step's formula
    (the decoupled rope score, one softmax per head) restricted to the
    selected positions.

Pins (tests/test_oracle_dsa_pins.py, CPU only): a hand-computed index score,
a pure-Python loop over the definition, the ReLU's positive homogeneity and
its zeroing of opposed heads, a rank-count brute force of the selection with
ties, the pages' pair counts, k >= T equal to the dense oracle, and the sparse
decode equal to the dense oracle on a cache rebuilt from only the selected
tokens.  No function here is parity unpinned.
"""
from __future__ import annotations

import numpy as np

from .mla_oracle import _head_explicit, decode_storage


# --------------------------------------------------------------------------
# lightning indexer
# --------------------------------------------------------------------------

def indexer_scores(q_I: np.ndarray, w: np.ndarray, K_I: np.ndarray) -> np.ndarray:
    """[LESSON] Chapter 6, "The lightning indexer": the index score of a
    candidate key is a weighted sum over the indexer heads of the rectified
    query-key inner product (no softmax anywhere).
    q_I [H_I, d_I], w [H_I], K_I [T, d_I]; returns [T] in fp64."""
    q = np.asarray(q_I, dtype=np.float64)
    k = np.asarray(K_I, dtype=np.float64)
    rectified = np.maximum(np.einsum("hd,td->th", q, k), 0.0)
    return np.einsum("th,h->t", rectified, np.asarray(w, dtype=np.float64))


def decode_scaled_e4m3(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """E4M3FN codes [..., d] times their per-row fp32 scale [...] (reading D1)."""
    return decode_storage(codes, "e4m3") * np.asarray(scale, dtype=np.float64)[..., None]


def gather_index_keys(k_I_pool, k_I_scale, block_table, seq_len, b, page_size):
    """Decoded indexer keys of sequence b's positions 0 .. T-1 through the
    block table (position t in block block_table[b][t // P], slot t % P)."""
    T = int(seq_len)
    d = k_I_pool.shape[-1]
    K = np.empty((T, d), dtype=np.float64)
    for t in range(0, T, page_size):
        blk = int(block_table[b][t // page_size])
        n = min(page_size, T - t)
        K[t: t + n] = decode_scaled_e4m3(k_I_pool[blk, :n], k_I_scale[blk, :n])
    return K


def sequence_index_scores(q_codes, q_scale, w, k_I_pool, k_I_scale, block_table, seq_lens,
                          page_size, b):
    """Index scores of every cached position of sequence b (reading D1, D3)."""
    q = decode_scaled_e4m3(q_codes[b], q_scale[b])
    K = gather_index_keys(k_I_pool, k_I_scale, block_table, seq_lens[b], b, page_size)
    return indexer_scores(q, w[b], K)


# --------------------------------------------------------------------------
# top-k selection
# --------------------------------------------------------------------------

def topk_select(scores: np.ndarray, k: int) -> np.ndarray:
    """[LESSON] Chapter 6, "Fine-grained token selection": the k highest
    scores; ties go to the earlier position (reading D2).  Returns the chosen
    positions in increasing order, min(T, k) of them."""
    s = np.asarray(scores)
    T = s.shape[0]
    if T <= k:
        return np.arange(T, dtype=np.int64)
    # order by score descending, then position ascending (lexsort: last key first)
    order = np.lexsort((np.arange(T), -s.astype(np.float64)))
    return np.sort(order[:k]).astype(np.int64)


def pair_count(L: int, k: int, sparse: bool) -> int:
    """Query-key pairs over a causal generation of L tokens, where the query
    at step t sees t candidates (dense) or min(t, k) (sparse) — [LESSON]
    Chapter 6, "Worked arithmetic"; counted with topk_select's rule in
    closed form (sum of min(t, k))."""
    if not sparse:
        return L * (L + 1) // 2
    m = min(L, k)
    return m * (m + 1) // 2 + (L - m) * k


# --------------------------------------------------------------------------
# MLA decode over the selected tokens
# --------------------------------------------------------------------------

def gather_positions(c_kv, k_rope, c_kv_scale, block_table, positions, b, page_size,
                     cache_tag, rope_tag):
    """Decoded latent rows and rope keys of sequence b at the given positions."""
    pos = np.asarray(positions, dtype=np.int64)
    d_c, d_r = c_kv.shape[-1], k_rope.shape[-1]
    C = np.empty((pos.shape[0], d_c), dtype=np.float64)
    R = np.empty((pos.shape[0], d_r), dtype=np.float64)
    for n, t in enumerate(pos):
        blk, off = int(block_table[b][t // page_size]), int(t % page_size)
        C[n] = decode_storage(c_kv[blk, off], cache_tag)
        if cache_tag == "e4m3":
            C[n] *= float(c_kv_scale[blk, off])
        R[n] = decode_storage(k_rope[blk, off], rope_tag)
    return C, R


def sparse_decode(q, c_kv, c_kv_scale, k_rope, block_table, selections, W_UK, W_UV, sm_scale,
                  page_size, q_tag="f32", cache_tag="f32", rope_tag="f32", weight_tag="f32",
                  batches=None, heads=None):
    """out[b, i, :] of the decode step attending only to the positions
    selections[b] (reading D4; [LESSON] Chapter 7: one selection shared by all
    heads).  Same shapes as the dense oracle; entries not computed are NaN."""
    B, h, _ = q.shape
    d_nope = W_UK.shape[1]
    d_v = W_UV.shape[1]
    Qf = decode_storage(q, q_tag)
    WK = decode_storage(W_UK, weight_tag)
    WV = decode_storage(W_UV, weight_tag)
    batches = range(B) if batches is None else batches
    heads = range(h) if heads is None else heads
    out = np.full((B, h, d_v), np.nan, dtype=np.float64)
    for b in batches:
        C, R = gather_positions(c_kv, k_rope, c_kv_scale, block_table, selections[b], b,
                                page_size, cache_tag, rope_tag)
        for i in heads:
            out[b, i] = _head_explicit(Qf[b, i, :d_nope], Qf[b, i, d_nope:], C, R, WK[i], WV[i],
                                       float(sm_scale))
    return out


def dsa_decode(inp, k: int, batches=None, heads=None):
    """The whole DSA decode step for a generated input set: index scores,
    top-k, and the sparse decode.  Returns (out, selections, scores)."""
    cfg = inp.cfg
    B = inp.q.shape[0]
    scores, sel = [], []
    for b in range(B):
        s = sequence_index_scores(inp.q_I, inp.q_I_scale, inp.w_I, inp.k_I, inp.k_I_scale,
                                  inp.block_table, inp.seq_lens, cfg.page_size, b)
        scores.append(s)
        sel.append(topk_select(s, k))
    out = sparse_decode(inp.q, inp.c_kv, inp.c_kv_scale, inp.k_rope, inp.block_table, sel,
                        inp.W_UK, inp.W_UV, cfg.sm_scale, cfg.page_size, q_tag=cfg.q_dtype,
                        cache_tag=cfg.cache_dtype, rope_tag=cfg.rope_dtype,
                        weight_tag=cfg.weight_dtype, batches=batches, heads=heads)
    return out, sel, scores
