"""Pins of the DSA oracle (CPU only): the indexer score against a hand-worked
case and a loop over its definition, the selection against a rank-count brute
force and the pages' pair counts, and the sparse decode against the dense
oracle (k >= T, and a cache rebuilt from only the selected tokens)."""
import itertools

import numpy as np
import pytest

from mla_inputs.configs import MLAConfig
from mla_inputs.dsa import DSA_CONFIGS, generate_dsa
from mla_inputs.generate import generate
from oracle import mla_decode_explicit
from oracle.dsa import (dsa_decode, gather_index_keys, indexer_scores, pair_count,
                        sequence_index_scores, sparse_decode, topk_select)


# ------------------------------------------------------------------ indexer

def test_indexer_hand_worked(golden):
    g = golden("dsa_indexer_toy.json")
    got = indexer_scores(np.array(g["q_I"]), np.array(g["w"]), np.array(g["keys"]))
    assert np.array_equal(got, np.array(g["scores"]))
    assert list(topk_select(got, 2)) == g["top2"]
    assert list(topk_select(got, 3)) == g["top3"]


def test_indexer_matches_loop_over_definition():
    """Plain Python loops over heads, dimensions and candidates."""
    rng = np.random.default_rng(11)
    H, d, T = 5, 7, 9
    q, w, K = rng.standard_normal((H, d)), rng.standard_normal(H), rng.standard_normal((T, d))
    want = []
    for s in range(T):
        tot = 0.0
        for j in range(H):
            dot = 0.0
            for i in range(d):
                dot += q[j, i] * K[s, i]
            tot += w[j] * (dot if dot > 0 else 0.0)
        want.append(tot)
    assert np.allclose(indexer_scores(q, w, K), want, rtol=1e-13, atol=1e-13)


def test_indexer_relu_properties():
    rng = np.random.default_rng(12)
    H, d, T = 6, 16, 20
    q, w, K = rng.standard_normal((H, d)), rng.standard_normal(H), rng.standard_normal((T, d))
    base = indexer_scores(q, w, K)
    # positive homogeneity in the key (the per-token scale factors out)
    assert np.allclose(indexer_scores(q, w, 3.5 * K), 3.5 * base, rtol=1e-12)
    # a head whose query opposes every key contributes nothing
    q2 = q.copy()
    q2[0] = -K.sum(axis=0) * 1e3
    K2 = K + 0.0
    keep = (K2 @ q2[0]) <= 0
    w_no0 = w.copy()
    w_no0[0] = 0.0
    assert np.allclose(indexer_scores(q2, w, K2)[keep], indexer_scores(q2, w_no0, K2)[keep])
    # a key equal to a single head's query with all other heads opposed: w_j |q_j|^2
    q3 = np.zeros((2, 3))
    q3[0] = [1.0, 2.0, 2.0]
    q3[1] = [-1.0, -2.0, -2.0]
    assert indexer_scores(q3, np.array([0.25, 7.0]), q3[:1])[0] == pytest.approx(0.25 * 9.0)
    # no softmax: scores of other candidates do not change a candidate's score
    assert np.allclose(indexer_scores(q, w, K[:5]), base[:5], rtol=1e-14)


# ------------------------------------------------------------------ top-k

def _rank_select(scores, k):
    """Brute force by definition: position s is kept when fewer than k
    positions beat it (a higher score, or an equal score earlier)."""
    T = len(scores)
    out = []
    for s in range(T):
        beat = sum(1 for u in range(T)
                   if scores[u] > scores[s] or (scores[u] == scores[s] and u < s))
        if beat < k:
            out.append(s)
    return out


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_rank_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    T = int(rng.integers(1, 40))
    # a few distinct values so that ties are common
    scores = rng.integers(-3, 4, size=T).astype(np.float64) * 0.5
    for k in (1, 2, 5, T - 1, T, T + 3):
        if k < 1:
            continue
        got = list(topk_select(scores, k))
        assert got == _rank_select(list(scores), k), (T, k)
        assert len(got) == min(T, k)


def test_topk_is_the_best_subset_on_tiny_inputs():
    """Among all subsets of size k, the selection has the largest score sum
    and, among those, the earliest positions."""
    rng = np.random.default_rng(7)
    for _ in range(20):
        T, k = int(rng.integers(2, 8)), int(rng.integers(1, 5))
        scores = rng.integers(0, 3, size=T).astype(np.float64)
        if k >= T:
            assert list(topk_select(scores, k)) == list(range(T))
            continue
        best = max(itertools.combinations(range(T), k),
                   key=lambda c: (sum(scores[list(c)]), [-x for x in c]))
        assert list(topk_select(scores, k)) == list(best)


def test_short_sequences_select_everything():
    s = np.random.default_rng(3).standard_normal(2048)
    assert np.array_equal(topk_select(s, 2048), np.arange(2048))
    assert np.array_equal(topk_select(s[:5], 2048), np.arange(5))
    assert topk_select(s[:0], 2048).shape == (0,)


def test_pair_counts_match_page(golden):
    g = golden("dsa_pair_counts.json")
    toy = g["toy"]
    # the toy by running the selection at every causal step
    rng = np.random.default_rng(0)
    pairs = sum(len(topk_select(rng.standard_normal(t), toy["k"])) for t in range(1, toy["L"] + 1))
    assert pairs == toy["dsa_pairs"]
    assert sum(range(1, toy["L"] + 1)) == toy["dense_pairs"]
    assert pair_count(toy["L"], toy["k"], sparse=True) == toy["dsa_pairs"]
    assert pair_count(toy["L"], toy["k"], sparse=False) == toy["dense_pairs"]
    assert round(toy["dense_pairs"] / toy["dsa_pairs"], 2) == toy["ratio_approx"]
    full = g["full"]
    L, k = full["L"], full["k"]
    assert pair_count(L, k, sparse=True) == full["dsa_pairs"]
    assert round(pair_count(L, k, False) / pair_count(L, k, True), 1) == full["ratio_approx"]
    # one late step: L candidates dense, k sparse -- checked through the selection
    assert L // len(topk_select(np.zeros(L), k)) == full["single_step_ratio"]
    for t in (1, k - 1, k, k + 1, 3 * k + 5):
        assert len(topk_select(rng.standard_normal(t), k)) == min(t, k)
    mid = g["mid"]
    assert round(pair_count(mid["L"], mid["k"], False) / pair_count(mid["L"], mid["k"], True),
                 1) == mid["ratio_approx"]


# ------------------------------------------------------------------ sparse decode

def _dense_cfg():
    return MLAConfig(name="pin", batch=3, heads=4, d_nope=8, d_latent=16, d_rope=4, d_v=8,
                     page_size=8, seq_len_range=(1, 2), cache_dtype="f32", q_dtype="f32",
                     rope_dtype="f32", weight_dtype="f32", seed=77)


def test_sparse_with_k_at_least_T_is_dense():
    """Lesson, Chapter 6: a sequence no longer than k selects everything and
    the step is identical to dense attention."""
    inp = generate(_dense_cfg(), seq_lens=[5, 21, 40])
    sel = [topk_select(np.zeros(int(T)), 64) for T in inp.seq_lens]
    cfg = inp.cfg
    want = mla_decode_explicit(inp.q, inp.c_kv, inp.c_kv_scale, inp.k_rope, inp.block_table,
                               inp.seq_lens, inp.W_UK, inp.W_UV, cfg.sm_scale, cfg.page_size)
    got = sparse_decode(inp.q, inp.c_kv, inp.c_kv_scale, inp.k_rope, inp.block_table, sel,
                        inp.W_UK, inp.W_UV, cfg.sm_scale, cfg.page_size)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-13)


def test_sparse_equals_dense_on_the_selected_tokens():
    """Rebuild a contiguous cache holding only the selected tokens (in position
    order) and run the dense oracle on it."""
    inp = generate(_dense_cfg(), seq_lens=[30, 17, 40])
    cfg = inp.cfg
    rng = np.random.default_rng(8)
    sel = [np.sort(rng.choice(int(T), size=min(int(T), 9), replace=False)) for T in inp.seq_lens]
    got = sparse_decode(inp.q, inp.c_kv, inp.c_kv_scale, inp.k_rope, inp.block_table, sel,
                        inp.W_UK, inp.W_UV, cfg.sm_scale, cfg.page_size)
    P = cfg.page_size
    for b in range(cfg.batch):
        n = len(sel[b])
        pages = (n + P - 1) // P
        c = np.zeros((pages, P, cfg.d_latent), np.float32)
        r = np.zeros((pages, P, cfg.d_rope), np.float32)
        for m, t in enumerate(sel[b]):
            blk, off = inp.block_table[b, t // P], t % P
            c[m // P, m % P] = inp.c_kv[blk, off]
            r[m // P, m % P] = inp.k_rope[blk, off]
        table = np.arange(pages, dtype=np.int32)[None, :]
        want = mla_decode_explicit(inp.q[b:b + 1], c, None, r, table, np.array([n]), inp.W_UK,
                                   inp.W_UV, cfg.sm_scale, P)
        assert np.allclose(got[b], want[0], rtol=1e-12, atol=1e-13)
    # a set function: the order of the list does not matter
    shuffled = [s[::-1].copy() for s in sel]
    again = sparse_decode(inp.q, inp.c_kv, inp.c_kv_scale, inp.k_rope, inp.block_table, shuffled,
                          inp.W_UK, inp.W_UV, cfg.sm_scale, cfg.page_size)
    assert np.allclose(again, got, rtol=1e-12, atol=1e-13)


def test_dsa_step_on_generated_inputs():
    """The composed step on the tiny workload: selection sizes min(T, k), the
    selected positions beat the rest under the scores, and the output equals
    the sparse decode over exactly that selection."""
    inp = generate_dsa(DSA_CONFIGS["dsa_tiny"])
    k = inp.topk
    out, sel, scores = dsa_decode(inp, k)
    for b, T in enumerate(inp.seq_lens):
        assert len(sel[b]) == min(int(T), k)
        rest = np.setdiff1d(np.arange(int(T)), sel[b])
        if len(rest):
            assert scores[b][sel[b]].min() >= scores[b][rest].max()
        # keys read back through the table are the stored rows
        K = gather_index_keys(inp.k_I, inp.k_I_scale, inp.block_table, T, b, inp.cfg.page_size)
        assert np.isfinite(K).all()
        assert np.array_equal(scores[b], sequence_index_scores(
            inp.q_I, inp.q_I_scale, inp.w_I, inp.k_I, inp.k_I_scale, inp.block_table,
            inp.seq_lens, inp.cfg.page_size, b))
    assert np.isfinite(out).all()


def test_index_keys_read_back_through_a_permuted_table():
    """Keys written page by page under a random physical permutation read back
    in logical order, scaled by their row's scale."""
    rng = np.random.default_rng(21)
    P, d, T = 4, 8, 23
    codes = rng.integers(0, 0x7E, size=(T, d), dtype=np.uint8)   # finite E4M3 codes
    codes[codes == 0x7F] = 0
    scale = rng.uniform(0.5, 2.0, size=T).astype(np.float32)
    pages = (T + P - 1) // P
    perm = rng.permutation(pages + 2)
    pool = np.full((pages + 2, P, d), 0x7F, np.uint8)
    pscale = np.full((pages + 2, P), np.nan, np.float32)
    for t in range(T):
        pool[perm[t // P], t % P] = codes[t]
        pscale[perm[t // P], t % P] = scale[t]
    table = perm[None, :pages].astype(np.int32)
    K = gather_index_keys(pool, pscale, table, T, 0, P)
    import torch
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(K, want * scale.astype(np.float64)[:, None])
