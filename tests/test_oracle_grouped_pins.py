"""Pins of the grouped-MLA oracle (CPU only)."""
import numpy as np

from mla_inputs.configs import MLAConfig
from mla_inputs.generate import generate
from oracle import build_selectors, gqa_decode, mla_decode_explicit
from oracle.grouped import group_of_head, grouped_decode, values_per_token


def _cfg(**kw):
    d = dict(name="pin", batch=2, heads=4, d_nope=8, d_latent=16, d_rope=4, d_v=8, page_size=8,
             seq_len_range=(1, 2), cache_dtype="f32", q_dtype="f32", rope_dtype="f32",
             weight_dtype="f32", seed=131)
    d.update(kw)
    return MLAConfig(**d)


def _pools(inp, G, seed):
    """G latent pools: the generated one first, then seeded others."""
    rng = np.random.default_rng(seed)
    extra = [rng.standard_normal(inp.c_kv.shape).astype(np.float32) for _ in range(G - 1)]
    return np.stack([inp.c_kv] + extra)


def _grouped(inp, pools):
    c = inp.cfg
    return grouped_decode(inp.q, pools, None, inp.k_rope, inp.block_table, inp.seq_lens, inp.W_UK,
                          inp.W_UV, c.sm_scale, c.page_size)


def _dense(inp, c_kv=None):
    c = inp.cfg
    return mla_decode_explicit(inp.q, inp.c_kv if c_kv is None else c_kv, None, inp.k_rope,
                               inp.block_table, inp.seq_lens, inp.W_UK, inp.W_UV, c.sm_scale,
                               c.page_size)


def test_kv_rank_of_the_discussion(golden):
    g = golden("grouped_kv_rank.json")
    assert values_per_token(g["groups"], g["d_latent"], g["d_rope"]) == g["kv_rank"]
    assert values_per_token(1, g["d_latent"], g["d_rope"]) == g["per_group_as_served"]


def test_one_group_is_dense():
    inp = generate(_cfg(), seq_lens=[11, 26])
    assert np.allclose(_grouped(inp, inp.c_kv[None]), _dense(inp), rtol=1e-12, atol=1e-13)


def test_equal_pools_give_dense():
    inp = generate(_cfg(), seq_lens=[19, 7])
    assert np.allclose(_grouped(inp, np.stack([inp.c_kv] * 2)), _dense(inp), rtol=1e-12,
                       atol=1e-13)


def test_a_head_reads_only_its_group():
    inp = generate(_cfg(), seq_lens=[19, 23])
    pools = _pools(inp, 2, 5)
    base = _grouped(inp, pools)
    pools2 = pools.copy()
    pools2[1] += 1.0
    moved = _grouped(inp, pools2)
    h = inp.cfg.heads
    for i in range(h):
        same = np.allclose(moved[:, i], base[:, i], rtol=0, atol=0)
        assert same == (group_of_head(i, h, 2) == 0), i
    # group 0's heads see the dense result of pool 0, group 1's that of pool 1
    d0, d1 = _dense(inp, pools[0]), _dense(inp, pools[1])
    assert np.allclose(base[:, : h // 2], d0[:, : h // 2], rtol=1e-12, atol=1e-13)
    assert np.allclose(base[:, h // 2:], d1[:, h // 2:], rtol=1e-12, atol=1e-13)


def test_gqa_is_grouped_mla_with_selectors():
    """Lesson Chapter 2 per group: group j's latent holds [k_j, v_j]; the
    selectors pick the key and value halves, and grouped MLA reproduces GQA."""
    rng = np.random.default_rng(17)
    h, G, d, T, P = 6, 3, 4, 13, 4
    q = rng.standard_normal((h, d))
    K, V = rng.standard_normal((T, G, d)), rng.standard_normal((T, G, d))
    want = gqa_decode(q, K, V, 0.5)
    pages = (T + P - 1) // P
    pools = np.zeros((G, pages, P, 2 * d))
    for t in range(T):
        pools[:, t // P, t % P, :d] = K[t]
        pools[:, t // P, t % P, d:] = V[t]
    WK1, WV1 = build_selectors(1, 1, d)          # one group of width 2d: [k, v]
    W_UK = np.repeat(WK1, h, axis=0)
    W_UV = np.repeat(WV1, h, axis=0)
    got = grouped_decode(q[None], pools, None, np.zeros((pages, P, 0)),
                         np.arange(pages, dtype=np.int32)[None], np.array([T]), W_UK, W_UV, 0.5,
                         P, cache_tag="f64", weight_tag="f64", q_tag="f64", rope_tag="f64")
    assert np.allclose(got[0], want, rtol=1e-12, atol=1e-13)
