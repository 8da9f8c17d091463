"""Pins of the TPLA oracle (CPU only): the dense limit, the page's equality
condition, a hand-worked case, the Sylvester matrices and the page's
counterexample, basis invariance of the dense step, and the page's per-device
cache figures."""
import numpy as np

from mla_inputs.configs import MLAConfig
from mla_inputs.generate import generate
from oracle import mla_decode_explicit
from oracle.tpla import (cache_values_per_device, hadamard, orthonormal_hadamard,
                         reparameterize, shard_slices, tpla_decode, tpla_latent)


def _cfg(**kw):
    d = dict(name="pin", batch=2, heads=3, d_nope=8, d_latent=16, d_rope=4, d_v=8, page_size=8,
             seq_len_range=(1, 2), cache_dtype="f32", q_dtype="f32", rope_dtype="f32",
             weight_dtype="f32", seed=91)
    d.update(kw)
    return MLAConfig(**d)


def _dense(inp):
    c = inp.cfg
    return mla_decode_explicit(inp.q, inp.c_kv, inp.c_kv_scale, inp.k_rope, inp.block_table,
                               inp.seq_lens, inp.W_UK, inp.W_UV, c.sm_scale, c.page_size)


def _tpla(inp, shards=2, mu=None):
    c = inp.cfg
    return tpla_decode(inp.q, inp.c_kv, inp.c_kv_scale, inp.k_rope, inp.block_table,
                       inp.seq_lens, inp.W_UK, inp.W_UV, c.sm_scale, c.page_size, shards=shards,
                       mu=mu)


def test_hand_worked_two_tokens(golden):
    g = golden("tpla_toy.json")
    got = tpla_latent(np.array(g["q_lat"]), np.array(g["q_rope"]), np.array(g["C"]),
                      np.array(g["R"]), g["sm_scale"], shards=2)
    assert np.allclose(got, g["tpla"], rtol=0, atol=g["tolerance"])
    one = tpla_latent(np.array(g["q_lat"]), np.array(g["q_rope"]), np.array(g["C"]),
                      np.array(g["R"]), g["sm_scale"], shards=1)
    assert np.allclose(one, g["dense"], rtol=0, atol=g["tolerance"])


def test_one_shard_is_the_dense_step():
    inp = generate(_cfg(), seq_lens=[9, 30])
    assert np.allclose(_tpla(inp, shards=1), _dense(inp), rtol=1e-12, atol=1e-13)


def test_constant_missing_shard_gives_the_dense_step():
    """The page: the per-shard softmaxes equal the joint one when the other
    shard adds the same score to every token.  With every token's shard-1
    latent equal, shard 1's score is constant and its weighted sum is that
    row, so both shards reproduce the dense result."""
    inp = generate(_cfg(), seq_lens=[12, 25])
    S1 = shard_slices(inp.cfg.d_latent, 2)[1]
    row = np.random.default_rng(3).standard_normal(S1.stop - S1.start).astype(np.float32)
    for b, T in enumerate(inp.seq_lens):
        for t in range(int(T)):
            inp.c_kv[inp.block_table[b, t // 8], t % 8, S1] = row
    assert np.allclose(_tpla(inp), _dense(inp), rtol=1e-11, atol=1e-12)


def test_tpla_differs_from_dense_in_general():
    inp = generate(_cfg(), seq_lens=[20, 31])
    assert np.max(np.abs(_tpla(inp) - _dense(inp))) > 1e-3


def test_zero_content_factor_attends_by_position_only():
    """mu_j = 0 leaves shard j weighted by the positional scores alone."""
    rng = np.random.default_rng(5)
    q_lat, q_rope = rng.standard_normal(8), rng.standard_normal(2)
    C, R = rng.standard_normal((6, 8)), rng.standard_normal((6, 2))
    got = tpla_latent(q_lat, q_rope, C, R, 0.7, shards=2, mu=[0.0, 1.0])
    p = np.exp(0.7 * (R @ q_rope))
    p /= p.sum()
    assert np.allclose(got[:4], p @ C[:, :4], rtol=1e-12)


def test_sylvester_hadamard():
    H4 = hadamard(4)
    assert np.array_equal(H4, [[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]])
    for d in (1, 2, 8, 64, 512):
        H = hadamard(d)
        assert np.array_equal(H @ H.T, d * np.eye(d))
        if d > 1:
            h = hadamard(d // 2)
            assert np.array_equal(H, np.block([[h, h], [h, -h]]))


def test_page_counterexample(golden):
    g = golden("tpla_page_figures.json")["counterexample"]
    U = orthonormal_hadamard(4)
    Qp, cp = np.array(g["Q"]) @ U, np.array(g["c"]) @ U
    assert np.allclose(Qp, g["Q_prime"]) and np.allclose(cp, g["c_prime"])
    prod = Qp * cp
    assert np.allclose(prod, g["product"])
    halves = [prod[S].sum() for S in shard_slices(4, 2)]
    assert np.allclose(halves, g["half_sums"]) and abs(prod.sum() - g["full"]) < 1e-9


def test_change_of_basis_leaves_the_dense_step_unchanged():
    inp = generate(_cfg(), seq_lens=[17, 24])
    c = inp.cfg
    signs = np.random.default_rng(8).choice([-1.0, 1.0], c.d_latent)
    U = orthonormal_hadamard(c.d_latent, signs)
    assert np.allclose(U @ U.T, np.eye(c.d_latent), atol=1e-14)
    C2, WK2, WV2 = reparameterize(U, inp.c_kv, inp.W_UK, inp.W_UV)
    got = mla_decode_explicit(inp.q, C2, None, inp.k_rope, inp.block_table, inp.seq_lens, WK2,
                              WV2, c.sm_scale, c.page_size, cache_tag="f64", weight_tag="f64")
    assert np.allclose(got, _dense(inp), rtol=1e-11, atol=1e-12)
    t2 = tpla_decode(inp.q, C2, None, inp.k_rope, inp.block_table, inp.seq_lens, WK2, WV2,
                     c.sm_scale, c.page_size, cache_tag="f64", weight_tag="f64")
    assert np.max(np.abs(t2 - _tpla(inp))) > 1e-4     # TPLA depends on the basis


def test_page_per_device_cache(golden):
    g = golden("tpla_page_figures.json")["per_device"]
    n = cache_values_per_device(g["d_c"], g["d_r"], g["shards"])
    assert n == g["values_per_token"]
    mla = g["tokens"] * (g["d_c"] + g["d_r"]) * g["bytes_per_value"] / 1e6
    tpla = g["tokens"] * n * g["bytes_per_value"] / 1e6
    assert round(mla, 1) == g["mla_tp_MB"] and round(tpla, 1) == g["tpla_MB"]
    assert round(mla / tpla, 1) == g["ratio"]
