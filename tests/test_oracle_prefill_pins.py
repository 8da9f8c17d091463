"""Pins of the MHA-mode prefill oracle (CPU only): each row is the pinned
decode oracle on the prefix it may see (absorbed or not), and causality."""
import numpy as np

from mla_inputs.configs import MLAConfig
from mla_inputs.generate import generate
from oracle import mla_decode_absorbed, mla_decode_explicit
from oracle.prefill import mha_prefill, query_position


def _inputs(lens, L, seed=61):
    cfg = MLAConfig(name="pin", batch=len(lens), heads=3, d_nope=8, d_latent=16, d_rope=4, d_v=8,
                    page_size=8, seq_len_range=(1, 2), cache_dtype="f32", q_dtype="f32",
                    rope_dtype="f32", weight_dtype="f32", seed=seed)
    inp = generate(cfg, seq_lens=lens)
    rng = np.random.default_rng(seed + 1)
    q = rng.standard_normal((len(lens), L, cfg.heads, cfg.d_nope + cfg.d_rope)).astype(np.float32)
    return inp, q


def _prefill(inp, q, q_lens, **kw):
    c = inp.cfg
    return mha_prefill(q, q_lens, inp.c_kv, inp.c_kv_scale, inp.k_rope, inp.block_table,
                       inp.seq_lens, inp.W_UK, inp.W_UV, c.sm_scale, c.page_size, **kw)


def test_positions():
    assert query_position(10, 10, 0) == 0 and query_position(10, 10, 9) == 9
    assert query_position(25, 4, 0) == 21 and query_position(25, 4, 3) == 24


def test_every_row_is_decode_on_its_prefix():
    inp, q = _inputs([13, 21], L=6)
    q_lens = np.array([6, 4])
    got = _prefill(inp, q, q_lens)
    c = inp.cfg
    for b in range(2):
        T = int(inp.seq_lens[b])
        for l in range(int(q_lens[b])):
            p = query_position(T, int(q_lens[b]), l)
            lens = inp.seq_lens.copy()
            lens[b] = p + 1
            qq = np.repeat(q[:, l], 1, axis=0)
            for fn in (mla_decode_explicit, mla_decode_absorbed):
                want = fn(qq, inp.c_kv, None, inp.k_rope, inp.block_table, lens, inp.W_UK,
                          inp.W_UV, c.sm_scale, c.page_size, batches=[b])
                assert np.allclose(got[b, l], want[b], rtol=1e-11, atol=1e-12), (b, l)
        assert np.isnan(got[b, int(q_lens[b]):]).all()


def test_future_tokens_do_not_matter():
    inp, q = _inputs([17], L=5)
    base = _prefill(inp, q, np.array([5]))
    # overwrite the last cached token: only the last row may change
    T = int(inp.seq_lens[0])
    blk, off = inp.block_table[0, (T - 1) // 8], (T - 1) % 8
    inp.c_kv[blk, off] += 3.0
    moved = _prefill(inp, q, np.array([5]))
    assert np.array_equal(moved[0, :4], base[0, :4])
    assert not np.allclose(moved[0, 4], base[0, 4])
