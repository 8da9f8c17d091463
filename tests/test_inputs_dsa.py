"""The DSA input generator: deterministic, shapes, and NaN in every pool slot
that holds no token."""
import numpy as np

from mla_inputs.dsa import DSA_CONFIGS, generate_dsa


def test_dsa_inputs_are_seeded_and_poisoned():
    a = generate_dsa(DSA_CONFIGS["dsa_tiny"])
    b = generate_dsa(DSA_CONFIGS["dsa_tiny"])
    for f in ("q_I", "q_I_scale", "w_I", "k_I", "k_I_scale"):
        assert np.array_equal(getattr(a, f).view(np.uint8), getattr(b, f).view(np.uint8)), f
    cfg, d = a.cfg, a.dcfg
    assert a.q_I.shape == (cfg.batch, d.index_heads, d.index_dim)
    assert a.k_I.shape == (a.num_blocks, cfg.page_size, d.index_dim)
    used = np.zeros(a.k_I_scale.shape, bool)
    for s, T in enumerate(a.seq_lens):
        for t in range(int(T)):
            used[a.block_table[s, t // cfg.page_size], t % cfg.page_size] = True
    assert np.isfinite(a.k_I_scale[used]).all() and np.isnan(a.k_I_scale[~used]).all()
    assert (a.k_I[~used] == 0x7F).all()
    assert list(a.seq_lens) == list(d.seq_lens)
    # the dense part is the dense generator's (same seed, same lengths)
    assert a.q.shape == (cfg.batch, cfg.heads, cfg.d_nope + cfg.d_rope)
