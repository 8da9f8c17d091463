"""Seeded input generator: determinism, layout, poisoning and storage rounding (no GPU)."""
import numpy as np
import pytest
import torch

from mla_inputs import CONFIGS, generate
from mla_inputs.generate import quantize_e4m3_rows, repermute, round_to
from oracle import decode_storage, oracle_from_inputs


def _small(name, **kw):
    cfg = CONFIGS[name]
    small = dict(batch=3, heads=min(cfg.heads, 4), d_nope=16, d_latent=32, d_rope=8, d_v=16,
                 seq_len=None, seq_len_range=(1, 150), page_size=16)
    small.update(kw)
    return cfg.replace(**small)


def test_deterministic():
    cfg = _small("dsv3_ragged_32k")
    a, b = generate(cfg), generate(cfg)
    for f in ("seq_lens", "block_table", "q", "c_kv", "k_rope", "W_UK", "W_UV"):
        assert np.array_equal(getattr(a, f).view(np.uint8), getattr(b, f).view(np.uint8)), f


def test_table_is_injective_and_padding_points_at_poison():
    cfg = _small("dsv3_ragged_32k")
    inp = generate(cfg)
    P = cfg.page_size
    used = []
    for b, T in enumerate(inp.seq_lens):
        n = -(-int(T) // P)
        used.extend(inp.block_table[b, :n].tolist())
        assert np.all(inp.block_table[b, n:] == inp.poison_block)
    assert len(used) == len(set(used))
    assert inp.poison_block not in used


def test_unused_slots_are_nan():
    cfg = _small("dsv3_fp8_16k", cache_dtype="e4m3")
    inp = generate(cfg)
    P = cfg.page_size
    C = decode_storage(inp.c_kv, "e4m3")
    R = decode_storage(inp.k_rope, "bf16")
    live = np.zeros(inp.c_kv.shape[:2], bool)
    for b, T in enumerate(inp.seq_lens):
        for t in range(int(T)):
            live[inp.block_table[b, t // P], t % P] = True
    assert np.all(np.isnan(C[~live])) and np.all(np.isnan(R[~live]))
    assert np.all(np.isnan(inp.c_kv_scale[~live]))
    assert np.all(np.isfinite(C[live])) and np.all(np.isfinite(R[live]))


def test_bf16_rounding_is_nearest():
    x = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
    y = decode_storage(round_to("bf16", x), "bf16")
    assert np.all(np.abs(y - x) <= np.abs(x) * 2.0 ** -8)   # half an ulp of an 8-bit significand


def test_e4m3_quantizer_properties():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((200, 64)).astype(np.float32)
    x[3] = 0.0                                   # all-zero row
    codes, scale = quantize_e4m3_rows(x)
    assert scale[3] == 0 and np.all(codes[3] == 0)
    deq = decode_storage(codes, "e4m3") * scale[:, None].astype(np.float64)
    amax_idx = np.argmax(np.abs(x), axis=1)
    for r in range(200):
        if r == 3:
            continue
        assert abs(decode_storage(codes[r, amax_idx[r]:amax_idx[r] + 1], "e4m3")[0]) == 448.0
    s = np.broadcast_to(scale[:, None].astype(np.float64), x.shape)
    normal = np.abs(x) >= s * 2.0 ** -6          # e4m3 normal range, relative bound
    err = np.abs(deq - x)
    assert np.all(err[normal] <= np.abs(x[normal]) * 2.0 ** -4 * (1 + 1e-6))
    assert np.all(err[~normal] <= s[~normal] * 2.0 ** -10 * (1 + 1e-6))  # half a subnormal step


def test_e4m3_quantizer_matches_torch_dequant():
    x = np.random.default_rng(2).standard_normal((10, 32)).astype(np.float32)
    codes, scale = quantize_e4m3_rows(x)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(ref, decode_storage(codes, "e4m3"))


def test_repermute_keeps_oracle_output_bitwise():
    cfg = _small("dsv3_ragged_32k")
    inp = generate(cfg)
    other = repermute(inp, seed=77)
    assert not np.array_equal(inp.block_table, other.block_table)
    a = oracle_from_inputs(inp)
    b = oracle_from_inputs(other)
    assert np.array_equal(a, b)


def test_configs_match_workloads():
    c = CONFIGS
    assert (c["tiny_fp32"].batch, c["tiny_fp32"].heads, c["tiny_fp32"].d_latent) == (2, 4, 32)
    assert c["transmla_llama2_7b"].d_latent + c["transmla_llama2_7b"].d_rope == 576
    assert c["dsv3_b64_4k"].heads == 128 and c["dsv3_b64_4k"].batch == 64
    assert c["dsv3_ragged_32k"].seq_len_range == (1024, 32768)
    assert c["dsv3_fp8_16k"].cache_dtype == "e4m3"
    assert abs(c["dsv3_b64_4k"].sm_scale - 1 / np.sqrt(192)) < 1e-15


@pytest.mark.parametrize("lens", [[0, 5, 16], [1, 1, 1], [17, 0, 0]])
def test_explicit_lengths(lens):
    inp = generate(_small("dsv3_ragged_32k"), seq_lens=lens)
    assert inp.seq_lens.tolist() == lens
    out = oracle_from_inputs(inp)
    for b, T in enumerate(lens):
        if T == 0:
            assert np.all(out[b] == 0)
        else:
            assert np.all(np.isfinite(out[b]))
