"""Pins of the CPU oracle to what the pages and the mathematics fix (no GPU).

Each test checks the oracle against something other than itself: values the
pages print (tests/golden), an independently written grouped-query attention,
closed forms, a long-double brute force, or torch's own storage casts.
"""
import math

import numpy as np
import pytest
import torch

from oracle import (bf16_bits_to_f64, build_selectors, decode_storage, e4m3_code_to_f64,
                    gqa_decode, mla_decode_absorbed, mla_decode_explicit, softmax)


def _contiguous_single(C, R, P=None):
    """Pack one sequence's fp64 rows into a one-sequence paged pool (identity table)."""
    T = C.shape[0]
    P = P or max(T, 1)
    nb = max(1, -(-T // P))
    ck = np.zeros((nb, P, C.shape[1]), dtype=np.float32)
    kr = np.zeros((nb, P, R.shape[1]), dtype=np.float32)
    ck.reshape(nb * P, C.shape[1])[:T] = C
    kr.reshape(nb * P, R.shape[1])[:T] = R
    table = np.arange(nb, dtype=np.int32)[None, :]
    return ck, kr, table, P


def _mla(q, C, R, W_UK, W_UV, sm_scale, P=None, absorbed=False):
    """Run the oracle on one sequence given as fp32-exact rows."""
    ck, kr, table, P = _contiguous_single(C, R, P)
    fn = mla_decode_absorbed if absorbed else mla_decode_explicit
    return fn(q[None].astype(np.float32), ck, None, kr, table,
              np.array([C.shape[0]], np.int32), W_UK.astype(np.float32),
              W_UV.astype(np.float32), sm_scale, P)[0]


# ---------------------------------------------------------------- page values

def test_gqa_toy_direct(golden):
    g = golden("gqa_toy.json")
    q = np.array(g["queries"])[:, None]
    K = np.array(g["group_keys"])[None, :, None]
    V = np.array(g["group_values"])[None, :, None]
    out = gqa_decode(q, K, V, 1.0)
    assert out[:, 0].tolist() == g["expected_outputs"]


def test_gqa_toy_through_mla_selectors(golden):
    g = golden("gqa_toy.json")
    h, G, d = g["h"], g["g"], g["d"]
    W_UK, W_UV = build_selectors(h, G, d)
    latent = np.array(g["group_keys"] + g["group_values"])[None, :]   # one token, width 2gd
    q = np.array(g["queries"])[:, None]                              # q_nope, d_rope = 0
    out = _mla(q, latent, np.zeros((1, 0)), W_UK, W_UV, 1.0)
    assert out[:, 0].tolist() == g["expected_outputs"]


def test_selector_reconstruction_toy(golden):
    g = golden("selector_toy.json")
    W_UK, W_UV = build_selectors(g["h"], g["g"], g["d"])
    c = np.array(g["latent"])
    for r in g["reconstructions"]:
        i = r["head_index"]
        assert (W_UK[i] @ c).tolist() == r["key"]
        if "value" in r:
            assert (W_UV[i] @ c).tolist() == r["value"]


def test_selector_group_of_head_index(golden):
    g = golden("selector_assert.json")
    h, G, d = g["h"], g["g"], g["d"]
    W_UK, _ = build_selectors(h, G, d)
    rng = np.random.default_rng(0)
    keys = rng.standard_normal(G * d)           # concatenated group keys
    W = W_UK[g["head_index"], :, : G * d]       # key half of the selector
    j = g["expected_group"]
    assert np.array_equal(W @ keys, keys[j * d:(j + 1) * d])


def test_dense_blend_one_token(golden):
    """One cached token: softmax weight 1, output = W_UV c (explicit decompression)."""
    g = golden("blend_toy.json")
    W = np.array(g["up_projection"])[None]       # one head, d_v = 2, d_c = 4
    c = np.array(g["latent"])[None, :]
    out = _mla(np.array([[1.0, -2.0]]), c, np.zeros((1, 0)), W, W, 0.7)
    assert out[0].tolist() == g["expected"]


def test_rope_scores_match_page(golden):
    """Positional scores of pre-rotated keys (content term off) reproduce the
    page's 0.540 / 0.284, seen through the softmax weights of the output."""
    g = golden("rope_toy.json")
    th = g["theta"]
    R = np.array([[math.cos(t * th), math.sin(t * th)] for t in g["positions"]])  # R(t) [1,0]
    C = np.eye(2)                                  # latent rows pick out each token's weight
    W_UK = np.zeros((1, 1, 2))
    W_UV = np.eye(2)[None]
    q = np.array([[0.0] + g["query"]])             # q_nope = 0, q_rope = [1, 0]
    out = _mla(q, C, R, W_UK, W_UV, 1.0)[0]
    want = softmax(np.array(g["scores"]))
    # each printed score is off by at most `rounding`; the weights move by < 2x that
    assert np.max(np.abs(out - want)) < 2 * g["rounding"]
    assert np.all(np.abs(np.log(out[0] / out[1]) - (g["scores"][0] - g["scores"][1]))
                  < 2 * g["rounding"])


# ---------------------------------------------------------- identities

def _random_gqa(rng, h, G, d, T):
    q = rng.standard_normal((h, d))
    K = rng.standard_normal((T, G, d))
    V = rng.standard_normal((T, G, d))
    return q, K, V


@pytest.mark.parametrize("h,G,d,T,P", [(8, 2, 4, 7, 3), (4, 4, 3, 5, 2), (6, 1, 5, 9, 4),
                                       (32, 8, 16, 33, 16)])
def test_gqa_equals_mla_with_selectors(h, G, d, T, P):
    """GQA rewritten with identity selectors computes the same outputs."""
    rng = np.random.default_rng(h * 100 + T)
    q, K, V = _random_gqa(rng, h, G, d, T)
    # fp32-exact inputs so the fp32 pool holds them unchanged
    q, K, V = (x.astype(np.float32).astype(np.float64) for x in (q, K, V))
    ref = gqa_decode(q, K, V, 1 / math.sqrt(d))
    W_UK, W_UV = build_selectors(h, G, d)
    latent = np.concatenate([K.reshape(T, G * d), V.reshape(T, G * d)], axis=1)
    out = _mla(q, latent, np.zeros((T, 0)), W_UK, W_UV, 1 / math.sqrt(d), P=P)
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-13)


def test_gqa_with_shared_rope_part_equals_mla():
    """Keys whose last d_r dims are shared by every group (a decoupled rope key)
    map to MLA with the shared part as k_rope: pins the positional term."""
    rng = np.random.default_rng(7)
    h, G, da, dr, T = 8, 2, 4, 3, 6
    q = rng.standard_normal((h, da + dr)).astype(np.float32).astype(np.float64)
    Ka = rng.standard_normal((T, G, da)).astype(np.float32).astype(np.float64)
    Kr = rng.standard_normal((T, dr)).astype(np.float32).astype(np.float64)
    V = rng.standard_normal((T, G, da)).astype(np.float32).astype(np.float64)
    K = np.concatenate([Ka, np.repeat(Kr[:, None, :], G, axis=1)], axis=2)
    Vpad = np.concatenate([V, np.zeros((T, G, dr))], axis=2)
    sm = 1 / math.sqrt(da + dr)
    ref = gqa_decode(q, K, Vpad, sm)[:, :da]
    W_UK, W_UV = build_selectors(h, G, da)
    latent = np.concatenate([Ka.reshape(T, -1), V.reshape(T, -1)], axis=1)
    out = _mla(q, latent, Kr, W_UK, W_UV, sm, P=4)
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_absorbed_equals_explicit(seed):
    rng = np.random.default_rng(seed)
    B, h, dn, dc, dr, dv, P = 3, 5, 6, 12, 4, 7, 4
    lens = np.array([9, 1, 13], np.int32)
    nb = 14
    ck = rng.standard_normal((nb, P, dc)).astype(np.float32)
    kr = rng.standard_normal((nb, P, dr)).astype(np.float32)
    table = rng.permutation(nb)[: 4 * B].reshape(B, 4).astype(np.int32)
    q = rng.standard_normal((B, h, dn + dr)).astype(np.float32)
    WK = rng.standard_normal((h, dn, dc)).astype(np.float32)
    WV = rng.standard_normal((h, dv, dc)).astype(np.float32)
    a = mla_decode_explicit(q, ck, None, kr, table, lens, WK, WV, 0.3, P)
    b = mla_decode_absorbed(q, ck, None, kr, table, lens, WK, WV, 0.3, P)
    np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------- closed forms

def _rand_head(rng, T, dn=5, dc=8, dr=3, dv=6):
    return (rng.standard_normal(dn + dr), rng.standard_normal((T, dc)),
            rng.standard_normal((T, dr)), rng.standard_normal((1, dn, dc)),
            rng.standard_normal((1, dv, dc)))


def _f32(*xs):
    return [np.asarray(x, np.float32).astype(np.float64) for x in xs]


def test_one_token_is_up_projected_latent():
    rng = np.random.default_rng(1)
    q, C, R, WK, WV = _f32(*_rand_head(rng, 1))
    out = _mla(q[None], C, R, WK, WV, 0.4)[0]
    np.testing.assert_allclose(out, WV[0] @ C[0], rtol=1e-13, atol=1e-14)


def test_zero_query_averages_tokens():
    rng = np.random.default_rng(2)
    q, C, R, WK, WV = _f32(*_rand_head(rng, 11))
    out = _mla(np.zeros_like(q)[None], C, R, WK, WV, 0.4)[0]
    np.testing.assert_allclose(out, WV[0] @ C.mean(axis=0), rtol=1e-12, atol=1e-13)


def test_dominant_token_takes_all_weight():
    rng = np.random.default_rng(3)
    q, C, R, WK, WV = _f32(*_rand_head(rng, 9))
    k = 4
    q = q.copy()
    q[5:] = 0.0
    R = R.copy()
    R[:] = 0.0
    R[k] = [1.0, 0.0, 0.0]
    q[5] = 60.0                                 # positional score of token k = 60*sm
    out = _mla(q[None], C, R, WK, WV, 1.0)[0]
    np.testing.assert_allclose(out, WV[0] @ C[k], rtol=1e-6, atol=1e-6)


def test_constant_score_shift_is_invisible():
    """An extra rope dimension adding the same amount to every token's score
    leaves the output unchanged (softmax shift invariance)."""
    rng = np.random.default_rng(4)
    q, C, R, WK, WV = _f32(*_rand_head(rng, 10))
    base = _mla(q[None], C, R, WK, WV, 0.5)[0]
    q2 = np.concatenate([q, [1.0]])
    R2 = np.concatenate([R, np.full((R.shape[0], 1), 7.25)], axis=1)
    shifted = _mla(q2[None], C, R2, WK, WV, 0.5)[0]
    np.testing.assert_allclose(shifted, base, rtol=1e-12, atol=1e-13)


def test_huge_scores_stay_finite():
    rng = np.random.default_rng(5)
    q, C, R, WK, WV = _f32(*_rand_head(rng, 6))
    out = _mla((q * 1e3)[None], C, R, WK * 1e3, WV, 1.0)[0]
    assert np.all(np.isfinite(out))


def test_empty_sequence_gives_zeros():
    q = np.ones((1, 2, 4), np.float32)
    ck = np.full((1, 4, 3), np.nan, np.float32)
    kr = np.full((1, 4, 1), np.nan, np.float32)
    out = mla_decode_explicit(q, ck, None, kr, np.zeros((1, 1), np.int32),
                              np.zeros(1, np.int32), np.ones((2, 3, 3), np.float32),
                              np.ones((2, 5, 3), np.float32), 1.0, 4)
    assert np.array_equal(out, np.zeros((1, 2, 5)))


# ---------------------------------------------------------- brute force

def _brute(q, C, R, WK, WV, sm):
    """Independent long-double direct sums over every index."""
    L = np.longdouble
    T, dc = C.shape
    dn = WK.shape[0]
    dv = WV.shape[0]
    dr = R.shape[1]
    scores = []
    for t in range(T):
        s = L(0)
        for n in range(dn):
            k = L(0)
            for c in range(dc):
                k += L(WK[n, c]) * L(C[t, c])
            s += L(q[n]) * k
        for r in range(dr):
            s += L(q[dn + r]) * L(R[t, r])
        scores.append(L(sm) * s)
    m = max(scores)
    w = [np.exp(s - m) for s in scores]
    z = sum(w)
    out = []
    for v in range(dv):
        acc = L(0)
        for t in range(T):
            val = L(0)
            for c in range(dc):
                val += L(WV[v, c]) * L(C[t, c])
            acc += w[t] / z * val
        out.append(acc)
    return np.array(out, dtype=np.float64)


@pytest.mark.parametrize("T,dn,dc,dr,dv", [(1, 2, 3, 1, 2), (4, 3, 5, 2, 3), (8, 2, 4, 0, 3)])
def test_brute_force_tiny(T, dn, dc, dr, dv):
    rng = np.random.default_rng(T * 10 + dc)
    q = rng.standard_normal(dn + dr)
    C = rng.standard_normal((T, dc))
    R = rng.standard_normal((T, dr))
    WK = rng.standard_normal((dn, dc))
    WV = rng.standard_normal((dv, dc))
    q, C, R, WK, WV = _f32(q, C, R, WK, WV)
    out = _mla(q[None], C, R, WK[None], WV[None], 0.6, P=3)[0]
    np.testing.assert_allclose(out, _brute(q, C, R, WK, WV, 0.6), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------- storage decoders

def test_bf16_decoder_matches_torch():
    rng = np.random.default_rng(9)
    bits = rng.integers(0, 1 << 16, size=20000, dtype=np.uint16)
    ours = bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().double().numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_e4m3_decoder_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_code_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().double().numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()
    assert np.nanmax(ours) == 448.0 and np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])


def test_decode_storage_tags():
    assert decode_storage(np.array([1.5], np.float32), "f32")[0] == 1.5
    assert decode_storage(np.array([0x3FC0], np.uint16), "bf16")[0] == 1.5
    assert decode_storage(np.array([0x3C], np.uint8), "e4m3")[0] == 1.5
    with pytest.raises(ValueError):
        decode_storage(np.zeros(1), "fp16")
