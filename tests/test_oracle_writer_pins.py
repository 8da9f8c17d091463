"""Pins of the latent-cache writer oracle (CPU only): page values, closed
forms and identities of RMSNorm and RoPE, and the E4M3FN code points."""
import math

import numpy as np
import pytest
import torch

from oracle.cache_writer import (cache_write, e4m3_encode, e4m3_value, page_slot,
                                 quantize_row_e4m3, rmsnorm, rope, rope_angles)


# ------------------------------------------------------------------ RoPE

def test_rope_scores_match_page(golden):
    """Lesson, 'RoPE Breaks the Trick': the query [1, 0] against the key [1, 0]
    rotated to t = 1 and t = 5 scores 0.540 and 0.284.  The first pair turns by
    t rad for any base."""
    g = golden("rope_toy.json")
    q = np.array(g["query"])
    for t, want in zip(g["positions"], g["scores"]):
        got = float(q @ rope(np.array(g["key"]), t, base=10000.0))
        assert abs(got - want) <= g["rounding"]


def test_rope_adjacent_frequency_ratio_matches_page(golden):
    """FreqFold: theta_63 / theta_64 at d = 128 is printed as about 1.15.  The
    angles are read back from rotations of unit pairs, not from the formula."""
    g = golden("freqfold_ratio.json")
    d = g["d"]
    e = np.zeros(d)
    e[0::2] = 1.0
    r = rope(e, 1, g["base"])
    ang = np.arctan2(r[1::2], r[0::2])           # angle of each pair at t = 1
    l1, l2 = g["l_pair"]
    assert abs(ang[l1 - 1] / ang[l2 - 1] - g["ratio"]) <= g["rounding"]


def test_rope_identities():
    rng = np.random.default_rng(5)
    v = rng.standard_normal(64)
    q = rng.standard_normal(64)
    assert np.array_equal(rope(v, 0, 10000.0), v)                   # position 0
    np.testing.assert_allclose(rope(rope(v, 7, 1e4), 11, 1e4), rope(v, 18, 1e4), atol=1e-12)
    # each pair keeps its length
    r = rope(v, 1234, 1e4)
    np.testing.assert_allclose(np.hypot(r[0::2], r[1::2]), np.hypot(v[0::2], v[1::2]), atol=1e-12)
    # scores depend on the relative position only
    s1 = rope(q, 100, 1e4) @ rope(v, 37, 1e4)
    s2 = rope(q, 563, 1e4) @ rope(v, 500, 1e4)
    assert abs(s1 - s2) < 1e-9
    # a plain pair: rotating [x, y] by a quarter turn gives [-y, x]
    base = 1.0  # every pair then turns by t rad
    w = rope(np.array([0.3, -0.8]), math.pi / 2, base)
    np.testing.assert_allclose(w, [0.8, 0.3], atol=1e-12)


def test_rope_frequencies_decrease_geometrically():
    a = rope_angles(64, 1.0, 10000.0)
    assert a[0] == 1.0 and np.all(np.diff(a) < 0)
    ratios = a[:-1] / a[1:]
    np.testing.assert_allclose(ratios, ratios[0], rtol=1e-12)        # one common ratio
    assert abs(a[-1] - 10000.0 ** (-62 / 64)) < 1e-15                # the last pair, l = d/2


# ------------------------------------------------------------------ RMSNorm

def test_rmsnorm_hand_values():
    # y = [3, 4]: mean square 12.5, RMS 3.5355..., output [0.8485..., 1.1313...]
    out = rmsnorm(np.array([3.0, 4.0]), np.ones(2), 0.0)
    np.testing.assert_allclose(out, [3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], rtol=1e-15)
    # gamma scales each dimension; eps enters under the square root
    out = rmsnorm(np.array([1.0, 1.0, 1.0, 1.0]), np.array([1.0, 2.0, 3.0, 4.0]), 3.0)
    np.testing.assert_allclose(out, [0.5, 1.0, 1.5, 2.0], rtol=1e-15)   # sqrt(1 + 3) = 2


def test_rmsnorm_identities():
    rng = np.random.default_rng(9)
    y = rng.standard_normal((5, 512))
    out = rmsnorm(y, np.ones(512), 0.0)
    np.testing.assert_allclose(np.mean(out * out, axis=-1), 1.0, rtol=1e-12)
    np.testing.assert_allclose(rmsnorm(7.5 * y, np.ones(512), 0.0), out, rtol=1e-12)
    assert np.all(rmsnorm(np.zeros((2, 8)), np.ones(8), 1e-6) == 0.0)


# ------------------------------------------------------------------ E4M3FN

@pytest.mark.parametrize("value,code", [
    (448.0, 0x7E), (-448.0, 0xFE), (1.0, 0x38), (0.5, 0x30), (240.0, 0x77),
    (2.0 ** -6, 0x08), (2.0 ** -9, 0x01), (7 * 2.0 ** -9, 0x07), (0.0, 0x00), (-0.0, 0x80),
])
def test_e4m3_code_points(value, code):
    """Code points of the format definition (bias 7, 3-bit mantissa, subnormals)."""
    assert int(e4m3_encode(value)) == code
    assert e4m3_value(code) == value
    assert math.isnan(e4m3_value(0x7F)) and math.isnan(e4m3_value(0xFF))


def test_e4m3_ties_go_to_even():
    assert int(e4m3_encode(1.0625)) == 0x38        # between 1.0 (m=0) and 1.125 (m=1)
    assert int(e4m3_encode(1.1875)) == 0x3A        # between 1.125 (m=1) and 1.25 (m=2)
    assert int(e4m3_encode(2.0 ** -10)) == 0x00    # half the smallest subnormal -> 0
    assert int(e4m3_encode(3 * 2.0 ** -10)) == 0x02  # between 1 and 2 subnormal units
    assert int(e4m3_encode(432.0)) == 0x7E         # between 416 (m=5) and 448 (m=6)


def test_e4m3_matches_torch_cast():
    """An independent implementation: torch's float8_e4m3fn cast (RNE)."""
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(4000) * s for s in (1e-3, 0.1, 1.0, 30.0)])
    x = np.clip(x, -448, 448).astype(np.float32)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(x), want)


def test_quantize_row_rules():
    codes, s = quantize_row_e4m3(np.zeros(16, np.float32))
    assert s == 0 and not codes.any()
    row = np.array([0.25, -3.0, 1.5, 0.0], np.float32)
    codes, s = quantize_row_e4m3(row)
    assert s == np.float32(np.float32(3.0) / np.float32(448.0))
    assert codes[1] == 0xFE                         # the largest magnitude maps to -448
    dec = np.array([e4m3_value(int(c)) for c in codes]) * float(s)
    np.testing.assert_allclose(dec, row, rtol=2.0 ** -4)   # within half an E4M3 step


# ------------------------------------------------------------------ the writer

def test_page_slots():
    bt = np.array([[5, 2, -1], [0, 7, 3]])
    assert page_slot(bt, 0, 0, 16, 8) == (5, 0)
    assert page_slot(bt, 0, 17, 16, 8) == (2, 1)
    assert page_slot(bt, 0, 33, 16, 8) is None     # table entry -1
    assert page_slot(bt, 1, 47, 16, 8) == (3, 15)
    assert page_slot(bt, 1, 48, 16, 8) is None     # past the table row
    assert page_slot(bt, 1, 20, 16, 7) is None     # block 7 outside a pool of 7
    assert page_slot(bt, 1, -1, 16, 8) is None


def test_cache_write_small_case():
    """Hand-checkable: W_DKV picks [x0, x1] and [x1, 0]; W_KR picks [x0, x1]."""
    x = np.array([[3.0, 4.0], [1.0, 0.0]])
    W_DKV = np.array([[1.0, 0.0], [0.0, 1.0]])
    W_KR = np.array([[1.0, 0.0], [0.0, 1.0]])
    bt = np.array([[1, 0], [0, 1]])
    c, k, slots = cache_write(x, W_DKV, np.array([1.0, 2.0]), W_KR, [3, 17], bt, 16, 2, 0.0, 1.0)
    np.testing.assert_allclose(c[0], [3 / math.sqrt(12.5), 8 / math.sqrt(12.5)], rtol=1e-15)
    np.testing.assert_allclose(c[1], [math.sqrt(2), 0.0], rtol=1e-15)
    np.testing.assert_allclose(k[0], [3 * math.cos(3) - 4 * math.sin(3),
                                      3 * math.sin(3) + 4 * math.cos(3)], rtol=1e-13)
    np.testing.assert_allclose(k[1], [math.cos(17), math.sin(17)], rtol=1e-13)
    assert slots == [(1, 3), (1, 1)]
