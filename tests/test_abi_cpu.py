"""The C-ABI library without a GPU: it loads, exports every declared entry
point, rejects bad arguments before touching HIP, and its split arithmetic
partitions the tiles exactly."""
import ctypes
import os
import re

import pytest

from head_latent_attention_10_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "mla.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load_library()


def test_every_declared_symbol_is_exported_and_bound(lib):
    names = _declared_functions()
    assert "mla_decode" in names and len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(_lib.exported_symbols()) == names


def test_status_strings(lib):
    assert _lib.mla_status_string(0) == "ok"
    assert "workspace" in _lib.mla_status_string(-3)
    assert _lib.mla_status_string(42) == "unknown status"


def _params(**kw):
    base = dict(batch=2, num_heads=4, d_nope=16, d_rope=8, d_latent=32, d_v=16, page_size=64,
                max_blocks_per_seq=2, num_blocks=4, q_dtype="f32", cache_dtype="f32",
                rope_dtype="f32", weight_dtype="f32", out_dtype="f32", sm_scale=0.0, num_splits=8)
    base.update(kw)
    return _lib.make_params(**base)


def test_workspace_size_without_device():
    n = _lib.mla_decode_workspace_size(_params())
    # q_lat + cu_tiles + tile descriptors (B * ceil(2 blocks * 64 / 32) of 16 B)
    # + partials ((8 + 2) slots) + lse + o_lat, each 256-aligned
    B, h, dc, dr = 2, 4, 32, 8
    expect = 0
    for size in (B * h * (dc + dr) * 4, (B + 1) * 4, B * 4 * 16, 10 * h * dc * 4, 10 * h * 4,
                 B * h * dc * 4):
        expect += (size + 255) // 256 * 256
    assert n == expect


@pytest.mark.parametrize("bad,status", [
    (dict(batch=0), _lib.MLA_ERR_INVALID_ARG),
    (dict(batch=65536, max_blocks_per_seq=1 << 14), _lib.MLA_ERR_UNSUPPORTED),  # 2^31 tiles
    (dict(num_heads=-1), _lib.MLA_ERR_INVALID_ARG),
    (dict(page_size=0), _lib.MLA_ERR_INVALID_ARG),
    (dict(page_size=5000), _lib.MLA_ERR_INVALID_ARG),
    (dict(num_blocks=0), _lib.MLA_ERR_INVALID_ARG),
    (dict(cache_dtype=7), _lib.MLA_ERR_INVALID_ARG),
    (dict(q_dtype=2), _lib.MLA_ERR_INVALID_ARG),         # fp8 queries are not accepted
    (dict(num_splits=-2), _lib.MLA_ERR_INVALID_ARG),
    (dict(sm_scale=float("nan")), _lib.MLA_ERR_INVALID_ARG),
    (dict(d_latent=2048), _lib.MLA_ERR_UNSUPPORTED),
])
def test_validation_errors(bad, status):
    with pytest.raises(_lib.MlaError) as ei:
        _lib.mla_decode_workspace_size(_params(**bad))
    assert ei.value.status == status
    assert _lib.mla_last_error()


def test_decode_rejects_null_and_small_workspace_before_launch():
    p = _params()
    fake = 0x10000  # never dereferenced: validation fails first
    with pytest.raises(_lib.MlaError) as ei:
        _lib.mla_decode(p, fake, None, None, fake, fake, fake, fake, fake, fake, fake, 1 << 20)
    assert ei.value.status == _lib.MLA_ERR_INVALID_ARG
    with pytest.raises(_lib.MlaError) as ei:   # fp32 cache with a scale pointer
        _lib.mla_decode(p, fake, fake, fake, fake, fake, fake, fake, fake, fake, fake, 1 << 20)
    assert ei.value.status == _lib.MLA_ERR_INVALID_ARG
    with pytest.raises(_lib.MlaError) as ei:
        _lib.mla_decode(p, fake, fake, None, fake, fake, fake, fake, fake, fake, fake, 16)
    assert ei.value.status == _lib.MLA_ERR_WORKSPACE
    with pytest.raises(_lib.MlaError) as ei:
        _lib.mla_decode(p, fake, fake, None, fake, fake, fake, fake, fake, fake, fake + 8, 1 << 20)
    assert ei.value.status == _lib.MLA_ERR_INVALID_ARG
    with pytest.raises(_lib.MlaError) as ei:
        _lib.mla_decode(p, fake, fake, None, fake, fake, fake, fake, fake, fake, None, 1 << 20)
    assert ei.value.status == _lib.MLA_ERR_WORKSPACE


def test_fp8_needs_scale_pointer():
    p = _params(cache_dtype="e4m3", q_dtype="bf16", rope_dtype="bf16", weight_dtype="bf16")
    fake = 0x10000
    with pytest.raises(_lib.MlaError) as ei:
        _lib.mla_attend_latent(p, fake, fake, None, fake, fake, fake, fake, fake, 1 << 20)
    assert ei.value.status == _lib.MLA_ERR_INVALID_ARG


def test_absorbed_dtype():
    assert _lib.mla_absorbed_dtype(_params()) == _lib.MLA_F32
    assert _lib.mla_absorbed_dtype(_params(cache_dtype="bf16")) == _lib.MLA_BF16


@pytest.mark.parametrize("n,G", [(1, 1), (1, 256), (7, 3), (64, 256), (300, 256), (4096, 256),
                                 (135168 // 64, 256), (1000003, 977)])
def test_split_arithmetic_partitions_tiles(n, G):
    begins = [_lib.mla_split_begin(n, G, g) for g in range(G + 1)]
    assert begins[0] == 0 and begins[-1] == n
    assert all(b0 <= b1 for b0, b1 in zip(begins, begins[1:]))
    sizes = [b1 - b0 for b0, b1 in zip(begins, begins[1:])]
    assert max(sizes) - min(sizes) <= 1            # balanced to one tile
    step = max(1, n // 2000)
    for t in list(range(0, n, step)) + [n - 1]:
        g = _lib.mla_split_owner(n, G, t)
        assert begins[g] <= t < begins[g + 1]


def test_split_slots_are_unique():
    """Slot (split + sequence) is unique over all (split, sequence) pairs that
    share tiles, for ragged lengths including empty sequences."""
    lens_tiles = [3, 0, 5, 1, 0, 0, 9, 2]
    cu = [0]
    for x in lens_tiles:
        cu.append(cu[-1] + x)
    n = cu[-1]
    for G in (1, 2, 3, 7, 16, 40):
        slots = set()
        for b in range(len(lens_tiles)):
            if cu[b + 1] == cu[b]:
                continue
            g_lo = _lib.mla_split_owner(n, G, cu[b])
            g_hi = _lib.mla_split_owner(n, G, cu[b + 1] - 1)
            for g in range(g_lo, g_hi + 1):
                s = g + b
                assert s not in slots
                assert s < G + len(lens_tiles)
                slots.add(s)


def _prefill_params(**kw):
    base = dict(batch=3, num_heads=4, d_nope=128, d_rope=64, d_latent=512, d_v=128, page_size=64,
                max_blocks_per_seq=5, num_blocks=16, q_dtype="bf16", cache_dtype="bf16",
                rope_dtype="bf16", weight_dtype="bf16", out_dtype="bf16", sm_scale=0.0,
                num_splits=0)
    base.update(kw)
    return _lib.make_params(**base)


def test_prefill_workspace_size_without_device():
    # keys with their rope part and transposed values: B x h x Tpad x (192 + 128)
    # bf16, Tpad = 5 blocks x 64 rounded up to 128
    assert _lib.mla_prefill_workspace_size(_prefill_params()) == 3 * 4 * 384 * (192 + 128) * 2


@pytest.mark.parametrize("bad", [dict(cache_dtype="f32"), dict(q_dtype="f32"),
                                 dict(weight_dtype="f32"), dict(d_nope=64), dict(d_v=64),
                                 dict(d_latent=256), dict(d_rope=32)])
def test_prefill_unsupported_shapes(bad):
    with pytest.raises(_lib.MlaError) as ei:
        _lib.mla_prefill_workspace_size(_prefill_params(**bad))
    assert ei.value.status == _lib.MLA_ERR_UNSUPPORTED


def test_prefill_rejects_bad_arguments_before_launch():
    p = _prefill_params()
    fake = 0x10000
    n = _lib.mla_prefill_workspace_size(p)
    args = [fake, fake, fake, None, fake, fake, fake, fake, fake, fake]  # no scale: bf16 cache
    for bad_len in (0, -1, (1 << 24) + 1):
        with pytest.raises(_lib.MlaError) as ei:
            _lib.mla_prefill(p, bad_len, *args, fake, n)
        assert ei.value.status == _lib.MLA_ERR_INVALID_ARG
    for i in range(10):
        if i == 3:
            continue
        a = list(args)
        a[i] = None
        with pytest.raises(_lib.MlaError) as ei:
            _lib.mla_prefill(p, 16, *a, fake, n)
        assert ei.value.status == _lib.MLA_ERR_INVALID_ARG, i
    with pytest.raises(_lib.MlaError) as ei:
        _lib.mla_prefill(p, 16, *args, fake, n - 1)
    assert ei.value.status == _lib.MLA_ERR_WORKSPACE
    with pytest.raises(_lib.MlaError) as ei:
        _lib.mla_prefill(p, 16, *args, fake + 128, n)
    assert ei.value.status == _lib.MLA_ERR_INVALID_ARG
    with pytest.raises(_lib.MlaError) as ei:  # misaligned query
        _lib.mla_prefill(p, 16, fake + 2, *args[1:], fake, n)
    assert ei.value.status == _lib.MLA_ERR_INVALID_ARG
    with pytest.raises(_lib.MlaError) as ei:  # a scale pointer with a bf16 cache
        _lib.mla_prefill(p, 16, *args[:3], fake, *args[4:], fake, n)
    assert ei.value.status == _lib.MLA_ERR_INVALID_ARG
    p8 = _prefill_params(cache_dtype="e4m3")
    with pytest.raises(_lib.MlaError) as ei:  # an fp8 cache without its scales
        _lib.mla_prefill(p8, 16, *args, fake, _lib.mla_prefill_workspace_size(p8))
    assert ei.value.status == _lib.MLA_ERR_INVALID_ARG
