"""Plant plausible mistakes in the cache-writer oracle (CPU only) and check
that its pins catch every one of them."""
import math

import numpy as np
import pytest

import oracle.cache_writer as cw
import tests.test_oracle_writer_pins as pins
from tests.conftest import load_golden

_orig = {n: getattr(cw, n) for n in ("rope", "rope_angles", "rmsnorm", "e4m3_encode",
                                      "quantize_row_e4m3", "page_slot")}


def _rope_rotate_half(v, t, base):
    v = np.asarray(v, dtype=np.float64)
    d = v.shape[-1]
    a = cw.rope_angles(d, t, base)
    x, y = v[..., : d // 2], v[..., d // 2:]
    out = np.empty_like(v)
    out[..., : d // 2] = x * np.cos(a) - y * np.sin(a)
    out[..., d // 2:] = x * np.sin(a) + y * np.cos(a)
    return out


def _rope_turns_backwards(v, t, base):
    return _orig["rope"](v, -t, base)


def _angles_half_exponent(d, t, base):
    i = np.arange(d // 2, dtype=np.float64)
    return float(t) * np.power(float(base), -1.0 * i / d)


def _rmsnorm_eps_outside(y, gamma, eps):
    y = np.asarray(y, dtype=np.float64)
    return y / (np.sqrt(np.mean(y * y, axis=-1, keepdims=True)) + eps) * gamma


def _rmsnorm_sum(y, gamma, eps):
    y = np.asarray(y, dtype=np.float64)
    return y / np.sqrt(np.sum(y * y, axis=-1, keepdims=True) + eps) * gamma


def _rmsnorm_no_gamma(y, gamma, eps):
    return _orig["rmsnorm"](y, np.ones_like(np.asarray(gamma, dtype=np.float64)), eps)


def _e4m3_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    out = _orig["e4m3_encode"](x)
    flat, res = x.reshape(-1), out.reshape(-1).copy()
    for k, v in enumerate(flat):
        a = abs(v)
        lo = cw._POS_VALS[cw._POS_VALS <= a].max()
        hi = cw._POS_VALS[cw._POS_VALS >= a].min()
        if lo != hi and a - lo == hi - a:           # a tie: take the larger magnitude
            res[k] = int(cw._POS_CODES[list(cw._POS_VALS).index(hi)]) | (0x80 if v < 0 else 0)
    return res.reshape(x.shape)


def _e4m3_truncate(x):
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(-1)
    res = np.empty(flat.shape, dtype=np.uint8)
    for k, v in enumerate(flat):
        a = abs(v)
        code = int(cw._POS_CODES[np.flatnonzero(cw._POS_VALS <= a).max()])
        res[k] = code | (0x80 if (v < 0 or math.copysign(1, v) < 0) else 0)
    return res.reshape(x.shape)


def _quantize_scale_447(row):
    r = np.asarray(row, dtype=np.float32)
    s = np.float32(np.max(np.abs(r)) / np.float32(447.0))
    if s == 0:
        return np.zeros(r.shape, np.uint8), np.float32(0)
    return cw.e4m3_encode(np.clip(r / s, -448, 448)), s


def _slot_off_by_one(block_table, b, t, P, num_blocks):
    return _orig["page_slot"](block_table, b, t + 1, P, num_blocks)


MUTANTS = {
    "rope rotates halves instead of pairs": ("rope", _rope_rotate_half),
    "rope turns backwards": ("rope", _rope_turns_backwards),
    "rope exponent -i/d": ("rope_angles", _angles_half_exponent),
    "rmsnorm eps outside the root": ("rmsnorm", _rmsnorm_eps_outside),
    "rmsnorm sum instead of mean": ("rmsnorm", _rmsnorm_sum),
    "rmsnorm drops gamma": ("rmsnorm", _rmsnorm_no_gamma),
    "e4m3 ties away from zero": ("e4m3_encode", _e4m3_ties_away),
    "e4m3 truncates": ("e4m3_encode", _e4m3_truncate),
    "scale from 447": ("quantize_row_e4m3", _quantize_scale_447),
    "page slot off by one": ("page_slot", _slot_off_by_one),
}


def _run_pins():
    failed = []
    for name in dir(pins):
        if not name.startswith("test_"):
            continue
        fn = getattr(pins, name)
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        argnames, cases = [], [()]
        if params:
            argnames = [a.strip() for a in params[0].args[0].split(",")]
            cases = [c if isinstance(c, tuple) else (c,) for c in params[0].args[1]]
        for case in cases:
            kw = dict(zip(argnames, case))
            if "golden" in fn.__code__.co_varnames[: fn.__code__.co_argcount]:
                kw["golden"] = load_golden
            try:
                with np.errstate(all="ignore"):
                    fn(**kw)
            except Exception:
                failed.append(name)
                break
    return failed


def test_writer_pins_pass_unmutated():
    assert _run_pins() == []


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_writer_pins_catch(mutant, monkeypatch):
    attr, fn = MUTANTS[mutant]
    monkeypatch.setattr(cw, attr, fn)
    # the pins module imported the names directly: patch them there too
    if hasattr(pins, attr):
        monkeypatch.setattr(pins, attr, fn)
    assert _run_pins(), f"no pin caught: {mutant}"
