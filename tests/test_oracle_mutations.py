"""Plant plausible mistakes in the oracle (CPU only) and check that the pins
catch every one of them: a pin set that lets a mistake through is too weak."""
import numpy as np
import pytest

import oracle.mla_oracle as om
import tests.test_oracle_pins as pins
from tests.conftest import load_golden


def _no_rope(q_nope, q_rope, C, R, WK, WV, sm):
    K = C @ WK.T
    p = om.softmax(sm * (K @ q_nope))
    return p @ (C @ WV.T) if C.shape[0] else np.zeros(WV.shape[0])


def _rope_sign(q_nope, q_rope, C, R, WK, WV, sm):
    if C.shape[0] == 0:
        return np.zeros(WV.shape[0])
    p = om.softmax(sm * (C @ WK.T @ q_nope - R @ q_rope))
    return p @ (C @ WV.T)


def _swap_kv(q_nope, q_rope, C, R, WK, WV, sm):
    if C.shape[0] == 0:
        return np.zeros(WV.shape[0])
    if WK.shape != WV.shape:
        raise AssertionError("shape mismatch exposes the swap")
    p = om.softmax(sm * (C @ WV.T @ q_nope + R @ q_rope))
    return p @ (C @ WK.T)


def _scale_content_only(q_nope, q_rope, C, R, WK, WV, sm):
    if C.shape[0] == 0:
        return np.zeros(WV.shape[0])
    p = om.softmax(sm * (C @ WK.T @ q_nope) + R @ q_rope)
    return p @ (C @ WV.T)


def _no_max_subtract(s):
    e = np.exp(np.asarray(s, dtype=np.float64))
    return e / np.sum(e, axis=-1, keepdims=True)


def _unnormalised(s):
    s = np.asarray(s, dtype=np.float64)
    return np.exp(s - np.max(s, axis=-1, keepdims=True))


def _selectors_wrong_group(h, g, d):
    WK = np.zeros((h, d, 2 * g * d))
    WV = np.zeros((h, d, 2 * g * d))
    for i in range(h):
        j = i % g                                  # interleaved instead of contiguous groups
        WK[i, :, j * d:(j + 1) * d] = np.eye(d)
        WV[i, :, (g + j) * d:(g + j + 1) * d] = np.eye(d)
    return WK, WV


def _selectors_v_in_k_half(h, g, d):
    WK, WV = _orig_selectors(h, g, d)
    WV2 = np.zeros_like(WV)
    for i in range(h):
        j = i // (h // g)
        WV2[i, :, j * d:(j + 1) * d] = np.eye(d)   # value read from the key block
    return WK, WV2


_orig_selectors = om.build_selectors


def _gather_off_by_one_page(c_kv, k_rope, c_kv_scale, block_table, seq_len, b, P, ct, rt):
    T = int(seq_len)
    C = np.empty((T, c_kv.shape[-1]))
    R = np.empty((T, k_rope.shape[-1]))
    for t in range(T):
        blk = int(block_table[b][min((t + 1) // P, block_table.shape[1] - 1)])
        C[t] = om.decode_storage(c_kv[blk, t % P], ct)
        R[t] = om.decode_storage(k_rope[blk, t % P], rt)
    return C, R


def _e4m3_bias8():
    t = om._e4m3_table()
    return t / 2.0


def _bf16_shift15(bits):
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(15)
    return u32.view(np.float32).astype(np.float64)


MUTANTS = {
    "drop rope term": [("_head_explicit", _no_rope)],
    "rope term sign": [("_head_explicit", _rope_sign)],
    "keys from W_UV, values from W_UK": [("_head_explicit", _swap_kv)],
    "scale on content only": [("_head_explicit", _scale_content_only)],
    "softmax without max subtraction": [("softmax", _no_max_subtract)],
    "softmax without normalisation": [("softmax", _unnormalised)],
    "interleaved head groups": [("build_selectors", _selectors_wrong_group)],
    "value selector over key block": [("build_selectors", _selectors_v_in_k_half)],
    "page index off by one": [("gather_sequence", _gather_off_by_one_page)],
    "e4m3 exponent bias 8": [("_E4M3", _e4m3_bias8())],
    "bf16 bits shifted by 15": [("bf16_bits_to_f64", _bf16_shift15)],
}


def _run_pins():
    """Run every pin; return the names of those that fail."""
    failed = []
    for name in dir(pins):
        if not name.startswith("test_"):
            continue
        fn = getattr(pins, name)
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        cases = [()]
        if params:
            argnames = [a.strip() for a in params[0].args[0].split(",")]
            cases = [c if isinstance(c, tuple) else (c,) for c in params[0].args[1]]
        else:
            argnames = []
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


def test_pins_pass_unmutated():
    assert _run_pins() == []


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_mutant(mutant, monkeypatch):
    for attr, repl in MUTANTS[mutant]:
        monkeypatch.setattr(om, attr, repl)
        if hasattr(pins, attr):
            monkeypatch.setattr(pins, attr, repl)
    failed = _run_pins()
    assert failed, f"no pin caught the planted mistake: {mutant}"
