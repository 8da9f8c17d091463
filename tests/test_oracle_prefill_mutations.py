"""Plant plausible mistakes in the prefill oracle (CPU only) and check that its
pins catch every one of them."""
import numpy as np
import pytest

import oracle.prefill as pf
import tests.test_oracle_prefill_pins as pins

_orig_pos = pf.query_position


def _positions_from_zero(seq_len, q_len, l):
    return l


def _one_short(seq_len, q_len, l):
    return seq_len - q_len + l - 1


def _one_long(seq_len, q_len, l):
    return min(seq_len - 1, seq_len - q_len + l + 1)


MUTANTS = {
    "queries placed from position 0": _positions_from_zero,
    "a row misses its own token": _one_short,
    "a row sees the next token": _one_long,
}


def _run_pins():
    failed = []
    for name in dir(pins):
        if name.startswith("test_"):
            try:
                with np.errstate(all="ignore"):
                    getattr(pins, name)()
            except Exception:
                failed.append(name)
    return failed


def test_prefill_pins_pass_unmutated():
    assert _run_pins() == []


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_prefill_pins_catch(mutant, monkeypatch):
    monkeypatch.setattr(pf, "query_position", MUTANTS[mutant])
    monkeypatch.setattr(pins, "query_position", MUTANTS[mutant])
    assert _run_pins(), f"no pin caught: {mutant}"
