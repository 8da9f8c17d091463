"""Plant plausible mistakes in the grouped-MLA oracle (CPU only) and check that
its pins catch every one of them."""
import numpy as np
import pytest

import oracle.grouped as gm
import tests.test_oracle_grouped_pins as pins
from tests.conftest import load_golden


def _interleaved_heads(i, heads, groups):
    return i % groups


def _last_group_first(i, heads, groups):
    return groups - 1 - i // (heads // groups)


def _rope_per_group(groups, d_latent, d_rope):
    return groups * (d_latent + d_rope)


MUTANTS = {
    "heads interleaved over the groups": ("group_of_head", _interleaved_heads),
    "groups in reverse order": ("group_of_head", _last_group_first),
    "rope key stored per group": ("values_per_token", _rope_per_group),
}


def _run_pins():
    failed = []
    for name in dir(pins):
        if not name.startswith("test_"):
            continue
        fn = getattr(pins, name)
        kw = {}
        if "golden" in fn.__code__.co_varnames[: fn.__code__.co_argcount]:
            kw["golden"] = load_golden
        try:
            with np.errstate(all="ignore"):
                fn(**kw)
        except Exception:
            failed.append(name)
    return failed


def test_grouped_pins_pass_unmutated():
    assert _run_pins() == []


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_grouped_pins_catch(mutant, monkeypatch):
    attr, fn = MUTANTS[mutant]
    monkeypatch.setattr(gm, attr, fn)
    if hasattr(pins, attr):
        monkeypatch.setattr(pins, attr, fn)
    assert _run_pins(), f"no pin caught: {mutant}"
