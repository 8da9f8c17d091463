"""Plant plausible mistakes in the TPLA oracle (CPU only) and check that its
pins catch every one of them."""
import numpy as np
import pytest

import oracle.tpla as tp
import tests.test_oracle_tpla_pins as pins
from oracle.mla_oracle import softmax
from tests.conftest import load_golden

_orig = {n: getattr(tp, n) for n in ("tpla_latent", "shard_slices", "hadamard",
                                      "cache_values_per_device", "reparameterize")}


def _joint_softmax(q_lat, q_rope, C, R, sm_scale, shards=2, mu=None):
    return _orig["tpla_latent"](q_lat, q_rope, C, R, sm_scale, shards=1)


def _interleaved(d_c, shards):
    return [slice(j, d_c, shards) for j in range(shards)]


def _no_rope_past_first(q_lat, q_rope, C, R, sm_scale, shards=2, mu=None):
    d_c = C.shape[1]
    out = np.zeros(d_c)
    if C.shape[0] == 0:
        return out
    for j, S in enumerate(tp.shard_slices(d_c, shards)):
        s = sm_scale * (C[:, S] @ q_lat[S] + (R @ q_rope if j == 0 else 0.0))
        out[S] = softmax(s) @ C[:, S]
    return out


def _mu_on_everything(q_lat, q_rope, C, R, sm_scale, shards=2, mu=None):
    d_c = C.shape[1]
    mu = [1.0] * shards if mu is None else list(mu)
    out = np.zeros(d_c)
    if C.shape[0] == 0:
        return out
    for j, S in enumerate(tp.shard_slices(d_c, shards)):
        s = sm_scale * mu[j] * (C[:, S] @ q_lat[S] + R @ q_rope)
        out[S] = softmax(s) @ C[:, S]
    return out


def _hadamard_flipped(d):
    H = np.ones((1, 1))
    while H.shape[0] < d:
        H = np.block([[H, -H], [H, H]])
    return H


def _values_full(d_c, d_r, shards):
    return d_c // shards



MUTANTS = {
    "one joint softmax": ("tpla_latent", _joint_softmax),
    "interleaved shards": ("shard_slices", _interleaved),
    "positional score on the first shard only": ("tpla_latent", _no_rope_past_first),
    "content factor scales the positional score too": ("tpla_latent", _mu_on_everything),
    "Sylvester blocks in the wrong places": ("hadamard", _hadamard_flipped),
    "rope key not counted per device": ("cache_values_per_device", _values_full),
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


def test_tpla_pins_pass_unmutated():
    assert _run_pins() == []


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_tpla_pins_catch(mutant, monkeypatch):
    attr, fn = MUTANTS[mutant]
    monkeypatch.setattr(tp, attr, fn)
    if hasattr(pins, attr):
        monkeypatch.setattr(pins, attr, fn)
    assert _run_pins(), f"no pin caught: {mutant}"
