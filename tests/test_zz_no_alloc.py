"""mla_decode_no_alloc (the decode step in the library's fixed device scratch)
against mla_decode with a caller-allocated workspace, through the C ABI
(needs an MI355X): two calls in a row, the second on a smaller input, each
bit for bit equal to mla_decode on the same inputs and split count; the
fixed scratch keeps the first call's contents, so the second also shows that
no call relies on it starting at zero."""
import sys

import numpy as np
import pytest
import torch

from head_latent_attention_10_amd import _lib
from head_latent_attention_10_amd.device import Decoder, DeviceInputs, out_torch_dtype
from mla_inputs import CONFIGS, generate
from oracle import oracle_from_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load_library()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _no_alloc(dev, num_splits):
    c = dev.cfg
    p = dev.params(num_splits=num_splits)
    out = torch.empty((c.batch, c.heads, c.d_v), dtype=out_torch_dtype(c.out_dtype), device="cuda")
    _lib.mla_decode_no_alloc(p, dev.q, dev.c_kv, dev.c_kv_scale, dev.k_rope, dev.block_table,
                             dev.seq_lens, dev.W_UK, dev.W_UV, out)
    return out


def _run_pair(cfg, lens, num_splits):
    inp = generate(cfg, seq_lens=lens)
    dev = DeviceInputs(inp)
    got = _no_alloc(dev, num_splits)
    dec = Decoder(dev, num_splits=num_splits)
    want = dec()
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    return inp, got


PAIRS = {
    # (first call, second call on a smaller input)
    "dsv3_bf16": ((CONFIGS["dsv3_b64_4k"].replace(batch=4), [700, 1, 333, 64], 0),
                  (CONFIGS["dsv3_b64_4k"].replace(batch=2, seed=91), [130, 9], 16)),
    "dsv3_fp8": ((CONFIGS["dsv3_fp8_16k"].replace(batch=3), [2100, 64, 5], 0),
                 (CONFIGS["dsv3_fp8_16k"].replace(batch=1, seed=92), [77], 8)),
    "tiny_fp32": ((CONFIGS["tiny_fp32"].replace(batch=3, seq_len=None, seq_len_range=(1, 200)),
                   [200, 3, 64], 5),
                  (CONFIGS["tiny_fp32"].replace(batch=2, seed=93), [17, 1], 2)),
}


@pytest.mark.parametrize("case", sorted(PAIRS))
def test_no_alloc_matches_decode_on_two_calls(case):
    for k, (cfg, lens, splits) in enumerate(PAIRS[case]):
        _say(f"no-alloc {case} call {k}: batch={cfg.batch} lens={lens} splits={splits}")
        inp, got = _run_pair(cfg, lens, splits)
        if k == 1:   # the smaller call also against the oracle
            ref = oracle_from_inputs(inp)
            g = got.float() if cfg.out_dtype == "f32" else got.view(torch.bfloat16).float()
            g = g.double().cpu().numpy()
            rms = float(np.sqrt(np.mean(ref ** 2)))
            tol = {"f32": 1e-5, "bf16": 2e-2, "e4m3": 6e-2}[cfg.cache_dtype]
            assert float(np.max(np.abs(g - ref))) <= tol * rms


def test_no_alloc_rejects_a_step_beyond_the_scratch():
    cfg = CONFIGS["dsv3_b64_4k"].replace(batch=2)
    inp = generate(cfg, seq_lens=[64, 64])
    dev = DeviceInputs(inp)
    p = dev.params(num_splits=4096)           # partials of 4098 slots: ~1 GiB
    assert _lib.mla_decode_workspace_size(p) > _lib.MLA_NO_ALLOC_SCRATCH_BYTES
    out = torch.zeros((2, cfg.heads, cfg.d_v), dtype=torch.float32, device="cuda")
    with pytest.raises(_lib.MlaError) as ei:
        _lib.mla_decode_no_alloc(p, dev.q, dev.c_kv, dev.c_kv_scale, dev.k_rope, dev.block_table,
                                 dev.seq_lens, dev.W_UK, dev.W_UV, out)
    assert ei.value.status == _lib.MLA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert not out.any()
