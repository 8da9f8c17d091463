"""Grouped-MLA decode on the GPU vs its CPU oracle, through the C ABI (needs an
MI355X): two and four latent groups, fp32 (generic kernels), bf16 and fp8
caches, head splits that the matrix-core kernels serve (64 heads per group)
and that they do not (the generic kernel), at the dense decode's bars; one
group is mla_decode bit for bit."""
import sys

import numpy as np
import pytest
import torch

from head_latent_attention_10_amd import _lib
from head_latent_attention_10_amd.device import Decoder, DeviceInputs, out_torch_dtype, to_device_array
from mla_inputs import CONFIGS
from mla_inputs.grouped import generate_grouped
from oracle.grouped import grouped_decode

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2, "e4m3": 6e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load_library()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_grouped(gi):
    dev = DeviceInputs(gi.dense)
    pools = to_device_array(gi.c_pools, dev.device)
    scales = None if gi.scale_pools is None else to_device_array(gi.scale_pools, dev.device)
    p = dev.params()
    n = _lib.mla_decode_workspace_size(p)
    ws = torch.empty(n, dtype=torch.uint8, device=dev.device)
    c = gi.cfg
    out = torch.empty((c.batch, c.heads, c.d_v), dtype=out_torch_dtype(c.out_dtype),
                      device=dev.device)
    _lib.mla_grouped_decode(p, gi.groups, dev.q, pools, scales, dev.k_rope, dev.block_table,
                            dev.seq_lens, dev.W_UK, dev.W_UV, out, ws, n)
    torch.cuda.synchronize()
    return out


def check(gi, out, heads=None, batches=None, label=""):
    c = gi.cfg
    ref = grouped_decode(gi.q, gi.c_pools, gi.scale_pools, gi.k_rope, gi.block_table,
                         gi.seq_lens, gi.W_UK, gi.W_UV, c.sm_scale, c.page_size, q_tag=c.q_dtype,
                         cache_tag=c.cache_dtype, rope_tag=c.rope_dtype, weight_tag=c.weight_dtype,
                         heads=heads, batches=batches)
    got = (out.float() if c.out_dtype == "f32" else out.view(torch.bfloat16).float()).double().cpu().numpy()
    mask = ~np.isnan(ref)
    r, g = ref[mask], got[mask]
    assert np.all(np.isfinite(g))
    rms = float(np.sqrt(np.mean(r * r)))
    err = float(np.max(np.abs(g - r)))
    _say(f"  {label}: max err {err:.3e}, RMS {rms:.3e}, ratio {err / rms:.3e}")
    assert err <= TOL[c.cache_dtype] * rms


CASES = {
    "fp32": (CONFIGS["tiny_fp32"].replace(seq_len=None, seq_len_range=(1, 150), batch=3,
                                          seed=5100, page_size=16), [2, 4]),
    "bf16": (CONFIGS["dsv3_ragged_32k"].replace(seq_len_range=(1, 900), batch=3, seed=5101), [2]),
    "bf16_generic_split": (CONFIGS["dsv3_ragged_32k"].replace(seq_len_range=(1, 300), batch=2,
                                                              seed=5103), [4]),
    "fp8": (CONFIGS["dsv3_fp8_16k"].replace(seq_len=None, seq_len_range=(1, 700), batch=3,
                                            seed=5102), [2]),
    "transmla": (CONFIGS["transmla_llama2_7b"].replace(seq_len=None, seq_len_range=(1, 500),
                                                       batch=2, seed=5104), [2]),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_grouped_matches_oracle(case):
    cfg, groups = CASES[case]
    for G in groups:
        _say(f"grouped {case} G={G}")
        gi = generate_grouped(cfg, G)
        out = run_grouped(gi)
        heads = None if cfg.heads <= 8 else [0, cfg.heads // G - 1, cfg.heads // G, cfg.heads - 1]
        check(gi, out, heads=heads, label=f"{case} G={G}")


def test_one_group_is_mla_decode_bitwise():
    gi = generate_grouped(CASES["bf16"][0], 1)
    out = run_grouped(gi)
    dec = Decoder(DeviceInputs(gi.dense))
    dec()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.uint8), dec.out.view(torch.uint8))


def test_grouped_full_size_sampled():
    """kv_rank 1088 (two 512-wide groups + rope 64) at the 32K ragged DeepSeek-V3 shape."""
    gi = generate_grouped(CONFIGS["dsv3_ragged_32k"], 2)
    out = run_grouped(gi)
    check(gi, out, heads=[5, 70], batches=[1, 6], label="dsv3_ragged_32k G=2")
