"""TPLA decode on the GPU vs its CPU oracle, through the C ABI (needs an
MI355X): element by element at the dense decode's bars (fp32 1e-5, bf16 2e-2,
fp8 6e-2 of RMS), for two and four shards and per-shard content factors, on
small cases over several tiles and ragged tails and on sampled (sequence,
head) pairs of the 32K ragged DeepSeek-V3 workload; one shard reproduces
mla_decode bit for bit."""
import sys

import numpy as np
import pytest
import torch

from head_latent_attention_10_amd import _lib
from head_latent_attention_10_amd.device import Decoder, DeviceInputs, out_torch_dtype
from mla_inputs import CONFIGS, generate
from oracle.tpla import tpla_decode

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


def run_tpla(inp, shards, mu=None, repeats=1, num_splits=0):
    dev = DeviceInputs(inp)
    p = dev.params(num_splits=num_splits)
    t = _lib.make_tpla_params(shards, mu)
    n = _lib.mla_tpla_decode_workspace_size(p, t)
    ws = torch.empty(n, dtype=torch.uint8, device=dev.device)
    c = inp.cfg
    outs = []
    for _ in range(repeats):
        out = torch.empty((c.batch, c.heads, c.d_v), dtype=out_torch_dtype(c.out_dtype),
                          device=dev.device)
        _lib.mla_tpla_decode(p, t, dev.q, dev.c_kv, dev.c_kv_scale, dev.k_rope, dev.block_table,
                             dev.seq_lens, dev.W_UK, dev.W_UV, out, ws, n)
        torch.cuda.synchronize()
        outs.append(out)
    return outs if repeats > 1 else outs[0]


def as_float(out, tag):
    return (out.float() if tag == "f32" else out.view(torch.bfloat16).float()).double().cpu().numpy()


def check(inp, out, shards, mu=None, batches=None, heads=None, label=""):
    c = inp.cfg
    ref = tpla_decode(inp.q, inp.c_kv, inp.c_kv_scale, inp.k_rope, inp.block_table, inp.seq_lens,
                      inp.W_UK, inp.W_UV, c.sm_scale, c.page_size, shards=shards, mu=mu,
                      q_tag=c.q_dtype, cache_tag=c.cache_dtype, rope_tag=c.rope_dtype,
                      weight_tag=c.weight_dtype, batches=batches, heads=heads)
    got = as_float(out, c.out_dtype)
    mask = ~np.isnan(ref)
    r, g = ref[mask], got[mask]
    assert np.all(np.isfinite(g))
    rms = float(np.sqrt(np.mean(r * r)))
    err = float(np.max(np.abs(g - r)))
    _say(f"  {label}: max err {err:.3e}, RMS {rms:.3e}, ratio {err / rms:.3e} "
         f"(tol {TOL[c.cache_dtype]})")
    assert err <= TOL[c.cache_dtype] * rms


def small(name, **kw):
    return CONFIGS[name].replace(**kw)


CASES = {
    "fp32": small("tiny_fp32", seq_len=None, seq_len_range=(1, 200), batch=3, seed=4100,
                  page_size=16),
    "bf16": small("dsv3_ragged_32k", seq_len_range=(1, 700), batch=3, seed=4101),
    "fp8": small("dsv3_fp8_16k", seq_len=None, seq_len_range=(1, 600), batch=3, seed=4102),
    # 64 heads on 16-token pages: the shard heads still come in whole 64-head
    # groups (one per shard for two shards), and steps span pages
    "bf16_h64_p16": small("dsv3_ragged_32k", heads=64, page_size=16, seq_len_range=(1, 500),
                          batch=3, seed=4103),
    # 32 heads: whole 32-head blocks (merged by shard) but no 64-head shard groups
    "bf16_h32": small("dsv3_ragged_32k", heads=32, seq_len_range=(1, 400), batch=2, seed=4104),
    # 16 heads: shard heads merged whole, then gathered
    "bf16_h16": small("dsv3_ragged_32k", heads=16, seq_len_range=(1, 400), batch=2, seed=4105),
}


@pytest.mark.parametrize("case", sorted(CASES))
@pytest.mark.parametrize("shards,mu", [(2, None), (4, None), (2, [0.8, 1.25])])
def test_tpla_matches_oracle(case, shards, mu):
    cfg = CASES[case]
    _say(f"tpla {case} shards={shards} mu={mu}")
    inp = generate(cfg)
    out = run_tpla(inp, shards, mu)
    h = cfg.heads
    heads = None if h <= 16 else sorted({0, 1, h // 2 - 1, h // 2, h - 1})
    check(inp, out, shards, mu, heads=heads, label=f"{case} g={shards}")


@pytest.mark.parametrize("shards", [2, 4])
def test_tpla_many_splits_per_sequence(shards):
    """200 splits over two long sequences: each sequence's merge runs over more
    than 64 slots (the weights of a second 64-slot chunk) in every shard."""
    cfg = small("dsv3_ragged_32k", batch=2, seed=4106)
    inp = generate(cfg, seq_lens=[5000, 3100])
    _say(f"tpla many splits shards={shards}")
    out = run_tpla(inp, shards, num_splits=200)
    h = cfg.heads
    check(inp, out, shards, heads=sorted({0, 1, h // 2 - 1, h // 2, h - 1}),
          label=f"200 splits g={shards}")


def test_one_shard_is_mla_decode_bitwise():
    inp = generate(CASES["bf16"])
    out = run_tpla(inp, 1)
    dec = Decoder(DeviceInputs(inp))
    dec()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.uint8), dec.out.view(torch.uint8))


def test_tpla_is_deterministic():
    inp = generate(CASES["bf16"])
    a, b = run_tpla(inp, 2, repeats=2)
    assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


@pytest.mark.parametrize("shards", [2, 4])
def test_tpla_full_size_sampled(shards):
    """The 32K ragged DeepSeek-V3 workload, two or four shards, sampled pairs."""
    _say(f"tpla dsv3_ragged_32k shards={shards}")
    inp = generate(CONFIGS["dsv3_ragged_32k"])
    out = run_tpla(inp, shards)
    check(inp, out, shards, batches=[0, 5], heads=[3, 77, 127], label=f"dsv3_ragged_32k g={shards}")
