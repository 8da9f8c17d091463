"""MHA-mode prefill on the GPU vs its CPU oracle, through the C ABI (needs an
MI355X): ragged chunks over ragged cached contexts (one row, a partial first
query tile, a ragged last one, whole-sequence prefill from an empty cache),
pages smaller than a key tile, both output types, the fp8 cache, q_lens of zero and beyond
the context, and the DeepSeek-V3 head count at a longer context on sampled
rows and heads; rows past each chunk stay untouched."""
import sys

import numpy as np
import pytest
import torch

from head_latent_attention_10_amd import _lib
from head_latent_attention_10_amd.device import DeviceInputs, out_torch_dtype, to_device_array
from mla_inputs import CONFIGS
from mla_inputs.prefill import generate_prefill
from oracle.prefill import mha_prefill

pytestmark = pytest.mark.gpu

# Bars (bf16 arithmetic with fp32 accumulation, as for the decode step):
#  * per output row (b, l, i): max |err| <= 2e-2 RMS of that row, on every
#    case.  Rows that average many keys are small, and so are their rounding
#    errors;
#  * whole output: max |err| <= 2e-2 RMS over every computed value, on the
#    cases where every row sees many keys (the 128-head long contexts, the
#    benchmark's call, the small-page fp8 case).  On the small ragged cases a
#    row with one or a few keys has outputs ~15x the overall RMS, and the bf16
#    rounding of its value vectors alone exceeds 2e-2 of that RMS
#    (tests/test_prefill_bar_cpu.py shows it on the oracle's own output).
TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load_library()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_prefill(pi, q_lens=None, units=None):
    """Run mla_prefill; `units` sizes the workspace at that many (sequence,
    head) units (the call then runs in chunks), else the size the library asks for."""
    dev = DeviceInputs(pi.dense)
    c = pi.cfg
    q = to_device_array(pi.q, dev.device)
    ql = to_device_array(np.asarray(pi.q_lens if q_lens is None else q_lens, np.int32), dev.device)
    p = dev.params()
    n = _lib.mla_prefill_workspace_size(p)
    if units is not None:
        n = units * _lib.prefill_unit_bytes(dev.max_blocks_per_seq, c.page_size)
    ws = torch.empty(n, dtype=torch.uint8, device=dev.device)
    out = torch.empty((c.batch, pi.max_q_len, c.heads, c.d_v), dtype=out_torch_dtype(c.out_dtype),
                      device=dev.device)
    if c.out_dtype == "f32":
        out.fill_(float("nan"))
    else:
        out.fill_(0x7FC0)
    _lib.mla_prefill(p, pi.max_q_len, q, ql, dev.c_kv, dev.c_kv_scale, dev.k_rope, dev.block_table,
                     dev.seq_lens, dev.W_UK, dev.W_UV, out, ws, n)
    torch.cuda.synchronize()
    return (out if c.out_dtype == "f32" else out.view(torch.bfloat16)).float().double().cpu().numpy()


def check(pi, got, heads=None, batches=None, rows=None, label="", whole=False):
    c = pi.cfg
    ref = mha_prefill(pi.q, pi.q_lens, pi.c_kv, pi.c_kv_scale, pi.k_rope, pi.block_table,
                      pi.seq_lens, pi.W_UK, pi.W_UV, c.sm_scale, c.page_size, q_tag=c.q_dtype,
                      cache_tag=c.cache_dtype, rope_tag=c.rope_dtype, weight_tag=c.weight_dtype,
                      heads=heads, batches=batches, rows=rows)
    mask = ~np.isnan(ref)
    assert mask.any()
    assert np.all(np.isfinite(got[mask]))
    # the bar per output row (b, l, i): rows that average many keys are small,
    # and so are their rounding errors
    rows_done = mask.all(axis=-1)
    err = np.abs(got - ref).max(axis=-1)
    rms = np.sqrt(np.mean(ref * ref, axis=-1))
    ratio = np.where(rows_done, err / np.where(rows_done, rms, 1.0), 0.0)
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    b, l, i = (int(x) for x in worst)
    _say(f"  {label}: {int(rows_done.sum())} rows, worst (b={b}, l={l}, i={i}, "
         f"keys={int(pi.seq_lens[b]) - int(pi.q_lens[b]) + l + 1}): err {err[worst]:.3e}, "
         f"row RMS {rms[worst]:.3e}, ratio {ratio[worst]:.3e}; overall max err "
         f"{float(err[rows_done].max()):.3e}, RMS {float(np.sqrt(np.mean(ref[mask] ** 2))):.3e}")
    assert ratio[worst] <= TOL
    if whole:
        w = float(err[rows_done].max()) / float(np.sqrt(np.mean(ref[mask] ** 2)))
        assert w <= TOL, w
    # rows past each chunk are never written
    for b in range(c.batch):
        assert np.isnan(got[b, int(pi.q_lens[b]):]).all(), b


DSV3 = CONFIGS["dsv3_ragged_32k"]

CASES = {
    # T = 1, 70, 200, 333 with one row, the whole sequence, one full tile, a ragged chunk
    "ragged_bf16": dict(cfg=DSV3.replace(heads=4, batch=4, seed=5200, out_dtype="bf16"),
                        seq_lens=[1, 70, 200, 333], max_q_len=160, q_lens=[1, 70, 64, 150]),
    # pages of 16 tokens, prefill from an empty cache, f32 output
    "whole_f32_p16": dict(cfg=DSV3.replace(heads=3, batch=2, seed=5201, page_size=16),
                          seq_lens=[129, 64], max_q_len=129, q_lens=[129, 64]),
    # the fp8 cache (E4M3 codes and per-token scales; the oracle dequantises the same codes)
    "fp8_ragged": dict(cfg=CONFIGS["dsv3_fp8_16k"].replace(heads=4, batch=3, seed=5205,
                                                           seq_len=None, seq_len_range=(1, 400)),
                       seq_lens=[1, 150, 333], max_q_len=140, q_lens=[1, 140, 77]),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_prefill_matches_oracle(case):
    k = CASES[case]
    _say(f"prefill {case}")
    pi = generate_prefill(k["cfg"], k["max_q_len"], seq_lens=k["seq_lens"], q_lens=k["q_lens"])
    check(pi, run_prefill(pi), label=case)


@pytest.mark.parametrize("case", ["ragged_bf16", "fp8_ragged"])
def test_prefill_in_unit_chunks_matches_one_pass(case):
    """A workspace of 1, 3 or 5 (sequence, head) units runs the call in chunks
    of consecutive units (16 units: chunks of 1; 3 with a last chunk of 1; 4);
    each unit's keys, values and attention are computed as in one pass, so the
    outputs are the same bits, and they match the oracle."""
    k = CASES[case]
    pi = generate_prefill(k["cfg"], k["max_q_len"], seq_lens=k["seq_lens"], q_lens=k["q_lens"])
    units = pi.cfg.batch * pi.cfg.heads
    _say(f"prefill {case} in one pass ({units} units)")
    full = run_prefill(pi, units=units)
    check(pi, full, label=f"{case} one pass")
    for per in (1, 3, 5):
        _say(f"prefill {case} with a workspace of {per} units")
        got = run_prefill(pi, units=per)
        np.testing.assert_array_equal(got, full)


def test_prefill_clamps_q_lens():
    """q_lens of 0 writes nothing; q_lens beyond the context or max_q_len is
    clamped to min(max_q_len, T_b)."""
    cfg = DSV3.replace(heads=2, batch=3, seed=5202, page_size=32)
    _say("prefill clamps")
    pi = generate_prefill(cfg, 48, seq_lens=[40, 90, 17], q_lens=[0, 48, 17])
    got = run_prefill(pi, q_lens=[0, 500, 999])
    check(pi, got, label="clamped")


CACHES = ["bf16", "e4m3"]


@pytest.mark.parametrize("cache", CACHES)
def test_prefill_dsv3_heads_long_context_sampled(cache):
    """128 heads, contexts of 4000 and 8192 cached tokens, chunks of 512 and 300
    new tokens, over a bf16 or fp8 cache: every output is finite; sampled rows
    (tile edges, last row) and heads match the oracle."""
    cfg = DSV3.replace(batch=2, seed=5203, cache_dtype=cache)
    _say(f"prefill dsv3 long ({cache})")
    pi = generate_prefill(cfg, 512, seq_lens=[4000, 8192], q_lens=[512, 300])
    got = run_prefill(pi)
    for b in range(2):
        assert np.all(np.isfinite(got[b, :int(pi.q_lens[b])])), b
    check(pi, got, heads=[0, 37, 127], rows=[0, 63, 64, 255, 299, 511], label=f"dsv3 long {cache}", whole=True)


def test_prefill_fp8_small_pages_many_tiles():
    """fp8 cache with 16-token pages (eight pages per 128-token key tile),
    contexts of 1500 and 2047 tokens (many key tiles, ragged last page) and
    chunks crossing several query tiles."""
    cfg = DSV3.replace(heads=4, batch=2, seed=5206, cache_dtype="e4m3", page_size=16)
    _say("prefill fp8 small pages")
    pi = generate_prefill(cfg, 400, seq_lens=[1500, 2047], q_lens=[400, 257])
    check(pi, run_prefill(pi), label="fp8 p16", whole=True)


def test_prefill_empty_sequences():
    """A sequence with no cached tokens writes nothing, whatever q_lens says;
    its neighbours are unaffected."""
    cfg = DSV3.replace(heads=2, batch=3, seed=5204)
    _say("prefill empty sequences")
    pi = generate_prefill(cfg, 40, seq_lens=[0, 90, 0], q_lens=[0, 40, 0])
    got = run_prefill(pi, q_lens=[7, 40, 40])
    check(pi, got, label="empty")


@pytest.mark.parametrize("cache", CACHES)
def test_prefill_bench_configuration_sampled(cache):
    """The benchmark's call (2 sequences of 16384 cached tokens, the last 4096
    new, 128 heads, bf16 output, seed 1200) over a bf16 or fp8 cache: every
    output finite; rows at the chunk's start, q-tile edges and end match the
    oracle on sampled heads."""
    cfg = CONFIGS["dsv3_b8_32k"].replace(batch=2, seq_len=16384, out_dtype="bf16", seed=1200,
                                         cache_dtype=cache)
    _say(f"prefill bench configuration ({cache})")
    pi = generate_prefill(cfg, 4096)
    got = run_prefill(pi)
    assert np.all(np.isfinite(got))
    check(pi, got, heads=[0, 127], batches=[0, 1], rows=[0, 255, 256, 4095],
          label=f"bench config {cache}", whole=True)
