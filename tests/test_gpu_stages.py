"""The decode step's stages through the C ABI (needs an MI355X): the split
attention (mla_attend_partial) followed by the log-sum-exp merge (mla_combine)
is mla_attend_latent bit for bit, and with the up-projection it is mla_decode
bit for bit; a merge over a single split returns the split's partial
unchanged; the generic kernel, serving misaligned pools of a matrix-core
shape, writes the partials as the same bf16 rows and the step still meets the
oracle."""
import sys

import numpy as np
import pytest
import torch

from head_latent_attention_10_amd import _lib
from head_latent_attention_10_amd.device import Decoder, DeviceInputs
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


def _cfg(name, **kw):
    base = dict(batch=3, seq_len=None, seq_len_range=(1, 700))
    base.update(kw)
    return CONFIGS[name].replace(**base)


CASES = {
    "dsv3_bf16": _cfg("dsv3_b64_4k", seed=7100),
    "dsv3_fp8": _cfg("dsv3_fp8_16k", seed=7101),
    "transmla_h32": _cfg("transmla_llama2_7b", seed=7102, heads=32),
    "tiny_fp32": CONFIGS["tiny_fp32"].replace(seed=7103),
    # more than 16 sequences: the step merges and up-projects in two launches
    "dsv3_bf16_b24": _cfg("dsv3_b64_4k", seed=7104, batch=24, seq_len_range=(1, 300)),
}


def _stages(dec, dev, cfg, **over):
    """absorb -> partial -> combine -> up-projection on fresh buffers."""
    p = dec.p
    qlat = torch.empty((cfg.batch, cfg.heads, cfg.d_latent + cfg.d_rope),
                       dtype=torch.float32 if _lib.mla_absorbed_dtype(p) == _lib.MLA_F32 else torch.int16,
                       device="cuda")
    _lib.mla_absorb_q(p, dev.q, dev.W_UK, qlat)
    c_kv = over.get("c_kv", dev.c_kv)
    ws = torch.empty(dec.ws_bytes, dtype=torch.uint8, device="cuda")
    _lib.mla_attend_partial(p, qlat, c_kv, dev.c_kv_scale, dev.k_rope, dev.block_table,
                            dev.seq_lens, ws)
    olat = torch.full((cfg.batch, cfg.heads, cfg.d_latent), float("nan"), device="cuda")
    _lib.mla_combine(p, olat, ws)
    out = torch.empty_like(dec.out)
    _lib.mla_up_project(p, olat, dev.W_UV, out)
    olat2 = torch.full_like(olat, float("nan"))
    ws2 = torch.empty_like(ws)
    _lib.mla_attend_latent(p, qlat, c_kv, dev.c_kv_scale, dev.k_rope, dev.block_table,
                           dev.seq_lens, olat2, ws2)
    torch.cuda.synchronize()
    return olat, olat2, out, ws


@pytest.mark.parametrize("case", sorted(CASES))
def test_partial_then_combine_is_attend_latent_and_decode(case):
    cfg = CASES[case]
    _say(f"stages {case}")
    inp = generate(cfg)
    dev = DeviceInputs(inp)
    dec = Decoder(dev, num_splits=13)
    dec()
    olat, olat2, out, _ = _stages(dec, dev, cfg)
    assert torch.isfinite(olat).all()
    assert torch.equal(olat, olat2)
    assert torch.equal(out, dec.out)


@pytest.mark.parametrize("case", ["dsv3_bf16", "tiny_fp32"])
def test_single_split_combine_returns_the_partial(case):
    """A sequence that one split holds whole gets that split's partial back
    bit for bit; the partial is read at the offsets mla_partials_layout gives,
    in the type (bf16 or fp32) and layout it states."""
    cfg = CASES[case].replace(batch=8)
    _say(f"single split {case}")
    inp = generate(cfg)
    dev = DeviceInputs(inp)
    dec = Decoder(dev, num_splits=1)
    olat, _, _, ws = _stages(dec, dev, cfg)
    off_o, off_l, slots, bf16 = _lib.mla_partials_layout(dec.p)
    splits = _lib.mla_decode_num_splits(dec.p)
    assert slots == splits + cfg.batch
    tiles = [(int(t) + 31) // 32 for t in inp.seq_lens]
    _, seq = _lib.mla_split_plan(tiles, splits)
    h, dc = cfg.heads, cfg.d_latent
    if bf16:   # bf16 rows, widened exactly
        part = ws[off_o: off_o + slots * h * dc * 2].view(torch.bfloat16).float().cpu().numpy()
    else:
        part = ws[off_o: off_o + slots * h * dc * 4].view(torch.float32).cpu().numpy()
    part = part.reshape(slots, h * dc)
    got = olat.cpu().numpy()
    whole = 0
    for b in range(cfg.batch):
        if tiles[b] == 0:
            assert not got[b].any()
            continue
        g0, g1 = int(seq[b, 0]), int(seq[b, 1])
        if g0 != g1:
            continue
        blk = part[g0 + b]                 # pair (split g, sequence b) -> slot g + b
        ref = blk.reshape(h, dc)
        assert np.array_equal(got[b], ref), b
        whole += 1
    assert whole >= cfg.batch // 2, whole


def test_misaligned_pools_take_the_generic_kernel_with_bf16_partials():
    """A 2-byte offset of the latent pool sends a matrix-core shape to the
    generic kernel; its partials are the same bf16 rows, so the merge and the
    whole step still match the oracle."""
    cfg = CASES["dsv3_bf16"]
    _say("misaligned pools")
    inp = generate(cfg)
    dev = DeviceInputs(inp)
    n = dev.c_kv.numel()
    buf = torch.empty(n + 8, dtype=dev.c_kv.dtype, device="cuda")
    mis = buf[1:1 + n].view(dev.c_kv.shape)
    mis.copy_(dev.c_kv)
    assert mis.data_ptr() % 16 != 0
    dec = Decoder(dev, num_splits=7)
    assert _lib.mla_partials_layout(dec.p)[3] == 1
    dec(c_kv=mis)
    torch.cuda.synchronize()
    gpu = dec.out_float().double().cpu().numpy()
    ref = oracle_from_inputs(inp)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.max(np.abs(gpu - ref)))
    _say(f"  max|err|/RMS = {err / rms:.3e}")
    assert err <= 2e-2 * rms
    olat, olat2, out, _ = _stages(dec, dev, cfg, c_kv=mis)
    assert torch.equal(olat, olat2)
    assert torch.equal(out, dec.out)
