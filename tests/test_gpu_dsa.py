"""DSA sparse decode on the GPU vs its CPU oracle, through the C ABI (needs an
MI355X).

  * top-k: bit-exact against the oracle's selection on the same fp32 scores
    (seeded, with planted ties and signed zeros);
  * indexer scores: against the oracle's fp64 scores of the same E4M3 codes,
    within an fp32 accumulation bound per score,
        |gpu - oracle| <= 2e-5 * sum_j |w_j| qs_j ks_s sum_d |q8_jd k8_sd|;
  * sparse decode over given index lists: element by element against the
    oracle, with the dense decode's bars (fp32 1e-5, bf16 2e-2, fp8 6e-2 of
    RMS);
  * the composed step: the selection is checked for what is unique (every
    position whose oracle score clears the k-th by more than the bound is
    selected, every one below it by more than the bound is not, exactly
    min(T, k) positions, increasing); where no oracle score lies within the
    bound of the k-th, the selection must equal the oracle's and the output is
    compared with the oracle's sparse decode; and the composed call is bitwise
    equal to its three stage entry points run in sequence (each of which is
    compared with the oracle above).  At long contexts several scores lie
    within the (worst-case) bound of the k-th, so there the output is covered
    through the stages.
"""
import sys

import numpy as np
import pytest
import torch

from head_latent_attention_10_amd import _lib
from head_latent_attention_10_amd.device import DeviceInputs, out_torch_dtype, to_device_array
from mla_inputs.dsa import DSA_CONFIGS, generate_dsa
from oracle.dsa import (decode_scaled_e4m3, gather_index_keys, sequence_index_scores,
                        sparse_decode, topk_select)

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2, "e4m3": 6e-2}
SCORE_TOL = 2e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load_library()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# ------------------------------------------------------------------ helpers

class DsaDevice:
    def __init__(self, inp):
        self.inp = inp
        self.dense = DeviceInputs(inp.dense)
        dev = self.dense.device
        for f in ("q_I", "q_I_scale", "w_I", "k_I", "k_I_scale"):
            setattr(self, f, to_device_array(getattr(inp, f), dev))
        d = inp.dcfg
        self.d = _lib.make_dsa_params(d.index_heads, d.index_dim, d.topk)
        self.p = self.dense.params()

    def out_tensor(self):
        c = self.inp.cfg
        return torch.empty((c.batch, c.heads, c.d_v), dtype=out_torch_dtype(c.out_dtype),
                           device=self.dense.device)


def _out_float(t, tag):
    return (t.float() if tag == "f32" else t.view(torch.bfloat16).float()).double().cpu().numpy()


def score_bound(inp, b):
    """Per-position bound on |gpu - oracle| for the index scores of sequence b."""
    Q = np.abs(decode_scaled_e4m3(inp.q_I[b], inp.q_I_scale[b]))
    K = np.abs(gather_index_keys(inp.k_I, inp.k_I_scale, inp.block_table, inp.seq_lens[b], b,
                                 inp.cfg.page_size))
    return SCORE_TOL * ((K @ Q.T) @ np.abs(inp.w_I[b].astype(np.float64))) + 1e-30


def check_out(ref, got, tag, label):
    mask = ~np.isnan(ref)
    r, g = ref[mask], got[mask]
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    rms = float(np.sqrt(np.mean(r * r)))
    err = float(np.max(np.abs(g - r)))
    _say(f"  {label}: max err {err:.3e}, RMS {rms:.3e}, ratio {err / max(rms, 1e-30):.3e} "
         f"(tol {TOL[tag]})")
    assert err <= TOL[tag] * rms


# ------------------------------------------------------------------ top-k

def _scores_with_ties(rng, T):
    s = rng.standard_normal(T).astype(np.float32)
    if T > 8:
        # plant ties: runs of equal values, signed zeros, repeated maxima
        idx = rng.choice(T, size=max(1, T // 10), replace=False)
        s[idx] = np.float32(0.75)
        z = rng.choice(T, size=max(1, T // 20), replace=False)
        s[z[: len(z) // 2]] = np.float32(0.0)
        s[z[len(z) // 2:]] = np.float32(-0.0)
        s[rng.choice(T, size=3, replace=False)] = np.float32(3.5)
    return s


TOPK = ["one_group", "split"]


def run_topk(variant, scores, stride, lens, B, k, idx, index_stride, cnt):
    """mla_topk_select (one work group per sequence) or mla_topk_select_split
    (candidate pass over several work groups per sequence)."""
    if variant == "one_group":
        _lib.mla_topk_select(scores, stride, lens, B, k, idx, index_stride, cnt)
    else:
        n = _lib.mla_topk_select_split_workspace_size(B, stride)
        ws = torch.empty(n, dtype=torch.uint8, device=scores.device)
        ws.fill_(0xAB)  # stale contents must not matter
        _lib.mla_topk_select_split(scores, stride, lens, B, k, idx, index_stride, cnt, ws, n)


@pytest.mark.parametrize("variant", TOPK)
@pytest.mark.parametrize("k,lens", [
    (300, [0, 1, 299, 300, 301, 5000, 4096, 777]),
    (2048, [131072, 2047, 2049, 65536]),
    (1, [1, 2, 50, 9]),
    # one candidate chunk, chunk edges, a ragged last chunk, 128 chunks
    (700, [2048, 2049, 4095, 6145, 262144, 9000]),
])
def test_topk_bit_exact(k, lens, variant):
    _say(f"top-k {variant} k={k} lens={lens}")
    rng = np.random.default_rng(900 + k)
    B, stride = len(lens), max(lens) + 3
    scores = np.full((B, stride), np.nan, np.float32)
    for b, T in enumerate(lens):
        scores[b, :T] = _scores_with_ties(rng, T)
    dev = torch.device("cuda")
    st = torch.from_numpy(scores).to(dev)
    lt = torch.tensor(lens, dtype=torch.int32, device=dev)
    idx = torch.full((B, k + 5), -7, dtype=torch.int32, device=dev)
    cnt = torch.full((B,), -7, dtype=torch.int32, device=dev)
    run_topk(variant, st, stride, lt, B, k, idx, k + 5, cnt)
    torch.cuda.synchronize()
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    for b, T in enumerate(lens):
        want = topk_select(scores[b, :T], k)
        assert cnt[b] == len(want), (b, cnt[b], len(want))
        assert np.array_equal(idx[b, :len(want)], want), (b, T)
        assert (idx[b, len(want):] == -7).all()


@pytest.mark.parametrize("variant", TOPK)
def test_topk_paths_past_the_sample_bound(variant):
    """Inputs the sampled lower bound cannot serve: a sequence longer than the
    in-LDS path allows, large scores only between the sampled positions, and k
    close to T -- all must still match the oracle bit for bit."""
    _say(f"top-k {variant} past the sample bound")
    rng = np.random.default_rng(4242)
    T1, T2, T3 = 300000, 20000, 20000
    lens, ks = [T1, T2, T3], 2048
    stride = T1
    scores = np.full((3, stride), np.nan, np.float32)
    scores[0, :T1] = _scores_with_ties(rng, T1)
    s2 = rng.standard_normal(T2).astype(np.float32)
    sampled = (np.arange(1024, dtype=np.int64) * T2) // 1024
    s2 += 10.0
    s2[sampled] -= 20.0          # the sample sees only the small scores
    scores[1, :T2] = s2
    scores[2, :T3] = _scores_with_ties(rng, T3)
    dev = torch.device("cuda")
    st = torch.from_numpy(scores).to(dev)
    for k in (ks, 19000):
        lt = torch.tensor(lens, dtype=torch.int32, device=dev)
        idx = torch.full((3, k), -7, dtype=torch.int32, device=dev)
        cnt = torch.empty((3,), dtype=torch.int32, device=dev)
        run_topk(variant, st, stride, lt, 3, k, idx, k, cnt)
        torch.cuda.synchronize()
        got, c = idx.cpu().numpy(), cnt.cpu().numpy()
        for b, T in enumerate(lens):
            want = topk_select(scores[b, :T], k)
            assert c[b] == len(want) and np.array_equal(got[b, :len(want)], want), (k, b)


@pytest.mark.parametrize("variant", TOPK)
def test_topk_all_equal_scores_take_the_earliest(variant):
    _say(f"top-k {variant} all equal")
    dev = torch.device("cuda")
    T, k = 10000, 2048
    s = torch.zeros((2, T), dtype=torch.float32, device=dev)
    s[1, ::2] = -0.0
    lens = torch.tensor([T, T], dtype=torch.int32, device=dev)
    idx = torch.empty((2, k), dtype=torch.int32, device=dev)
    cnt = torch.empty((2,), dtype=torch.int32, device=dev)
    run_topk(variant, s, T, lens, 2, k, idx, k, cnt)
    torch.cuda.synchronize()
    assert (cnt.cpu().numpy() == k).all()
    assert np.array_equal(idx.cpu().numpy(), np.tile(np.arange(k), (2, 1)))


# ------------------------------------------------------------------ indexer

@pytest.mark.parametrize("name", ["dsa_tiny", "dsa_dsv3_small"])
def test_indexer_scores_within_bound(name):
    _say(f"indexer {name}")
    inp = generate_dsa(DSA_CONFIGS[name])
    D = DsaDevice(inp)
    stride = int(inp.block_table.shape[1] * inp.cfg.page_size)
    scores = torch.full((inp.cfg.batch, stride), float("nan"), dtype=torch.float32,
                        device=D.dense.device)
    _lib.mla_indexer_scores(D.p, D.d, D.q_I, D.q_I_scale, D.w_I, D.k_I, D.k_I_scale,
                            D.dense.block_table, D.dense.seq_lens, scores, stride)
    torch.cuda.synchronize()
    got = scores.double().cpu().numpy()
    for b, T in enumerate(inp.seq_lens):
        T = int(T)
        want = sequence_index_scores(inp.q_I, inp.q_I_scale, inp.w_I, inp.k_I, inp.k_I_scale,
                                     inp.block_table, inp.seq_lens, inp.cfg.page_size, b)
        bound = score_bound(inp, b)
        err = np.abs(got[b, :T] - want)
        assert np.all(err <= bound), (b, float(np.max(err / bound)))
        assert np.isnan(got[b, T:]).all()   # nothing written past T
        _say(f"  seq {b}: T={T}, max err/bound {float(np.max(err / bound)):.3f}")


# ------------------------------------------------------------------ sparse decode

def _random_lists(rng, lens, k, dup=False):
    B = len(lens)
    idx = np.full((B, k), -1, np.int32)
    cnt = np.zeros(B, np.int32)
    sel = []
    for b, T in enumerate(lens):
        n = min(int(T), k)
        s = (rng.integers(0, T, size=n) if dup else
             np.sort(rng.choice(int(T), size=n, replace=False))) if n else np.zeros(0, np.int64)
        idx[b, :n] = s
        cnt[b] = n
        sel.append(s.astype(np.int64))
    return idx, cnt, sel


@pytest.mark.parametrize("name,dup", [("dsa_tiny", False), ("dsa_tiny", True),
                                      ("dsa_dsv3_small", False), ("dsa_dsv3_fp8_16k", False),
                                      ("dsa_dsv3_ragged_32k", False),
                                      ("dsa_dsv3_ragged_32k", True)])
def test_sparse_decode_matches_oracle(name, dup):
    _say(f"sparse decode {name} dup={dup}")
    inp = generate_dsa(DSA_CONFIGS[name])
    cfg = inp.cfg
    k = inp.topk
    rng = np.random.default_rng(55)
    idx, cnt, sel = _random_lists(rng, inp.seq_lens, k, dup)
    D = DsaDevice(inp)
    dev = D.dense.device
    it, ct = to_device_array(idx, dev), to_device_array(cnt, dev)
    ws_bytes = _lib.mla_decode_sparse_workspace_size(D.p, k)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = D.out_tensor()
    d = D.dense
    _lib.mla_decode_sparse(D.p, d.q, d.c_kv, d.c_kv_scale, d.k_rope, d.block_table, it, k, ct,
                           d.W_UK, d.W_UV, out, ws, ws_bytes)
    torch.cuda.synchronize()
    got = _out_float(out, cfg.out_dtype)
    heads = None if cfg.heads <= 8 else [0, 37, 127]
    batches = None if cfg.batch <= 4 else [0, 2, cfg.batch - 1]
    ref = sparse_decode(inp.q, inp.c_kv, inp.c_kv_scale, inp.k_rope, inp.block_table, sel,
                        inp.W_UK, inp.W_UV, cfg.sm_scale, cfg.page_size, q_tag=cfg.q_dtype,
                        cache_tag=cfg.cache_dtype, rope_tag=cfg.rope_dtype,
                        weight_tag=cfg.weight_dtype, batches=batches, heads=heads)
    check_out(ref, got, cfg.cache_dtype, name)


# ------------------------------------------------------------------ composed step

def run_dsa(inp, repeats=1):
    D = DsaDevice(inp)
    dev = D.dense.device
    k = inp.topk
    ws_bytes = _lib.mla_dsa_decode_workspace_size(D.p, D.d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    d = D.dense
    res = []
    for _ in range(repeats):
        out = D.out_tensor()
        idx = torch.full((inp.cfg.batch, k), -1, dtype=torch.int32, device=dev)
        _lib.mla_dsa_decode(D.p, D.d, d.q, d.c_kv, d.c_kv_scale, d.k_rope, d.block_table,
                            d.seq_lens, D.q_I, D.q_I_scale, D.w_I, D.k_I, D.k_I_scale, d.W_UK,
                            d.W_UV, out, idx, ws, ws_bytes)
        torch.cuda.synchronize()
        res.append((out.clone(), idx.cpu().numpy()))
    return res if repeats > 1 else res[0]


def check_selection(inp, b, got_idx):
    """The unique part of the selection of sequence b.  Returns the oracle's
    selection and whether it is unambiguous (no other score within the error
    bound of the k-th), in which case the GPU's must equal it."""
    T, k = int(inp.seq_lens[b]), inp.topk
    s = sequence_index_scores(inp.q_I, inp.q_I_scale, inp.w_I, inp.k_I, inp.k_I_scale,
                              inp.block_table, inp.seq_lens, inp.cfg.page_size, b)
    want = topk_select(s, k)
    n = len(want)
    sel = got_idx[:n]
    assert (got_idx[n:] == -1).all()
    if T <= k:
        assert np.array_equal(sel, np.arange(T))
        return want, True
    assert np.all(np.diff(sel) > 0) and sel[0] >= 0 and sel[-1] < T
    bound = score_bound(inp, b)
    order = np.argsort(-s, kind="stable")
    kth_pos = order[k - 1]
    kth, kb = s[kth_pos], bound[kth_pos]
    chosen = np.zeros(T, bool)
    chosen[sel] = True
    # clear winners and clear losers under the bound
    assert chosen[s - bound > kth + kb].all()
    assert not chosen[s + bound < kth - kb].any()
    near = np.abs(s - kth) <= bound + kb
    unambiguous = int(near.sum()) <= 1
    if unambiguous:
        assert np.array_equal(sel, want)
    _say(f"  seq {b}: T={T}, positions within the bound of the k-th: {int(near.sum())}")
    return want, unambiguous


def run_stages(inp):
    """The three stage entry points in sequence (indexer, top-k, sparse decode)."""
    D = DsaDevice(inp)
    dev = D.dense.device
    cfg, k = inp.cfg, inp.topk
    stride = int(inp.block_table.shape[1] * cfg.page_size)
    scores = torch.empty((cfg.batch, stride), dtype=torch.float32, device=dev)
    d = D.dense
    _lib.mla_indexer_scores(D.p, D.d, D.q_I, D.q_I_scale, D.w_I, D.k_I, D.k_I_scale,
                            d.block_table, d.seq_lens, scores, stride)
    idx = torch.full((cfg.batch, k), -1, dtype=torch.int32, device=dev)
    cnt = torch.empty((cfg.batch,), dtype=torch.int32, device=dev)
    _lib.mla_topk_select(scores, stride, d.seq_lens, cfg.batch, k, idx, k, cnt)
    ws_bytes = _lib.mla_decode_sparse_workspace_size(D.p, k)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = D.out_tensor()
    _lib.mla_decode_sparse(D.p, d.q, d.c_kv, d.c_kv_scale, d.k_rope, d.block_table, idx, k, cnt,
                           d.W_UK, d.W_UV, out, ws, ws_bytes)
    torch.cuda.synchronize()
    return out, idx.cpu().numpy()


@pytest.mark.parametrize("name", ["dsa_tiny", "dsa_dsv3_small", "dsa_dsv3_ragged_32k",
                                  "dsa_dsv3_fp8_16k"])
def test_dsa_step_matches_oracle(name):
    """Selection checked against the oracle's scores; the output against the
    oracle on every sequence whose selection is unambiguous; the composed call
    bitwise equal to its three stages (each compared with the oracle above)."""
    _say(f"dsa step {name}")
    inp = generate_dsa(DSA_CONFIGS[name])
    cfg = inp.cfg
    out, idx = run_dsa(inp)
    checked = [check_selection(inp, b, idx[b]) for b in range(cfg.batch)]
    sure = [b for b, (_, u) in enumerate(checked) if u]
    _say(f"  unambiguous selections: {len(sure)}/{cfg.batch}")
    if name in ("dsa_tiny", "dsa_dsv3_small"):
        assert sure, "no sequence with an unambiguous selection"
    if sure:
        heads = None if cfg.heads <= 8 else [0, 64, 127]
        batches = sure if len(sure) <= 4 else [sure[0], sure[len(sure) // 2], sure[-1]]
        ref = sparse_decode(inp.q, inp.c_kv, inp.c_kv_scale, inp.k_rope, inp.block_table,
                            [w for w, _ in checked], inp.W_UK, inp.W_UV, cfg.sm_scale,
                            cfg.page_size, q_tag=cfg.q_dtype, cache_tag=cfg.cache_dtype,
                            rope_tag=cfg.rope_dtype, weight_tag=cfg.weight_dtype,
                            batches=batches, heads=heads)
        check_out(ref, _out_float(out, cfg.out_dtype), cfg.cache_dtype, name)
    out2, idx2 = run_stages(inp)
    assert np.array_equal(idx, idx2)
    assert torch.equal(out.view(torch.uint8), out2.view(torch.uint8))


def test_dsa_step_full_context_sampled():
    """The pages' design point: 128K context, top-2048, sampled sequences and heads."""
    _say("dsa step dsa_dsv3_b4_128k")
    inp = generate_dsa(DSA_CONFIGS["dsa_dsv3_b4_128k"])
    cfg = inp.cfg
    out, idx = run_dsa(inp)
    checked = [check_selection(inp, b, idx[b]) for b in range(cfg.batch)]
    sure = [b for b, (_, u) in enumerate(checked) if u]
    _say(f"  unambiguous selections: {len(sure)}/{cfg.batch}")
    if sure:
        ref = sparse_decode(inp.q, inp.c_kv, inp.c_kv_scale, inp.k_rope, inp.block_table,
                            [w for w, _ in checked], inp.W_UK, inp.W_UV, cfg.sm_scale,
                            cfg.page_size, q_tag=cfg.q_dtype, cache_tag=cfg.cache_dtype,
                            rope_tag=cfg.rope_dtype, weight_tag=cfg.weight_dtype,
                            batches=sure[:2], heads=[5, 100])
        check_out(ref, _out_float(out, cfg.out_dtype), cfg.cache_dtype, "dsa_dsv3_b4_128k")
    out2, idx2 = run_stages(inp)
    assert np.array_equal(idx, idx2)
    assert torch.equal(out.view(torch.uint8), out2.view(torch.uint8))


def test_dsa_step_is_deterministic_and_handles_empty_sequences():
    inp = generate_dsa(DSA_CONFIGS["dsa_dsv3_small"])
    (o1, i1), (o2, i2) = run_dsa(inp, repeats=2)
    assert torch.equal(o1.view(torch.uint8), o2.view(torch.uint8)) and np.array_equal(i1, i2)
    # an empty sequence attends to nothing: zero output, no selection
    inp.dense.seq_lens[1] = 0
    out, idx = run_dsa(inp)
    o = _out_float(out, inp.cfg.out_dtype)
    assert (o[1] == 0).all() and (idx[1] == -1).all()
    assert np.isfinite(o).all()
