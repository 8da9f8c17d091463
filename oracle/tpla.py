"""Plain CPU oracle of TPLA decode: the latent dimension cut into g shards,
a softmax per shard, the shard outputs summed after the value projection.

TEST INFRASTRUCTURE ONLY.  Imported by the tests and the benchmark's checks;
never by the HIP library, with which it shares no code.  Arithmetic is fp64.

Source: "TPLA: Tensor Parallel Latent Attention for Efficient Disaggregated
Prefill and Decode Inference":
  * "The Core TPLA Computation and Structural Differences from GLA"
    (Eqs. 6-7): shard j of the absorbed query meets shard j of the latent
    cache, every head on every shard; each shard takes its own softmax and
    weighted sum, and the up-projected shard outputs are added; the rope key
    is replicated, so every shard adds the full positional score;
  * "The softmax non-linearity problem": the sum of per-shard softmaxes
    differs from the joint one unless the missing shard adds the same score
    to every token;
  * "Reparameterization Methods: Hadamard vs. PCA" (Section 4.3.1): the
    Sylvester construction H_2n = [[H_n, H_n], [H_n, -H_n]], H_d H_d^T = d I,
    and the counterexample Q = (100, 0, 0, 0), c = (0, 0, 80, 0);
  * the complexity analysis: a device holding one of two shards stores
    d_c / 2 + d_r values per token (320 for DeepSeek-V3).

Readings taken where the page is silent or inconsistent:
  * T1: one softmax scale for the content and positional terms, as in the
    dense decode step (the page's "RoPE handling" form; its softmax-slicing
    section scales the two terms differently), times an optional per-shard
    factor mu_j on the content term (default 1; the page gives both mu = alpha
    and mu ~ 1/alpha for PCA);
  * T2: shards are contiguous, equal slices of the latent dimension, in order;
  * T3: the reparameterisation U (Hadamard or PCA) is an offline change of
    basis applied to the cache and to W_UK, W_UV; the decode step consumes the
    transformed tensors as they are.

Pins (tests/test_oracle_tpla_pins.py, CPU only): one shard is the dense
oracle; a shard whose latent rows are equal for every token gives the dense
result (the page's equality condition); a hand-worked two-token case; the
Sylvester matrices and the page's counterexample; an orthogonal change of
basis leaves the dense step unchanged; the page's per-device cache figures.
No function here is parity unpinned.
"""
from __future__ import annotations

import numpy as np

from .mla_oracle import decode_storage, gather_sequence, softmax


def hadamard(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix H_d (entries +-1), d a power of two."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    H = np.ones((1, 1))
    while H.shape[0] < d:
        H = np.block([[H, H], [H, -H]])
    return H


def orthonormal_hadamard(d: int, signs=None) -> np.ndarray:
    """H_d / sqrt(d), optionally times a diagonal sign matrix on the left."""
    U = hadamard(d) / np.sqrt(d)
    if signs is not None:
        U = np.asarray(signs, dtype=np.float64)[:, None] * U
    return U


def reparameterize(U, C, W_UK, W_UV):
    """Change of latent basis: cached rows c -> c U, and W -> W U for the
    up-projections ([h, rows, d_c]), so that W_UK c = (W_UK U)(c U)^T."""
    U = np.asarray(U, dtype=np.float64)
    return (np.asarray(C, np.float64) @ U, np.asarray(W_UK, np.float64) @ U,
            np.asarray(W_UV, np.float64) @ U)


def shard_slices(d_c: int, shards: int):
    """Contiguous equal slices of the latent dimension (reading T2)."""
    if d_c % shards:
        raise ValueError("d_c must divide into equal shards")
    w = d_c // shards
    return [slice(j * w, (j + 1) * w) for j in range(shards)]


def tpla_latent(q_lat, q_rope, C, R, sm_scale, shards=2, mu=None):
    """o_lat of one head: per shard j, softmax_t(sm (mu_j q_lat[S_j] . C[t, S_j]
    + q_rope . R[t])) applied to C[:, S_j]; the shard results side by side."""
    d_c = C.shape[1]
    mu = [1.0] * shards if mu is None else list(mu)
    out = np.zeros(d_c, dtype=np.float64)
    if C.shape[0] == 0:
        return out
    pos = R @ q_rope
    for j, S in enumerate(shard_slices(d_c, shards)):
        s = sm_scale * (mu[j] * (C[:, S] @ q_lat[S]) + pos)
        out[S] = softmax(s) @ C[:, S]
    return out


def tpla_decode(q, c_kv, c_kv_scale, k_rope, block_table, seq_lens, W_UK, W_UV, sm_scale,
                page_size, shards=2, mu=None, q_tag="f32", cache_tag="f32", rope_tag="f32",
                weight_tag="f32", batches=None, heads=None):
    """out[b, i, :] = sum over shards j of W_UV[i][:, S_j] o_j (Eqs. 6-7), with
    o_j from tpla_latent; same shapes as the dense oracle (NaN where not
    computed)."""
    B, h, _ = q.shape
    d_nope = W_UK.shape[1]
    d_v = W_UV.shape[1]
    Qf = decode_storage(q, q_tag)
    WK = decode_storage(W_UK, weight_tag)
    WV = decode_storage(W_UV, weight_tag)
    batches = range(B) if batches is None else batches
    heads = range(h) if heads is None else heads
    out = np.full((B, h, d_v), np.nan, dtype=np.float64)
    for b in batches:
        C, R = gather_sequence(c_kv, k_rope, c_kv_scale, block_table, seq_lens[b], b,
                               page_size, cache_tag, rope_tag)
        for i in heads:
            q_lat = WK[i].T @ Qf[b, i, :d_nope]
            o = tpla_latent(q_lat, Qf[b, i, d_nope:], C, R, float(sm_scale), shards, mu)
            out[b, i] = sum(WV[i][:, S] @ o[S] for S in shard_slices(C.shape[1], shards))
    return out


def cache_values_per_device(d_c: int, d_r: int, shards: int) -> int:
    """Values per token a device holds when it keeps one latent shard and the
    replicated rope key."""
    return d_c // shards + d_r
