"""Plain fp64 CPU oracle of one MLA decode step over a paged latent cache.

TEST INFRASTRUCTURE ONLY.  Imported by the tests, the smoke check and the
benchmark's CPU-baseline leg; never by the HIP library, with which it shares no
code.  It is slow on purpose: it decompresses per-head keys and values
explicitly and runs textbook softmax attention, exactly as the pages write the
unabsorbed computation.

Sources (cited by page title and section):
  [TPLA]  "TPLA: Tensor Parallel Latent Attention for Efficient Disaggregated
          Prefill and Decode Inference", section 3.4, subsections "MLA Matrix
          Absorption" (unabsorbed form, Eq. 4; key absorption, Eq. 5) and
          "The RoPE handling" (decoupled positional score, one softmax scale
          1/sqrt(d_h + d_r)).
  [LESSON] "TransMLA & Sparse Latent Attention", Chapter 1 "GQA, Precisely"
          (grouped attention, head-to-group map) and Chapter 2 "GQA Is MLA in
          Disguise" (identity-selector up-projections).
  [TransMLA] "TransMLA: Multi-Head Latent Attention Is All You Need", the MLA
          equations with a decoupled RoPE key shared by all heads.

Readings taken where the pages are silent or inconsistent:
  * indices are 0-based; head i belongs to group i // (h / g);
  * the rope halves of q and of the cached key arrive already rotated;
  * the cache holds every token the new query attends to (no causal mask);
  * a sequence with no cached token produces a zero output;
  * fp8 latent rows decode as OCP E4M3FN value times the row's fp32 scale.

Pins (tests/test_oracle_pins.py, CPU only): the lesson's hand-worked GQA toy
and selector examples, the GQA == MLA-with-selectors identity, absorbed ==
explicit, closed forms (one token, zero query, dominant token, score shift),
the lesson's RoPE score values, a long-double brute force on tiny shapes, and
the storage decoders against torch's own casts.  No function here is parity
unpinned.
"""
from __future__ import annotations

import numpy as np


# --------------------------------------------------------------------------
# storage decoders
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64: the 16 bits are the top half of an fp32."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def _e4m3_table() -> np.ndarray:
    """All 256 OCP E4M3FN codes -> float64 (bias 7, subnormals, S.1111.111 = NaN)."""
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp = (code >> 3) & 0xF
        man = code & 0x7
        if exp == 0xF and man == 0x7:
            out[code] = np.nan
        elif exp == 0:
            out[code] = sign * (man / 8.0) * 2.0 ** (1 - 7)
        else:
            out[code] = sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return out


_E4M3 = _e4m3_table()


def e4m3_code_to_f64(codes: np.ndarray) -> np.ndarray:
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def decode_storage(raw: np.ndarray, tag: str) -> np.ndarray:
    if tag == "f64":   # values already in fp64 (oracle-side transforms)
        return np.asarray(raw, dtype=np.float64)
    if tag == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if tag == "bf16":
        return bf16_bits_to_f64(raw)
    if tag == "e4m3":
        return e4m3_code_to_f64(raw)
    raise ValueError(f"unknown storage tag {tag!r}")


# --------------------------------------------------------------------------
# paged cache walk
# --------------------------------------------------------------------------

def gather_sequence(c_kv, k_rope, c_kv_scale, block_table, seq_len, b, page_size,
                    cache_tag, rope_tag):
    """Logical token t of sequence b lives in block block_table[b][t // P] at
    slot t % P.  Returns the decoded latent rows C [T, d_c] and rope keys
    R [T, d_r] in fp64 (fp8 rows multiplied by their per-token scale)."""
    T = int(seq_len)
    d_c = c_kv.shape[-1]
    d_r = k_rope.shape[-1]
    C = np.empty((T, d_c), dtype=np.float64)
    R = np.empty((T, d_r), dtype=np.float64)
    for t in range(0, T, page_size):
        blk = int(block_table[b][t // page_size])
        n = min(page_size, T - t)
        C[t: t + n] = decode_storage(c_kv[blk, :n], cache_tag)
        if cache_tag == "e4m3":
            C[t: t + n] *= np.asarray(c_kv_scale[blk, :n], dtype=np.float64)[:, None]
        R[t: t + n] = decode_storage(k_rope[blk, :n], rope_tag)
    return C, R


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def softmax(s: np.ndarray) -> np.ndarray:
    """Max-subtracted softmax over the last axis."""
    s = np.asarray(s, dtype=np.float64)
    e = np.exp(s - np.max(s, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def _head_explicit(q_nope, q_rope, C, R, W_UK_i, W_UV_i, sm_scale):
    """[TPLA] 3.4, unabsorbed form: k = c W_UK, v = c W_UV per head, score
    (q k^T + q_pe k_pe^T) / sqrt(d_h + d_r), softmax over cached tokens,
    output = p v.  Here W_UK_i is [d_nope, d_c] so k_t = W_UK_i c_t."""
    if C.shape[0] == 0:
        return np.zeros(W_UV_i.shape[0], dtype=np.float64)
    K = C @ W_UK_i.T            # [T, d_nope]  explicit key decompression
    V = C @ W_UV_i.T            # [T, d_v]     explicit value decompression
    s = sm_scale * (K @ q_nope + R @ q_rope)
    p = softmax(s)
    return p @ V


def _head_absorbed(q_nope, q_rope, C, R, W_UK_i, W_UV_i, sm_scale):
    """[TPLA] 3.4, key absorption (Eq. 5): the absorbed query W_UK^T q_nope is
    scored directly against the latent rows; the latent-space output p C is
    then up-projected by W_UV.  Used only to pin the explicit form."""
    if C.shape[0] == 0:
        return np.zeros(W_UV_i.shape[0], dtype=np.float64)
    q_lat = W_UK_i.T @ q_nope   # [d_c]
    s = sm_scale * (C @ q_lat + R @ q_rope)
    p = softmax(s)
    o_lat = p @ C               # [d_c]
    return W_UV_i @ o_lat


def _decode(head_fn, q, c_kv, c_kv_scale, k_rope, block_table, seq_lens, W_UK, W_UV,
            sm_scale, page_size, q_tag, cache_tag, rope_tag, weight_tag,
            batches=None, heads=None):
    B, h, dq = q.shape
    d_nope = W_UK.shape[1]
    d_v = W_UV.shape[1]
    if dq != d_nope + k_rope.shape[-1]:
        raise ValueError("q width must be d_nope + d_rope")
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
            out[b, i] = head_fn(Qf[b, i, :d_nope], Qf[b, i, d_nope:], C, R, WK[i], WV[i],
                                float(sm_scale))
    return out


def mla_decode_explicit(q, c_kv, c_kv_scale, k_rope, block_table, seq_lens, W_UK, W_UV,
                        sm_scale, page_size, q_tag="f32", cache_tag="f32", rope_tag="f32",
                        weight_tag="f32", batches=None, heads=None):
    """out[b, i, :] for every (or the selected) sequence b and head i, in fp64.
    Shapes: q [B,h,d_nope+d_rope]; c_kv [num_blocks,P,d_c]; k_rope
    [num_blocks,P,d_r]; c_kv_scale [num_blocks,P] or None; block_table
    [B,max_blocks]; seq_lens [B]; W_UK [h,d_nope,d_c]; W_UV [h,d_v,d_c].
    Entries not computed (outside ``batches``/``heads``) are NaN."""
    return _decode(_head_explicit, q, c_kv, c_kv_scale, k_rope, block_table, seq_lens,
                   W_UK, W_UV, sm_scale, page_size, q_tag, cache_tag, rope_tag,
                   weight_tag, batches, heads)


def mla_decode_absorbed(q, c_kv, c_kv_scale, k_rope, block_table, seq_lens, W_UK, W_UV,
                        sm_scale, page_size, q_tag="f32", cache_tag="f32", rope_tag="f32",
                        weight_tag="f32", batches=None, heads=None):
    """Same result through the absorbed form; pins the explicit form only."""
    return _decode(_head_absorbed, q, c_kv, c_kv_scale, k_rope, block_table, seq_lens,
                   W_UK, W_UV, sm_scale, page_size, q_tag, cache_tag, rope_tag,
                   weight_tag, batches, heads)


def oracle_from_inputs(inp, batches=None, heads=None, absorbed=False):
    """Convenience wrapper taking any object with the generator's fields."""
    cfg = inp.cfg
    fn = mla_decode_absorbed if absorbed else mla_decode_explicit
    return fn(inp.q, inp.c_kv, inp.c_kv_scale, inp.k_rope, inp.block_table, inp.seq_lens,
              inp.W_UK, inp.W_UV, cfg.sm_scale, cfg.page_size, q_tag=cfg.q_dtype,
              cache_tag=cfg.cache_dtype, rope_tag=cfg.rope_dtype,
              weight_tag=cfg.weight_dtype, batches=batches, heads=heads)


# --------------------------------------------------------------------------
# grouped-query attention and the identity selectors
# --------------------------------------------------------------------------

def gqa_decode(q, K, V, sm_scale):
    """[LESSON] Chapter 1: h query heads in g groups; head i reads the key and
    value of group i // (h / g).  q [h, d], K [T, g, d], V [T, g, d] -> [h, d]."""
    h = q.shape[0]
    g = K.shape[1]
    if h % g:
        raise ValueError("h must be a multiple of g")
    out = np.empty((h, V.shape[2]), dtype=np.float64)
    for i in range(h):
        j = i // (h // g)
        s = sm_scale * (K[:, j, :] @ q[i])
        out[i] = softmax(s) @ V[:, j, :]
    return out


def build_selectors(h, g, d):
    """[LESSON] Chapter 2 "GQA Is MLA in Disguise": the latent row is the
    concatenation of every group's key and then every group's value (width
    2gd); head i's key up-projection picks its own group's key block out of it
    and its value up-projection its group's value block.

    Written as a Kronecker product: with e_j the one-hot row of length g for
    the head's group j = i // (h/g), the key selector is [e_j, 0] (x) I_d and
    the value selector [0, e_j] (x) I_d, each d x 2gd."""
    if h % g:
        raise ValueError("h must be a multiple of g")
    group_of_head = np.arange(h) // (h // g)
    onehot = np.eye(g)[group_of_head]                  # [h, g]
    zeros = np.zeros_like(onehot)
    key_pick = np.concatenate([onehot, zeros], axis=1)  # [h, 2g]
    val_pick = np.concatenate([zeros, onehot], axis=1)
    eye = np.eye(d)
    W_UK = np.stack([np.kron(key_pick[i][None, :], eye) for i in range(h)])
    W_UV = np.stack([np.kron(val_pick[i][None, :], eye) for i in range(h)])
    return W_UK, W_UV
