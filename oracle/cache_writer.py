"""Plain CPU oracle of the latent-cache writer: one new token per sequence
appended to the paged cache.

TEST INFRASTRUCTURE ONLY.  Imported by the tests and the benchmark's checks;
never by the HIP library, with which it shares no code.  Arithmetic is fp64
except where a reading below fixes another precision.

Sources (cited by page title and section):
  [TransMLA] "TransMLA: Multi-Head Latent Attention Is All You Need", the full
          MLA structure after conversion: the stored latent is a down
          projection of the hidden state, and the decoupled RoPE key is a
          second projection rotated to the token's position; both are cached.
          The same summary's FreqFold subsection gives the RoPE frequencies,
          theta_l = 10000^(-2(l-1)/d) for l = 1 .. d/2, the l-th frequency
          acting on the pair of dimensions (2l-1, 2l) as real and imaginary
          parts.
  [TPLA]  "TPLA: Tensor Parallel Latent Attention ...", "RMSNorm Slicing: The
          Problem and Solution" (Eqs. 8-9): RMS(x) = sqrt(mean(x^2) + eps),
          RMSNorm(gamma, x) = x / RMS(x) * gamma, applied to the KV latent.
  [LESSON] "TransMLA & Sparse Latent Attention", Chapter 3 "RoPE Breaks the
          Trick": the rotation of a 2-d pair by angle t*theta, with the
          printed scores 0.540 (t = 1) and 0.284 (t = 5) for theta = 1 rad.

Readings taken where the pages are silent:
  * the latent written to the cache is RMSNorm(gamma, W_DKV x); the rope key is
    RoPE(W_KR x, t) with t the token's 0-based position in its sequence, which
    also selects its page slot (block_table[b][t // P], offset t % P);
  * the rotation of pair i (0-based dims 2i, 2i+1) by angle a is
    (x, y) -> (x cos a - y sin a, x sin a + y cos a), a = t * base^(-2i/d);
  * an fp8 (OCP E4M3FN) latent row is quantised from its fp32 value with the
    per-row scale s = fp32(max|x| / 448) and codes RNE(clamp(fp32(x / s),
    +-448)), ties to the even code; an all-zero row has scale 0 and zero codes
    (the same rule the benchmark inputs use);
  * a position below zero, or whose page entry lies outside the table row or
    the pool, writes nothing.

Pins (tests/test_oracle_writer_pins.py, CPU only): the lesson's 0.540 / 0.284,
the FreqFold ratio of adjacent frequencies at d = 128 (about 1.15), RoPE's
identities (position 0, composition, relative position, norm), RMSNorm hand
values and identities, the E4M3FN code points of the format definition, ties
to even, and agreement with torch's own float8 cast.  No function here is
parity unpinned.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0


# --------------------------------------------------------------------------
# RMSNorm and RoPE
# --------------------------------------------------------------------------

def rmsnorm(y: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """[TPLA] Eqs. 8-9 along the last axis, in fp64."""
    y = np.asarray(y, dtype=np.float64)
    rms = np.sqrt(np.mean(y * y, axis=-1, keepdims=True) + float(eps))
    return y / rms * np.asarray(gamma, dtype=np.float64)


def rope_angles(d: int, t: float, base: float) -> np.ndarray:
    """Rotation angle of each of the d/2 pairs at position t ([TransMLA] FreqFold)."""
    i = np.arange(d // 2, dtype=np.float64)
    return float(t) * np.power(float(base), -2.0 * i / d)


def rope(v: np.ndarray, t: float, base: float) -> np.ndarray:
    """Rotate consecutive pairs (2i, 2i+1) of the last axis by rope_angles."""
    v = np.asarray(v, dtype=np.float64)
    d = v.shape[-1]
    a = rope_angles(d, t, base)
    x, y = v[..., 0::2], v[..., 1::2]
    out = np.empty_like(v)
    out[..., 0::2] = x * np.cos(a) - y * np.sin(a)
    out[..., 1::2] = x * np.sin(a) + y * np.cos(a)
    return out


# --------------------------------------------------------------------------
# OCP E4M3FN encoding
# --------------------------------------------------------------------------

def e4m3_value(code: int) -> float:
    """Value of an E4M3FN code: sign, 4-bit exponent (bias 7), 3-bit mantissa,
    subnormals at exponent 0, no infinities, S.1111.111 is NaN."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * m * 2.0 ** -9            # (m / 8) * 2^(1 - 7)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def _finite_nonneg_codes():
    codes = [c for c in range(0x80) if not math.isnan(e4m3_value(c))]
    vals = np.array([e4m3_value(c) for c in codes], dtype=np.float64)
    order = np.argsort(vals, kind="stable")
    return np.array(codes)[order], vals[order]


_POS_CODES, _POS_VALS = _finite_nonneg_codes()


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3FN code to each value (|x| <= 448), ties to the even code.

    Brute force over the 127 non-negative finite codes; fp32 inputs, the code
    values and their midpoints are all exact in fp64."""
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    for k, v in enumerate(flat):
        a = abs(v)
        if a > E4M3_MAX:
            raise ValueError("e4m3_encode expects |x| <= 448 (clamp first)")
        dist = np.abs(_POS_VALS - a)
        best = np.flatnonzero(dist == dist.min())
        if len(best) > 1:  # a tie: the code with an even mantissa bit
            best = [b for b in best if (_POS_CODES[b] & 1) == 0]
        code = int(_POS_CODES[best[0]])
        if v < 0 or (v == 0 and math.copysign(1.0, v) < 0):
            code |= 0x80
        out[k] = code
    return out.reshape(x.shape)


def quantize_row_e4m3(row_f32: np.ndarray):
    """One latent row (fp32 values) -> (codes uint8 [d], scale float32).

    The scale and the scaled values are computed in fp32 (IEEE division), the
    precision the reading fixes, so that an implementation doing the same
    arithmetic reaches the same codes."""
    r = np.asarray(row_f32, dtype=np.float32)
    amax = np.float32(np.max(np.abs(r))) if r.size else np.float32(0.0)
    scale = np.float32(amax / np.float32(E4M3_MAX))
    if scale == 0:
        return np.zeros(r.shape, dtype=np.uint8), np.float32(0.0)
    y = (r / scale).astype(np.float32)
    y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX)).astype(np.float32)
    return e4m3_encode(y), scale


# --------------------------------------------------------------------------
# the writer
# --------------------------------------------------------------------------

def page_slot(block_table: np.ndarray, b: int, t: int, page_size: int, num_blocks: int):
    """(block, offset) of token t of sequence b, or None when it has no slot."""
    if t < 0:
        return None
    j = t // page_size
    if j >= block_table.shape[1]:
        return None
    blk = int(block_table[b, j])
    if blk < 0 or blk >= num_blocks:
        return None
    return blk, t % page_size


def cache_write(x, W_DKV, gamma, W_KR, positions, block_table, page_size: int,
                num_blocks: int, eps: float, base: float):
    """The values the writer stores for each sequence's new token.

    x [B, d_model], W_DKV [d_c, d_model], gamma [d_c], W_KR [d_r, d_model] (all
    already decoded to float64).  Returns (c [B, d_c], k [B, d_r], slots) with
    slots[b] = (block, offset) or None; the projections are plain matrix
    products."""
    x = np.asarray(x, dtype=np.float64)
    c = rmsnorm(x @ np.asarray(W_DKV, dtype=np.float64).T, gamma, eps)
    r = x @ np.asarray(W_KR, dtype=np.float64).T
    k = np.stack([rope(r[b], int(positions[b]), base) for b in range(x.shape[0])])
    slots = [page_slot(block_table, b, int(positions[b]), page_size, num_blocks)
             for b in range(x.shape[0])]
    return c, k, slots
