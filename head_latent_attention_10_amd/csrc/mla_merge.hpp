// The log-sum-exp merge of bf16 split partials, one (sequence, head) row per
// wave (gfx950).  The merge kernel and the merge + up-projection kernel both
// call merge_row, so the decode step and its stages give the same bits.
//
// "TPLA: Tensor Parallel Latent Attention ...", Section 3.4 ("MLA Matrix
// Absorption", Eq. 5): the attention output of a head is the softmax-weighted
// sum of the latent rows.  Split over disjoint token ranges, split s holds
// o_s = sum_t p_t c_t / sum_t p_t and lse_s = m_s + ln sum_t exp(s_t - m_s);
// the whole sum is  o = sum_s e^(lse_s - M) o_s / sum_s e^(lse_s - M)  with
// M = max_s lse_s, exactly (up to rounding).
#pragma once

#include "mla_kernels.hpp"

namespace mla {

typedef unsigned merge_u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMergeLat = 512;   // latent values of a bf16 partial row
constexpr int kMergeGroup = 8;   // partial rows a lane loads at a time (two groups in flight)

// Wave-wide reductions as xor butterflies: each step adds a lane's value and
// its partner's in either order, which gives the same bits, so every lane
// ends with the same result.
__device__ inline float merge_wave_max(float v) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}
__device__ inline float merge_wave_sum(float v) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) v += __shfl_xor(v, m);
  return v;
}
__device__ inline float merge_readlane(float v, int32_t k) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), k));
}

// One wave merges row (sequence b, output head i) of the bf16 partials
// (row-major [slot][h][512], slot g + b for split g): lane l returns latent
// values 8 l .. 8 l + 7 in o.  With G > 1 TPLA shards the partials are those
// of G h_out shard heads (shard-major: shard head j h_out + i), and the lane's
// columns lie in shard j = l / (64 / G), each shard with its own weights.  The
// sequence's splits are seq_splits[b]; a split that owns no tiles wrote
// nothing and weighs 0 (its row is never multiplied in).  A sequence without
// tokens gets zeros.  The sums run in slot order, so the result depends only
// on the inputs.  The code is kept small (rolled loops): a launch runs it
// once per wave, with a cold instruction cache.
template <int G>
__device__ __forceinline__ void merge_row(const AttnArgs& a, int32_t b, int32_t i,
                                         int lane, float o[8]) {
  static_assert(G == 1 || G == 2 || G == 4, "1, 2 or 4 shards");
#pragma unroll
  for (int e = 0; e < 8; e++) o[e] = 0.f;
  const int32_t g_lo = load_ro(a.seq_splits, 2 * b);
  const int32_t n = load_ro(a.seq_splits, 2 * b + 1) - g_lo + 1;
  if (n <= 0) return;
  const int32_t h_out = a.h / G;
  const int j_lane = lane / (64 / G);
  const int64_t slot0 = (int64_t)g_lo + b;
  const int64_t row_stride = (int64_t)a.h * kMergeLat;
  const uint16_t* rows = static_cast<const uint16_t*>(a.part_o) + slot0 * row_stride +
                         (int64_t)(j_lane * h_out + i) * kMergeLat + 8 * lane;
  // log-sum-exp of slot k for shard j, -inf past the range or without tiles
  auto lse_of = [&](int32_t k, int j) -> float {
    const int32_t kk = min(k, n - 1);
    const bool owns = load_ro(a.split_first, g_lo + kk) < load_ro(a.split_first, g_lo + kk + 1);
    const float l = a.part_lse[(slot0 + kk) * a.h + j * h_out + i];
    return (k < n && owns) ? l : -INFINITY;
  };
  auto weight = [](float l, float M) -> float { return l == -INFINITY ? 0.f : expf(l - M); };
  // a group of partial rows from slot k0 on; rows past the range are not read
  auto load_group = [&](merge_u32x4* x, int32_t k0) {
#pragma unroll
    for (int u = 0; u < kMergeGroup; u++)
      x[u] = k0 + u < n ? *reinterpret_cast<const merge_u32x4*>(rows + (int64_t)(k0 + u) * row_stride)
                        : merge_u32x4{0u, 0u, 0u, 0u};
  };
  // the first 64 log-sum-exps (lane k: slot k) and the first group, in flight together
  float lc[G];
#pragma unroll
  for (int j = 0; j < G; j++) lc[j] = lse_of(lane, j);
  merge_u32x4 xa[kMergeGroup], xb[kMergeGroup];
  load_group(xa, 0);
  float M[G], W[G], wl[G];
#pragma unroll
  for (int j = 0; j < G; j++) M[j] = merge_wave_max(lc[j]);
#pragma unroll 1
  for (int32_t c0 = 64; c0 < n; c0 += 64)
#pragma unroll
    for (int j = 0; j < G; j++) M[j] = fmaxf(M[j], merge_wave_max(lse_of(c0 + lane, j)));
#pragma unroll
  for (int j = 0; j < G; j++) {
    wl[j] = weight(lc[j], M[j]);
    W[j] = merge_wave_sum(wl[j]);
  }
#pragma unroll 1
  for (int32_t c0 = 64; c0 < n; c0 += 64)
#pragma unroll
    for (int j = 0; j < G; j++) W[j] += merge_wave_sum(weight(lse_of(c0 + lane, j), M[j]));
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
  for (int32_t k0 = 0; k0 < n; k0 += kMergeGroup) {
    if (k0 + kMergeGroup < n) load_group(xb, k0 + kMergeGroup);  // the next group, in flight
    if (k0 > 0 && (k0 & 63) == 0) {
#pragma unroll
      for (int j = 0; j < G; j++) wl[j] = weight(lse_of(k0 + lane, j), M[j]);
    }
#pragma unroll
    for (int u = 0; u < kMergeGroup; u++) {
      const int32_t k = k0 + u;
      if (k >= n) break;  // wave-uniform
      float w = merge_readlane(wl[0], k & 63);
#pragma unroll
      for (int j = 1; j < G; j++) {
        const float wj = merge_readlane(wl[j], k & 63);
        w = j_lane == j ? wj : w;
      }
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const uint32_t xq = xa[u][q];
        const float lo = __uint_as_float(xq << 16), hi = __uint_as_float(xq & 0xffff0000u);
        acc[2 * q] = w != 0.f ? fmaf(w, lo, acc[2 * q]) : acc[2 * q];
        acc[2 * q + 1] = w != 0.f ? fmaf(w, hi, acc[2 * q + 1]) : acc[2 * q + 1];
      }
    }
#pragma unroll
    for (int u = 0; u < kMergeGroup; u++) xa[u] = xb[u];
  }
  float Wl = W[0];
#pragma unroll
  for (int j = 1; j < G; j++) Wl = j_lane == j ? W[j] : Wl;
  const float inv = Wl > 0.f ? 1.f / Wl : 0.f;
  {
    // a plain product: fused into a caller's next operation it would round
    // differently in the two kernels
#pragma clang fp contract(off)
#pragma unroll
    for (int e = 0; e < 8; e++) o[e] = acc[e] * inv;
  }
}

}  // namespace mla
