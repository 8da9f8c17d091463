// Generic split attention in the latent space: any latent/rope width, any
// storage type.  Work group = (token split g, head); it walks the tiles of its
// split, keeps an online-softmax state per sequence segment and writes one
// normalised partial plus its log-sum-exp per segment.  This is the exact-fp32
// path (fp32 caches) and the fallback for shapes the matrix-core kernel does
// not cover.
#include "mla_kernels.hpp"

namespace mla {

constexpr int kSimtMaxDc = 1024;               // latent values per thread: 4
constexpr int kSimtPerThread = kSimtMaxDc / 256;

template <int CT, int RT, int QT>
__global__ __launch_bounds__(256) void attend_simt_kernel(AttnArgs a) {
  extern __shared__ float smem[];
  float* qs = smem;                      // [d_c + d_r] absorbed query of this head
  float* ps = smem + a.d_c + a.d_r;      // [kTile] scores, then weights
  __shared__ float red[8];
  __shared__ float bcast;

  const int32_t g = blockIdx.x, head = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  select_latent_group(a, head);
  const int32_t n_total = a.cu_tiles[a.B];
  if (n_total == 0) return;
  const int64_t t_begin = load_ro(a.split_first, g);
  const int64_t t_end = load_ro(a.split_first, g + 1);
  if (t_begin >= t_end) return;
  const int32_t d_c = a.d_c, d_r = a.d_r, dl = d_c + d_r;
  const float sm = a.sm_scale_log2 * 0.69314718055994530942f;  // back to natural units

  int32_t b = 0;
  while (a.cu_tiles[b + 1] <= t_begin) b++;

  float o[kSimtPerThread];
  float m = -INFINITY, l = 0.f;
  bool fresh = true;

  for (int64_t tile = t_begin; tile < t_end; tile++) {
    while (a.cu_tiles[b + 1] <= tile) b++;
    if (fresh) {
      __syncthreads();
      for (int32_t i = tid; i < dl; i += 256)
        qs[i] = load_elem<QT>(a.q_lat, ((int64_t)b * a.h + head) * dl + i);
#pragma unroll
      for (int k = 0; k < kSimtPerThread; k++) o[k] = 0.f;
      m = -INFINITY;
      l = 0.f;
      fresh = false;
      __syncthreads();
    }
    const int32_t T = attn_len(a, b);
    const int32_t t0 = (int32_t)(tile - a.cu_tiles[b]) * kTile;
    const int32_t nvalid = min(kTile, T - t0);

    // scores: 4 threads per token
    {
      const int32_t tt = tid >> 2, part = tid & 3;
      float s = 0.f;
      if (tt < nvalid) {
        const int64_t slot = entry_slot(a, b, t0 + tt);
        float cs = 1.f;
        if (CT == MLA_FP8_E4M3) cs = a.c_kv_scale[slot];
        float sc = 0.f, sr = 0.f;
        for (int32_t d = part; d < d_c; d += 4) sc = fmaf(qs[d], load_elem<CT>(a.c_kv, slot * d_c + d), sc);
        for (int32_t d = part; d < d_r; d += 4) sr = fmaf(qs[d_c + d], load_elem<RT>(a.k_rope, slot * d_r + d), sr);
        s = sc * cs + sr;
      }
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      if (part == 0) ps[tt] = (tt < nvalid) ? s * sm : -INFINITY;
    }
    __syncthreads();
    // tile max and weights
    static_assert(kTile <= 64, "one wave reduces a tile");
    if (wave == 0) {
      float v = lane < kTile ? ps[lane] : -INFINITY;
      for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
      if (lane == 0) bcast = v;
    }
    __syncthreads();
    const float m_new = fmaxf(m, bcast);
    const float alpha = (m == -INFINITY) ? 0.f : expf(m - m_new);
    __syncthreads();
    if (tid < kTile) ps[tid] = (tid < nvalid) ? expf(ps[tid] - m_new) : 0.f;
    __syncthreads();
    if (wave == 0) {
      float v = lane < kTile ? ps[lane] : 0.f;
      for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
      if (lane == 0) red[0] = v;
    }
    __syncthreads();
    l = l * alpha + red[0];
    m = m_new;
    // o = o * alpha + sum_t p_t c_t
#pragma unroll
    for (int k = 0; k < kSimtPerThread; k++) {
      const int32_t d = tid + 256 * k;
      if (d < d_c) {
        float acc = o[k] * alpha;
        for (int32_t tt = 0; tt < nvalid; tt++) {
          const int64_t slot = entry_slot(a, b, t0 + tt);
          float c = load_elem<CT>(a.c_kv, slot * d_c + d);
          if (CT == MLA_FP8_E4M3) c *= a.c_kv_scale[slot];
          acc = fmaf(ps[tt], c, acc);
        }
        o[k] = acc;
      }
    }
    // segment end: write the normalised partial and its log-sum-exp
    const bool last_of_seq = (tile + 1 == t_end) || (a.cu_tiles[b + 1] <= tile + 1);
    if (last_of_seq) {
      const int64_t slot = (int64_t)(g + b) * a.streams;
      const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
      for (int k = 0; k < kSimtPerThread; k++) {
        const int32_t d = tid + 256 * k;
        if (d >= d_c) continue;
        // the matrix-core shapes keep their partials bf16 (what the merge
        // reads for them), whichever kernel wrote them
        if (a.part_bf16) {
          static_cast<uint16_t*>(a.part_o)[slot * a.h * d_c + (int64_t)head * d_c + d] =
              f32_to_bf16_bits(o[k] * inv);
        } else {
          static_cast<float*>(a.part_o)[slot * a.h * d_c + (int64_t)head * d_c + d] = o[k] * inv;
        }
      }
      if (tid == 0) a.part_lse[slot * a.h + head] = l > 0.f ? m + logf(l) : -INFINITY;
      fresh = true;
    }
    __syncthreads();
  }
}

template <int CT, int RT, int QT>
static hipError_t simt_t(const AttnArgs& a, hipStream_t s) {
  dim3 grid(a.splits, a.h);
  size_t lds = (size_t)(a.d_c + a.d_r + kTile) * sizeof(float);
  hipLaunchKernelGGL((attend_simt_kernel<CT, RT, QT>), grid, dim3(256), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_attend_simt(const AttnArgs& a, int32_t ct, int32_t rt, int32_t qt,
                              hipStream_t s) {
  if (a.d_c > kSimtMaxDc) return hipErrorInvalidValue;
#define MLA_SIMT(C, R, Q) \
  if (ct == C && rt == R && qt == Q) return simt_t<C, R, Q>(a, s);
  MLA_SIMT(MLA_F32, MLA_F32, MLA_F32)
  MLA_SIMT(MLA_F32, MLA_BF16, MLA_F32)
  MLA_SIMT(MLA_BF16, MLA_F32, MLA_BF16)
  MLA_SIMT(MLA_BF16, MLA_BF16, MLA_BF16)
  MLA_SIMT(MLA_FP8_E4M3, MLA_F32, MLA_BF16)
  MLA_SIMT(MLA_FP8_E4M3, MLA_BF16, MLA_BF16)
#undef MLA_SIMT
  return hipErrorInvalidValue;
}

}  // namespace mla
