// Planner, absorption, log-sum-exp merge, up-projection and cache gather.
#include "mla_kernels.hpp"

namespace mla {

// ------------------------------------------------------------------ planner
// One work group scans the batch: cu_tiles[b] = sum_{j<b} ceil(T_j / kTile).
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ seq_lens, int32_t B,
                                                     int32_t max_blocks, int32_t P,
                                                     int32_t* __restrict__ cu_tiles) {
  __shared__ int32_t buf[1024];
  __shared__ int32_t carry;
  const int tid = threadIdx.x;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int32_t base = 0; base < B; base += 1024) {
    int32_t b = base + tid;
    int32_t n = 0;
    if (b < B) n = (seq_len_clamped(seq_lens, b, max_blocks, P) + kTile - 1) / kTile;
    buf[tid] = n;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {  // inclusive Hillis-Steele scan
      int32_t v = tid >= off ? buf[tid - off] : 0;
      __syncthreads();
      buf[tid] += v;
      __syncthreads();
    }
    if (b < B) cu_tiles[b + 1] = carry + buf[tid];
    __syncthreads();
    if (tid == 1023) carry += buf[1023];
    __syncthreads();
  }
  if (tid == 0) cu_tiles[0] = 0;
}

hipError_t launch_plan(const int32_t* seq_lens, int32_t B, int32_t max_blocks, int32_t P,
                       int32_t* cu_tiles, hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, s, seq_lens, B, max_blocks, P, cu_tiles);
  return hipGetLastError();
}

// ------------------------------------------------------------------ absorb
// Work group = (head, 256 output columns); 16 sequences at a time share each
// W_UK element loaded.  fp32 accumulation.
constexpr int kAbsorbB = 16;

template <int QT, int WT, int OT>
__global__ __launch_bounds__(256) void absorb_kernel(const void* __restrict__ q,
                                                     const void* __restrict__ W_UK,
                                                     void* __restrict__ q_lat, int32_t B, int32_t h,
                                                     int32_t d_n, int32_t d_r, int32_t d_c) {
  extern __shared__ float qs[];  // [kAbsorbB][d_n]
  const int32_t head = blockIdx.x;
  const int32_t col = blockIdx.y * 256 + threadIdx.x;
  const int32_t dq = d_n + d_r, dl = d_c + d_r;
  for (int32_t b0 = 0; b0 < B; b0 += kAbsorbB) {
    const int32_t nb = min(kAbsorbB, B - b0);
    __syncthreads();
    for (int32_t i = threadIdx.x; i < nb * d_n; i += 256) {
      int32_t j = i / d_n, n = i % d_n;
      qs[i] = load_elem<QT>(q, ((int64_t)(b0 + j) * h + head) * dq + n);
    }
    __syncthreads();
    if (col < d_c) {
      float acc[kAbsorbB];
#pragma unroll
      for (int j = 0; j < kAbsorbB; j++) acc[j] = 0.f;
      const int64_t wbase = (int64_t)head * d_n * d_c + col;
      for (int32_t n = 0; n < d_n; n++) {
        float w = load_elem<WT>(W_UK, wbase + (int64_t)n * d_c);
#pragma unroll
        for (int j = 0; j < kAbsorbB; j++) acc[j] = fmaf(w, qs[j * d_n + n], acc[j]);
      }
      for (int j = 0; j < nb; j++)
        store_elem<OT>(q_lat, ((int64_t)(b0 + j) * h + head) * dl + col, acc[j]);
    } else if (col < dl) {
      for (int j = 0; j < nb; j++) {
        float v = load_elem<QT>(q, ((int64_t)(b0 + j) * h + head) * dq + d_n + (col - d_c));
        store_elem<OT>(q_lat, ((int64_t)(b0 + j) * h + head) * dl + col, v);
      }
    }
  }
}

template <int QT, int WT, int OT>
static hipError_t absorb_t(const mla_decode_params& p, const void* q, const void* W, void* ql,
                           hipStream_t s) {
  dim3 grid(p.num_heads, (p.d_latent + p.d_rope + 255) / 256);
  size_t lds = (size_t)kAbsorbB * p.d_nope * sizeof(float);
  hipLaunchKernelGGL((absorb_kernel<QT, WT, OT>), grid, dim3(256), lds, s, q, W, ql, p.batch,
                     p.num_heads, p.d_nope, p.d_rope, p.d_latent);
  return hipGetLastError();
}

hipError_t launch_absorb(const mla_decode_params& p, const void* q, const void* W_UK, void* q_lat,
                         int32_t ot, hipStream_t s) {
  const int32_t qt = p.q_dtype, wt = p.weight_dtype;
#define MLA_ABSORB(Q, W, O) \
  if (qt == Q && wt == W && ot == O) return absorb_t<Q, W, O>(p, q, W_UK, q_lat, s);
  MLA_ABSORB(MLA_F32, MLA_F32, MLA_F32)
  MLA_ABSORB(MLA_F32, MLA_F32, MLA_BF16)
  MLA_ABSORB(MLA_F32, MLA_BF16, MLA_F32)
  MLA_ABSORB(MLA_F32, MLA_BF16, MLA_BF16)
  MLA_ABSORB(MLA_BF16, MLA_F32, MLA_F32)
  MLA_ABSORB(MLA_BF16, MLA_F32, MLA_BF16)
  MLA_ABSORB(MLA_BF16, MLA_BF16, MLA_F32)
  MLA_ABSORB(MLA_BF16, MLA_BF16, MLA_BF16)
#undef MLA_ABSORB
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------------ combine
// out = sum_s w_s o_s / sum_s w_s with w_s = exp(lse_s - max lse): the exact
// merge of softmax partials taken over disjoint token ranges.
__global__ __launch_bounds__(256) void combine_kernel(AttnArgs a, float* __restrict__ o_lat) {
  const int32_t b = blockIdx.x, head = blockIdx.y;
  const int32_t d_c = a.d_c;
  float* dst = o_lat + ((int64_t)b * a.h + head) * d_c;
  const int32_t n_total = a.cu_tiles[a.B];
  const int32_t first = a.cu_tiles[b], last = a.cu_tiles[b + 1] - 1;
  if (last < first) {
    for (int32_t d = threadIdx.x; d < d_c; d += 256) dst[d] = 0.f;
    return;
  }
  const int32_t g_lo = split_owner(n_total, a.splits, first);
  const int32_t g_hi = split_owner(n_total, a.splits, last);
  // Splits in [g_lo, g_hi] that own no tile at all (possible when there are
  // more splits than tiles) wrote nothing: skip them.
  auto owns_tiles = [&](int32_t g) {
    return split_begin(n_total, a.splits, g) < split_begin(n_total, a.splits, g + 1);
  };
  float M = -INFINITY;
  for (int32_t g = g_lo; g <= g_hi; g++) {
    if (!owns_tiles(g)) continue;
    for (int32_t ts = 0; ts < a.streams; ts++)
      M = fmaxf(M, a.part_lse[((int64_t)(g + b) * a.streams + ts) * a.h + head]);
  }
  float wsum = 0.f;
  for (int32_t g = g_lo; g <= g_hi; g++) {
    if (!owns_tiles(g)) continue;
    for (int32_t ts = 0; ts < a.streams; ts++) {
      const float l = a.part_lse[((int64_t)(g + b) * a.streams + ts) * a.h + head];
      wsum += (l == -INFINITY) ? 0.f : expf(l - M);
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  for (int32_t d = threadIdx.x; d < d_c; d += 256) {
    float acc = 0.f;
    for (int32_t g = g_lo; g <= g_hi; g++) {
      if (!owns_tiles(g)) continue;
      for (int32_t ts = 0; ts < a.streams; ts++) {
        const int64_t s = (int64_t)(g + b) * a.streams + ts;
        const float l = a.part_lse[s * a.h + head];
        if (l == -INFINITY) continue;
        acc = fmaf(expf(l - M), a.part_o[(s * a.h + head) * d_c + d], acc);
      }
    }
    dst[d] = acc * inv;
  }
}

hipError_t launch_combine(const AttnArgs& a, float* o_lat, hipStream_t s) {
  hipLaunchKernelGGL(combine_kernel, dim3(a.B, a.h), dim3(256), 0, s, a, o_lat);
  return hipGetLastError();
}

// ------------------------------------------------------------------ up-projection
constexpr int kUpB = 16;

template <int WT, int OT>
__global__ __launch_bounds__(256) void up_project_kernel(const float* __restrict__ o_lat,
                                                         const void* __restrict__ W_UV,
                                                         void* __restrict__ out, int32_t B,
                                                         int32_t h, int32_t d_c, int32_t d_v) {
  extern __shared__ float os[];  // [kUpB][d_c]
  const int32_t head = blockIdx.x;
  const int32_t b0 = blockIdx.y * kUpB;
  const int32_t nb = min(kUpB, B - b0);
  for (int32_t i = threadIdx.x; i < nb * d_c; i += 256) {
    int32_t j = i / d_c, c = i % d_c;
    os[i] = o_lat[((int64_t)(b0 + j) * h + head) * d_c + c];
  }
  __syncthreads();
  for (int32_t v = threadIdx.x; v < d_v; v += 256) {
    float acc[kUpB];
#pragma unroll
    for (int j = 0; j < kUpB; j++) acc[j] = 0.f;
    const int64_t wrow = ((int64_t)head * d_v + v) * d_c;
    for (int32_t c = 0; c < d_c; c++) {
      float w = load_elem<WT>(W_UV, wrow + c);
#pragma unroll
      for (int j = 0; j < kUpB; j++) acc[j] = fmaf(w, os[j * d_c + c], acc[j]);
    }
    for (int j = 0; j < nb; j++) store_elem<OT>(out, ((int64_t)(b0 + j) * h + head) * d_v + v, acc[j]);
  }
}

template <int WT, int OT>
static hipError_t up_t(const mla_decode_params& p, const float* o, const void* W, void* out,
                       hipStream_t s) {
  dim3 grid(p.num_heads, (p.batch + kUpB - 1) / kUpB);
  size_t lds = (size_t)kUpB * p.d_latent * sizeof(float);
  hipLaunchKernelGGL((up_project_kernel<WT, OT>), grid, dim3(256), lds, s, o, W, out, p.batch,
                     p.num_heads, p.d_latent, p.d_v);
  return hipGetLastError();
}

hipError_t launch_up_project(const mla_decode_params& p, const float* o_lat, const void* W_UV,
                             void* out, hipStream_t s) {
  const int32_t wt = p.weight_dtype, ot = p.out_dtype;
  if (wt == MLA_F32 && ot == MLA_F32) return up_t<MLA_F32, MLA_F32>(p, o_lat, W_UV, out, s);
  if (wt == MLA_F32 && ot == MLA_BF16) return up_t<MLA_F32, MLA_BF16>(p, o_lat, W_UV, out, s);
  if (wt == MLA_BF16 && ot == MLA_F32) return up_t<MLA_BF16, MLA_F32>(p, o_lat, W_UV, out, s);
  if (wt == MLA_BF16 && ot == MLA_BF16) return up_t<MLA_BF16, MLA_BF16>(p, o_lat, W_UV, out, s);
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------------ gather (test aid)
__global__ __launch_bounds__(256) void gather_kernel(
    const uint8_t* __restrict__ c_kv, const float* __restrict__ c_kv_scale,
    const uint8_t* __restrict__ k_rope, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, int32_t P, int32_t max_blocks, int32_t num_blocks,
    int32_t max_tokens, int32_t c_row_bytes, int32_t r_row_bytes, uint8_t* __restrict__ c_out,
    float* __restrict__ scale_out, uint8_t* __restrict__ rope_out) {
  const int32_t b = blockIdx.x;
  const int32_t T = min(seq_len_clamped(seq_lens, b, max_blocks, P), max_tokens);
  for (int32_t t = blockIdx.y; t < max_tokens; t += gridDim.y) {
    const int64_t row = (int64_t)b * max_tokens + t;
    if (t < T) {
      const int64_t slot = phys_slot(block_table, b, t, P, max_blocks, num_blocks);
      for (int32_t i = threadIdx.x; i < c_row_bytes; i += 256)
        c_out[row * c_row_bytes + i] = c_kv[slot * c_row_bytes + i];
      for (int32_t i = threadIdx.x; i < r_row_bytes; i += 256)
        rope_out[row * r_row_bytes + i] = k_rope[slot * r_row_bytes + i];
      if (scale_out && threadIdx.x == 0) scale_out[row] = c_kv_scale[slot];
    } else {
      for (int32_t i = threadIdx.x; i < c_row_bytes; i += 256) c_out[row * c_row_bytes + i] = 0;
      for (int32_t i = threadIdx.x; i < r_row_bytes; i += 256) rope_out[row * r_row_bytes + i] = 0;
      if (scale_out && threadIdx.x == 0) scale_out[row] = 0.f;
    }
  }
}

hipError_t launch_gather(const mla_decode_params& p, const void* c_kv, const float* c_kv_scale,
                         const void* k_rope, const int32_t* block_table, const int32_t* seq_lens,
                         int32_t max_tokens, void* c_out, float* scale_out, void* rope_out,
                         hipStream_t s) {
  if (max_tokens == 0) return hipSuccess;
  dim3 grid(p.batch, min(max_tokens, 1024));
  hipLaunchKernelGGL(gather_kernel, grid, dim3(256), 0, s, (const uint8_t*)c_kv, c_kv_scale,
                     (const uint8_t*)k_rope, block_table, seq_lens, p.page_size,
                     p.max_blocks_per_seq, p.num_blocks, max_tokens,
                     p.d_latent * dtype_size(p.cache_dtype), p.d_rope * dtype_size(p.rope_dtype),
                     (uint8_t*)c_out, p.cache_dtype == MLA_FP8_E4M3 ? scale_out : nullptr,
                     (uint8_t*)rope_out);
  return hipGetLastError();
}

}  // namespace mla
