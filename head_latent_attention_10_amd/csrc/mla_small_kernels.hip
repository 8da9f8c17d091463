// Planner, absorption, log-sum-exp merge, up-projection and cache gather.
#include "mla_kernels.hpp"
#include "mla_merge.hpp"

namespace mla {

// ------------------------------------------------------------------ planner
// kPlanGroups work groups running plan_block.
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanInput in) {
  __shared__ PlanShared sh;
  plan_block(in, blockIdx.x, gridDim.x, sh);
}

hipError_t launch_plan(const PlanInput& in, hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, dim3(kPlanGroups), dim3(kPlanThreads), 0, s, in);
  return hipGetLastError();
}

// ------------------------------------------------------------------ absorb
// Work group = (head, 256 output columns); thread = 4 adjacent columns for a
// quarter of the sequences.  Per row n of W_UK the 4 weights are one 8-byte
// (bf16) or 16-byte (fp32) load, reused for up to 16 sequences whose q_nope
// sits in LDS; loads of 8 rows are issued before they are used.  fp32
// accumulation; the rope part of the row is copied.
constexpr int kAbsCols = 256;
constexpr int kAbsSeq = 64;        // sequences staged in LDS at a time
constexpr int kAbsPerThread = 16;  // sequences per thread (kAbsSeq / 4 waves)
constexpr int kAbsRows = 8;        // W rows loaded ahead

template <int WT>
__device__ inline void load4(const void* W, int64_t idx, float* w);
template <>
__device__ inline void load4<MLA_F32>(const void* W, int64_t idx, float* w) {
  const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(W) + idx);
  w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
}
template <>
__device__ inline void load4<MLA_BF16>(const void* W, int64_t idx, float* w) {
  const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(W) + idx);
  w[0] = __uint_as_float(u.x << 16);
  w[1] = __uint_as_float(u.x & 0xffff0000u);
  w[2] = __uint_as_float(u.y << 16);
  w[3] = __uint_as_float(u.y & 0xffff0000u);
}

template <int QT, int WT, int OT>
__global__ __launch_bounds__(256) void absorb_kernel(const void* __restrict__ q,
                                                     const void* __restrict__ W_UK,
                                                     void* __restrict__ q_lat, int32_t B, int32_t h,
                                                     int32_t d_n, int32_t d_r, int32_t d_c) {
  extern __shared__ float qs[];  // [kAbsSeq][d_n]
  const int32_t head = blockIdx.x;
  const int32_t dq = d_n + d_r, dl = d_c + d_r;
  const int cq = threadIdx.x & 63, ph = threadIdx.x >> 6;
  const int32_t col = blockIdx.y * kAbsCols + 4 * cq;
  // vector loads need 4 whole columns inside the latent part and an aligned base
  const bool vec = col + 3 < d_c && (d_c & 3) == 0 &&
                   (reinterpret_cast<uintptr_t>(W_UK) & (WT == MLA_F32 ? 15 : 7)) == 0;
  const int64_t wbase = (int64_t)head * d_n * d_c + col;
  for (int32_t b0 = 0; b0 < B; b0 += kAbsSeq) {
    const int32_t nb = min(kAbsSeq, B - b0);
    __syncthreads();
    for (int32_t i = threadIdx.x; i < nb * d_n; i += 256) {
      const int32_t j = i / d_n, n = i % d_n;
      qs[i] = load_elem<QT>(q, ((int64_t)(b0 + j) * h + head) * dq + n);
    }
    __syncthreads();
    // sequences of this thread: b0 + ph + 4k, k < mine
    const int32_t mine = nb > ph ? (nb - ph + 3) / 4 : 0;
    if (col < d_c && mine > 0) {
      float acc[kAbsPerThread][4];
#pragma unroll
      for (int k = 0; k < kAbsPerThread; k++)
#pragma unroll
        for (int c = 0; c < 4; c++) acc[k][c] = 0.f;
      for (int32_t n0 = 0; n0 < d_n; n0 += kAbsRows) {
        float w[kAbsRows][4];
#pragma unroll
        for (int r = 0; r < kAbsRows; r++) {
          const int32_t n = n0 + r;
          if (n < d_n) {
            if (vec) {
              load4<WT>(W_UK, wbase + (int64_t)n * d_c, w[r]);
            } else {
#pragma unroll
              for (int c = 0; c < 4; c++)
                w[r][c] = col + c < d_c ? load_elem<WT>(W_UK, wbase + (int64_t)n * d_c + c) : 0.f;
            }
          } else {
#pragma unroll
            for (int c = 0; c < 4; c++) w[r][c] = 0.f;
          }
        }
#pragma unroll
        for (int k = 0; k < kAbsPerThread; k++) {
          // rows past d_n carry zero weights; sequences past `mine` read a valid row
          const float* qrow = qs + (ph + 4 * (k < mine ? k : 0)) * d_n + n0;
#pragma unroll
          for (int r = 0; r < kAbsRows; r++) {
            const float qv = n0 + r < d_n ? qrow[r] : 0.f;
#pragma unroll
            for (int c = 0; c < 4; c++) acc[k][c] = fmaf(w[r][c], qv, acc[k][c]);
          }
        }
      }
#pragma unroll
      for (int k = 0; k < kAbsPerThread; k++) {
        if (k < mine) {
          const int32_t b = b0 + ph + 4 * k;
#pragma unroll
          for (int c = 0; c < 4; c++)
            if (col + c < d_c) store_elem<OT>(q_lat, ((int64_t)b * h + head) * dl + col + c, acc[k][c]);
        }
      }
    }
    // rope part: copy
    for (int k = 0; k < 4; k++) {
      const int32_t cc = col + k;
      if (cc < d_c || cc >= dl) continue;
      for (int32_t j = ph; j < nb; j += 4) {
        const int32_t b = b0 + j;
        const float v = load_elem<QT>(q, ((int64_t)b * h + head) * dq + d_n + (cc - d_c));
        store_elem<OT>(q_lat, ((int64_t)b * h + head) * dl + cc, v);
      }
    }
  }
}

template <int QT, int WT, int OT>
static hipError_t absorb_t(const mla_decode_params& p, const void* q, const void* W, void* ql,
                           hipStream_t s) {
  dim3 grid(p.num_heads, (p.d_latent + p.d_rope + kAbsCols - 1) / kAbsCols);
  size_t lds = (size_t)kAbsSeq * p.d_nope * sizeof(float);
  hipLaunchKernelGGL((absorb_kernel<QT, WT, OT>), grid, dim3(256), lds, s, q, W, ql, p.batch,
                     p.num_heads, p.d_nope, p.d_rope, p.d_latent);
  return hipGetLastError();
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

bool absorb_mfma_ok(const mla_decode_params& p, const void* q, const void* W_UK, const void* q_lat) {
  return proj_mfma_supported(p) && aligned16(q) && aligned16(W_UK) && aligned16(q_lat) &&
         (p.d_nope + p.d_rope) % 8 == 0;
}

hipError_t launch_absorb(const mla_decode_params& p, const void* q, const void* W_UK, void* q_lat,
                         int32_t ot, const PlanRequest* plan, bool* planned, hipStream_t s) {
  if (planned) *planned = false;
  if (absorb_mfma_ok(p, q, W_UK, q_lat)) {
    if (planned) *planned = plan != nullptr;
    return launch_absorb_mfma(p, q, W_UK, q_lat, ot, plan, s);
  }
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
// merge of softmax partials taken over disjoint token ranges.  Work group =
// (sequence, head); the split weights are computed once per chunk of 256
// slots into LDS, then each thread merges 4 adjacent latent values.
constexpr int kCombThreads = 128;
constexpr int kCombChunk = 256;

__global__ __launch_bounds__(kCombThreads) void combine_kernel(AttnArgs a, float* __restrict__ o_lat) {
  __shared__ float s_w[kCombChunk];
  __shared__ int64_t s_slot[kCombChunk];
  __shared__ float s_red[kCombThreads / 64];
  const int32_t b = blockIdx.x, head = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int32_t d_c = a.d_c;
  float* dst = o_lat + ((int64_t)b * a.h + head) * d_c;
  const int32_t first = a.cu_tiles[b], last = a.cu_tiles[b + 1] - 1;
  if (last < first) {
    for (int32_t d = tid; d < d_c; d += kCombThreads) dst[d] = 0.f;
    return;
  }
  const int32_t g_lo = a.seq_splits[2 * b];
  const int32_t g_hi = a.seq_splits[2 * b + 1];
  const int32_t n_cand = (g_hi - g_lo + 1) * a.streams;
  // candidate slot k -> (split, stream); splits that own no tile wrote nothing
  auto cand_lse = [&](int32_t k, int64_t* slot_out) -> float {
    const int32_t gg = g_lo + k / a.streams, ts = k % a.streams;
    const bool owns = a.split_first[gg] < a.split_first[gg + 1];
    const int64_t slot = (int64_t)(gg + b) * a.streams + ts;
    *slot_out = slot;
    return owns ? a.part_lse[slot * a.h + head] : -INFINITY;
  };
  auto block_reduce = [&](float v, bool is_max) -> float {
    for (int off = 32; off > 0; off >>= 1) {
      const float o = __shfl_xor(v, off);
      v = is_max ? fmaxf(v, o) : v + o;
    }
    if (lane == 0) s_red[wv] = v;
    __syncthreads();
    float r = s_red[0];
    for (int i = 1; i < kCombThreads / 64; i++) r = is_max ? fmaxf(r, s_red[i]) : r + s_red[i];
    __syncthreads();
    return r;
  };
  float m = -INFINITY;
  for (int32_t k = tid; k < n_cand; k += kCombThreads) {
    int64_t sl;
    m = fmaxf(m, cand_lse(k, &sl));
  }
  const float M = block_reduce(m, true);
  float ws = 0.f;
  for (int32_t k = tid; k < n_cand; k += kCombThreads) {
    int64_t sl;
    const float l = cand_lse(k, &sl);
    ws += l == -INFINITY ? 0.f : expf(l - M);
  }
  const float W = block_reduce(ws, false);
  const float inv = W > 0.f ? 1.f / W : 0.f;
  for (int32_t d0 = 0; d0 < d_c; d0 += 4 * kCombThreads) {
    const int32_t d = d0 + 4 * tid;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int32_t k0 = 0; k0 < n_cand; k0 += kCombChunk) {
      const int32_t n = min(kCombChunk, n_cand - k0);
      __syncthreads();
      for (int32_t k = tid; k < n; k += kCombThreads) {
        int64_t sl;
        const float l = cand_lse(k0 + k, &sl);
        s_w[k] = l == -INFINITY ? 0.f : expf(l - M) * inv;
        s_slot[k] = sl;
      }
      __syncthreads();
      if (d < d_c) {
        const bool v4 = d + 3 < d_c && (d_c & 3) == 0;
        for (int32_t k0b = 0; k0b < n; k0b += 8) {
          float4 v[8];
#pragma unroll
          for (int u = 0; u < 8; u++) {  // issue the loads of 8 splits first
            const int32_t k = k0b + u;
            v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (k < n && s_w[k] != 0.f) {
              const float* src = static_cast<const float*>(a.part_o) + (s_slot[k] * a.h + head) * d_c + d;
              if (v4) {
                v[u] = *reinterpret_cast<const float4*>(src);
              } else {
                v[u].x = src[0];
                if (d + 1 < d_c) v[u].y = src[1];
                if (d + 2 < d_c) v[u].z = src[2];
                if (d + 3 < d_c) v[u].w = src[3];
              }
            }
          }
#pragma unroll
          for (int u = 0; u < 8; u++) {
            const int32_t k = k0b + u;
            const float w = k < n ? s_w[k] : 0.f;
            acc[0] = fmaf(w, v[u].x, acc[0]);
            acc[1] = fmaf(w, v[u].y, acc[1]);
            acc[2] = fmaf(w, v[u].z, acc[2]);
            acc[3] = fmaf(w, v[u].w, acc[3]);
          }
        }
      }
    }
    for (int i = 0; i < 4; i++)
      if (d + i < d_c) dst[d + i] = acc[i];
  }
}

// The same merge over bf16 partial rows (512 latent values): one wave per
// (sequence, output head) row, merge_row; each lane writes its 8 values.
// With TPLA shards (a.shards = G > 1) output head i takes the columns of
// shard j from shard head j (h / G) + i, into an output of h / G heads.
template <int G>
__global__ __launch_bounds__(256) void merge_kernel(AttnArgs a, float* __restrict__ o_lat) {
  const int32_t b = blockIdx.x, h_out = a.h / G;
  const int32_t i = blockIdx.y * 4 + (int32_t)(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= h_out) return;  // wave-uniform
  float o[8];
  merge_row<G>(a, b, i, lane, o);
  float4* dst = reinterpret_cast<float4*>(o_lat + ((int64_t)b * h_out + i) * kMergeLat + 8 * lane);
  dst[0] = make_float4(o[0], o[1], o[2], o[3]);
  dst[1] = make_float4(o[4], o[5], o[6], o[7]);
}

hipError_t launch_combine(const AttnArgs& a, float* o_lat, hipStream_t s) {
  if (a.part_bf16) {
    const int32_t G = a.shards > 1 ? a.shards : 1;
    if (a.d_c != kMergeLat || a.h % G || a.streams != 1) return hipErrorInvalidValue;
    const dim3 grid(a.B, (a.h / G + 3) / 4);
    if (G == 1)
      hipLaunchKernelGGL(merge_kernel<1>, grid, dim3(256), 0, s, a, o_lat);
    else if (G == 2)
      hipLaunchKernelGGL(merge_kernel<2>, grid, dim3(256), 0, s, a, o_lat);
    else if (G == 4)
      hipLaunchKernelGGL(merge_kernel<4>, grid, dim3(256), 0, s, a, o_lat);
    else
      return hipErrorInvalidValue;
  } else {
    hipLaunchKernelGGL(combine_kernel, dim3(a.B, a.h), dim3(kCombThreads), 0, s, a, o_lat);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ up-projection
// Work group = (head, 32 output rows).  Thread = (row, one of 8 interleaved
// column segments); W_UV row segments are read once (coalesced 16-byte loads)
// and kept in registers, o_lat rows of 16 sequences at a time sit in LDS, and
// the 8 segment sums of a row are added with lane shuffles.
constexpr int kUpRows = 32;
constexpr int kUpSeq = 16;
constexpr int kUpMaxDc = 512;              // row length of the register-resident fast path
constexpr int kUpChunks = kUpMaxDc / 64;   // 8-wide chunks per thread

template <int WT>
__device__ inline void load8(const void* W, int64_t idx, float* w);
template <>
__device__ inline void load8<MLA_F32>(const void* W, int64_t idx, float* w) {
  const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(W) + idx);
  const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(W) + idx + 4);
  w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w; w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
}
template <>
__device__ inline void load8<MLA_BF16>(const void* W, int64_t idx, float* w) {
  const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(W) + idx);
  const uint32_t p[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    w[2 * i] = __uint_as_float(p[i] << 16);
    w[2 * i + 1] = __uint_as_float(p[i] & 0xffff0000u);
  }
}

template <int WT, int OT>
__global__ __launch_bounds__(256) void up_project_kernel(const float* __restrict__ o_lat,
                                                         const void* __restrict__ W_UV,
                                                         void* __restrict__ out, int32_t B,
                                                         int32_t h, int32_t d_c, int32_t d_v) {
  extern __shared__ float os[];  // [kUpSeq][d_c]
  const int32_t head = blockIdx.x;
  const int32_t v = blockIdx.y * kUpRows + (threadIdx.x >> 3);
  const int seg = threadIdx.x & 7;
  // interleaved 8-wide segments tile the row; 16-byte loads need an aligned base
  const bool vec = d_c == kUpMaxDc && (reinterpret_cast<uintptr_t>(W_UV) & 15) == 0;
  const int64_t wrow = ((int64_t)head * d_v + min(v, d_v - 1)) * d_c;
  float w[kUpChunks][8];
  if (vec) {  // the whole row share of this thread, loaded once up front
#pragma unroll
    for (int k = 0; k < kUpChunks; k++) load8<WT>(W_UV, wrow + 8 * seg + 64 * k, w[k]);
  }
  for (int32_t b0 = 0; b0 < B; b0 += kUpSeq) {
    const int32_t nb = min(kUpSeq, B - b0);
    __syncthreads();
    for (int32_t i = threadIdx.x; i < nb * d_c; i += 256) {
      const int32_t j = i / d_c, c = i % d_c;
      os[i] = o_lat[((int64_t)(b0 + j) * h + head) * d_c + c];
    }
    __syncthreads();
    float acc[kUpSeq];
#pragma unroll
    for (int j = 0; j < kUpSeq; j++) acc[j] = 0.f;
    if (v < d_v) {
      if (vec) {
#pragma unroll
        for (int j = 0; j < kUpSeq; j++) {
          if (j >= nb) break;
#pragma unroll
          for (int k = 0; k < kUpChunks; k++) {
            const float* orow = os + j * d_c + 8 * seg + 64 * k;
#pragma unroll
            for (int i = 0; i < 8; i++) acc[j] = fmaf(w[k][i], orow[i], acc[j]);
          }
        }
      } else {
        for (int32_t c = seg; c < d_c; c += 8) {
          const float wc = load_elem<WT>(W_UV, wrow + c);
          for (int j = 0; j < nb; j++) acc[j] = fmaf(wc, os[j * d_c + c], acc[j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kUpSeq; j++) {
      acc[j] += __shfl_xor(acc[j], 1);
      acc[j] += __shfl_xor(acc[j], 2);
      acc[j] += __shfl_xor(acc[j], 4);
    }
    if (v < d_v && seg == 0)
      for (int j = 0; j < nb; j++) store_elem<OT>(out, ((int64_t)(b0 + j) * h + head) * d_v + v, acc[j]);
  }
}

template <int WT, int OT>
static hipError_t up_t(const mla_decode_params& p, const float* o, const void* W, void* out,
                       hipStream_t s) {
  dim3 grid(p.num_heads, (p.d_v + kUpRows - 1) / kUpRows);
  size_t lds = (size_t)kUpSeq * p.d_latent * sizeof(float);
  hipLaunchKernelGGL((up_project_kernel<WT, OT>), grid, dim3(256), lds, s, o, W, out, p.batch,
                     p.num_heads, p.d_latent, p.d_v);
  return hipGetLastError();
}

hipError_t launch_up_project(const mla_decode_params& p, const float* o_lat, const void* W_UV,
                             void* out, hipStream_t s) {
  if (proj_mfma_supported(p) && aligned16(o_lat) && aligned16(W_UV))
    return launch_up_project_mfma(p, o_lat, W_UV, out, s);
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
