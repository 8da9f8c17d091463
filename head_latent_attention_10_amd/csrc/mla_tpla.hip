// TPLA decode on one GPU (gfx950): the latent dimension cut into g shards,
// each head attending to every shard with its own softmax.
//
// "TPLA: Tensor Parallel Latent Attention ...", "The Core TPLA Computation and
// Structural Differences from GLA" (Eqs. 6-7) and "TPLA as a special case of
// GLA" (Section 4.4): per head i and shard j the score is the shard's content
// score (times a factor mu_j) plus the replicated positional score, softmaxed
// over the tokens, and the result is the softmax-weighted sum of the shard's
// latent columns; the up-projected shard outputs are added.  That is the
// ordinary decode step with g h heads whose absorbed queries are zero outside
// their shard.  The shard heads are numbered shard-major (shard head j h + i is
// head i's shard j), so that a block of consecutive shard heads shares one
// shard and the matrix-core attention reads only that shard's latent columns.
// These kernels build the shard heads' queries from the absorbed ones
// (expand) and, where the merge does not already do it, take each head's own
// shard columns back out of the g h head outputs (gather); absorption,
// attention, merge and up-projection are the decode step's own kernels.
#include "mla_kernels.hpp"

namespace mla {
namespace {

constexpr int kTplaThreads = 256;

// q2[b, j h + i, x] = mu_j q1[b, i, x] for x in shard j of the latent part,
// 0 elsewhere in it, and q1[b, i, x] for the rope part.
template <int QT>
__global__ __launch_bounds__(kTplaThreads) void tpla_expand_kernel(const void* __restrict__ q1,
                                                                   void* __restrict__ q2,
                                                                   int64_t n, int32_t g,
                                                                   int32_t h, int32_t d_c,
                                                                   int32_t d_r, TplaMu mu) {
  const int64_t e = (int64_t)blockIdx.x * kTplaThreads + threadIdx.x;
  if (e >= n) return;
  const int32_t dl = d_c + d_r;
  const int32_t x = (int32_t)(e % dl);
  const int64_t row2 = e / dl;  // b g h + j h + i
  const int64_t b = row2 / ((int64_t)g * h);
  const int32_t ji = (int32_t)(row2 - b * g * h);
  const int32_t j = ji / h;
  const int64_t row1 = b * h + (ji - j * h);
  const float v = load_elem<QT>(q1, row1 * dl + x);
  float o = v;
  if (x < d_c) o = (x / (d_c / g) == j) ? mu.v[j] * v : 0.f;
  store_elem<QT>(q2, e, o);
}

// The same for bf16 queries, 8 values (16 bytes) a thread: with d_c / g and
// d_c + d_r multiples of 8 the 8 values of a chunk lie in one shard or in the
// rope part.  Chunk c of the output is row c / cpr, values 8 (c % cpr) ..
// (32-bit index arithmetic: rows and chunks are counted in int32).
__global__ __launch_bounds__(kTplaThreads) void tpla_expand_bf16x8_kernel(
    const uint16_t* __restrict__ q1, uint16_t* __restrict__ q2, int32_t chunks, int32_t cpr,
    int32_t g, int32_t h, int32_t d_c, TplaMu mu) {
  const int32_t c = blockIdx.x * kTplaThreads + threadIdx.x;
  if (c >= chunks) return;
  const int32_t row2 = c / cpr, k = c - row2 * cpr, x = 8 * k;
  const int32_t gh = g * h, b = row2 / gh, ji = row2 - b * gh, j = ji / h;
  const int32_t row1 = b * h + (ji - j * h);
  const uint4 v = *reinterpret_cast<const uint4*>(q1 + (int64_t)row1 * cpr * 8 + x);
  uint4 o = v;
  if (x < d_c) {
    if (x / (d_c / g) != j) {
      o = make_uint4(0u, 0u, 0u, 0u);
    } else {
      const float m = mu.v[j];
      uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int p = 0; p < 4; p++) {
        const float lo = __uint_as_float(w[p] << 16) * m, hi = __uint_as_float(w[p] & 0xffff0000u) * m;
        w[p] = (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
      }
      o = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
  *reinterpret_cast<uint4*>(q2 + (int64_t)c * 8) = o;
}

// o1[b, i, x] = o2[b, j h + i, x], j = x / (d_c / g).
__global__ __launch_bounds__(kTplaThreads) void tpla_gather_kernel(const float* __restrict__ o2,
                                                                   float* __restrict__ o1,
                                                                   int64_t n, int32_t g, int32_t h,
                                                                   int32_t d_c) {
  const int64_t e = (int64_t)blockIdx.x * kTplaThreads + threadIdx.x;
  if (e >= n) return;
  const int32_t x = (int32_t)(e % d_c);
  const int64_t row1 = e / d_c;  // b h + i
  const int64_t b = row1 / h;
  const int32_t j = x / (d_c / g);
  o1[e] = o2[((b * g + j) * h + (row1 - b * h)) * d_c + x];
}

}  // namespace

hipError_t launch_tpla_expand(const void* q1, void* q2, int32_t q_dtype, int32_t B, int32_t h,
                              int32_t g, int32_t d_c, int32_t d_r, const TplaMu& mu,
                              hipStream_t s) {
  const int64_t n = (int64_t)B * h * g * (d_c + d_r);
  const int32_t dl = d_c + d_r;
  if (q_dtype == MLA_BF16 && dl % 8 == 0 && (d_c / g) % 8 == 0 && n / 8 < INT32_MAX &&
      (reinterpret_cast<uintptr_t>(q1) & 15) == 0 && (reinterpret_cast<uintptr_t>(q2) & 15) == 0) {
    const int32_t chunks = (int32_t)(n / 8);
    const dim3 grid8((uint32_t)((chunks + kTplaThreads - 1) / kTplaThreads));
    hipLaunchKernelGGL(tpla_expand_bf16x8_kernel, grid8, dim3(kTplaThreads), 0, s,
                       static_cast<const uint16_t*>(q1), static_cast<uint16_t*>(q2), chunks,
                       dl / 8, g, h, d_c, mu);
    return hipGetLastError();
  }
  const dim3 grid((uint32_t)((n + kTplaThreads - 1) / kTplaThreads));
  if (q_dtype == MLA_F32)
    hipLaunchKernelGGL(tpla_expand_kernel<MLA_F32>, grid, dim3(kTplaThreads), 0, s, q1, q2, n, g,
                       h, d_c, d_r, mu);
  else
    hipLaunchKernelGGL(tpla_expand_kernel<MLA_BF16>, grid, dim3(kTplaThreads), 0, s, q1, q2, n, g,
                       h, d_c, d_r, mu);
  return hipGetLastError();
}

hipError_t launch_tpla_gather(const float* o2, float* o1, int32_t B, int32_t h, int32_t g,
                              int32_t d_c, hipStream_t s) {
  const int64_t n = (int64_t)B * h * d_c;
  const dim3 grid((uint32_t)((n + kTplaThreads - 1) / kTplaThreads));
  hipLaunchKernelGGL(tpla_gather_kernel, grid, dim3(kTplaThreads), 0, s, o2, o1, n, g, h, d_c);
  return hipGetLastError();
}

}  // namespace mla
