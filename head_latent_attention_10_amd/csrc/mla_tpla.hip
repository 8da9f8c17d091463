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
