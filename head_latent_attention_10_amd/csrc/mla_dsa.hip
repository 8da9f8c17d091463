// DeepSeek Sparse Attention at decode time (gfx950): the lightning indexer
// and the top-k selection that feed the sparse decode step.
//
// "TransMLA & Sparse Latent Attention", Chapter 6 ("The lightning indexer",
// "Fine-grained token selection"): the index score of cached position s for
// the new token of sequence b is
//   I[b, s] = sum_j w[b, j] * ReLU(q_I[b, j] . k_I[s])
// over the H_I indexer heads (no softmax), and the k positions with the
// highest scores are attended to.  Chapter 7: one selection per token, shared
// by all heads; each cached position keeps a d_I-wide indexer key.
//
// Storage: q_I as E4M3FN codes with one fp32 scale per (sequence, head), the
// key pool as E4M3FN codes with one fp32 scale per slot (paged like the latent
// cache).  Both scales are positive, so they factor out of the ReLU:
//   I[b, s] = ks[s] * sum_j (w[b, j] qs[b, j]) * ReLU(q8[b, j] . k8[s]).
// The code dot products run on the fp8 matrix core (32x32x64, fp32
// accumulation): indexer heads on M, tokens on N, so one lane's accumulator
// holds 16 heads of one token and the head sum is in-lane plus one exchange.
//
// Top-k: one work group per sequence.  Scores map to unsigned keys that order
// like the floats (-0 taken as +0); an MSB-first radix select (11 + 11 + 10
// bits, LDS histograms) finds the k-th largest key K and how many keys equal
// to K are taken (the earliest positions); a final pass writes the selected
// positions in increasing order.
#include "mla_mfma_util.hpp"

namespace mla {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kIdxHeads = 64;      // matrix-core indexer: H_I
constexpr int kIdxDim = 128;       // d_I (two 64-byte k-steps)
constexpr int kIdxWaves = 4;
constexpr int kIdxTokWave = 64;    // tokens per wave (two 32-token N blocks)
constexpr int kIdxTokWG = kIdxWaves * kIdxTokWave;
constexpr int kIdxSimt = 256;

struct IndexerArgs {
  const uint8_t* q;        // [B, H, d]
  const float* q_scale;    // [B, H]
  const float* w;          // [B, H]
  const uint8_t* k;        // [nb, P, d]
  const float* k_scale;    // [nb, P]
  const int32_t* block_table;
  const int32_t* seq_lens;
  float* scores;           // [B, stride]
  int32_t B, H, d, P, max_blocks, num_blocks, stride;
};

// Positions of sequence b that get a score.
__device__ inline int32_t scored_len(const IndexerArgs& a, int32_t b) {
  int32_t T = a.seq_lens[b];
  const int32_t cap = min(a.max_blocks * a.P, a.stride);
  return T < 0 ? 0 : (T > cap ? cap : T);
}

// Work group = 256 tokens of one sequence; wave = 64 tokens (two N blocks).
// A operand: q codes of heads 32 mb + (lane & 31), bytes 64 ks + 32 (lane >> 5)
// .. +31; B operand: key codes of token (lane & 31) of the block, same bytes.
// (Any consistent assignment of the 64 bytes of a k-step to the two lane
// halves gives the same dot products.)
__global__ __launch_bounds__(64 * kIdxWaves) void indexer_mfma_kernel(IndexerArgs a) {
  const int32_t b = blockIdx.y;
  const int32_t T = scored_len(a, b);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, c = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t t_wave = blockIdx.x * kIdxTokWG + wave * kIdxTokWave;
  if (t_wave >= T) return;
  // keys of the wave's 64 tokens first (their loads are the long ones)
  i32x8 kb[2][2];
  float ks[2];
#pragma unroll
  for (int nb = 0; nb < 2; nb++) {
    const int32_t t = min(t_wave + 32 * nb + c, T - 1);
    const int64_t slot = phys_slot(a.block_table, b, t, a.P, a.max_blocks, a.num_blocks);
    const uint8_t* row = a.k + slot * kIdxDim + 32 * g;
#pragma unroll
    for (int s = 0; s < 2; s++) {
      const i32x4 lo = *reinterpret_cast<const i32x4*>(row + 64 * s);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(row + 64 * s + 16);
      kb[nb][s] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    ks[nb] = a.k_scale[slot];
  }
  i32x8 qa[2][2];
  float wq[2][16];
#pragma unroll
  for (int mb = 0; mb < 2; mb++) {
    const uint8_t* row = a.q + ((int64_t)b * kIdxHeads + 32 * mb + c) * kIdxDim + 32 * g;
#pragma unroll
    for (int s = 0; s < 2; s++) {
      const i32x4 lo = *reinterpret_cast<const i32x4*>(row + 64 * s);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(row + 64 * s + 16);
      qa[mb][s] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    // accumulator row j of block mb is head 32 mb + 8 (j / 4) + 4 g + j % 4
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const int32_t head = 32 * mb + 8 * (j >> 2) + 4 * g + (j & 3);
      const int64_t o = (int64_t)b * kIdxHeads + head;
      wq[mb][j] = a.w[o] * a.q_scale[o];
    }
  }
#pragma unroll
  for (int nb = 0; nb < 2; nb++) {
    float v = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; mb++) {
      f32x16 acc = f32x16{};
#pragma unroll
      for (int s = 0; s < 2; s++)
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[mb][s], kb[nb][s], acc, 0, 0, 0,
                                                              127, 0, 127);
#pragma unroll
      for (int j = 0; j < 16; j++) v = fmaf(wq[mb][j], fmaxf(acc[j], 0.f), v);
    }
    v += __shfl_xor(v, 32);  // the other 32 heads of this token
    const int32_t t = t_wave + 32 * nb + c;
    if (g == 0 && t < T) a.scores[(int64_t)b * a.stride + t] = v * ks[nb];
  }
}

// Generic indexer (any H, d): thread = one token, heads in order.
__global__ __launch_bounds__(kIdxSimt) void indexer_simt_kernel(IndexerArgs a) {
  const int32_t b = blockIdx.y;
  const int32_t t = blockIdx.x * kIdxSimt + threadIdx.x;
  if (t >= scored_len(a, b)) return;
  const int64_t slot = phys_slot(a.block_table, b, t, a.P, a.max_blocks, a.num_blocks);
  const uint8_t* kr = a.k + slot * a.d;
  float v = 0.f;
  for (int32_t j = 0; j < a.H; j++) {
    const uint8_t* qr = a.q + ((int64_t)b * a.H + j) * a.d;
    float dot = 0.f;
    for (int32_t i = 0; i < a.d; i++) dot = fmaf(e4m3_to_f32(qr[i]), e4m3_to_f32(kr[i]), dot);
    const int64_t o = (int64_t)b * a.H + j;
    v = fmaf(a.w[o] * a.q_scale[o], fmaxf(dot, 0.f), v);
  }
  a.scores[(int64_t)b * a.stride + t] = v * a.k_scale[slot];
}

// ------------------------------------------------------------------ top-k
constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kBins = 2048;

// Unsigned key ordering like the float (-0 is +0; larger float, larger key).
__device__ inline uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the work group (one value per thread).
__device__ inline uint32_t block_scan(uint32_t v, uint32_t* s_wave) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  __syncthreads();
  if (lane == 63) s_wave[wave] = v;
  __syncthreads();
  uint32_t add = 0;
  for (int w = 0; w < wave; w++) add += s_wave[w];
  return v + add;
}

struct TopkArgs {
  const float* scores;
  int32_t score_stride;
  const int32_t* seq_lens;
  int32_t k;
  int32_t* indices;
  int32_t index_stride;
  int32_t* counts;
};

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a) {
  __shared__ uint32_t s_hist[kBins];
  __shared__ uint32_t s_wave[kTopkWaves];
  __shared__ uint32_t s_pick[2];
  const int32_t b = blockIdx.x;
  const int tid = threadIdx.x;
  int32_t T = a.seq_lens[b];
  T = T < 0 ? 0 : (T > a.score_stride ? a.score_stride : T);
  int32_t* out = a.indices + (int64_t)b * a.index_stride;
  if (T <= a.k) {  // everything is selected
    for (int32_t i = tid; i < T; i += kTopkThreads) out[i] = i;
    if (tid == 0) a.counts[b] = T;
    return;
  }
  const float* sc = a.scores + (int64_t)b * a.score_stride;
  // radix select, most significant digit first
  uint32_t prefix = 0, rem = (uint32_t)a.k;
  constexpr int kShift[3] = {21, 10, 0};
  constexpr int kWidth[3] = {11, 11, 10};
#pragma unroll
  for (int pass = 0; pass < 3; pass++) {
    const int shift = kShift[pass], width = kWidth[pass];
    const uint32_t hi_mask = pass == 0 ? 0u : ~((1u << (shift + width)) - 1u);
    for (int i = tid; i < kBins; i += kTopkThreads) s_hist[i] = 0;
    __syncthreads();
    for (int32_t i = tid; i < T; i += kTopkThreads) {
      const uint32_t key = score_key(sc[i]);
      if ((key & hi_mask) == prefix) atomicAdd(&s_hist[(key >> shift) & ((1u << width) - 1u)], 1u);
    }
    __syncthreads();
    // counts from the top bin down: thread t owns bins 2047 - 2t and 2046 - 2t
    const int hb = kBins - 1 - 2 * tid;
    const uint32_t c0 = s_hist[hb], c1 = s_hist[hb - 1];
    const uint32_t incl = block_scan(c0 + c1, s_wave);  // keys in bins >= hb - 1
    const uint32_t above = incl - c0 - c1;                // keys in bins > hb
    // the bin holding the rem-th largest key
    if (above < rem && rem <= above + c0) {
      s_pick[0] = hb;
      s_pick[1] = above;
    } else if (above + c0 < rem && rem <= incl) {
      s_pick[0] = hb - 1;
      s_pick[1] = above + c0;
    }
    __syncthreads();
    prefix |= s_pick[0] << shift;
    rem -= s_pick[1];
    __syncthreads();
  }
  // prefix = K (the k-th largest key); take every key above it and the first
  // rem keys equal to it, in position order.  Thread t walks positions
  // [t * chunk, (t + 1) * chunk).
  const uint32_t K = prefix;
  const int32_t chunk = (T + kTopkThreads - 1) / kTopkThreads;
  const int32_t p0 = min(T, tid * chunk), p1 = min(T, p0 + chunk);
  uint32_t n_gt = 0, n_eq = 0;
  for (int32_t i = p0; i < p1; i++) {
    const uint32_t key = score_key(sc[i]);
    n_gt += key > K;
    n_eq += key == K;
  }
  uint32_t gt = block_scan(n_gt, s_wave) - n_gt;
  __syncthreads();
  uint32_t eq = block_scan(n_eq, s_wave) - n_eq;
  for (int32_t i = p0; i < p1; i++) {
    const uint32_t key = score_key(sc[i]);
    if (key > K) {
      out[gt + min(eq, rem)] = i;
      gt++;
    } else if (key == K) {
      if (eq < rem) out[gt + eq] = i;
      eq++;
    }
  }
  if (tid == 0) a.counts[b] = a.k;
}

}  // namespace

bool indexer_mfma_ok(int32_t heads, int32_t dim) { return heads == kIdxHeads && dim == kIdxDim; }

hipError_t launch_indexer(const uint8_t* q, const float* q_scale, const float* w, const uint8_t* k,
                          const float* k_scale, const int32_t* block_table,
                          const int32_t* seq_lens, float* scores, int32_t B, int32_t H, int32_t d,
                          int32_t P, int32_t max_blocks, int32_t num_blocks, int32_t stride,
                          hipStream_t s) {
  IndexerArgs a{q, q_scale, w, k, k_scale, block_table, seq_lens, scores,
                B, H, d, P, max_blocks, num_blocks, stride};
  const int64_t cap = std::min<int64_t>((int64_t)max_blocks * P, stride);
  if (indexer_mfma_ok(H, d)) {
    const dim3 grid((uint32_t)((cap + kIdxTokWG - 1) / kIdxTokWG), B);
    hipLaunchKernelGGL(indexer_mfma_kernel, grid, dim3(64 * kIdxWaves), 0, s, a);
  } else {
    const dim3 grid((uint32_t)((cap + kIdxSimt - 1) / kIdxSimt), B);
    hipLaunchKernelGGL(indexer_simt_kernel, grid, dim3(kIdxSimt), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_topk(const float* scores, int32_t score_stride, const int32_t* seq_lens,
                       int32_t B, int32_t k, int32_t* indices, int32_t index_stride,
                       int32_t* counts, hipStream_t s) {
  TopkArgs a{scores, score_stride, seq_lens, k, indices, index_stride, counts};
  hipLaunchKernelGGL(topk_kernel, dim3(B), dim3(kTopkThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
