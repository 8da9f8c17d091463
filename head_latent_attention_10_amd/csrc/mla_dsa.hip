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
// Top-k.  Scores map to unsigned keys that order like the floats (-0 taken as
// +0).  A sample bounds the k-th largest key from below, the keys above the
// bound are gathered in position order, and the k-th largest key K and how
// many keys equal to K are taken (the earliest positions) are found by
// counting; the selected positions come out in increasing order.  Either one
// work group per sequence does all of it (topk_kernel), or work groups of 2048
// positions gather the candidates and one work group per sequence selects
// (topk_cand_kernel, topk_pick_kernel); both give the same selection.
#include <algorithm>

#include "mla_mfma_util.hpp"

namespace mla {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kIdxHeads = 64;      // matrix-core indexer: H_I
constexpr int kIdxDim = 128;       // d_I (two 64-byte k-steps)
constexpr int kIdxWaves = 4;
constexpr int kIdxBlocks = 4;      // 32-token N blocks per wave
constexpr int kIdxTokWave = 32 * kIdxBlocks;
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

// Work group = kIdxTokWG tokens of one sequence; wave = kIdxBlocks 32-token N
// blocks, whose key loads (table entry, then the row pieces and the scale) are
// all issued before the first product.  The sequence's query codes (8 KiB) and
// its per-head factors w q_scale are staged in LDS once per work group, so a
// wave's vector-memory instructions are its keys' alone.
// A operand: q codes of heads 32 mb + (lane & 31), bytes 64 ks + 32 (lane >> 5)
// .. +31; B operand: key codes of token (lane & 31) of the block, same bytes.
// (Any consistent assignment of the 64 bytes of a k-step to the two lane
// halves gives the same dot products.)
// (At most 168 VGPRs, so that three waves fit on a SIMD: 152 without spills.)
__global__ __launch_bounds__(64 * kIdxWaves) __attribute__((amdgpu_waves_per_eu(3)))
void indexer_mfma_kernel(IndexerArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_q[kIdxHeads * kIdxDim];
  __shared__ __attribute__((aligned(16))) float s_wq[kIdxHeads];
  const int32_t b = blockIdx.y;
  const int32_t T = scored_len(a, b);
  const int32_t t_wg = blockIdx.x * kIdxTokWG;
  if (t_wg >= T) return;  // the whole work group
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, c = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t t_wave = t_wg + wave * kIdxTokWave;
  const bool active = t_wave < T;
  i32x8 kb[kIdxBlocks][2];
  float ks[kIdxBlocks];
  if (active) {
#pragma unroll
    for (int nb = 0; nb < kIdxBlocks; nb++) {
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
  }
  {
    const i32x4* src = reinterpret_cast<const i32x4*>(a.q + (int64_t)b * kIdxHeads * kIdxDim);
    for (int i = tid; i < kIdxHeads * kIdxDim / 16; i += 64 * kIdxWaves)
      reinterpret_cast<i32x4*>(s_q)[i] = src[i];
    if (tid < kIdxHeads) {
      const int64_t o = (int64_t)b * kIdxHeads + tid;
      s_wq[tid] = a.w[o] * a.q_scale[o];
    }
  }
  __syncthreads();
  if (!active) return;
  i32x8 qa[2][2];
  float wq[2][16];
#pragma unroll
  for (int mb = 0; mb < 2; mb++) {
    const uint8_t* row = s_q + (32 * mb + c) * kIdxDim + 32 * g;
#pragma unroll
    for (int s = 0; s < 2; s++) {
      const i32x4 lo = *reinterpret_cast<const i32x4*>(row + 64 * s);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(row + 64 * s + 16);
      qa[mb][s] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    // accumulator row j of block mb is head 32 mb + 8 (j / 4) + 4 g + j % 4
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const f32x4 f = *reinterpret_cast<const f32x4*>(s_wq + 32 * mb + 8 * i + 4 * g);
#pragma unroll
      for (int r = 0; r < 4; r++) wq[mb][4 * i + r] = f[r];
    }
  }
#pragma unroll
  for (int nb = 0; nb < kIdxBlocks; nb++) {
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
constexpr int kCandCap = 12288;                 // candidates kept in LDS
constexpr int kSeg = kCandCap / kTopkWaves;     // candidates per wave segment (768)
constexpr int kSegLane = kSeg / 64;             // per lane (12)
constexpr int kSample = 4096;                   // sampled keys (4 per thread)
constexpr int kAllCand = 6144;                  // up to this length every key is a candidate
constexpr int kMaxBlocks = 256;                 // 1024-position blocks of the fast path
constexpr int kFastMaxT = kMaxBlocks * kTopkThreads;
constexpr int kGrp = 32;                        // position blocks whose loads go out together

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

// Sum over the work group.
__device__ inline uint32_t block_sum_u32(uint32_t v, uint32_t* s_wave) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s_wave[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; w++) t += s_wave[w];
  return t;
}

// Maximum over the work group (two barriers).
__device__ inline uint32_t block_max_u32(uint32_t v, uint32_t* s_wave) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s_wave[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; w++) t = max(t, s_wave[w]);
  return t;
}

// Two maxima over the work group in one exchange (two barriers); s_wave holds
// 2 kTopkWaves values.
__device__ inline void block_max2_u32(uint32_t& a, uint32_t& b, uint32_t* s_wave) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    a = max(a, (uint32_t)__shfl_xor((int)a, o));
    b = max(b, (uint32_t)__shfl_xor((int)b, o));
  }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    s_wave[threadIdx.x >> 6] = a;
    s_wave[kTopkWaves + (threadIdx.x >> 6)] = b;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kTopkWaves; w++) {
    a = max(a, s_wave[w]);
    b = max(b, s_wave[kTopkWaves + w]);
  }
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

// What a radix round over register-held keys shares (radix_rank).
struct RadixShared {
  uint32_t whist[kTopkWaves][256];  // per-wave digit histograms
  uint32_t wave[2 * kTopkWaves];    // per-wave values of the work-group reductions
  uint32_t pick[4];
};

struct TopkShared {
  uint32_t cand_key[kCandCap];
  int32_t cand_pos[kCandCap];
  union {
    uint32_t bits[kFastMaxT / 32];  // selected positions (fast path)
    uint32_t hist[kBins];           // radix histogram (general path)
  };
  RadixShared r;
  uint32_t seg[kTopkWaves];  // candidates of each wave's segment
};

// Inclusive prefix sum over the 64 lanes of a wave (DPP: row shifts, then
// the row totals broadcast to the rows after them).
__device__ inline uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Radix select over keys held by the threads (key[i] for i < n, n
// wave-uniform, where ok[i]): K = the rank-th largest key, searched over bits
// [low, top) eight at a time from the top (bits at and above top are base's,
// those below low stay zero).  Each wave counts its keys' digits in its own
// LDS histogram; wave 0 then adds the sixteen histograms (lane l: bins
// 255 - 4l down to 252 - 4l), scans them from the top bin down and publishes
// the digit, so a round costs two barriers.  With low = 0, *rem = rank -
// #(keys > K) and *eq = #(keys == K).
template <int N>
__device__ uint32_t radix_rank(const uint32_t (&key)[N], const bool (&ok)[N], int n, uint32_t rank,
                               uint32_t base, int top, int low, RadixShared& sh, uint32_t* rem_out,
                               uint32_t* eq_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t K = base, rem = rank, eq = 0;
  for (int hi = top; hi > low;) {
    const int width = min(8, hi - low);
    const int sft = hi - width;
    reinterpret_cast<u32x4*>(sh.whist[wave])[lane] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < N; i++) {
      if (i < n && ok[i] && (hi >= 32 || (key[i] >> hi) == (K >> hi)))
        atomicAdd(&sh.whist[wave][(key[i] >> sft) & ((1u << width) - 1u)], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // lane l: bins 4 (63 - l) .. 4 (63 - l) + 3, i.e. descending with l
      const int b0 = 4 * (63 - lane);
      u32x4 t = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int w = 0; w < kTopkWaves; w++) t += reinterpret_cast<const u32x4*>(sh.whist[w])[63 - lane];
      const uint32_t mine = t[0] + t[1] + t[2] + t[3];
      const uint32_t incl = wave_incl_scan(mine);      // keys in bins >= b0
      uint32_t above = incl - mine;                     // keys in bins >= b0 + 4
#pragma unroll
      for (int e = 3; e >= 0; e--) {
        if (above < rem && rem <= above + t[e]) {
          sh.pick[0] = (uint32_t)(b0 + e);
          sh.pick[1] = above;
          sh.pick[2] = t[e];
        }
        above += t[e];
      }
    }
    __syncthreads();
    K |= sh.pick[0] << sft;
    rem -= sh.pick[1];
    eq = sh.pick[2];
    hi = sft;
  }
  if (rem_out) *rem_out = rem;
  if (eq_out) *eq_out = eq;
  return K;
}

// Radix select over all T keys in global memory (11 + 11 + 10 bits, LDS
// histograms): the k-th largest key K and how many keys equal to K are taken.
template <typename SH>
__device__ void radix_select_global(const float* sc, int32_t T, uint32_t k, SH& sh,
                                    uint32_t* K_out, uint32_t* rem_out) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, rem = k;
  constexpr int kShift[3] = {21, 10, 0};
  constexpr int kWidth[3] = {11, 11, 10};
#pragma unroll
  for (int pass = 0; pass < 3; pass++) {
    const int shift = kShift[pass], width = kWidth[pass];
    const uint32_t hi_mask = pass == 0 ? 0u : ~((1u << (shift + width)) - 1u);
    for (int i = tid; i < kBins; i += kTopkThreads) sh.hist[i] = 0;
    __syncthreads();
    for (int32_t i = tid; i < T; i += kTopkThreads) {
      const uint32_t key = score_key(sc[i]);
      if ((key & hi_mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & ((1u << width) - 1u)], 1u);
    }
    __syncthreads();
    // counts from the top bin down: thread t owns bins 2047 - 2t and 2046 - 2t
    const int hb = kBins - 1 - 2 * tid;
    const uint32_t c0 = sh.hist[hb], c1 = sh.hist[hb - 1];
    const uint32_t incl = block_scan(c0 + c1, sh.r.wave);  // keys in bins >= hb - 1
    const uint32_t above = incl - c0 - c1;                // keys in bins > hb
    if (above < rem && rem <= above + c0) {
      sh.r.pick[0] = hb;
      sh.r.pick[1] = above;
    } else if (above + c0 < rem && rem <= incl) {
      sh.r.pick[0] = hb - 1;
      sh.r.pick[1] = above + c0;
    }
    __syncthreads();
    prefix |= sh.r.pick[0] << shift;
    rem -= sh.r.pick[1];
    __syncthreads();
  }
  *K_out = prefix;
  *rem_out = rem;
}

// Step 1 of the fast path below: a lower bound L of the k-th largest key, the
// top 16 bits of the R-th largest of 4096 keys at evenly spaced positions, R
// a few standard deviations above the sample rank of the k-th largest key, so
// that at least k keys are >= L and not many more (L = 0, every key, when
// T <= 6144).  False when the fast path does not apply (T too long, or R past
// the sample).  The same scores always give the same L.
__device__ bool sample_bound(const float* sc, int32_t T, uint32_t k, RadixShared& sh, uint32_t* L) {
  const int tid = threadIdx.x;
  *L = 0;
  if (T > kFastMaxT) return false;
  if (T <= kAllCand) return true;
  const uint32_t r = (uint32_t)(((uint64_t)k * kSample + T - 1) / T);
  const uint32_t R = r + 4 * (uint32_t)ceilf(sqrtf((float)r)) + 16;
  if (R >= kSample) return false;
  uint32_t key[4];
  bool ok[4];
#pragma unroll
  for (int e = 0; e < 4; e++) {
    key[e] = score_key(sc[((int64_t)(tid + kTopkThreads * e) * T) / kSample]);
    ok[e] = true;
  }
  // the top 16 bits of the R-th largest sampled key: a lower bound is all
  // the candidate pass needs
  *L = radix_rank<4>(key, ok, 4, R, 0u, 32, 16, sh, nullptr, nullptr);
  return true;
}

// The general path: a radix select over all T keys in global memory gives the
// k-th largest key K and how many keys equal to K are taken, then thread t
// walks positions [t chunk, (t + 1) chunk) twice, counting and then writing
// the selected positions in increasing order.
template <typename SH>
__device__ void select_general(const float* sc, int32_t T, uint32_t k, int32_t* out, SH& sh) {
  const int tid = threadIdx.x;
  uint32_t K, rem;
  radix_select_global(sc, T, k, sh, &K, &rem);
  const int32_t chunk = (T + kTopkThreads - 1) / kTopkThreads;
  const int32_t p0 = min(T, tid * chunk), p1 = min(T, p0 + chunk);
  uint32_t n_gt = 0, n_eq = 0;
  for (int32_t i = p0; i < p1; i++) {
    const uint32_t key = score_key(sc[i]);
    n_gt += key > K;
    n_eq += key == K;
  }
  uint32_t gt = block_scan(n_gt, sh.r.wave) - n_gt;
  uint32_t eq = block_scan(n_eq, sh.r.wave) - n_eq;
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
}

// Over candidates held N per thread (key, position, ok; every key >= L), the
// k-th largest key K and the last position `last` up to which keys equal to K
// are taken: a position is selected when its key is > K, or == K at a
// position <= last.  ne (wave-uniform) bounds the register slots in use.  The
// radix select runs on key - L (order kept, all candidates being >= L): only
// the bits of max - L are searched, and its leading digit spreads the
// candidates over many bins.
// kmax: the largest candidate key.
template <int N>
__device__ void candidate_cut(const uint32_t (&key)[N], const int32_t (&pos)[N], const bool (&ok)[N],
                              int ne, uint32_t k, uint32_t L, uint32_t kmax_key, RadixShared& sh,
                              uint32_t* K_out, uint32_t* last_out) {
  uint32_t dk[N];
#pragma unroll
  for (int e = 0; e < N; e++) dk[e] = ok[e] ? key[e] - L : 0u;
  const uint32_t kmax = kmax_key - L;
  const int bits = kmax == 0 ? 0 : 32 - __clz(kmax);
  const int top = max(8, bits);  // at least one pass (it counts the equal keys)
  uint32_t rem, eq;
  const uint32_t K = L + radix_rank<N>(dk, ok, ne, k, 0u, top, 0, sh, &rem, &eq);
  uint32_t last = 0xffffffffu;  // equal keys at positions <= last are taken
  if (eq > rem) {
    uint32_t pk[N];  // larger for earlier positions, among the equal keys
    bool pok[N];
#pragma unroll
    for (int e = 0; e < N; e++) {
      pok[e] = ok[e] && key[e] == K;
      pk[e] = ~(uint32_t)pos[e];
    }
    last = ~radix_rank<N>(pk, pok, ne, rem, 0u, 32, 0, sh, nullptr, nullptr);
  }
  *K_out = K;
  *last_out = last;
}

// One work group per sequence.  Fast path (k < T <= 262144):
//  1. L = sample_bound;
//  2. one pass over the scores: each wave appends its keys >= L (the
//     candidates) with their positions to its own LDS segment (ballots, no
//     atomics);
//  3. K = the k-th largest candidate key, by counting; the keys above K and,
//     of those equal to K, the rem = k - #(keys > K) earliest (the rem-th
//     smallest position found the same way when there are more) are marked in
//     a bitmap of the positions;
//  4. a scan of the bitmap writes the positions in increasing order.
// When the sample bound misses (fewer than k candidates, or a full segment)
// or T is larger, select_general.
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a) {
  __shared__ TopkShared sh;
  const int32_t b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t T = a.seq_lens[b];
  T = T < 0 ? 0 : (T > a.score_stride ? a.score_stride : T);
  int32_t* out = a.indices + (int64_t)b * a.index_stride;
  const uint32_t k = (uint32_t)a.k;
  if (T <= a.k) {  // everything is selected
    for (int32_t i = tid; i < T; i += kTopkThreads) out[i] = i;
    if (tid == 0) a.counts[b] = T;
    return;
  }
  const float* sc = a.scores + (int64_t)b * a.score_stride;
  uint32_t L;
  bool fast = sample_bound(sc, T, k, sh.r, &L);
  if (fast) {
    const int32_t nwords = (T + 31) / 32;
    for (int32_t w = tid; w < nwords; w += kTopkThreads) sh.bits[w] = 0;
    // one pass: wave w appends its candidates to segment w
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int32_t nblk = (T + kTopkThreads - 1) / kTopkThreads;
    const int32_t seg0 = wave * kSeg;
    uint32_t cnt = 0;  // wave-uniform
    for (int32_t j0 = 0; j0 < nblk; j0 += kGrp) {
      float v[kGrp];
#pragma unroll
      for (int g = 0; g < kGrp; g++) {
        const int32_t i = (j0 + g) * kTopkThreads + tid;
        v[g] = i < T ? sc[i] : 0.f;
      }
#pragma unroll
      for (int g = 0; g < kGrp; g++) {
        const int32_t i = (j0 + g) * kTopkThreads + tid;
        const uint32_t key = score_key(v[g]);
        const bool c = i < T && key >= L;
        const uint64_t m = __ballot(c);
        const uint32_t o = cnt + (uint32_t)__popcll(m & below);
        if (c && o < (uint32_t)kSeg) {
          sh.cand_key[seg0 + o] = key;
          sh.cand_pos[seg0 + o] = i;
        }
        cnt += (uint32_t)__popcll(m);
      }
    }
    if (lane == 0) sh.seg[wave] = cnt;
    __syncthreads();
    uint32_t ncand = 0;
    bool full = false;
#pragma unroll
    for (int w = 0; w < kTopkWaves; w++) {
      ncand += sh.seg[w];
      full |= sh.seg[w] > (uint32_t)kSeg;
    }
    fast = ncand >= k && !full;
  }
  if (fast) {
    // this wave's segment: lane l holds entries l, l + 64, ...
    const uint32_t n_seg = sh.seg[wave];
    const int ne = (int)((n_seg + 63) / 64);  // wave-uniform
    uint32_t key[kSegLane];
    int32_t pos[kSegLane];
    bool ok[kSegLane];
#pragma unroll
    for (int e = 0; e < kSegLane; e++) {
      const uint32_t x = lane + 64 * e;
      ok[e] = x < n_seg;
      key[e] = ok[e] ? sh.cand_key[wave * kSeg + x] : 0u;
      pos[e] = ok[e] ? sh.cand_pos[wave * kSeg + x] : 0;
    }
    uint32_t kmax = 0;
#pragma unroll
    for (int e = 0; e < kSegLane; e++) kmax = max(kmax, key[e]);
    kmax = block_max_u32(kmax, sh.r.wave);
    uint32_t K, last;
    candidate_cut<kSegLane>(key, pos, ok, ne, k, L, kmax, sh.r, &K, &last);
#pragma unroll
    for (int e = 0; e < kSegLane; e++) {
      if (ok[e] && (key[e] > K || (key[e] == K && (uint32_t)pos[e] <= last)))
        atomicOr(&sh.bits[pos[e] >> 5], 1u << (pos[e] & 31));
    }
    __syncthreads();
    // positions in increasing order: thread t scans words [8t, 8t + 8)
    const int32_t nwords = (T + 31) / 32;
    uint32_t wv[8], nb = 0;
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const int32_t w = 8 * tid + e;
      wv[e] = w < nwords ? sh.bits[w] : 0u;
      nb += (uint32_t)__popc(wv[e]);
    }
    uint32_t o = block_scan(nb, sh.r.wave) - nb;
#pragma unroll
    for (int e = 0; e < 8; e++) {
      uint32_t x = wv[e];
      while (x) {
        const int bit = __ffs(x) - 1;
        out[o++] = (8 * tid + e) * 32 + bit;
        x &= x - 1;
      }
    }
  } else {
    select_general(sc, T, k, out, sh);
  }
  if (tid == 0) a.counts[b] = a.k;
}

// ------------------------------------------------------------------ split top-k
// The same selection with the candidate pass spread over work groups of
// kSplitChunk positions each (several per sequence), for batches too small
// to fill the chip with one work group per sequence:
//  * topk_cand_kernel, work group (chunk c, sequence b): L = sample_bound
//    (every chunk of a sequence computes the same L), then the positions of
//    the chunk whose keys are >= L, in increasing order, into the chunk's
//    region of the candidate list and their count into ccount; chunk 0 also
//    records whether the fast path applies;
//  * topk_pick_kernel, work group b: the chunks' candidates concatenated in
//    LDS (in position order), kCandCap at most, thread t holding candidates
//    [12 t, 12 t + 12); K and last as above (candidate_cut); the selected
//    positions written in order by a scan over the threads.  Fewer than k or
//    more than kCandCap candidates, or no fast path: select_general.
constexpr int kSplitChunk = 2048;                        // positions per candidate work group
constexpr int kSplitMaxChunks = kFastMaxT / kSplitChunk;  // 128
constexpr int kPickLane = kCandCap / kTopkThreads;       // 12

struct TopkSplit {
  int32_t* cand;    // [B][nch * kSplitChunk] candidate positions
  uint32_t* ckey;   // [B][nch * kSplitChunk] their keys
  int32_t* ccount;  // [B][nch] candidates per chunk
  int32_t* fast;    // [B] the fast path applies (written by chunk 0)
  int32_t nch;      // chunks per sequence: those of the longest sequence the fast path takes
};

__device__ inline int32_t topk_len(const TopkArgs& a, int32_t b) {
  const int32_t T = a.seq_lens[b];
  return T < 0 ? 0 : (T > a.score_stride ? a.score_stride : T);
}

__global__ __launch_bounds__(kTopkThreads) void topk_cand_kernel(TopkArgs a, TopkSplit sp) {
  __shared__ RadixShared sh;
  __shared__ uint32_t s_cnt[kSplitChunk / kTopkThreads][kTopkWaves];
  const int32_t c = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t T = topk_len(a, b);
  const int32_t p0 = c * kSplitChunk;
  if (T <= a.k || p0 >= T) return;
  const float* sc = a.scores + (int64_t)b * a.score_stride;
  // the chunk's keys (position p0 + 1024 e + tid), requested with the sample's
  constexpr int E = kSplitChunk / kTopkThreads;
  float v[E];
#pragma unroll
  for (int e = 0; e < E; e++) {
    const int32_t i = p0 + kTopkThreads * e + tid;
    v[e] = i < T ? sc[i] : 0.f;
  }
  uint32_t L;
  const bool fast = sample_bound(sc, T, (uint32_t)a.k, sh, &L);
  if (c == 0 && tid == 0) sp.fast[b] = fast ? 1 : 0;
  if (!fast) return;
  // wave w's candidates of round e go after those of the rounds before and of
  // the waves before it in round e
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  bool cnd[E];
  uint32_t kv[E];
  uint32_t rank[E];  // among the wave's candidates of its round
#pragma unroll
  for (int e = 0; e < E; e++) {
    const int32_t i = p0 + kTopkThreads * e + tid;
    kv[e] = score_key(v[e]);
    cnd[e] = i < T && kv[e] >= L;
    const uint64_t m = __ballot(cnd[e]);
    rank[e] = (uint32_t)__popcll(m & below);
    if (lane == 0) s_cnt[e][wave] = (uint32_t)__popcll(m);
  }
  __syncthreads();
  const int64_t base = ((int64_t)b * sp.nch + c) * kSplitChunk;
  uint32_t total = 0;  // candidates of the rounds before e, then of the chunk
#pragma unroll
  for (int e = 0; e < E; e++) {
    uint32_t waves_before = 0, round = 0;
#pragma unroll
    for (int w = 0; w < kTopkWaves; w++) {
      const uint32_t n = s_cnt[e][w];
      waves_before += w < wave ? n : 0u;
      round += n;
    }
    if (cnd[e]) {
      sp.cand[base + total + waves_before + rank[e]] = p0 + kTopkThreads * e + tid;
      sp.ckey[base + total + waves_before + rank[e]] = kv[e];
    }
    total += round;
  }
  if (tid == 0) sp.ccount[(int64_t)b * sp.nch + c] = (int32_t)total;
}

struct PickShared {
  uint32_t cand_key[kCandCap];
  int32_t cand_pos[kCandCap];
  uint32_t hist[kBins];  // radix histogram (general path)
  RadixShared r;
  uint32_t first[kSplitMaxChunks + 1];  // first candidate of each chunk
};

__global__ __launch_bounds__(kTopkThreads) void topk_pick_kernel(TopkArgs a, TopkSplit sp) {
  __shared__ PickShared sh;
  const int32_t b = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t T = topk_len(a, b);
  int32_t* out = a.indices + (int64_t)b * a.index_stride;
  const uint32_t k = (uint32_t)a.k;
  if (T <= a.k) {  // everything is selected
    for (int32_t i = tid; i < T; i += kTopkThreads) out[i] = i;
    if (tid == 0) a.counts[b] = T;
    return;
  }
  const float* sc = a.scores + (int64_t)b * a.score_stride;
  bool fast = sp.fast[b] != 0;  // uniform
  if (fast) {
    const int32_t nc = (T + kSplitChunk - 1) / kSplitChunk;  // <= nch <= 128 on the fast path
    if (tid < 64) {  // wave 0: chunks 2 l and 2 l + 1, scanned across the lanes
      const int32_t c0 = 2 * tid, c1 = 2 * tid + 1;
      const uint32_t n0 = c0 < nc ? (uint32_t)sp.ccount[(int64_t)b * sp.nch + c0] : 0u;
      const uint32_t n1 = c1 < nc ? (uint32_t)sp.ccount[(int64_t)b * sp.nch + c1] : 0u;
      const uint32_t incl = wave_incl_scan(n0 + n1);
      const uint32_t f0 = incl - n0 - n1;
      if (c0 <= nc) sh.first[c0] = f0;
      if (c1 <= nc) sh.first[c1] = f0 + n0;  // entry nc: the total
      if (c1 + 1 == nc) sh.first[nc] = incl;  // (nc = 128: past the last lane's pair)
    }
    __syncthreads();
    const uint32_t n = sh.first[nc];
    fast = n >= k && n <= (uint32_t)kCandCap;
    if (fast) {
      // the chunks' lists concatenated in LDS (position order): G threads a
      // chunk, each copying every G-th candidate, eight requests in flight
      const int lg = 32 - __clz((uint32_t)(nc - 1));  // ceil(log2(nc)), nc >= 1
      const int G = kTopkThreads >> lg;
      const int32_t c = tid / G, j = tid % G;
      if (c < nc) {
        const uint32_t f = sh.first[c], m = sh.first[c + 1] - f;
        const int64_t src = ((int64_t)b * sp.nch + c) * kSplitChunk;
        for (uint32_t i0 = (uint32_t)j; i0 < m; i0 += 8u * G) {
          int32_t pv[8];
          uint32_t kv[8];
#pragma unroll
          for (int u = 0; u < 8; u++) {
            const uint32_t i = i0 + (uint32_t)(u * G);
            pv[u] = i < m ? sp.cand[src + i] : 0;
            kv[u] = i < m ? sp.ckey[src + i] : 0u;
          }
#pragma unroll
          for (int u = 0; u < 8; u++) {
            const uint32_t i = i0 + (uint32_t)(u * G);
            if (i < m) {
              sh.cand_pos[f + i] = pv[u];
              sh.cand_key[f + i] = kv[u];
            }
          }
        }
      }
      __syncthreads();
      // candidates 12 t .. 12 t + 11, in position order
      uint32_t key[kPickLane];
      int32_t pos[kPickLane];
      bool ok[kPickLane];
      uint32_t nmin = 0, kmax = 0;  // ~least and largest key
#pragma unroll
      for (int e = 0; e < kPickLane; e++) {
        const uint32_t x = (uint32_t)(kPickLane * tid + e);
        ok[e] = x < n;
        pos[e] = ok[e] ? sh.cand_pos[x] : 0;
        key[e] = ok[e] ? sh.cand_key[x] : 0u;
        nmin = max(nmin, ok[e] ? ~key[e] : 0u);
        kmax = max(kmax, key[e]);
      }
      block_max2_u32(nmin, kmax, sh.r.wave);
      // every candidate is >= the bound; the least candidate key is one too
      uint32_t K, last;
      candidate_cut<kPickLane>(key, pos, ok, kPickLane, k, ~nmin, kmax, sh.r, &K, &last);
      bool sel[kPickLane];
      uint32_t ns = 0;
#pragma unroll
      for (int e = 0; e < kPickLane; e++) {
        sel[e] = ok[e] && (key[e] > K || (key[e] == K && (uint32_t)pos[e] <= last));
        ns += sel[e];
      }
      uint32_t o = block_scan(ns, sh.r.wave) - ns;
#pragma unroll
      for (int e = 0; e < kPickLane; e++)
        if (sel[e]) out[o++] = pos[e];
    }
  }
  if (!fast) select_general(sc, T, k, out, sh);
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

static int32_t split_chunks(int32_t score_stride) {
  return (std::min(score_stride, kFastMaxT) + kSplitChunk - 1) / kSplitChunk;
}

size_t topk_split_ws_bytes(int32_t B, int32_t score_stride) {
  const size_t nch = (size_t)split_chunks(score_stride);
  return (size_t)B * (2 * nch * kSplitChunk + nch + 1) * sizeof(int32_t);
}

hipError_t launch_topk_split(const float* scores, int32_t score_stride, const int32_t* seq_lens,
                             int32_t B, int32_t k, int32_t* indices, int32_t index_stride,
                             int32_t* counts, void* workspace, hipStream_t s) {
  TopkArgs a{scores, score_stride, seq_lens, k, indices, index_stride, counts};
  TopkSplit sp;
  int32_t* w = static_cast<int32_t*>(workspace);
  sp.nch = split_chunks(score_stride);  // longer sequences go the general way
  sp.cand = w;
  sp.ckey = reinterpret_cast<uint32_t*>(w + (size_t)B * sp.nch * kSplitChunk);
  sp.ccount = w + 2 * (size_t)B * sp.nch * kSplitChunk;
  sp.fast = sp.ccount + (size_t)B * sp.nch;
  hipLaunchKernelGGL(topk_cand_kernel, dim3(sp.nch, B), dim3(kTopkThreads), 0, s, a, sp);
  hipLaunchKernelGGL(topk_pick_kernel, dim3(B), dim3(kTopkThreads), 0, s, a, sp);
  return hipGetLastError();
}

}  // namespace mla
