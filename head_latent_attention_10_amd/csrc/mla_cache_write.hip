// Latent-cache writer (gfx950): one new token per sequence appended to the
// paged cache.
//
// "TransMLA: Multi-Head Latent Attention Is All You Need", the MLA structure
// after conversion: the cached latent is a down projection of the hidden
// state and the decoupled RoPE key a second projection rotated to the token's
// position.  "TPLA: Tensor Parallel Latent Attention ...", "RMSNorm Slicing"
// (Eqs. 8-9): the latent is RMS-normalised before attention.  Per sequence b
// with position t = positions[b]:
//   y = [W_DKV; W_KR] x_b                       (d_latent + d_rope values)
//   c = y[:d_latent] / sqrt(mean(y[:d_latent]^2) + eps) * gamma
//   k = RoPE(y[d_latent:], t): pair i turned by t * base^(-2i / d_rope)
// stored at slot (block_table[b][t / P], t % P); an fp8 latent row is stored
// as E4M3FN codes of c / s with s = max|c| / 448 (fp32, ties to even).
//
// Projection: a matrix-core kernel (bf16 x and weights) or a generic kernel
// writes fp32 partial sums over KC chunks of the model dimension; the finish
// kernel (one work group per sequence) adds them in a fixed order, so the
// result is deterministic, then normalises, rotates, encodes and stores.
#include <algorithm>

#include "mla_mfma_util.hpp"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWrThreads = 256;   // quantiser, generic projection
constexpr int kFinThreads = 1024; // finish: one thread per value of a row (up to 1024)
constexpr int kProjWaves = 4;     // waves of a projection work group
constexpr int kProjBatch = 8;     // k-steps a wave loads before its products
constexpr int kMaxChunks = 32;    // K chunks of the direct-load projection
constexpr int kStageK = 512;      // model-dimension chunk of the LDS-staged projection
constexpr int kStageRow = kStageK * 2 + 16;  // LDS bytes per staged weight row (16 B pad)

// ------------------------------------------------------------------ E4M3FN
// The OCP E4M3FN code of y, |y| <= 448 (callers clamp), rounded to nearest
// with ties to even.  Every step is exact in fp32: scaling by powers of two,
// 2m - 1 for m in [0.5, 1), and rintf (round to nearest even).
__device__ inline uint32_t e4m3_encode(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 31) << 7;
  const float a = fabsf(y);
  uint32_t code;
  if (a < 0.015625f) {                       // below 2^-6: steps of 2^-9
    code = (uint32_t)rintf(a * 512.0f);      // 8 is the smallest normal, 0x08
  } else {
    int e;
    const float m = frexpf(a, &e);           // a = m 2^e, m in [0.5, 1)
    uint32_t q = (uint32_t)rintf((2.0f * m - 1.0f) * 8.0f);
    int be = e - 1 + 7;                      // biased exponent of 2^(e-1)
    if (q == 8) {
      q = 0;
      be += 1;
    }
    code = ((uint32_t)be << 3) | q;
  }
  return code | sign;
}

// Block reductions over NT threads (s_red holds one value per wave).
template <int NT>
__device__ inline float block_sum(float v, float* s_red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < NT / 64; i++) t += s_red[i];
  return t;
}

template <int NT>
__device__ inline float block_max(float v, float* s_red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = s_red[0];
#pragma unroll
  for (int i = 1; i < NT / 64; i++) t = fmaxf(t, s_red[i]);
  return t;
}

// Quantise the row vals[0..d) (LDS) into codes/scale; every thread of the
// block (NT threads) calls it.
template <int NT>
__device__ inline void quantize_row(const float* vals, int32_t d, uint8_t* codes, float* scale,
                                    float* s_red) {
  float am = 0.f;
  for (int i = threadIdx.x; i < d; i += NT) am = fmaxf(am, fabsf(vals[i]));
  am = block_max<NT>(am, s_red);
  const float s = am / 448.0f;  // IEEE division
  if (threadIdx.x == 0) *scale = s;
  for (int i = threadIdx.x; i < d; i += NT) {
    uint32_t c = 0;
    if (s > 0.f) c = e4m3_encode(fminf(fmaxf(vals[i] / s, -448.0f), 448.0f));
    codes[i] = (uint8_t)c;
  }
}

// ------------------------------------------------------------------ projection
// Matrix-core partial sums: work group = (32 output columns, K chunk, 64 rows
// of the batch); its four waves take consecutive quarters of the chunk's
// k-steps (so a wave's loads sweep whole lines of each weight row) and add
// their products in LDS.  Output column n < d_c is row n of W_DKV, else row
// n - d_c of W_KR; both operands are read straight from global memory (a lane
// reads 16 contiguous bytes of one x row and one weight row per k-step).
//   part[kc][b][n] = sum over the chunk's k of x[b][k] W[n][k]
__global__ __launch_bounds__(64 * kProjWaves) void writer_proj_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W_DKV,
    const uint16_t* __restrict__ W_KR, float* __restrict__ part, int32_t B, int32_t d_model,
    int32_t d_c, int32_t d_r, int32_t chunks) {
  __shared__ float s_acc[kProjWaves > 1 ? kProjWaves - 1 : 1][2][16][64];
  const int32_t N = d_c + d_r;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, r = lane & 31;
  const int32_t n = blockIdx.x * 32 + r;
  const int32_t kc = blockIdx.y, b0 = blockIdx.z * 64;
  const int32_t nks = d_model / 16;
  const int32_t c_lo = (int32_t)(((int64_t)nks * kc) / chunks);
  const int32_t c_hi = (int32_t)(((int64_t)nks * (kc + 1)) / chunks);
  const int32_t s_lo = c_lo + ((c_hi - c_lo) * wave) / kProjWaves;
  const int32_t s_hi = c_lo + ((c_hi - c_lo) * (wave + 1)) / kProjWaves;
  const uint16_t* wrow = n < d_c ? W_DKV + (int64_t)n * d_model : W_KR + (int64_t)(n - d_c) * d_model;
  const bool two = b0 + 32 < B;  // a second 32-row tile has rows
  const int32_t ra = min(b0 + r, B - 1), rb = min(b0 + 32 + r, B - 1);
  const uint16_t* xa = x + (int64_t)ra * d_model;
  const uint16_t* xb = x + (int64_t)rb * d_model;
  f32x16 acc0 = f32x16{}, acc1 = f32x16{};
  for (int32_t s0 = s_lo; s0 < s_hi; s0 += kProjBatch) {
    bf16x8 w[kProjBatch], p[kProjBatch], q[kProjBatch];
#pragma unroll
    for (int i = 0; i < kProjBatch; i++) {
      const int32_t s = min(s0 + i, s_hi - 1);
      const int32_t k = 16 * s + 8 * g;
      w[i] = *reinterpret_cast<const bf16x8*>(wrow + k);
      p[i] = *reinterpret_cast<const bf16x8*>(xa + k);
      q[i] = *reinterpret_cast<const bf16x8*>(xb + k);
    }
#pragma unroll
    for (int i = 0; i < kProjBatch; i++) {
      if (s0 + i >= s_hi) break;  // uniform
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(p[i], w[i], acc0, 0, 0, 0);
      if (two) acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q[i], w[i], acc1, 0, 0, 0);
    }
  }
  // add the four waves' products (fixed order) and store the chunk's partial
  if (wave > 0) {
#pragma unroll
    for (int j = 0; j < 16; j++) {
      s_acc[wave - 1][0][j][lane] = acc0[j];
      s_acc[wave - 1][1][j][lane] = acc1[j];
    }
  }
  __syncthreads();
  if (wave == 0 && n < N) {
#pragma unroll
    for (int j = 0; j < 16; j++) {
      float v0 = acc0[j], v1 = acc1[j];
#pragma unroll
      for (int w2 = 0; w2 < kProjWaves - 1; w2++) {
        v0 += s_acc[w2][0][j][lane];
        v1 += s_acc[w2][1][j][lane];
      }
      // D[m = row][n]: lane holds column n, rows 8(j/4) + 4g + j%4
      const int32_t m = 8 * (j >> 2) + 4 * g + (j & 3);
      if (b0 + m < B) part[((int64_t)kc * B + b0 + m) * N + n] = v0;
      if (b0 + 32 + m < B) part[((int64_t)kc * B + b0 + 32 + m) * N + n] = v1;
    }
  }
}

// The same partial sums with the weights staged in LDS: chunk kc is 512
// model dimensions, so each of a work group's 32 weight rows contributes 1 KiB
// contiguous, brought in by one direct-to-LDS load (every load instruction
// reads 1 KiB of one row; operand-layout loads straight from global memory
// read 32 bytes of each of 32 rows 14 KiB apart, which streams at about
// 1 TB/s).  Rows are 16 bytes apart in LDS beyond their 1 KiB, which spreads
// the operand reads over the banks.  Each wave then takes 8 of the chunk's 32
// k-steps; x comes from global memory (small, L2-resident).
__global__ __launch_bounds__(64 * kProjWaves) void writer_proj_lds_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W_DKV,
    const uint16_t* __restrict__ W_KR, float* __restrict__ part, int32_t B, int32_t d_model,
    int32_t d_c, int32_t d_r) {
  __shared__ __attribute__((aligned(16))) char s_w[32 * kStageRow];
  __shared__ float s_acc[kProjWaves - 1][2][16][64];
  const int32_t N = d_c + d_r;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, r = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: the loads' LDS base
  const int32_t n0 = blockIdx.x * 32, kc = blockIdx.y, b0 = blockIdx.z * 64;
  const int32_t k0 = kc * kStageK;
  // rows n0 + 8 wave .. + 7 of the tile: one 1 KiB load each
#pragma unroll
  for (int i = 0; i < 32 / kProjWaves; i++) {
    const int32_t rl = (32 / kProjWaves) * wave + i;
    const int32_t n = n0 + rl;
    const uint16_t* row = n < d_c ? W_DKV + (int64_t)n * d_model : W_KR + (int64_t)(n - d_c) * d_model;
    dma16(row + k0 + 8 * lane, (lds_t*)s_w + rl * kStageRow);
  }
  const bool two = b0 + 32 < B;
  const int32_t ra = min(b0 + r, B - 1), rb = min(b0 + 32 + r, B - 1);
  const uint16_t* xa = x + (int64_t)ra * d_model + k0;
  const uint16_t* xb = x + (int64_t)rb * d_model + k0;
  constexpr int kSteps = kStageK / 16 / kProjWaves;  // k-steps per wave
  bf16x8 p[kSteps], q[kSteps];
#pragma unroll
  for (int i = 0; i < kSteps; i++) {
    const int k = 16 * (kSteps * wave + i) + 8 * g;
    p[i] = *reinterpret_cast<const bf16x8*>(xa + k);
    q[i] = *reinterpret_cast<const bf16x8*>(xb + k);
  }
  wait_vmcnt<0>();
  __syncthreads();
  f32x16 acc0 = f32x16{}, acc1 = f32x16{};
#pragma unroll
  for (int i = 0; i < kSteps; i++) {
    const int s = kSteps * wave + i;
    const bf16x8 w = *reinterpret_cast<const bf16x8*>(s_w + r * kStageRow + 32 * s + 16 * g);
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(p[i], w, acc0, 0, 0, 0);
    if (two) acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q[i], w, acc1, 0, 0, 0);
  }
  if (wave > 0) {
#pragma unroll
    for (int j = 0; j < 16; j++) {
      s_acc[wave - 1][0][j][lane] = acc0[j];
      s_acc[wave - 1][1][j][lane] = acc1[j];
    }
  }
  __syncthreads();
  const int32_t n = n0 + r;
  if (wave == 0 && n < N) {
#pragma unroll
    for (int j = 0; j < 16; j++) {
      float v0 = acc0[j], v1 = acc1[j];
#pragma unroll
      for (int w2 = 0; w2 < kProjWaves - 1; w2++) {
        v0 += s_acc[w2][0][j][lane];
        v1 += s_acc[w2][1][j][lane];
      }
      const int32_t m = 8 * (j >> 2) + 4 * g + (j & 3);
      if (b0 + m < B) part[((int64_t)kc * B + b0 + m) * N + n] = v0;
      if (b0 + 32 + m < B) part[((int64_t)kc * B + b0 + 32 + m) * N + n] = v1;
    }
  }
}

// Generic projection (any x/weight dtype): thread = one output column of one
// sequence, one chunk (part[0]).
template <int XT, int WT>
__global__ __launch_bounds__(kWrThreads) void writer_proj_simt_kernel(
    const void* __restrict__ x, const void* __restrict__ W_DKV, const void* __restrict__ W_KR,
    float* __restrict__ part, int32_t B, int32_t d_model, int32_t d_c, int32_t d_r) {
  const int32_t N = d_c + d_r;
  const int32_t b = blockIdx.y, n = blockIdx.x * kWrThreads + threadIdx.x;
  if (n >= N) return;
  const void* W = n < d_c ? W_DKV : W_KR;
  const int64_t row = (int64_t)(n < d_c ? n : n - d_c) * d_model;
  float acc = 0.f;
  for (int32_t k = 0; k < d_model; k++)
    acc = fmaf(load_elem<XT>(x, (int64_t)b * d_model + k), load_elem<WT>(W, row + k), acc);
  part[(int64_t)b * N + n] = acc;
}

// ------------------------------------------------------------------ finish
struct FinishArgs {
  const float* part;
  const void* gamma;
  const int32_t* positions;
  const int32_t* block_table;
  void* c_kv;
  float* c_kv_scale;
  void* k_rope;
  int32_t B, d_c, d_r, chunks, P, max_blocks, num_blocks;
  float eps, base;
};

template <int WT, int CT, int RT>
__global__ __launch_bounds__(kFinThreads) void writer_finish_kernel(FinishArgs f) {
  extern __shared__ float s_y[];  // [d_c + d_r]
  __shared__ float s_red[kFinThreads / 64];
  const int32_t b = blockIdx.x, N = f.d_c + f.d_r;
  // the position and table entry first, so that their loads overlap the
  // partials' (which do not depend on them)
  const int32_t t = f.positions[b];
  const bool in_row = t >= 0 && t / f.P < f.max_blocks;
  const int32_t blk = in_row ? f.block_table[(int64_t)b * f.max_blocks + t / f.P] : -1;
  // the chunk partials, sixteen loads in flight before any is added (the sum
  // keeps chunk order)
  for (int32_t i = threadIdx.x; i < N; i += kFinThreads) {
    float v = 0.f;
    for (int32_t k0 = 0; k0 < f.chunks; k0 += 16) {
      float u[16];
#pragma unroll
      for (int j = 0; j < 16; j++)
        u[j] = k0 + j < f.chunks ? f.part[((int64_t)(k0 + j) * f.B + b) * N + i] : 0.f;
#pragma unroll
      for (int j = 0; j < 16; j++) v += u[j];
    }
    s_y[i] = v;
  }
  if (blk < 0 || blk >= f.num_blocks) return;  // no slot: nothing to write
  const int64_t slot = (int64_t)blk * f.P + t % f.P;
  __syncthreads();
  // RMSNorm of the latent
  float ss = 0.f;
  for (int32_t i = threadIdx.x; i < f.d_c; i += kFinThreads) ss = fmaf(s_y[i], s_y[i], ss);
  ss = block_sum<kFinThreads>(ss, s_red);
  const float inv = 1.0f / sqrtf(ss / (float)f.d_c + f.eps);
  for (int32_t i = threadIdx.x; i < f.d_c; i += kFinThreads)
    s_y[i] = s_y[i] * inv * load_elem<WT>(f.gamma, i);
  __syncthreads();
  if constexpr (CT == MLA_FP8_E4M3) {
    quantize_row<kFinThreads>(s_y, f.d_c, static_cast<uint8_t*>(f.c_kv) + slot * f.d_c, f.c_kv_scale + slot, s_red);
  } else {
    for (int32_t i = threadIdx.x; i < f.d_c; i += kFinThreads)
      store_elem<CT>(f.c_kv, slot * f.d_c + i, s_y[i]);
  }
  // RoPE of the rope key.  The angle t * theta reaches 10^5 rad and more, so
  // it is formed in fp64 and reduced by 2 pi there (Cody-Waite: 2 pi split
  // into two 26-bit parts and a tail, so k times each part is exact for
  // k < 2^27); the remainder's sine and cosine are taken in fp32 and the
  // rotation is done in fp32.
  for (int32_t i = threadIdx.x; i < f.d_r / 2; i += kFinThreads) {
    const double ang = (double)t * exp2(-2.0 * (double)i / (double)f.d_r * log2((double)f.base));
    constexpr double kTwoPi0 = 0x1.921fb5p+2;           // 2 pi, leading 26 bits
    constexpr double kTwoPi1 = 0x1.110b46p-24;          // next 26 bits
    constexpr double kTwoPi2 = 0x1.1a62633145c07p-52;   // the rest
    const double k = rint(ang * 0x1.45f306dc9c883p-3);  // ang / (2 pi)
    const float red = (float)(((ang - k * kTwoPi0) - k * kTwoPi1) - k * kTwoPi2);
    float sn, cs;
    sincosf(red, &sn, &cs);
    const float xv = s_y[f.d_c + 2 * i], yv = s_y[f.d_c + 2 * i + 1];
    store_elem<RT>(f.k_rope, slot * f.d_r + 2 * i, xv * cs - yv * sn);
    store_elem<RT>(f.k_rope, slot * f.d_r + 2 * i + 1, xv * sn + yv * cs);
  }
}

// ------------------------------------------------------------------ quantiser
__global__ __launch_bounds__(kWrThreads) void quantize_rows_kernel(const float* __restrict__ x,
                                                                   int32_t d, uint8_t* codes,
                                                                   float* scales) {
  extern __shared__ float s_row[];
  __shared__ float s_red[kWrThreads / 64];
  const int64_t row = blockIdx.x;
  for (int32_t i = threadIdx.x; i < d; i += kWrThreads) s_row[i] = x[row * d + i];
  __syncthreads();
  quantize_row<kWrThreads>(s_row, d, codes + row * d, scales + row, s_red);
}

}  // namespace

// Chunks of the model dimension the matrix-core projection splits into: about
// 32, fewer when the batch is large (the partials are KC x B x N fp32).
int32_t writer_chunks(const mla_cache_write_params& p) {
  if (!writer_mfma_ok(p)) return 1;
  if (p.d_model % kStageK == 0) return p.d_model / kStageK;
  int32_t kc = kMaxChunks;
  while (kc > 1 && (int64_t)kc * p.batch > 1024) kc /= 2;
  return std::min<int32_t>(kc, p.d_model / 16);
}

bool writer_mfma_ok(const mla_cache_write_params& p) {
  return p.x_dtype == MLA_BF16 && p.weight_dtype == MLA_BF16 && p.d_model % 16 == 0 &&
         (p.d_latent + p.d_rope) % 32 == 0;
}

hipError_t launch_cache_write(const mla_cache_write_params& p, const void* x, const void* W_DKV,
                              const void* gamma, const void* W_KR, const int32_t* positions,
                              const int32_t* block_table, void* c_kv, float* c_kv_scale,
                              void* k_rope, float* part, hipStream_t s) {
  const int32_t N = p.d_latent + p.d_rope;
  const int32_t chunks = writer_chunks(p);
  if (writer_mfma_ok(p) && p.d_model % kStageK == 0) {
    const dim3 grid(N / 32, chunks, (p.batch + 63) / 64);
    hipLaunchKernelGGL(writer_proj_lds_kernel, grid, dim3(64 * kProjWaves), 0, s,
                       static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(W_DKV),
                       static_cast<const uint16_t*>(W_KR), part, p.batch, p.d_model, p.d_latent,
                       p.d_rope);
  } else if (writer_mfma_ok(p)) {
    const dim3 grid(N / 32, chunks, (p.batch + 63) / 64);
    hipLaunchKernelGGL(writer_proj_mfma_kernel, grid, dim3(64 * kProjWaves), 0, s,
                       static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(W_DKV),
                       static_cast<const uint16_t*>(W_KR), part, p.batch, p.d_model, p.d_latent,
                       p.d_rope, chunks);
  } else {
    const dim3 grid((N + kWrThreads - 1) / kWrThreads, p.batch);
#define MLA_PROJ(XT, WT)                                                                        \
  hipLaunchKernelGGL((writer_proj_simt_kernel<XT, WT>), grid, dim3(kWrThreads), 0, s, x, W_DKV, \
                     W_KR, part, p.batch, p.d_model, p.d_latent, p.d_rope)
    if (p.x_dtype == MLA_F32 && p.weight_dtype == MLA_F32) MLA_PROJ(MLA_F32, MLA_F32);
    else if (p.x_dtype == MLA_F32) MLA_PROJ(MLA_F32, MLA_BF16);
    else if (p.weight_dtype == MLA_F32) MLA_PROJ(MLA_BF16, MLA_F32);
    else MLA_PROJ(MLA_BF16, MLA_BF16);
#undef MLA_PROJ
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  FinishArgs f;
  f.part = part;
  f.gamma = gamma;
  f.positions = positions;
  f.block_table = block_table;
  f.c_kv = c_kv;
  f.c_kv_scale = c_kv_scale;
  f.k_rope = k_rope;
  f.B = p.batch;
  f.d_c = p.d_latent;
  f.d_r = p.d_rope;
  f.chunks = chunks;
  f.P = p.page_size;
  f.max_blocks = p.max_blocks_per_seq;
  f.num_blocks = p.num_blocks;
  f.eps = p.rms_eps;
  f.base = p.rope_base;
  const size_t lds = (size_t)N * sizeof(float);
#define MLA_FIN(WT, CT, RT) \
  hipLaunchKernelGGL((writer_finish_kernel<WT, CT, RT>), dim3(p.batch), dim3(kFinThreads), lds, s, f)
  const bool wf = p.weight_dtype == MLA_F32, rf = p.rope_dtype == MLA_F32;
  switch (p.cache_dtype) {
    case MLA_F32:
      if (wf) { if (rf) MLA_FIN(MLA_F32, MLA_F32, MLA_F32); else MLA_FIN(MLA_F32, MLA_F32, MLA_BF16); }
      else { if (rf) MLA_FIN(MLA_BF16, MLA_F32, MLA_F32); else MLA_FIN(MLA_BF16, MLA_F32, MLA_BF16); }
      break;
    case MLA_BF16:
      if (wf) { if (rf) MLA_FIN(MLA_F32, MLA_BF16, MLA_F32); else MLA_FIN(MLA_F32, MLA_BF16, MLA_BF16); }
      else { if (rf) MLA_FIN(MLA_BF16, MLA_BF16, MLA_F32); else MLA_FIN(MLA_BF16, MLA_BF16, MLA_BF16); }
      break;
    default:
      if (wf) { if (rf) MLA_FIN(MLA_F32, MLA_FP8_E4M3, MLA_F32); else MLA_FIN(MLA_F32, MLA_FP8_E4M3, MLA_BF16); }
      else { if (rf) MLA_FIN(MLA_BF16, MLA_FP8_E4M3, MLA_F32); else MLA_FIN(MLA_BF16, MLA_FP8_E4M3, MLA_BF16); }
      break;
  }
#undef MLA_FIN
  return hipGetLastError();
}

hipError_t launch_quantize_rows(const float* x, int64_t rows, int32_t d, uint8_t* codes,
                                float* scales, hipStream_t s) {
  hipLaunchKernelGGL(quantize_rows_kernel, dim3((uint32_t)rows), dim3(kWrThreads),
                     (size_t)d * sizeof(float), s, x, d, codes, scales);
  return hipGetLastError();
}

}  // namespace mla
