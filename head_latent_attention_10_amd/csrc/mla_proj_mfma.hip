// Matrix-core query absorption and value up-projection (bf16 weights, gfx950).
//
// Both are per-head products with a short sequence dimension:
//   absorb:  q_lat[b, i, c] = sum_n q[b, i, n] W_UK[i, n, c]   (K = d_nope)
//   up-proj: out[b, i, v]   = sum_c o_lat[b, i, c] W_UV[i, v, c] (K = d_latent)
// computed with MFMA bf16 (fp32 accumulation), sequences on M (padded with
// zero rows).  For d_v = 128 the up-projection can also take its rows straight
// from the bf16 split partials (merge + up-projection in one launch).
#include "mla_kernels.hpp"
#include "mla_merge.hpp"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_t;

constexpr int kLat = 512;             // latent width of the fast path
constexpr int kUpKs = kLat / 16;      // k-steps of the up-projection

// ------------------------------------------------------------------ up-projection
// Work group = (head, 64 rows of W_UV), two waves of 32 rows.  Each wave keeps
// its 32 W_UV rows (32 KiB) in registers as the MFMA B operand.  The o_lat
// rows of 32 sequences at a time are staged in LDS, split into a bf16 high
// part and a bf16 remainder (16-byte chunks XOR-swizzled by the row); both
// are multiplied and the products summed in fp32, which keeps about 16
// significant bits of o_lat.  The first o_lat rows are loaded before the
// W_UV rows, so that (the load counter being in order) their conversion does
// not wait for W_UV, and the products run as four independent accumulator
// chains.
constexpr int kUpWaves = 2;

__device__ inline int up_swz(int row) { return row & 15; }

template <int OT>
__global__ __launch_bounds__(64 * kUpWaves) void up_project_mfma_kernel(
    const float* __restrict__ o_lat, const uint16_t* __restrict__ W_UV, void* __restrict__ out,
    int32_t B, int32_t h, int32_t d_v) {
  __shared__ __attribute__((aligned(16))) char os[2][32 * kLat * 2];  // high, low parts
  const int32_t head = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, r = lane & 31;
  const int32_t v0 = (blockIdx.y * kUpWaves + wave) * 32;
  const bool live_w = v0 < d_v;
  static_assert(64 * kUpWaves * 4 == kLat, "one float4 of a row per thread");
  // 8 o_lat rows (sequences b0 .. b0 + 7, clamped to the batch; rows past it
  // only feed outputs that are not stored)
  float4 x[8];
  auto load8 = [&](int32_t b0) {
#pragma unroll
    for (int u = 0; u < 8; u++) {
      const int32_t b = min(b0 + u, B - 1);
      x[u] = *reinterpret_cast<const float4*>(o_lat + ((int64_t)b * h + head) * kLat + 4 * tid);
    }
  };
  load8(0);
  asm volatile("" ::: "memory");  // keep the W_UV loads behind these
  bf16x8 wf[kUpKs];
  {
    const uint16_t* wrow = W_UV + ((int64_t)head * d_v + (live_w ? v0 : 0) + r) * kLat + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kUpKs; ks++) wf[ks] = *reinterpret_cast<const bf16x8*>(wrow + 16 * ks);
  }
  // x (8 rows) -> LDS rows i0 .. i0 + 7 as bf16 high and low parts
  auto convert = [&](int i0) {
#pragma unroll
    for (int u = 0; u < 8; u++) {
      const int row = i0 + u, c4 = tid;
      const f32x2 v01 = {x[u].x, x[u].y}, v23 = {x[u].z, x[u].w};
      const bf16x2 h01 = __builtin_convertvector(v01, bf16x2);
      const bf16x2 h23 = __builtin_convertvector(v23, bf16x2);
      const bf16x2 l01 = __builtin_convertvector(v01 - __builtin_convertvector(h01, f32x2), bf16x2);
      const bf16x2 l23 = __builtin_convertvector(v23 - __builtin_convertvector(h23, f32x2), bf16x2);
      const int off = row * 1024 + (((c4 >> 1) ^ up_swz(row)) << 4) + (c4 & 1) * 8;
      const u32x2 hv = {__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23)};
      const u32x2 lv = {__builtin_bit_cast(uint32_t, l01), __builtin_bit_cast(uint32_t, l23)};
      *reinterpret_cast<u32x2*>(os[0] + off) = hv;
      *reinterpret_cast<u32x2*>(os[1] + off) = lv;
    }
  };
  // products and stores for sequences b0 .. b0 + 31
  auto products = [&](int32_t b0) {
    f32x16 acc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
    // the o_lat operands are read kPre k-steps ahead of their products
    constexpr int kPre = 4;
    bf16x8 hi[kPre], lo[kPre];
    auto ld_o = [&](int ks, int slot) {
      const int off = r * 1024 + (((2 * ks + g) ^ up_swz(r)) << 4);
      hi[slot] = *reinterpret_cast<const bf16x8*>(os[0] + off);
      lo[slot] = *reinterpret_cast<const bf16x8*>(os[1] + off);
    };
#pragma unroll
    for (int ks = 0; ks < kPre; ks++) ld_o(ks, ks);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < kUpKs; ks++) {
      const int slot = ks % kPre;
      acc[2 * (ks & 1)] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hi[slot], wf[ks], acc[2 * (ks & 1)], 0, 0, 0);
      acc[2 * (ks & 1) + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lo[slot], wf[ks], acc[2 * (ks & 1) + 1], 0, 0, 0);
      if (ks + kPre < kUpKs) ld_o(ks + kPre, slot);
      __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of their products
    }
    const f32x16 sum = (acc[0] + acc[2]) + (acc[1] + acc[3]);
    // D[m = sequence][n = row]: lane holds row v0 + r, sequences 8(j/4) + 4g + j%4
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const int32_t bb = b0 + 8 * (j >> 2) + 4 * g + (j & 3);
      if (bb < B) store_elem<OT>(out, ((int64_t)bb * h + head) * d_v + v0 + r, sum[j]);
    }
  };
  // first block of sequences: the first 8 rows were loaded before W_UV
  convert(0);
  for (int32_t i0 = 8; i0 < min(32, B); i0 += 8) {
    load8(i0);
    convert(i0);
  }
  __syncthreads();
  if (live_w) products(0);
  for (int32_t b0 = 32; b0 < B; b0 += 32) {
    __syncthreads();  // the previous block has been read
    for (int32_t i0 = 0; i0 < min(32, B - b0); i0 += 8) {
      load8(b0 + i0);
      convert(i0);
    }
    __syncthreads();
    if (live_w) products(b0);
  }
}

// ------------------------------------------------------------------ up-projection, 16-row blocks
// For d_v = 128.  Work group = (head, 64-row half of W_UV, 16 sequences),
// eight waves; wave w takes rows 16 (w % 4) .. 16 (w % 4) + 15 of the half
// over latent half w / 4 and keeps them (8 KiB) in registers as the B operand
// of v_mfma_f32_16x16x32_bf16 (lane 16 q + c: row c of the block, latent
// values 32 k + 8 q .. 32 k + 8 q + 7 of k-step k); the two latent halves'
// sums are added through LDS.  In up16_mfma_kernel (the decode step up to 16
// sequences) the 16 o_lat rows are merged from the bf16 split partials by
// merge_row, wave w producing rows w and w + 8, each lane 8 values, so o_lat
// is never written; up16_olat_kernel (the up-projection stage, and the step
// of larger batches after the merge kernel) reads them from o_lat, up to
// kUp16Blocks blocks of 16 sequences per work group, which loads its W_UV
// rows once and the next block's rows while it multiplies the current one.
// The rows are staged in LDS as a bf16 high part and a bf16 remainder
// (16-byte chunk index XOR the row), both multiplied and the products summed
// in fp32, which keeps about 16 significant bits of o_lat.  Rows past the
// batch are zero.  Both kernels run the same conversion, products and sums,
// so the step and its stages agree bit for bit.
constexpr int kUp16Rows = 16;
constexpr int kUp16Waves = 8;
constexpr int kUp16Dv = 128;
constexpr int kUp16Ks = kLat / 32 / 2;  // k-steps of one latent half
constexpr int kUp16Blocks = 4;          // 16-sequence blocks per work group (rows from o_lat)

template <bool kFromParts, int OT>
__global__ __launch_bounds__(64 * kUp16Waves) void up16_mfma_kernel(
    AttnArgs a, const float* __restrict__ o_lat, const uint16_t* __restrict__ W_UV,
    void* __restrict__ out, int32_t B, int32_t h) {
  static_assert(kFromParts, "rows from o_lat: up16_olat_kernel");
  __shared__ __attribute__((aligned(16))) char os[2][kUp16Rows * kLat * 2];  // high, low parts
  __shared__ f32x4 red[4][64];  // sums of the second latent half
  const int32_t head = blockIdx.x, vh = blockIdx.y, b0 = blockIdx.z * kUp16Rows;
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, c = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), vb = wave & 3, kh = wave >> 2;
  const int32_t vrow = 64 * vh + 16 * vb + c;
  bf16x8 wf[kUp16Ks];
  auto load_w = [&] {
    const uint16_t* wrow = W_UV + ((int64_t)head * kUp16Dv + vrow) * kLat + 256 * kh + 8 * q;
#pragma unroll
    for (int ks = 0; ks < kUp16Ks; ks++) wf[ks] = *reinterpret_cast<const bf16x8*>(wrow + 32 * ks);
  };
  load_w();
#pragma unroll 1
  for (int rr = 0; rr < 2; rr++) {
    const int r = wave + 8 * rr;
    const int32_t b = b0 + r;
    float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (b < B) merge_row<1>(a, b, head, lane, x);
    uint32_t hv[4], lv[4];
#pragma unroll
    for (int p = 0; p < 4; p++) {
      const f32x2 v01 = {x[2 * p], x[2 * p + 1]};
      const bf16x2 hp = __builtin_convertvector(v01, bf16x2);
      const bf16x2 lp = __builtin_convertvector(v01 - __builtin_convertvector(hp, f32x2), bf16x2);
      hv[p] = __builtin_bit_cast(uint32_t, hp);
      lv[p] = __builtin_bit_cast(uint32_t, lp);
    }
    const int off = r * (kLat * 2) + ((lane ^ r) << 4);
    *reinterpret_cast<merge_u32x4*>(os[0] + off) = merge_u32x4{hv[0], hv[1], hv[2], hv[3]};
    *reinterpret_cast<merge_u32x4*>(os[1] + off) = merge_u32x4{lv[0], lv[1], lv[2], lv[3]};
  }
  __syncthreads();
  f32x4 acc[4] = {f32x4{}, f32x4{}, f32x4{}, f32x4{}};
#pragma unroll
  for (int kk = 0; kk < kUp16Ks; kk++) {
    const int ks = kUp16Ks * kh + kk;
    const int off = c * (kLat * 2) + (((4 * ks + q) ^ c) << 4);
    const bf16x8 ah = *reinterpret_cast<const bf16x8*>(os[0] + off);
    const bf16x8 al = *reinterpret_cast<const bf16x8*>(os[1] + off);
    acc[2 * (kk & 1)] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, wf[kk], acc[2 * (kk & 1)], 0, 0, 0);
    acc[2 * (kk & 1) + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, wf[kk], acc[2 * (kk & 1) + 1], 0, 0, 0);
  }
  const f32x4 sum = (acc[0] + acc[2]) + (acc[1] + acc[3]);
  if (kh == 1) red[vb][lane] = sum;
  __syncthreads();
  if (kh == 0) {
    const f32x4 tot = sum + red[vb][lane];
    // D[m = sequence 4 q + j][n = row c]
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int32_t bb = b0 + 4 * q + j;
      if (bb < B) store_elem<OT>(out, ((int64_t)bb * h + head) * kUp16Dv + vrow, tot[j]);
    }
  }
}

template <int OT>
__global__ __launch_bounds__(64 * kUp16Waves) void up16_olat_kernel(
    const float* __restrict__ o_lat, const uint16_t* __restrict__ W_UV,
    void* __restrict__ out, int32_t B, int32_t h) {
  __shared__ __attribute__((aligned(16))) char os[2][kUp16Rows * kLat * 2];  // high, low parts
  __shared__ f32x4 red[4][64];  // sums of the second latent half
  constexpr int NB = kUp16Blocks;
  const int32_t head = blockIdx.x, vh = blockIdx.y, bfirst = blockIdx.z * NB * kUp16Rows;
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, c = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), vb = wave & 3, kh = wave >> 2;
  const int32_t vrow = 64 * vh + 16 * vb + c;
  bf16x8 wf[kUp16Ks];
  auto load_w = [&] {
    const uint16_t* wrow = W_UV + ((int64_t)head * kUp16Dv + vrow) * kLat + 256 * kh + 8 * q;
#pragma unroll
    for (int ks = 0; ks < kUp16Ks; ks++) wf[ks] = *reinterpret_cast<const bf16x8*>(wrow + 32 * ks);
  };
  // the o_lat rows w and w + 8 of the block at b0 (zero past the batch)
  float xr[2][8];
  auto load_rows = [&](int32_t b0) {
#pragma unroll
    for (int rr = 0; rr < 2; rr++) {
      const int32_t b = b0 + wave + 8 * rr;
#pragma unroll
      for (int e = 0; e < 8; e++) xr[rr][e] = 0.f;
      if (b < B) {
        const float4* src = reinterpret_cast<const float4*>(o_lat + ((int64_t)b * h + head) * kLat + 8 * lane);
        const float4 u = src[0], v = src[1];
        xr[rr][0] = u.x; xr[rr][1] = u.y; xr[rr][2] = u.z; xr[rr][3] = u.w;
        xr[rr][4] = v.x; xr[rr][5] = v.y; xr[rr][6] = v.z; xr[rr][7] = v.w;
      }
    }
  };
  // row r of the block into LDS as bf16 high and low parts
  auto stage_row = [&](int r, const float* x) {
    uint32_t hv[4], lv[4];
#pragma unroll
    for (int p = 0; p < 4; p++) {
      const f32x2 v01 = {x[2 * p], x[2 * p + 1]};
      const bf16x2 hp = __builtin_convertvector(v01, bf16x2);
      const bf16x2 lp = __builtin_convertvector(v01 - __builtin_convertvector(hp, f32x2), bf16x2);
      hv[p] = __builtin_bit_cast(uint32_t, hp);
      lv[p] = __builtin_bit_cast(uint32_t, lp);
    }
    const int off = r * (kLat * 2) + ((lane ^ r) << 4);
    *reinterpret_cast<merge_u32x4*>(os[0] + off) = merge_u32x4{hv[0], hv[1], hv[2], hv[3]};
    *reinterpret_cast<merge_u32x4*>(os[1] + off) = merge_u32x4{lv[0], lv[1], lv[2], lv[3]};
  };
  load_w();
  load_rows(bfirst);
#pragma unroll 1
  for (int blk = 0; blk < NB; blk++) {
    const int32_t b0 = bfirst + blk * kUp16Rows;
    if (b0 >= B) break;  // uniform over the work group
    if (blk > 0) __syncthreads();  // the previous block's LDS rows and sums have been read
    stage_row(wave, xr[0]);
    stage_row(wave + 8, xr[1]);
    // the next block's rows, in flight during this block's products
    if (blk + 1 < NB && b0 + kUp16Rows < B) load_rows(b0 + kUp16Rows);
    __syncthreads();
    f32x4 acc[4] = {f32x4{}, f32x4{}, f32x4{}, f32x4{}};
#pragma unroll
    for (int kk = 0; kk < kUp16Ks; kk++) {
      const int ks = kUp16Ks * kh + kk;
      const int off = c * (kLat * 2) + (((4 * ks + q) ^ c) << 4);
      const bf16x8 ah = *reinterpret_cast<const bf16x8*>(os[0] + off);
      const bf16x8 al = *reinterpret_cast<const bf16x8*>(os[1] + off);
      acc[2 * (kk & 1)] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, wf[kk], acc[2 * (kk & 1)], 0, 0, 0);
      acc[2 * (kk & 1) + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, wf[kk], acc[2 * (kk & 1) + 1], 0, 0, 0);
    }
    const f32x4 sum = (acc[0] + acc[2]) + (acc[1] + acc[3]);
    if (kh == 1) red[vb][lane] = sum;
    __syncthreads();
    if (kh == 0) {
      const f32x4 tot = sum + red[vb][lane];
      // D[m = sequence 4 q + j][n = row c]
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int32_t bb = b0 + 4 * q + j;
        if (bb < B) store_elem<OT>(out, ((int64_t)bb * h + head) * kUp16Dv + vrow, tot[j]);
      }
    }
  }
}

template <bool kFromParts>
hipError_t launch_up16(const mla_decode_params& p, const AttnArgs& a, const float* o_lat,
                       const void* W_UV, void* out, hipStream_t s) {
  const uint16_t* w = static_cast<const uint16_t*>(W_UV);
  if constexpr (kFromParts) {
    const dim3 grid(p.num_heads, kUp16Dv / 64, (p.batch + kUp16Rows - 1) / kUp16Rows);
    if (p.out_dtype == MLA_BF16)
      hipLaunchKernelGGL((up16_mfma_kernel<true, MLA_BF16>), grid, dim3(64 * kUp16Waves), 0, s, a,
                         o_lat, w, out, p.batch, p.num_heads);
    else
      hipLaunchKernelGGL((up16_mfma_kernel<true, MLA_F32>), grid, dim3(64 * kUp16Waves), 0, s, a,
                         o_lat, w, out, p.batch, p.num_heads);
  } else {
    const int32_t per = kUp16Blocks * kUp16Rows;  // sequences per work group
    const dim3 grid(p.num_heads, kUp16Dv / 64, (p.batch + per - 1) / per);
    if (p.out_dtype == MLA_BF16)
      hipLaunchKernelGGL((up16_olat_kernel<MLA_BF16>), grid, dim3(64 * kUp16Waves), 0, s, o_lat, w,
                         out, p.batch, p.num_heads);
    else
      hipLaunchKernelGGL((up16_olat_kernel<MLA_F32>), grid, dim3(64 * kUp16Waves), 0, s, o_lat, w,
                         out, p.batch, p.num_heads);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ absorb
// Work group = (head, 128 latent columns), four waves of 32 columns each.  The
// W_UK rows of the group (d_nope x 128 bf16) are staged in LDS with the
// 16-byte chunk index XOR-swizzled by the row; the MFMA B operand (8
// consecutive rows n of one column) comes from the transposing LDS read.  All
// global loads of a work group are issued before the first is waited for.
//
// The first kPlanGroups work groups of the launch run the split planner
// instead (plan_block), which needs no result of the absorption, so that the
// two latency-bound steps share one launch.
constexpr int kAbsCols = 128;
constexpr int kAbsColGroups = kLat / kAbsCols;
constexpr int kAbsMaxN = 128;         // d_nope of the fast path (LDS 32 KiB)
constexpr int kAbsStage = kAbsMaxN * 16 / 256;  // 16-byte staging loads per thread
constexpr int kAbsKs = kAbsMaxN / 16;           // MFMA k-steps

__device__ inline int abs_swz(int row) { return row & 15; }

struct PlanArgs {
  int32_t groups;  // planning work groups at the start of the launch (0: none)
  PlanInput in;
};

template <int OT, bool kExpand>
__global__ __launch_bounds__(256) void absorb_mfma_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ W_UK,
                                                          void* __restrict__ q_lat, int32_t B,
                                                          int32_t h, int32_t d_n, int32_t d_r,
                                                          PlanArgs pl, ShardExpand ex) {
  __shared__ __attribute__((aligned(16))) char ws[kAbsMaxN * kAbsCols * 2];
  static_assert(sizeof(PlanShared) <= sizeof(ws), "planner LDS");
  if ((int32_t)blockIdx.x < pl.groups) {
    plan_block(pl.in, blockIdx.x, pl.groups, *reinterpret_cast<PlanShared*>(ws));
    return;
  }
  const int32_t id = blockIdx.x - pl.groups;
  const int32_t head = id / kAbsColGroups;
  const int32_t cgrp = id % kAbsColGroups;
  const int32_t c0 = cgrp * kAbsCols;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int32_t dq = d_n + d_r, dl = kLat + d_r;
  const int g = lane >> 5, r = lane & 31;
  const int nks = d_n / 16;
  // stage W_UK[head][0:d_n][c0:c0+128]: rows of 256 B, 16 chunks of 16 B
  // (loads are unconditional, from clamped addresses, so that none waits on a branch)
  uint4 wv[kAbsStage];
#pragma unroll
  for (int i = 0; i < kAbsStage; i++) {
    const int idx = tid + 256 * i, row = min(idx >> 4, d_n - 1), ch = idx & 15;
    wv[i] = *reinterpret_cast<const uint4*>(W_UK + ((int64_t)head * d_n + row) * kLat + c0 + 8 * ch);
  }
  // q_nope fragments of a block of 32 sequences (rows past B are zeroed where
  // they are used)
  bf16x8 qa[kAbsKs];
  auto load_q = [&](int32_t b0) {
    const int32_t b = b0 + r;
    const uint16_t* qrow = q + ((int64_t)(b < B ? b : 0) * h + head) * dq + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kAbsKs; ks++)
      qa[ks] = *reinterpret_cast<const bf16x8*>(qrow + 16 * min(ks, nks - 1));
  };
  load_q(0);
  // rows past d_n repeat row d_n - 1 (same value, same place)
#pragma unroll
  for (int i = 0; i < kAbsStage; i++) {
    const int idx = tid + 256 * i, row = min(idx >> 4, d_n - 1), ch = idx & 15;
    *reinterpret_cast<uint4*>(ws + row * 256 + ((ch ^ abs_swz(row)) << 4)) = wv[i];
  }
  // the rope part of the absorbed query is q_rope copied (once per head, to
  // each of its shard heads when expanding)
  const int32_t ng = kExpand ? ex.g : 1;
  auto out_row = [&](int32_t b, int32_t j) -> int64_t {
    return kExpand ? (int64_t)b * ng * h + (int64_t)j * h + head : (int64_t)b * h + head;
  };
  if (cgrp == 0 && OT == MLA_BF16 && d_r % 8 == 0) {
    const int32_t per = d_r / 8;  // 16-byte pieces per row
    for (int32_t i = tid; i < B * per; i += 256) {
      const int32_t b = i / per, k = 8 * (i % per);
      const uint4 v = *reinterpret_cast<const uint4*>(q + ((int64_t)b * h + head) * dq + d_n + k);
      for (int32_t j = 0; j < ng; j++)
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(q_lat) + out_row(b, j) * dl + kLat + k) = v;
    }
  } else if (cgrp == 0) {
    for (int32_t i0 = 0; i0 < B * d_r; i0 += 4 * 256) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const int32_t i = i0 + u * 256 + tid;
        if (i < B * d_r)
          v[u] = load_elem<MLA_BF16>(q, ((int64_t)(i / d_r) * h + head) * dq + d_n + i % d_r);
      }
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const int32_t i = i0 + u * 256 + tid;
        if (i < B * d_r)
          for (int32_t j = 0; j < ng; j++)
            store_elem<OT>(q_lat, out_row(i / d_r, j) * dl + kLat + i % d_r, v[u]);
      }
    }
  }
  __syncthreads();
  const int j16 = lane & 15, grp = lane >> 4, e = j16 >> 2, qd = j16 & 3;
  const int cw = 32 * wave;                      // this wave's columns within the group
  const int col_in = cw + 16 * (grp & 1) + 4 * qd;
  const int chunk = col_in >> 3, hoff = (col_in & 7) * 2;
  bf16x8 bw[kAbsKs];
#pragma unroll
  for (int ks = 0; ks < kAbsKs; ks++) {
    if (ks < nks) {
      const int row0 = 16 * ks + 8 * g + e, row1 = row0 + 4;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<i16x4 __attribute__((address_space(3)))*>(
          (lds_t*)ws + row0 * 256 + ((chunk ^ abs_swz(row0)) << 4) + hoff));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<i16x4 __attribute__((address_space(3)))*>(
          (lds_t*)ws + row1 * 256 + ((chunk ^ abs_swz(row1)) << 4) + hoff));
      bw[ks] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  }
  for (int32_t b0 = 0; b0 < B; b0 += 32) {
    if (b0 > 0) load_q(b0);
    const bool live = b0 + r < B;
    f32x16 acc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < kAbsKs; ks++)
      if (ks < nks)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            live ? qa[ks] : __builtin_bit_cast(bf16x8, i16x8{}), bw[ks], acc, 0, 0, 0);
    // D[m = sequence][n = column]: lane holds column c0 + cw + r
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const int32_t bb = b0 + 8 * (j >> 2) + 4 * g + (j & 3);
      if (bb < B) {
        const int32_t col = c0 + cw + r;
        if constexpr (!kExpand) {
          store_elem<OT>(q_lat, ((int64_t)bb * h + head) * dl + col, acc[j]);
        } else {
          // what absorption then expansion store: the stored query value,
          // times the factor of its column's shard, zero in the other shards
          const float v = OT == MLA_BF16 ? bf16_bits_to_f32(f32_to_bf16_bits(acc[j])) : acc[j];
          const int32_t js = col / (kLat / ng);
          for (int32_t jj = 0; jj < ng; jj++)
            store_elem<OT>(q_lat, out_row(bb, jj) * dl + col, jj == js ? ex.mu[jj] * v : 0.f);
        }
      }
    }
  }
}

}  // namespace

bool proj_mfma_supported(const mla_decode_params& p) {
  return p.q_dtype == MLA_BF16 && p.weight_dtype == MLA_BF16 && p.d_latent == kLat &&
         p.d_nope % 16 == 0 && p.d_nope <= kAbsMaxN && p.d_v % 32 == 0;
}

hipError_t launch_absorb_mfma(const mla_decode_params& p, const void* q, const void* W_UK,
                              void* q_lat, int32_t ot, const PlanRequest* plan, hipStream_t s,
                              const ShardExpand* ex) {
  PlanArgs pl{};
  if (plan) pl = PlanArgs{kPlanGroups, plan_input(p, *plan)};
  const dim3 grid(p.num_heads * kAbsColGroups + pl.groups);
  const ShardExpand e = ex ? *ex : ShardExpand{1, {1.f, 1.f, 1.f, 1.f}};
  if (ex && (e.g < 1 || e.g > 4 || kLat % e.g != 0)) return hipErrorInvalidValue;
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* w = static_cast<const uint16_t*>(W_UK);
#define MLA_ABSORB_MFMA(O, X)                                                                  \
  hipLaunchKernelGGL((absorb_mfma_kernel<O, X>), grid, dim3(256), 0, s, qq, w, q_lat, p.batch, \
                     p.num_heads, p.d_nope, p.d_rope, pl, e)
  if (ot == MLA_BF16) {
    if (ex) MLA_ABSORB_MFMA(MLA_BF16, true);
    else MLA_ABSORB_MFMA(MLA_BF16, false);
  } else {
    if (ex) MLA_ABSORB_MFMA(MLA_F32, true);
    else MLA_ABSORB_MFMA(MLA_F32, false);
  }
#undef MLA_ABSORB_MFMA
  return hipGetLastError();
}

hipError_t launch_up_project_mfma(const mla_decode_params& p, const float* o_lat,
                                  const void* W_UV, void* out, hipStream_t s) {
  if (p.d_v == kUp16Dv) return launch_up16<false>(p, AttnArgs{}, o_lat, W_UV, out, s);
  const dim3 grid(p.num_heads, (p.d_v + 32 * kUpWaves - 1) / (32 * kUpWaves));
  if (p.out_dtype == MLA_BF16)
    hipLaunchKernelGGL((up_project_mfma_kernel<MLA_BF16>), grid, dim3(64 * kUpWaves), 0, s, o_lat,
                       static_cast<const uint16_t*>(W_UV), out, p.batch, p.num_heads, p.d_v);
  else
    hipLaunchKernelGGL((up_project_mfma_kernel<MLA_F32>), grid, dim3(64 * kUpWaves), 0, s, o_lat,
                       static_cast<const uint16_t*>(W_UV), out, p.batch, p.num_heads, p.d_v);
  return hipGetLastError();
}

// One 16-row block of sequences: a larger batch would repeat every head's
// W_UV reads per block and its merges per W_UV half, and is faster as the
// merge (one wave per row over the whole chip) and the up-projection.
bool merge_up_supported(const mla_decode_params& p) {
  return proj_mfma_supported(p) && mfma_any_supported(p) && p.d_v == kUp16Dv &&
         p.batch <= kUp16Rows;
}

hipError_t launch_merge_up(const mla_decode_params& p, const AttnArgs& a, const void* W_UV,
                           void* out, hipStream_t s) {
  if (!merge_up_supported(p) || !a.part_bf16 || a.shards > 1 || a.d_c != kMergeLat ||
      a.streams != 1)
    return hipErrorInvalidValue;
  return launch_up16<true>(p, a, nullptr, W_UV, out, s);
}

}  // namespace mla
