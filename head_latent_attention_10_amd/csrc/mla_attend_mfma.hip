// Matrix-core split attention over the paged latent cache (gfx950).
//
// Shape: d_c = 512 latent values + d_r = 64 rope values per cached token,
// heads a multiple of 32, bf16 latent/rope rows, bf16 absorbed query.
//
// Work decomposition.  Work group = (token split g, block of up to 128 heads).
// Split g owns a contiguous run of 64-token tiles of the concatenated
// sequences ("split plan" in mla_common.hpp); every tile is read from HBM
// once and staged in LDS, where all heads of the work group use it.  A wave
// owns 32 heads and, per 32-token sub-tile, computes
//   S^T[t, i] = sum_d KV[t, d] Q[i, d]        (MFMA 32x32x16: M = tokens,
//                                              N = heads, K = 576)
//   online softmax over t (one lane = one head: in-lane reductions plus one
//                          exchange with the lane 32 away)
//   O^T[d, i] += sum_t C[t, d] P[i, t]        (MFMA: M = latent rows, N = heads,
//                                              K = tokens)
// The heads that share one latent row sit on the MFMA's N dimension, so each
// row is fetched once per 32 heads.  The softmax weights go from the score
// accumulator straight into the PV operand: the K order inside each 16-token
// step is permuted (slot i of lane group g is token 8*(i/4) + 4*g + i%4) so
// that it matches the accumulator layout, and the latent tile is read in the
// same permuted order with the gfx950 transposing LDS read.
//
// LDS ring.  Two stages of one 64-token tile: 64 latent rows of 1 KiB and 64
// rope rows of 128 B.  Rows are written by direct global->LDS 16-byte loads
// (one instruction per latent row, eight rope rows per instruction) with the
// 16-byte chunk index XOR-swizzled by the row so the MFMA operand reads are
// spread over the banks.  The loads of tile i+1 are in flight while tile i is
// computed.
//
// Softmax rescaling is lazy: the running maximum is only raised when a tile's
// maximum exceeds it by more than 2^8 in weight, so the 256-register
// accumulator is rarely rescaled; weights then stay below 2^8, well inside
// bf16 and fp32 range, and the final normalisation uses the same reference.
#include "mla_kernels.hpp"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_t;

constexpr int kDc = 512, kDr = 64;
constexpr int kKsC = kDc / 16;          // 32 score k-steps over the latent
constexpr int kKs = (kDc + kDr) / 16;   // 36 score k-steps in all
constexpr int kMd = kDc / 32;           // 16 output row blocks
constexpr int kCRow = kDc * 2;          // 1024 bytes per latent row
constexpr int kRRow = kDr * 2;          // 128 bytes per rope row
constexpr int kStageC = kTile * kCRow;  // 65536
constexpr int kStage = kStageC + kTile * kRRow;  // 73728
constexpr float kLazy = 8.0f;           // log2 of the largest unnormalised weight
constexpr int kQkDepth = 4;             // score operand reads in flight
constexpr int kPvDepth = 4;             // value operand reads in flight

__device__ inline int swz_c(int row) { return row & 15; }

// fp32 value of the round-to-nearest-even bf16 of a finite x.
__device__ inline float round_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return __uint_as_float(u & 0xffff0000u);
}
__device__ inline int swz_r(int row) { return (row >> 1) & 7; }

// Issue the direct-to-LDS loads of one tile (tokens t0.. of sequence b, T tokens
// in all; t0 is a multiple of 64).  Rows past the end repeat the last valid
// token so every load reads finite data; those rows are masked in the softmax.
// `wave` must be wave-uniform so the block-table lookups are scalar loads and
// never make the wave wait on the vector-memory counter.
template <int NW>
__device__ inline void issue_tile(const AttnArgs& a, lds_t* stage, int32_t b, int32_t t0,
                                  int32_t T, int wave, int lane) {
  const char* ckv = static_cast<const char*>(a.c_kv);
  const char* krp = static_cast<const char*>(a.k_rope);
  const int32_t rmax = T - 1 - t0;
  const int32_t* trow = a.block_table + (int64_t)b * a.max_blocks;
  if (a.P % kTile == 0) {
    // the whole tile lies in one block: one table lookup
    int32_t blk = trow[t0 / a.P];
    blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
    const int64_t base = (int64_t)blk * a.P + (t0 % a.P);
#pragma unroll
    for (int r0 = 0; r0 < kTile; r0 += NW) {
      const int r = r0 + wave;
      const char* src = ckv + (base + min(r, rmax)) * kCRow + ((lane ^ swz_c(r)) << 4);
      __builtin_amdgcn_global_load_lds(src, (void __attribute__((address_space(3)))*)(stage + r * kCRow), 16, 0, 0);
    }
#pragma unroll
    for (int j0 = 0; j0 < 8; j0 += NW) {
      const int j = j0 + wave;
      const int r = 8 * j + (lane >> 3);
      const char* src = krp + (base + min(r, rmax)) * kRRow + (((lane & 7) ^ swz_r(r)) << 4);
      __builtin_amdgcn_global_load_lds(src, (void __attribute__((address_space(3)))*)(stage + kStageC + j * 1024), 16, 0, 0);
    }
  } else {
#pragma unroll
    for (int r0 = 0; r0 < kTile; r0 += NW) {
      const int r = r0 + wave;
      const int64_t slot = phys_slot(a.block_table, b, t0 + min(r, rmax), a.P, a.max_blocks, a.num_blocks);
      const char* src = ckv + slot * kCRow + ((lane ^ swz_c(r)) << 4);
      __builtin_amdgcn_global_load_lds(src, (void __attribute__((address_space(3)))*)(stage + r * kCRow), 16, 0, 0);
    }
#pragma unroll
    for (int j0 = 0; j0 < 8; j0 += NW) {
      const int j = j0 + wave;
      const int r = 8 * j + (lane >> 3);
      const int64_t slot = phys_slot(a.block_table, b, t0 + min(r, rmax), a.P, a.max_blocks, a.num_blocks);
      const char* src = krp + slot * kRRow + (((lane & 7) ^ swz_r(r)) << 4);
      __builtin_amdgcn_global_load_lds(src, (void __attribute__((address_space(3)))*)(stage + kStageC + j * 1024), 16, 0, 0);
    }
  }
}

template <int NW>
constexpr int loads_per_tile() { return kTile / NW + (8 + NW - 1) / NW; }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

struct SoftmaxState {
  float m;  // running reference maximum, log2 units
  float l;  // lane-partial sum of weights
};

// HB = 32-head blocks per work group, TS = token streams (waves splitting the
// two 32-token halves of each tile, each with its own partial).
template <int HB, int TS>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * HB * TS, 64 * HB * TS),
                          amdgpu_waves_per_eu(1, 1)))
void attend_mfma_kernel(AttnArgs a) {
  constexpr int NW = HB * TS;
  __shared__ __attribute__((aligned(1024))) char lds_raw[2 * kStage];
  lds_t* lds = (lds_t*)(lds_raw);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int hb = wave % HB, ts = wave / HB;
  const int g32 = lane >> 5;                       // lane group within the MFMA
  const int32_t head = blockIdx.y * (32 * HB) + hb * 32 + (lane & 31);
  const int32_t g = blockIdx.x;

  const int32_t n_total = a.cu_tiles[a.B];
  if (n_total == 0) return;
  const int32_t t_begin = (int32_t)split_begin(n_total, a.splits, g);
  const int32_t t_end = (int32_t)split_begin(n_total, a.splits, g + 1);
  if (t_begin >= t_end) return;

  int32_t b = 0;
  while (a.cu_tiles[b + 1] <= t_begin) b++;
  int32_t T = seq_len_clamped(a.seq_lens, b, a.max_blocks, a.P);
  int32_t first = a.cu_tiles[b];

  issue_tile<NW>(a, lds, b, (t_begin - first) * kTile, T, wave, lane);

  bf16x8 qf[kKs];
  auto load_q = [&](int32_t bb) {
    const bf16x8* qp = reinterpret_cast<const bf16x8*>(
        static_cast<const uint16_t*>(a.q_lat) + ((int64_t)bb * a.h + head) * (kDc + kDr));
#pragma unroll
    for (int ks = 0; ks < kKs; ks++) qf[ks] = qp[2 * ks + g32];
  };
  load_q(b);

  f32x16 o[kMd];
#pragma unroll
  for (int md = 0; md < kMd; md++) o[md] = f32x16{};
  SoftmaxState st{-INFINITY, 0.f};
  const float sm = a.sm_scale_log2;

  for (int32_t tile = t_begin; tile < t_end; tile++) {
    lds_t* cur = lds + ((tile - t_begin) & 1) * kStage;
    lds_t* nxt = lds + (((tile - t_begin) & 1) ^ 1) * kStage;
    int32_t b_next = b;
    const bool more = tile + 1 < t_end;
    if (more) {
      while (a.cu_tiles[b_next + 1] <= tile + 1) b_next++;
      const int32_t T_next = b_next == b ? T : seq_len_clamped(a.seq_lens, b_next, a.max_blocks, a.P);
      issue_tile<NW>(a, nxt, b_next, (tile + 1 - a.cu_tiles[b_next]) * kTile, T_next, wave, lane);
      wait_vmcnt<loads_per_tile<NW>()>();
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();

    const int32_t nvalid = min(kTile, T - (tile - first) * kTile);
#pragma unroll
    for (int sub = 0; sub < 2; sub++) {
      if (TS == 2 && sub != ts) continue;
      // ---- scores S^T[t, i] for the 32 tokens of this sub-tile
      f32x16 s = f32x16{};
      const int row = 32 * sub + (lane & 31);
      auto ld_a = [&](int ks) -> bf16x8 {
        const int chunk = 2 * (ks < kKsC ? ks : ks - kKsC) + g32;
        const lds_t* p = ks < kKsC ? cur + row * kCRow + ((chunk ^ swz_c(row)) << 4)
                                   : cur + kStageC + row * kRRow + ((chunk ^ swz_r(row)) << 4);
        return *reinterpret_cast<const bf16x8 __attribute__((address_space(3)))*>(p);
      };
      bf16x8 av[kQkDepth];
#pragma unroll
      for (int k = 0; k < kQkDepth; k++) av[k] = ld_a(k);
#pragma unroll
      for (int ks = 0; ks < kKs; ks++) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[ks % kQkDepth], qf[ks], s, 0, 0, 0);
        if (ks + kQkDepth < kKs) av[ks % kQkDepth] = ld_a(ks + kQkDepth);
        __builtin_amdgcn_sched_barrier(0);
      }
      // ---- online softmax (one lane = one head; tokens split over g32)
      float sv[16];
      float mt = -INFINITY;
#pragma unroll
      for (int j = 0; j < 16; j++) {
        const int tok = 32 * sub + 8 * (j >> 2) + 4 * g32 + (j & 3);
        sv[j] = tok < nvalid ? s[j] * sm : -INFINITY;
        mt = fmaxf(mt, sv[j]);
      }
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const bool need = mt > st.m + kLazy;
      if (__any(need)) {
        const float m_new = fmaxf(st.m, mt);
        const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
#pragma unroll
        for (int md = 0; md < kMd; md++) o[md] *= alpha;
        st.l *= alpha;
        st.m = m_new;
      }
      const float mref = st.m == -INFINITY ? 0.f : st.m;
      // Weights to bf16 with whole-vector conversions only: element-wise
      // writes into bf16 vectors are not lowered correctly by this compiler.
      f32x8 pw[2];
      float lsum = 0.f;
#pragma unroll
      for (int j = 0; j < 16; j++) {
        const float pj = __builtin_amdgcn_exp2f(sv[j] - mref);
        pw[j >> 3][j & 7] = pj;
        lsum += round_to_bf16(pj);   // normalise by the weights the MFMA actually uses
      }
      const bf16x8 pf[2] = {__builtin_convertvector(pw[0], bf16x8),
                            __builtin_convertvector(pw[1], bf16x8)};
      st.l += lsum;
      // ---- O^T[d, i] += C[t, d] P[i, t]
      const int j16 = lane & 15, grp = lane >> 4;
      const int e = j16 >> 2, qd = j16 & 3;
      // A operand of (md, half): latent rows d, the 8 permuted tokens of the step
      auto ld_c = [&](int md, int half) -> bf16x8 {
        const int dd = 32 * md + 16 * (grp & 1) + 4 * qd;
        const int chunk = dd >> 3, hoff = (dd & 7) * 2;
        const int r0 = 32 * sub + 16 * half + 4 * g32 + e;
        const int r1 = r0 + 8;
        i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<i16x4 __attribute__((address_space(3)))*>(
            cur + r0 * kCRow + ((chunk ^ swz_c(r0)) << 4) + hoff));
        i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<i16x4 __attribute__((address_space(3)))*>(
            cur + r1 * kCRow + ((chunk ^ swz_c(r1)) << 4) + hoff));
        const i16x8 cat = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_bit_cast(bf16x8, cat);
      };
      bf16x8 cv[kPvDepth];
#pragma unroll
      for (int k = 0; k < kPvDepth; k++) cv[k] = ld_c(k >> 1, k & 1);
#pragma unroll
      for (int step = 0; step < 2 * kMd; step++) {
        const int md = step >> 1, half = step & 1;
        o[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cv[step % kPvDepth], pf[half], o[md], 0, 0, 0);
        const int nx = step + kPvDepth;
        if (nx < 2 * kMd) cv[step % kPvDepth] = ld_c(nx >> 1, nx & 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // ---- end of a sequence segment: write the normalised partial
    if (!more || b_next != b) {
      const float ltot = st.l + __shfl_xor(st.l, 32);
      const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
      const int64_t slot = (int64_t)(g + b) * TS + ts;
      float* dst = a.part_o + (slot * a.h + head) * kDc;
#pragma unroll
      for (int md = 0; md < kMd; md++) {
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
          f32x4 v = {o[md][4 * jj] * inv, o[md][4 * jj + 1] * inv, o[md][4 * jj + 2] * inv,
                     o[md][4 * jj + 3] * inv};
          *reinterpret_cast<f32x4*>(dst + 32 * md + 8 * jj + 4 * g32) = v;
        }
      }
      if (g32 == 0)
        a.part_lse[slot * a.h + head] =
            ltot > 0.f ? (st.m + log2f(ltot)) * 0.69314718055994530942f : -INFINITY;
      if (more) {
        b = b_next;
        T = seq_len_clamped(a.seq_lens, b, a.max_blocks, a.P);
        first = a.cu_tiles[b];
        load_q(b);
#pragma unroll
        for (int md = 0; md < kMd; md++) o[md] = f32x16{};
        st = SoftmaxState{-INFINITY, 0.f};
      }
    }
    __syncthreads();
  }
}

}  // namespace

bool mfma_supported(const mla_decode_params& p) {
  return p.cache_dtype == MLA_BF16 && p.rope_dtype == MLA_BF16 && p.d_latent == kDc &&
         p.d_rope == kDr && p.num_heads % 32 == 0;
}

int32_t mfma_streams(int32_t heads) { return (heads % 128 == 0) ? 1 : 2; }

hipError_t launch_attend_mfma(const AttnArgs& a, int32_t cache_dtype, hipStream_t s) {
  if (cache_dtype != MLA_BF16 || a.d_c != kDc || a.d_r != kDr || a.h % 32) return hipErrorInvalidValue;
  if (a.h % 128 == 0) {
    hipLaunchKernelGGL((attend_mfma_kernel<4, 1>), dim3(a.splits, a.h / 128), dim3(256), 0, s, a);
  } else if (a.h % 64 == 0) {
    hipLaunchKernelGGL((attend_mfma_kernel<2, 2>), dim3(a.splits, a.h / 64), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((attend_mfma_kernel<1, 2>), dim3(a.splits, a.h / 32), dim3(128), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace mla
