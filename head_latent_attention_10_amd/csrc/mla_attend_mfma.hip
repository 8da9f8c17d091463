// Matrix-core split attention over the paged latent cache (gfx950).
//
// Shape: d_c = 512 latent values + d_r = 64 rope values per cached token,
// heads a multiple of 32, bf16 latent/rope rows, bf16 absorbed query.
//
// Work decomposition.  A token split g owns a contiguous run of 64-token tiles
// of the concatenated sequences ("split plan" in mla_common.hpp).  Its heads
// are served by HG work groups of 32*HB heads each (HB = 2 for 64 heads, 1 for
// 32); the HG groups of one split get workgroup ids that differ by a multiple
// of 8 and are dispatched together, so they run on the same XCD and the
// second read of every tile is served by that XCD's L2.
//
// Inside a work group the waves specialise:
//  * 2*HB score waves.  Wave (hb, kh) holds the absorbed query of 32 heads for
//    half of the 576-wide key (kh = 0: latent 0..287; kh = 1: latent 288..511
//    and the 64 rope values) in registers and computes, for each 32-token step,
//      S^T[t, i] = sum_d KV[t, d] Q[i, d]      (MFMA 32x32x16 bf16, M = tokens,
//                                              N = heads, K = its 288 values)
//    The kh = 1 wave hands its partial scores to its partner through LDS; the
//    partner adds them, runs the online softmax (one lane = one head) and
//    publishes the bf16 weights P, the per-head rescale factors and, at the
//    end of a sequence segment, 1/l and the log-sum-exp.
//  * 4 (HB = 2) or 2 (HB = 1) value waves.  Each owns a slice of 128 (or 256)
//    latent rows of the output for all heads of the group and computes
//      O^T[d, i] += sum_t C[t, d] P[i, t]      (M = latent rows, N = heads,
//                                              K = tokens)
//    one step behind the score waves.  The latent tile is read with the
//    transposing LDS read; each such read feeds HB MFMAs.  The weights are in
//    a permuted token order (slot i of lane group g is token 8*(i/4) + 4*g +
//    i%4 of the 16-token k-step) that matches the score accumulator layout,
//    and the latent tile is read in the same order.
//
// LDS ring.  Four stages of one 32-token step: 32 latent rows of 1 KiB and 32
// rope rows of 128 B, written by direct global->LDS 16-byte loads (one
// instruction per latent row, eight rope rows per instruction) two steps
// ahead of use.  The 16-byte chunk index is XOR-swizzled with a permutation
// of the row's low four bits, which keeps both the row reads of the score
// product and the 4-row transposing reads of the value product free of bank
// conflicts.
//
// Step i (three work-group barriers):
//   wait for step i's loads; barrier
//   issue loads of step i+2 | score waves: partial S(i) | value waves: O += P(i-1) C(i-1)
//   barrier
//   score wave kh = 0: merge partial scores, softmax, publish P(i)
//   barrier
//
// Softmax rescaling is lazy: after the first four steps of a sequence segment
// (which track the exact maximum, so an early dominant token gets weight
// exactly 1), the running maximum is only raised when a step's maximum
// exceeds it by more than 2^8 in weight, so the output accumulator is rarely
// rescaled; weights stay below 2^8.  The normaliser is the sum of the
// bf16-rounded weights that the MFMA consumes.
#include "mla_kernels.hpp"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) char lds_t;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kDc = 512, kDr = 64;
constexpr int kStep = 32;                         // tokens per pipeline step
constexpr int kCRow = kDc * 2;                    // 1024 bytes per latent row
constexpr int kRRow = kDr * 2;                    // 128 bytes per rope row
constexpr int kStageC = kStep * kCRow;            // 32768
constexpr int kStage = kStageC + kStep * kRRow;   // 36864
constexpr int kStages = 4;
constexpr int kRing = kStages * kStage;           // 147456
constexpr int kLoadsPerStep = kStep + kStep / 8;  // 32 latent rows + 4 rope groups
constexpr int kKsHalf = 18;                       // score k-steps per score wave
constexpr int kXBytes = 64 * 64;                  // one wave's partial scores
constexpr int kPBytes = 2 * 64 * 16;              // weights of one head block, two k-steps
constexpr float kLazy = 8.0f;                     // log2 of the largest unnormalised weight
constexpr int kExactSteps = 4;                    // steps per segment with an exact maximum

template <int HB>
struct Shape {
  static constexpr int NQ = 2 * HB;             // score waves
  static constexpr int NP = HB == 2 ? 4 : 2;    // value waves
  static constexpr int NW = NQ + NP;
  static constexpr int MDP = kDc / 32 / NP;     // 32-row output blocks per value wave
  static constexpr int LDS = kRing + HB * (kXBytes + kPBytes) + HB * 32 * 4 * 2 + 16;
};

// Chunk swizzles: row bits (b3 b2 b1 b0) -> chunk bits (b2 b1 b0 b3) for latent
// rows; rope rows share 256-byte bank lines in pairs.
__device__ inline int swz_c(int r) { return ((r & 3) << 1) | (((r >> 2) & 1) << 3) | ((r >> 3) & 1); }
__device__ inline int swz_r(int r) { return (r >> 1) & 7; }

__device__ inline float round_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return __uint_as_float(u & 0xffff0000u);
}

template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Walks the 32-token steps of a split's tiles in order; a tile's second half
// is skipped when it holds no token of its sequence.
struct StepIter {
  int32_t t, t_end, half, b, T, first;  // first = first tile of sequence b
  bool valid;

  __device__ void init(const AttnArgs& a, int32_t t_begin, int32_t t_stop) {
    t = t_begin;
    t_end = t_stop;
    half = 0;
    b = 0;
    while (a.cu_tiles[b + 1] <= t) b++;
    T = seq_len_clamped(a.seq_lens, b, a.max_blocks, a.P);
    first = a.cu_tiles[b];
    valid = t < t_end;
  }
  __device__ int32_t t0() const { return (t - first) * kTile + half * kStep; }
  __device__ int32_t nvalid() const { return min(kStep, T - t0()); }
  __device__ bool has_second_half() const { return (t - first) * kTile + kStep < T; }
  // last step of its sequence within this split
  __device__ bool seg_last(const AttnArgs& a) const {
    const bool last_of_tile = half == 1 || !has_second_half();
    return last_of_tile && (t + 1 == t_end || a.cu_tiles[b + 1] <= t + 1);
  }
  __device__ void advance(const AttnArgs& a) {
    if (half == 0 && has_second_half()) {
      half = 1;
      return;
    }
    half = 0;
    t++;
    valid = t < t_end;
    if (valid && a.cu_tiles[b + 1] <= t) {
      while (a.cu_tiles[b + 1] <= t) b++;
      T = seq_len_clamped(a.seq_lens, b, a.max_blocks, a.P);
      first = a.cu_tiles[b];
    }
  }
};

// Direct-to-LDS loads of one step.  Rows past the end repeat the last valid
// token (finite data; masked in the softmax).  `wave` is wave-uniform, so the
// block-table lookups are scalar loads.
template <int NW>
__device__ inline void issue_step(const AttnArgs& a, lds_t* stage, const StepIter& it, int wave,
                                  int lane) {
  const char* ckv = static_cast<const char*>(a.c_kv);
  const char* krp = static_cast<const char*>(a.k_rope);
  const int32_t t0 = it.t0();
  const int32_t rmax = it.T - 1 - t0;
  const int32_t* trow = a.block_table + (int64_t)it.b * a.max_blocks;
  const bool one_block = (a.P % kStep) == 0;  // the step lies inside one block
  int64_t base = 0;
  if (one_block) {
    int32_t blk = trow[t0 / a.P];
    blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
    base = (int64_t)blk * a.P + (t0 % a.P);
  }
  for (int k = wave; k < kLoadsPerStep; k += NW) {
    if (k < kStep) {
      const int r = k;
      const int64_t slot = one_block ? base + min(r, rmax)
                                     : phys_slot(a.block_table, it.b, t0 + min(r, rmax), a.P,
                                                 a.max_blocks, a.num_blocks);
      const char* src = ckv + slot * kCRow + ((lane ^ swz_c(r)) << 4);
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(stage + r * kCRow), 16, 0, 0);
    } else {
      const int j = k - kStep;
      const int r = 8 * j + (lane >> 3);
      const int64_t slot = one_block ? base + min(r, rmax)
                                     : phys_slot(a.block_table, it.b, t0 + min(r, rmax), a.P,
                                                 a.max_blocks, a.num_blocks);
      const char* src = krp + slot * kRRow + (((lane & 7) ^ swz_r(r)) << 4);
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(stage + kStageC + j * 1024), 16, 0, 0);
    }
  }
}

template <int NW>
__device__ constexpr int loads_of_wave(int wave) { return (kLoadsPerStep - wave + NW - 1) / NW; }

// The load schedule every wave keeps identically.
template <int NW>
struct Loader {
  StepIter next;       // next step to load
  int32_t loaded;      // steps issued so far
  bool newer_issued;   // the batch after the awaited one was issued

  __device__ void start(const AttnArgs& a, lds_t* ring, int32_t tb, int32_t te, int wave,
                        int lane) {
    next.init(a, tb, te);
    loaded = 0;
    for (int s = 0; s < 2 && next.valid; s++) {
      issue_step<NW>(a, ring + (loaded % kStages) * kStage, next, wave, lane);
      next.advance(a);
      loaded++;
    }
    newer_issued = loaded == 2;
  }
  // Start of step i: wait for this wave's loads of step i (only the newer batch
  // i+1 may stay in flight), barrier, then issue step i+2.
  __device__ void begin_step(const AttnArgs& a, lds_t* ring, int wave, int lane) {
    if (!newer_issued)
      wait_vmcnt<0>();
    else if (loads_of_wave<NW>(wave) == loads_of_wave<NW>(0))
      wait_vmcnt<loads_of_wave<NW>(0)>();
    else
      wait_vmcnt<loads_of_wave<NW>(NW - 1)>();
    __syncthreads();
    if (next.valid) {
      issue_step<NW>(a, ring + (loaded % kStages) * kStage, next, wave, lane);
      next.advance(a);
      loaded++;
      newer_issued = true;
    } else {
      newer_issued = false;
    }
  }
};

template <int HB>
__global__ __attribute__((amdgpu_flat_work_group_size(Shape<HB>::NW * 64, Shape<HB>::NW * 64)))
void attend_mfma_kernel(AttnArgs a) {
  using S = Shape<HB>;
  constexpr int NW = S::NW;
  __shared__ __attribute__((aligned(1024))) char smem[S::LDS];
  lds_t* ring = (lds_t*)smem;
  lds_t* xbuf = ring + kRing;                       // [HB][64 lanes][16 floats]
  lds_t* pbuf = xbuf + HB * kXBytes;                // [HB][2 k-steps][64 lanes][16 B]
  float* s_alpha = (float*)(smem + kRing + HB * (kXBytes + kPBytes));  // [HB][32]
  float* s_invl = s_alpha + HB * 32;                // [HB][32]
  int* s_flag = (int*)(s_invl + HB * 32);           // [HB]

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g32 = lane >> 5;

  // workgroup id -> (split, head group); the HG groups of a split share an XCD
  const int32_t HG = a.h / (32 * HB);
  int32_t g, hg;
  if (HG > 1) {
    const int32_t L = blockIdx.x, span = 8 * HG;
    hg = (L % span) / 8;
    g = (L / span) * 8 + (L % 8);
  } else {
    hg = 0;
    g = blockIdx.x;
  }
  if (g >= a.splits) return;
  const int32_t n_total = a.cu_tiles[a.B];
  if (n_total == 0) return;
  const int32_t t_begin = (int32_t)split_begin(n_total, a.splits, g);
  const int32_t t_end = (int32_t)split_begin(n_total, a.splits, g + 1);
  if (t_begin >= t_end) return;

  Loader<NW> ld;
  ld.start(a, ring, t_begin, t_end, wave, lane);
  StepIter cur;
  cur.init(a, t_begin, t_end);
  const float sm = a.sm_scale_log2;

  if (wave < S::NQ) {
    // ================================================================ score waves
    const int hb = wave >> 1, kh = wave & 1;
    const int32_t head = hg * 32 * HB + hb * 32 + (lane & 31);
    bf16x8 qf[kKsHalf];
    auto load_q = [&](int32_t bb) {
      const bf16x8* qp = reinterpret_cast<const bf16x8*>(
          static_cast<const uint16_t*>(a.q_lat) + ((int64_t)bb * a.h + head) * (kDc + kDr));
#pragma unroll
      for (int k = 0; k < kKsHalf; k++) qf[k] = qp[2 * (kh * kKsHalf + k) + g32];
    };
    load_q(cur.b);
    float m_run = -INFINITY, l_run = 0.f;
    int32_t seg_step = 0;  // steps of the current segment seen so far
    lds_t* xb = xbuf + hb * kXBytes + lane * 64;
    lds_t* pb = pbuf + hb * kPBytes + lane * 16;
    // n steps of scores plus one final step in which only the value waves work
    for (int32_t i = 0;; i++) {
      ld.begin_step(a, ring, wave, lane);
      lds_t* st = ring + (i % kStages) * kStage;
      f32x16 s = f32x16{};
      if (cur.valid) {
        const int row = lane & 31;
        auto ld_a = [&](int k) -> bf16x8 {
          const int ks = kh * kKsHalf + k;
          const lds_t* p = ks < 32
              ? st + row * kCRow + (((2 * ks + g32) ^ swz_c(row)) << 4)
              : st + kStageC + row * kRRow + (((2 * (ks - 32) + g32) ^ swz_r(row)) << 4);
          return *reinterpret_cast<const bf16x8 __attribute__((address_space(3)))*>(p);
        };
        constexpr int D = 4;
        bf16x8 av[D];
#pragma unroll
        for (int k = 0; k < D; k++) av[k] = ld_a(k);
#pragma unroll
        for (int k = 0; k < kKsHalf; k++) {
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[k % D], qf[k], s, 0, 0, 0);
          if (k + D < kKsHalf) av[k % D] = ld_a(k + D);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (kh == 1) {
#pragma unroll
          for (int q = 0; q < 4; q++)
            *reinterpret_cast<f32x4 __attribute__((address_space(3)))*>(xb + 16 * q) =
                f32x4{s[4 * q], s[4 * q + 1], s[4 * q + 2], s[4 * q + 3]};
        }
      }
      __syncthreads();
      if (cur.valid && kh == 0) {
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const f32x4 o = *reinterpret_cast<const f32x4 __attribute__((address_space(3)))*>(xb + 16 * q);
          s[4 * q] += o[0];
          s[4 * q + 1] += o[1];
          s[4 * q + 2] += o[2];
          s[4 * q + 3] += o[3];
        }
        const int32_t nv = cur.nvalid();
        float sv[16];
        float mt = -INFINITY;
#pragma unroll
        for (int j = 0; j < 16; j++) {
          const int tok = 8 * (j >> 2) + 4 * g32 + (j & 3);
          sv[j] = tok < nv ? s[j] * sm : -INFINITY;
          mt = fmaxf(mt, sv[j]);
        }
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        // exact running maximum for the first steps of a segment (the largest
        // weight is then exactly 1 in bf16), lazy afterwards
        const float thr = seg_step < kExactSteps ? 0.f : kLazy;
        const bool any = __any(mt > m_run + thr);
        float alpha = 1.f;
        if (any) {
          const float m_new = fmaxf(m_run, mt);
          alpha = __builtin_amdgcn_exp2f(m_run - m_new);
          l_run *= alpha;
          m_run = m_new;
        }
        const float mref = m_run == -INFINITY ? 0.f : m_run;
        f32x8 pw[2];
        float lsum = 0.f;
#pragma unroll
        for (int j = 0; j < 16; j++) {
          const float pj = __builtin_amdgcn_exp2f(sv[j] - mref);
          pw[j >> 3][j & 7] = pj;
          lsum += round_to_bf16(pj);
        }
        l_run += lsum;
        seg_step++;
        // publish the weights in the value product's operand layout (whole-vector
        // conversions only: element-wise bf16 vector writes are not lowered correctly)
        *reinterpret_cast<bf16x8 __attribute__((address_space(3)))*>(pb) =
            __builtin_convertvector(pw[0], bf16x8);
        *reinterpret_cast<bf16x8 __attribute__((address_space(3)))*>(pb + 64 * 16) =
            __builtin_convertvector(pw[1], bf16x8);
        if (g32 == 0) s_alpha[hb * 32 + lane] = alpha;
        if (lane == 0) s_flag[hb] = any ? 1 : 0;
        if (cur.seg_last(a)) {
          const float ltot = l_run + __shfl_xor(l_run, 32);
          if (g32 == 0) {
            s_invl[hb * 32 + lane] = ltot > 0.f ? 1.f / ltot : 0.f;
            const int64_t slot = (int64_t)(g + cur.b);
            a.part_lse[slot * a.h + head] =
                ltot > 0.f ? (m_run + log2f(ltot)) * 0.69314718055994530942f : -INFINITY;
          }
        }
      }
      __syncthreads();
      if (!cur.valid) break;  // that was the value waves' final step
      const bool was_last = cur.seg_last(a);
      cur.advance(a);
      if (cur.valid && was_last) {
        load_q(cur.b);
        m_run = -INFINITY;
        l_run = 0.f;
        seg_step = 0;
      }
    }
  } else {
    // ================================================================ value waves
    constexpr int MDP = S::MDP;
    const int pw_id = wave - S::NQ;
    const int j16 = lane & 15, grp = lane >> 4, e = j16 >> 2, qd = j16 & 3;
    f32x16 o[MDP][HB];
#pragma unroll
    for (int md = 0; md < MDP; md++)
#pragma unroll
      for (int hb = 0; hb < HB; hb++) o[md][hb] = f32x16{};
    StepIter prev = cur;  // the step whose weights are consumed in this iteration
    bool prev_valid = false;
    for (int32_t i = 0;; i++) {
      if (!cur.valid && !prev_valid) break;
      ld.begin_step(a, ring, wave, lane);
      if (prev_valid) {
        lds_t* st = ring + ((i - 1) % kStages) * kStage;
        // rescale by the factors published with the step being consumed
#pragma unroll
        for (int hb = 0; hb < HB; hb++) {
          if (s_flag[hb]) {
            const float al = s_alpha[hb * 32 + (lane & 31)];
#pragma unroll
            for (int md = 0; md < MDP; md++) o[md][hb] *= al;
          }
        }
        bf16x8 pf[HB][2];
#pragma unroll
        for (int hb = 0; hb < HB; hb++)
#pragma unroll
          for (int kk = 0; kk < 2; kk++)
            pf[hb][kk] = *reinterpret_cast<const bf16x8 __attribute__((address_space(3)))*>(
                pbuf + hb * kPBytes + (kk * 64 + lane) * 16);
        auto ld_c = [&](int md, int kk) -> bf16x8 {
          const int dd = 32 * (pw_id * MDP + md) + 16 * (grp & 1) + 4 * qd;
          const int chunk = dd >> 3, hoff = (dd & 7) * 2;
          const int r0 = 16 * kk + 4 * g32 + e;
          const int r1 = r0 + 8;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              reinterpret_cast<i16x4 __attribute__((address_space(3)))*>(
                  st + r0 * kCRow + ((chunk ^ swz_c(r0)) << 4) + hoff));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              reinterpret_cast<i16x4 __attribute__((address_space(3)))*>(
                  st + r1 * kCRow + ((chunk ^ swz_c(r1)) << 4) + hoff));
          const i16x8 cat = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          return __builtin_bit_cast(bf16x8, cat);
        };
        constexpr int NSTEP = 2 * MDP;
        constexpr int D = 4;
        bf16x8 cv[D];
#pragma unroll
        for (int k = 0; k < D; k++) cv[k] = ld_c(k >> 1, k & 1);
#pragma unroll
        for (int s = 0; s < NSTEP; s++) {
          const int md = s >> 1, kk = s & 1;
#pragma unroll
          for (int hb = 0; hb < HB; hb++)
            o[md][hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cv[s % D], pf[hb][kk], o[md][hb], 0, 0, 0);
          if (s + D < NSTEP) cv[s % D] = ld_c((s + D) >> 1, (s + D) & 1);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (prev.seg_last(a)) {
          const int64_t slot = (int64_t)(g + prev.b);
#pragma unroll
          for (int hb = 0; hb < HB; hb++) {
            const int32_t head = hg * 32 * HB + hb * 32 + (lane & 31);
            const float inv = s_invl[hb * 32 + (lane & 31)];
            float* dst = a.part_o + (slot * a.h + head) * kDc + 32 * pw_id * MDP;
#pragma unroll
            for (int md = 0; md < MDP; md++) {
#pragma unroll
              for (int jj = 0; jj < 4; jj++) {
                const f32x4 v = {o[md][hb][4 * jj] * inv, o[md][hb][4 * jj + 1] * inv,
                                 o[md][hb][4 * jj + 2] * inv, o[md][hb][4 * jj + 3] * inv};
                *reinterpret_cast<f32x4*>(dst + 32 * md + 8 * jj + 4 * g32) = v;
              }
              o[md][hb] = f32x16{};
            }
          }
        }
      }
      __syncthreads();
      __syncthreads();
      prev = cur;
      prev_valid = cur.valid;
      if (cur.valid) cur.advance(a);
    }
  }
}

// heads served by one work group
int32_t heads_per_group(int32_t heads) { return heads % 64 == 0 ? 64 : 32; }

}  // namespace

bool mfma_supported(const mla_decode_params& p) {
  return p.cache_dtype == MLA_BF16 && p.rope_dtype == MLA_BF16 && p.d_latent == kDc &&
         p.d_rope == kDr && p.num_heads % 32 == 0;
}

int32_t mfma_streams(int32_t) { return 1; }

int32_t mfma_head_groups(int32_t heads) { return heads / heads_per_group(heads); }

hipError_t launch_attend_mfma(const AttnArgs& a, int32_t cache_dtype, hipStream_t s) {
  if (cache_dtype != MLA_BF16 || a.d_c != kDc || a.d_r != kDr || a.h % 32) return hipErrorInvalidValue;
  const int32_t hpg = heads_per_group(a.h);
  const int32_t HG = a.h / hpg;
  if (HG > 1 && a.splits % 8) return hipErrorInvalidValue;  // XCD pairing uses whole groups of 8
  const dim3 grid(a.splits * HG);
  if (hpg == 64)
    hipLaunchKernelGGL((attend_mfma_kernel<2>), grid, dim3(Shape<2>::NW * 64), 0, s, a);
  else
    hipLaunchKernelGGL((attend_mfma_kernel<1>), grid, dim3(Shape<1>::NW * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
