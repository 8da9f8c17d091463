// Matrix-core split attention over an fp8 latent cache (gfx950).
//
// Shape: d_c = 512 latent values stored as OCP E4M3FN bytes with one fp32
// scale per cached token (the row's value is scale * e4m3), d_r = 64 bf16 rope
// values per token, heads a multiple of 32, bf16 absorbed query.
//
// The work decomposition, split plan, tile descriptors and head groups are
// those of the bf16 kernels (mla_attend_mfma.hip).  Two schedules:
//  * attend64_fp8_kernel (64-head work groups, dense tables): the pipelined
//    schedule of the bf16 64-head kernel, described above it.
//  * attend_fp8_kernel (32-head work groups, and index lists): two work-group
//    barriers per step (one when the step's tile is in LDS, one after the
//    softmax wave has published the weights, after which the value waves run
//    the value product of that same step).
// Both consume the 8-bit latent tile the same way:
//
//  * Scores.  S^T[t, i] = scale_t * sum_d e4m3[t, d] q[i, d] + rope term.  The
//    latent part runs on the fp8 matrix core (32x32x64, both operands E4M3):
//    the A operand is the cached bytes as they are, the B operand is the
//    absorbed query split into two E4M3 terms, q * 2^k = hi + lo with
//    hi = e4m3(q * 2^k) and lo = e4m3(q * 2^k - hi), where 2^k (one power of two
//    per head and key half) brings the largest |q| into [128, 256).  The two
//    products share the accumulator; the split keeps about 8 significant bits
//    of q (one term would keep 4).  The result is multiplied by 2^-k (exact)
//    and by the token's scale.  The rope part is bf16 as in the bf16 kernel.
//  * Values.  O^T[d, i] += sum_t e4m3[t, d] (p[i, t] * scale_t): the token
//    scale is folded into the bf16 weight, and the latent tile is read with the
//    8-bit transposing LDS read (8 tokens of one latent column per lane) and
//    widened to bf16 exactly (every E4M3 value is a bf16 value), feeding the
//    bf16 matrix core.
//  * The per-token scales multiply the latent part of the score only, so the
//    latent and rope partial scores are handed to the softmax wave separately
//    and it applies the scales.  attend_fp8_kernel's softmax waves load the
//    scales from global memory one step ahead; attend64_fp8_kernel loads them
//    into the tile's LDS stage together with the tile.
//
// LDS ring of attend_fp8_kernel: six stages of 32 latent rows of 512 B plus 32
// rope rows of 128 B (20 KiB), loaded four steps ahead.  The 16-byte chunk index of a latent row
// is XOR-swizzled with a permutation of the row's low four bits chosen so that
// the 16-row reads of the score product and the 8-row transposing reads of the
// value product both spread over the 64 banks.
#include "mla_mfma_util.hpp"

#include <hip/hip_ext.h>

namespace mla {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int kDc8 = 512, kDr8 = 64;
constexpr int kStep8 = kTile;                         // tokens per pipeline step
constexpr int kCRow8 = kDc8;                          // 512 bytes per latent row
constexpr int kRRow8 = kDr8 * 2;                      // 128 bytes per rope row
constexpr int kStageC8 = kStep8 * kCRow8;             // 16384
constexpr int kStage8 = kStageC8 + kStep8 * kRRow8;   // 20480
constexpr int kStages8 = 6;
constexpr int kAhead8 = kStages8 - 2;                 // steps loaded ahead of use
constexpr int kRing8 = kStages8 * kStage8;            // 122880
constexpr int kLoadsPerStep8 = kStep8 / 2 + kStep8 / 8;  // 2 latent rows or 8 rope rows each
constexpr int kBlocksHalf = 4;                        // 64-byte key blocks per score wave
constexpr int kRopeKs = kDr8 / 16;                    // bf16 rope k-steps (kh = 1)
constexpr int kX8Bytes = 2 * 64 * 64;                 // latent and rope partial scores
constexpr int kP8Bytes = 2 * 64 * 16;
constexpr float kLazy8 = 8.0f;
constexpr int kExactSteps8 = 4;
static_assert(kStep8 == 32, "the score and value products are laid out for 32-token steps");

template <int HB>
struct Shape8 {
  static constexpr int NQ = 2 * HB;
  static constexpr int NP = HB == 2 ? 4 : 2;
  static constexpr int NW = NQ + NP;
  static constexpr int MDP = kDc8 / 32 / NP;
  static constexpr int LDS = kRing8 + kWinBytes + HB * (kX8Bytes + kP8Bytes) + HB * 32 * 4 * 2 + 16;
};

// Latent rows: row bits (b3 b2 b1 b0) -> chunk bits (b3 b1 b0 b2).
__device__ inline int swz8(int r) { return ((r & 3) << 1) | (((r >> 3) & 1) << 3) | ((r >> 2) & 1); }
__device__ inline int swz_r8(int r) { return (r >> 1) & 7; }

// Direct-to-LDS loads of one step by the NL loader waves: latent instruction
// q covers rows 2q and 2q+1 (lane l: row 2q + l/32, LDS chunk l%32), rope
// instruction j covers rows 8j..8j+7.  Fast path as in the bf16 kernel; rows
// past the end repeat the last valid token.
template <int NL, bool SP>
struct StepIssue8 {
  static constexpr int kLat = kStep8 / 2 / NL;
  static constexpr int kRope = kStep8 / 8 / NL;
  static constexpr int kPer = kLat + kRope;
  static_assert(kPer * NL == kLoadsPerStep8, "uniform load counts");

  __device__ __forceinline__ static void issue(const AttnArgs& a, lds_t* stage, const Tile& d, int lw, int lane) {
    const uint32_t st = (uint32_t)(uintptr_t)stage;
    const int64_t base = (int64_t)d.blk * a.P + d.off;
    if (d.blk >= 0 && d.nv == kStep8) {
      const char* cb = static_cast<const char*>(a.c_kv) + base * kCRow8;
      const char* rb = static_cast<const char*>(a.k_rope) + base * kRRow8;
#pragma unroll
      for (int m = 0; m < kLat; m++) {
        const int q = lw + NL * m;
        const int r = 2 * q + (lane >> 5);
        dma16s(cb, (uint32_t)(r * kCRow8 + (((lane & 31) ^ swz8(r)) << 4)), st + q * 1024);
      }
#pragma unroll
      for (int m = 0; m < kRope; m++) {
        const int j = lw + NL * m;
        const int r = 8 * j + (lane >> 3);
        dma16s(rb, (uint32_t)(r * kRRow8 + (((lane & 7) ^ swz_r8(r)) << 4)), st + kStageC8 + j * 1024);
      }
      return;
    }
    const char* ckv = static_cast<const char*>(a.c_kv);
    const char* krp = static_cast<const char*>(a.k_rope);
    const int32_t rmax = d.nv - 1;
    if constexpr (SP) {
      // sparse: slots from the planner's list, read with scalar loads (two
      // rows per latent load, eight per rope load, picked per lane)
#pragma unroll
      for (int m = 0; m < kLat; m++) {
        const int q = lw + NL * m;
        const int32_t s0 = sparse_slot_uniform(a, d.b, d.t0 + min(2 * q, rmax));
        const int32_t s1 = sparse_slot_uniform(a, d.b, d.t0 + min(2 * q + 1, rmax));
        const int64_t slot = (lane >> 5) ? s1 : s0;
        const int r = 2 * q + (lane >> 5);
        dma16(ckv + slot * kCRow8 + (((lane & 31) ^ swz8(r)) << 4), stage + q * 1024);
      }
#pragma unroll
      for (int m = 0; m < kRope; m++) {
        const int j = lw + NL * m;
        int32_t sl = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) {
          const int32_t si = sparse_slot_uniform(a, d.b, d.t0 + min(8 * j + i, rmax));
          sl = (lane >> 3) == i ? si : sl;
        }
        const int r = 8 * j + (lane >> 3);
        dma16(krp + (int64_t)sl * kRRow8 + (((lane & 7) ^ swz_r8(r)) << 4), stage + kStageC8 + j * 1024);
      }
      return;
    }
#pragma unroll
    for (int m = 0; m < kLat; m++) {
      const int q = lw + NL * m;
      const int r = 2 * q + (lane >> 5);
      const int64_t slot = d.blk >= 0 ? base + min(r, rmax)
                                      : phys_slot(a.block_table, d.b, d.t0 + min(r, rmax), a.P,
                                                  a.max_blocks, a.num_blocks);
      dma16(ckv + slot * kCRow8 + (((lane & 31) ^ swz8(r)) << 4), stage + q * 1024);
    }
#pragma unroll
    for (int m = 0; m < kRope; m++) {
      const int j = lw + NL * m;
      const int r = 8 * j + (lane >> 3);
      const int64_t slot = d.blk >= 0 ? base + min(r, rmax)
                                      : phys_slot(a.block_table, d.b, d.t0 + min(r, rmax), a.P,
                                                  a.max_blocks, a.num_blocks);
      dma16(krp + slot * kRRow8 + (((lane & 7) ^ swz_r8(r)) << 4), stage + kStageC8 + j * 1024);
    }
  }
};

// Wait until at most `newer` batches of kPer loads issued after the awaited
// one are outstanding.
template <int kPer>
__device__ inline void wait_batches(int newer) {
  switch (newer) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<kPer>(); break;
    case 2: wait_vmcnt<2 * kPer>(); break;
    default: wait_vmcnt<3 * kPer>(); break;
  }
}

// Load schedule of one loader wave: steps are loaded kAhead8 ahead.  Loader 0
// refills the descriptor window w + 1 into the buffer of window w - 1 with the
// loads of step kWin w + kAhead8 + 2, when the value waves (furthest behind,
// then at step kWin w + 1) have left window w - 1.
template <int NL, bool SP>
struct Loader8 {
  static constexpr int kPerWave = StepIssue8<NL, SP>::kPer;
  static_assert(3 * kPerWave + 1 < 64, "vmcnt range");
  static_assert(kAhead8 - 1 <= 3, "wait_batches cases");
  int32_t next, n;

  __device__ void issue_next(const AttnArgs& a, lds_t* ring, lds_t* win, int32_t t_begin, int lw,
                             int lane) {
    constexpr int kRefill = kAhead8 + 2;
    if (lw == 0 && next >= kWin + kRefill && next % kWin == kRefill && next + kWin - kRefill < n)
      load_window(a, win, t_begin, t_begin + n, next / kWin + 1, lane);
    const Tile d = read_tile(win, next);
    StepIssue8<NL, SP>::issue(a, ring + (next % kStages8) * kStage8, d, lw, lane);
    next++;
  }
  __device__ void start(const AttnArgs& a, lds_t* ring, lds_t* win, int32_t t_begin, int32_t steps,
                        int lw, int lane) {
    next = 0;
    n = steps;
    for (int s = 0; s < kAhead8 && next < n; s++) issue_next(a, ring, win, t_begin, lw, lane);
  }
  // before step i: its loads are complete (later batches may be in flight)
  __device__ void wait_for(int32_t i) const { wait_batches<kPerWave>(next - i - 1); }
};

// fp32 pair -> two E4M3 bytes (round to nearest even) in the low half of a word.
__device__ inline uint32_t e4m3_pair(float x, float y) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x, y, 0, false) & 0xffffu;
}

template <int HB, bool SP>
__global__ __attribute__((amdgpu_flat_work_group_size(Shape8<HB>::NW * 64, Shape8<HB>::NW * 64)))
void attend_fp8_kernel(AttnArgs a) {
  using S = Shape8<HB>;
  __shared__ __attribute__((aligned(1024))) char smem[S::LDS];
  lds_t* ring = (lds_t*)smem;
  lds_t* win = ring + kRing8;                       // [2][kWin] tile descriptors
  lds_t* xbuf = win + kWinBytes;                    // [HB][latent, rope][4][64 lanes][16 B]
  lds_t* pbuf = xbuf + HB * kX8Bytes;               // [HB][2 k-steps][64 lanes][16 B]
  float* s_alpha = (float*)(smem + kRing8 + kWinBytes + HB * (kX8Bytes + kP8Bytes));  // [HB][32]
  float* s_invl = s_alpha + HB * 32;                // [HB][32]
  int* s_flag = (int*)(s_invl + HB * 32);           // [HB]

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g32 = lane >> 5;

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
  select_latent_group(a, hg * 32 * HB);  // the host keeps a head group inside one latent group
  const int32_t n_total = load_ro(a.cu_tiles, a.B);
  if (n_total == 0) return;
  const int32_t t_begin = load_ro(a.split_first, g);
  const int32_t t_end = load_ro(a.split_first, g + 1);
  if (t_begin >= t_end) return;
  const int32_t n = t_end - t_begin;

  if (wave == 1) {
    load_window(a, win, t_begin, t_end, 0, lane);
    if (n > kWin) load_window(a, win, t_begin, t_end, 1, lane);
    wait_vmcnt<0>();
  }
  wg_barrier();
  const float sm = a.sm_scale_log2;

  if (wave < S::NQ) {
    // ================================================================ score waves
    const int hb = wave >> 1, kh = wave & 1;
    const int32_t head = hg * 32 * HB + hb * 32 + (lane & 31);
    const int row = lane & 31;
    // the absorbed query as two E4M3 terms per 64-byte key block, times 2^k
    i32x8 qhi[kBlocksHalf], qlo[kBlocksHalf];
    bf16x8 qr[kRopeKs];
    float qinv = 1.f;  // 2^-k
    auto load_q = [&](int32_t bb) {
      const uint16_t* qp = static_cast<const uint16_t*>(a.q_lat) + ((int64_t)bb * a.h + head) * (kDc8 + kDr8);
      // lane half g32 holds key bytes 32 g32 .. 32 g32 + 31 of every block
      // (bf16 pairs read as words and widened with integer operations); the
      // query is read twice, for the largest |q| and then block by block for
      // the split, which keeps few registers live
      auto chunk = [&](int kb, int c) -> u32x4 {
        return *reinterpret_cast<const u32x4*>(qp + 64 * (kh * kBlocksHalf + kb) + 32 * g32 + 8 * c);
      };
      auto elem = [](const u32x4& w, int e) -> float {  // element e (0..7) of a chunk
        const uint32_t x = w[e >> 1];
        return __uint_as_float((e & 1) ? (x & 0xffff0000u) : (x << 16));
      };
      float mx = 0.f;
#pragma unroll
      for (int kb = 0; kb < kBlocksHalf; kb++) {
        u32x4 w[4];
#pragma unroll
        for (int c = 0; c < 4; c++) w[c] = chunk(kb, c);
#pragma unroll
        for (int c = 0; c < 4; c++)
#pragma unroll
          for (int e = 0; e < 8; e++) mx = fmaxf(mx, fabsf(elem(w[c], e)));
      }
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      // 2^k with max|q| 2^k in [128, 256) (1 for an all-zero query)
      const int k = mx > 0.f ? min(max(8 - __builtin_amdgcn_frexp_expf(mx), -120), 120) : 0;
      const float qs = __builtin_amdgcn_ldexpf(1.f, k);
      qinv = __builtin_amdgcn_ldexpf(1.f, -k);
#pragma unroll
      for (int kb = 0; kb < kBlocksHalf; kb++) {
        u32x4 w[4];
#pragma unroll
        for (int c = 0; c < 4; c++) w[c] = chunk(kb, c);
        uint32_t h[8], l[8];
#pragma unroll
        for (int c = 0; c < 4; c++) {
#pragma unroll
          for (int hw = 0; hw < 2; hw++) {
            float x[4], r[4];
#pragma unroll
            for (int e = 0; e < 4; e++) x[e] = elem(w[c], 4 * hw + e) * qs;
            const uint32_t h01 = e4m3_pair(x[0], x[1]), h23 = e4m3_pair(x[2], x[3]);
            r[0] = x[0] - __builtin_amdgcn_cvt_f32_fp8((int)h01, 0);
            r[1] = x[1] - __builtin_amdgcn_cvt_f32_fp8((int)h01, 1);
            r[2] = x[2] - __builtin_amdgcn_cvt_f32_fp8((int)h23, 0);
            r[3] = x[3] - __builtin_amdgcn_cvt_f32_fp8((int)h23, 1);
            h[2 * c + hw] = h01 | (h23 << 16);
            l[2 * c + hw] = e4m3_pair(r[0], r[1]) | (e4m3_pair(r[2], r[3]) << 16);
          }
        }
        qhi[kb] = i32x8{(int)h[0], (int)h[1], (int)h[2], (int)h[3], (int)h[4], (int)h[5], (int)h[6], (int)h[7]};
        qlo[kb] = i32x8{(int)l[0], (int)l[1], (int)l[2], (int)l[3], (int)l[4], (int)l[5], (int)l[6], (int)l[7]};
      }
      if (kh == 1) {
#pragma unroll
        for (int kr = 0; kr < kRopeKs; kr++)
          qr[kr] = *reinterpret_cast<const bf16x8*>(qp + kDc8 + 16 * kr + 8 * g32);
      }
      // nothing the compiler tracks stays in flight: its per-use waits would
      // also count the tile loads
      wait_vmcnt<0>();
    };
    // per-token scales of a step, rows 8 (j/4) + 4 g32 + j%4 of accumulator slot j
    auto load_scales = [&](const Tile& d, float* sc) {
      const int32_t rmax = d.nv - 1;
      if (d.blk >= 0 && d.nv == kStep8) {
        const float* sb = a.c_kv_scale + (int64_t)d.blk * a.P + d.off + 4 * g32;
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(sb + 8 * q);
#pragma unroll
          for (int e = 0; e < 4; e++) sc[4 * q + e] = v[e];
        }
      } else {
#pragma unroll
        for (int j = 0; j < 16; j++) {
          const int r = min(8 * (j >> 2) + 4 * g32 + (j & 3), rmax);
          const int64_t slot = d.blk >= 0 ? (int64_t)d.blk * a.P + d.off + r
                                          : entry_slot(a, d.b, d.t0 + r);
          sc[j] = a.c_kv_scale[slot];
        }
      }
    };
    Tile cur = read_tile(win, 0);
    load_q(cur.b);
    float sc[16];
    if (kh == 0) load_scales(cur, sc);
    float m_run = -INFINITY, l_run = 0.f;
    int32_t seg_step = 0;
    lds_t* xb = xbuf + hb * kX8Bytes + lane * 16;
    lds_t* pb = pbuf + hb * kP8Bytes + lane * 16;
    Loader8<HB, SP> ld;
    if (kh == 1) ld.start(a, ring, win, t_begin, n, hb, lane);
    for (int32_t i = 0;; i++) {
      const bool valid = i < n;
      const bool seg_last = valid && (cur.last || i + 1 == n);
      if (kh == 1) {
        ld.wait_for(i);
        wg_barrier_nowait();  // step i's tile is in LDS
      } else {
        wg_barrier();
      }
      lds_t* st = ring + (i % kStages8) * kStage8;
      f32x16 s = f32x16{}, sr = f32x16{};
      if (valid) {
        auto ld_a = [&](int kb) -> i32x8 {  // key bytes 64 kb + 32 g32 .. +31 of row `row`
          const int c0 = 4 * (kh * kBlocksHalf + kb) + 2 * g32;
          const i32x4 x0 = *reinterpret_cast<const i32x4 __attribute__((address_space(3)))*>(
              st + row * kCRow8 + ((c0 ^ swz8(row)) << 4));
          const i32x4 x1 = *reinterpret_cast<const i32x4 __attribute__((address_space(3)))*>(
              st + row * kCRow8 + (((c0 + 1) ^ swz8(row)) << 4));
          return i32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        };
        i32x8 av = ld_a(0);
#pragma unroll
        for (int kb = 0; kb < kBlocksHalf; kb++) {
          const i32x8 an = kb + 1 < kBlocksHalf ? ld_a(kb + 1) : av;
          s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, qhi[kb], s, 0, 0, 0, 127, 0, 127);
          s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, qlo[kb], s, 0, 0, 0, 127, 0, 127);
          av = an;
          __builtin_amdgcn_sched_barrier(0);
        }
        if (kh == 1) {
#pragma unroll
          for (int k = 0; k < kRopeKs; k++) {
            const bf16x8 ar = *reinterpret_cast<const bf16x8 __attribute__((address_space(3)))*>(
                st + kStageC8 + row * kRRow8 + (((2 * k + g32) ^ swz_r8(row)) << 4));
            sr = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ar, qr[k], sr, 0, 0, 0);
          }
#pragma unroll
          for (int q = 0; q < 4; q++) {
            *reinterpret_cast<f32x4 __attribute__((address_space(3)))*>(xb + 1024 * q) =
                f32x4{s[4 * q] * qinv, s[4 * q + 1] * qinv, s[4 * q + 2] * qinv, s[4 * q + 3] * qinv};
            *reinterpret_cast<f32x4 __attribute__((address_space(3)))*>(xb + 4096 + 1024 * q) =
                f32x4{sr[4 * q], sr[4 * q + 1], sr[4 * q + 2], sr[4 * q + 3]};
          }
        }
      }
      wg_barrier();
      Tile nxt{};
      if (i + 1 < n) nxt = read_tile(win, i + 1);
      if (kh == 1) {
        // loads of step i + kAhead8, into the stage last read in step i - 2
        if (ld.next < n) ld.issue_next(a, ring, win, t_begin, hb, lane);
      } else if (valid) {
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const f32x4 xl = *reinterpret_cast<const f32x4 __attribute__((address_space(3)))*>(xb + 1024 * q);
          const f32x4 xr = *reinterpret_cast<const f32x4 __attribute__((address_space(3)))*>(xb + 4096 + 1024 * q);
#pragma unroll
          for (int e = 0; e < 4; e++)
            s[4 * q + e] = __builtin_fmaf(__builtin_fmaf(s[4 * q + e], qinv, xl[e]), sc[4 * q + e], xr[e]);
        }
        const int32_t nv = cur.nv;
        if (nv < kStep8) {
#pragma unroll
          for (int j = 0; j < 16; j++)
            if (8 * (j >> 2) + 4 * g32 + (j & 3) >= nv) s[j] = -INFINITY;
        }
        float mx = s[0];
#pragma unroll
        for (int j = 1; j < 16; j++) mx = fmaxf(mx, s[j]);
        {
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                           false, false);
          mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        const float mt = mx * sm;
        const float thr = seg_step < kExactSteps8 ? 0.f : kLazy8;
        const bool any = __any(mt > m_run + thr);
        float alpha = 1.f;
        if (any) {
          const float m_new = fmaxf(m_run, mt);
          alpha = __builtin_amdgcn_exp2f(m_run - m_new);
          l_run *= alpha;
          m_run = m_new;
        }
        const float mref = m_run == -INFINITY ? 0.f : m_run;
        // weights p * scale_t rounded to bf16 (the value product's operand);
        // the normaliser sums the weights that product consumes, those bf16
        // values divided by scale_t (p where the scale is 0), so that their
        // rounding cancels in the normalised output as in the bf16 path
        uint32_t pk[8];
        float lsum = 0.f;
#pragma unroll
        for (int q = 0; q < 8; q++) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * q], sm, -mref));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * q + 1], sm, -mref));
          const float c0 = sc[2 * q], c1 = sc[2 * q + 1];
          const f32x2 e = {p0 * c0, p1 * c1};
          const bf16x2 pr = __builtin_convertvector(e, bf16x2);
          pk[q] = __builtin_bit_cast(uint32_t, pr);
          const f32x2 back = __builtin_convertvector(pr, f32x2);
          lsum += (c0 != 0.f ? back[0] * __builtin_amdgcn_rcpf(c0) : p0) +
                  (c1 != 0.f ? back[1] * __builtin_amdgcn_rcpf(c1) : p1);
        }
        l_run += lsum;
        *reinterpret_cast<u32x4 __attribute__((address_space(3)))*>(pb) = u32x4{pk[0], pk[1], pk[2], pk[3]};
        *reinterpret_cast<u32x4 __attribute__((address_space(3)))*>(pb + 64 * 16) =
            u32x4{pk[4], pk[5], pk[6], pk[7]};
        seg_step++;
        if (g32 == 0) s_alpha[hb * 32 + lane] = alpha;
        if (lane == 0) s_flag[hb] = any ? 1 : 0;
        if (seg_last) {
          const float ltot = l_run + __shfl_xor(l_run, 32);
          if (g32 == 0) {
            s_invl[hb * 32 + lane] = ltot > 0.f ? 1.f / ltot : 0.f;
            a.part_lse[(int64_t)(g + cur.b) * a.h + head] =
                ltot > 0.f ? (m_run + log2f(ltot)) * 0.69314718055994530942f : -INFINITY;
          }
        }
      }
      if (!valid) break;
      if (i + 1 < n) {
        cur = nxt;
        // the next step's scales, used after its score products
        if (kh == 0) load_scales(cur, sc);
        if (seg_last) {
          load_q(cur.b);
          m_run = -INFINITY;
          l_run = 0.f;
          seg_step = 0;
        }
      }
    }
  } else {
    // ================================================================ value waves
    constexpr int MDP = S::MDP;
    const int pw_id = wave - S::NQ;
    const int grp16 = lane >> 4, i16 = lane & 15;
    f32x16 o[MDP][HB];
#pragma unroll
    for (int md = 0; md < MDP; md++)
#pragma unroll
      for (int hb = 0; hb < HB; hb++) o[md][hb] = f32x16{};
    for (int32_t i = 0; i <= n; i++) {
      wg_barrier();
      lds_t* st = ring + ((i + kStages8 - 1) % kStages8) * kStage8;
      const bool have = i > 0;
      Tile prev{};
      if (have) prev = read_tile(win, i - 1);
      const bool last = have && (prev.last || i == n);
      bf16x8 pf[HB][2];
      float inv[HB];
      if (have) {
#pragma unroll
        for (int hb = 0; hb < HB; hb++) {
          if (s_flag[hb]) {
            const float al = s_alpha[hb * 32 + (lane & 31)];
#pragma unroll
            for (int md = 0; md < MDP; md++) o[md][hb] *= al;
          }
          inv[hb] = last ? s_invl[hb * 32 + (lane & 31)] : 0.f;
#pragma unroll
          for (int kk = 0; kk < 2; kk++)
            pf[hb][kk] = *reinterpret_cast<const bf16x8 __attribute__((address_space(3)))*>(
                pbuf + hb * kP8Bytes + (kk * 64 + lane) * 16);
        }
      }
      wg_barrier();
      if (have) {
        // A operand: 8 tokens of latent column 32 mb + 16 (grp16 % 2) + i16 per
        // lane, from the 8-bit transposing read (lane 2 j + h of a 16-lane group
        // reads row j of the group's tokens, bytes 8 h .. 8 h + 7), widened to bf16
        auto ld_c = [&](int md, int kk) -> bf16x8 {
          const int mb = pw_id * MDP + md;
          const int jj = i16 >> 1, h = i16 & 1;
          const int r = 16 * kk + 8 * (jj >> 2) + 4 * (grp16 >> 1) + (jj & 3);
          const int cc = 2 * mb + (grp16 & 1);
          const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              reinterpret_cast<i32x2 __attribute__((address_space(3)))*>(
                  st + r * kCRow8 + ((cc ^ swz8(r)) << 4) + 8 * h));
          const bf16x2 b0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)w[0], 1.f, false);
          const bf16x2 b1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)w[0], 1.f, true);
          const bf16x2 b2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)w[1], 1.f, false);
          const bf16x2 b3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)w[1], 1.f, true);
          const u32x4 u = {__builtin_bit_cast(uint32_t, b0), __builtin_bit_cast(uint32_t, b1),
                           __builtin_bit_cast(uint32_t, b2), __builtin_bit_cast(uint32_t, b3)};
          return __builtin_bit_cast(bf16x8, u);
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
        if (last) {
          const int64_t slot = (int64_t)(g + prev.b);
#pragma unroll
          for (int hb = 0; hb < HB; hb++) {
            uint16_t* dst = static_cast<uint16_t*>(a.part_o) + slot * a.h * kDc8 +
                            part_row(hg * HB + hb, pw_id * MDP, lane);
#pragma unroll
            for (int md = 0; md < MDP; md++) {
              store_block_bf16(dst + md * 32, o[md][hb], inv[hb], lane);
              o[md][hb] = f32x16{};
            }
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 64 heads per work group on the pipelined schedule of the bf16 kernel's
// 64-head variant (eight waves, one barrier per step, value product two steps
// behind the scores), with this file's fp8 arithmetic:
//
//  * w0, w1: score waves, key half kh (latent bytes 256 kh .. 256 kh + 255: four
//    64-byte blocks, each against both query terms of both 32-head blocks, so
//    every A fragment feeds four fp8 products).  Each publishes its latent
//    partial times 2^-k of its half, then runs the rope part (bf16, four
//    products) of head block kh and publishes it separately: the token scale
//    applies to the latent part only.  The rope query waits in LDS.
//  * w4, w5: softmax waves for head blocks 0 and 1: in step j they form
//    s = scale_t (x0 + x1) + rope of step j - 1 (the token scale applies to the
//    latent part only; the scales sit in the tile's stage and are read in step
//    j - 1), run the online softmax (normaliser over p) and publish the bf16
//    weights p * scale_t.
//  * w2, w3, w6, w7: value waves, latent columns 128 v .. 128 v + 127 of both
//    head blocks; the 8-bit transposing read of tile j in step j (raw bytes
//    kept in registers), widened to bf16 in step j + 2 for the products with
//    that step's weights.  w2 and w3 are the two loader waves (eleven loads
//    each per step), issued after their products.
//
// A stage of the ring is the 20 KiB tile plus its 32 token scales (loaded with
// the tile, so that no wave waits on a global load in the step loop); three
// stages, loads two steps ahead.
constexpr int kStageF = kStage8 + 256;              // tile, then 128 B of scales
constexpr int kStagesF = 3;
constexpr int kRingF = kStagesF * kStageF;
constexpr int kXF = 3 * 2 * 64 * 64;                // one step's partials: [x0, x1, rope][hb][4][64][16 B]
constexpr int kPF = 2 * kP8Bytes;                   // one step's weights: [hb]
constexpr int kQrF = 2 * kRopeKs * 64 * 16;        // rope query of both head blocks, per lane
constexpr int kLdsF = kRingF + kWinBytes + 2 * kXF + 2 * kPF + kQrF + 2 * 2 * 32 * 4 * 2 + 2 * 2 * 4;
static_assert(kLdsF <= 160 * 1024, "LDS budget of one compute unit");

// Loads of the value-wave loaders (two steps ahead, as in the bf16 kernel):
// the loads of step i + 2 are issued in step i, into the stage step i - 1
// read.  Loader 0 refills descriptor window w + 1 into the buffer of window
// w - 1 together with the loads of step kWin w + 4, issued in step kWin w + 2,
// when every wave has left window w - 1.
template <int NL, bool SP>
struct LoaderF {
  static_assert(NL == 2 && !SP, "two loader waves, dense tables");
  // the tile's loads and one 4-byte load of 16 token scales (loader lw: tokens 16 lw ..)
  static constexpr int kPerWave = StepIssue8<NL, SP>::kPer + 1;
  int32_t next;
  int32_t n;
  bool newer_issued;

  __device__ void issue_next(const AttnArgs& a, lds_t* ring, lds_t* win, int32_t t_begin, int lw,
                             int lane, const Tile& d) {
    if (lw == 0 && next >= kWin + 4 && next % kWin == 4 && next + kWin - 4 < n)
      load_window(a, win, t_begin, t_begin + n, next / kWin + 1, lane);
    lds_t* stage = ring + (next % kStagesF) * kStageF;
    StepIssue8<NL, SP>::issue(a, stage, d, lw, lane);
    if (lane < 16) {
      const int32_t r = min(16 * lw + lane, d.nv - 1);  // rows past the end repeat the last token
      const int64_t slot = d.blk >= 0 ? (int64_t)d.blk * a.P + d.off + r
                                      : phys_slot(a.block_table, d.b, d.t0 + r, a.P, a.max_blocks,
                                                  a.num_blocks);
      dma4(a.c_kv_scale + slot, stage + kStage8 + 64 * lw);
    }
    next++;
  }
  __device__ void start(const AttnArgs& a, lds_t* ring, lds_t* win, int32_t t_begin, int32_t steps,
                        int lw, int lane) {
    next = 0;
    n = steps;
    for (int s = 0; s < 2 && next < n; s++)
      issue_next(a, ring, win, t_begin, lw, lane, global_tile(a, t_begin + next));
    newer_issued = next == 2;
  }
  __device__ Tile peek(const lds_t* win) const { return next < n ? read_tile(win, next) : Tile{}; }
  // Wait for this wave's loads of step i; what may stay in flight: the batch
  // of step i + 1 and sb groups of KS stores issued after the awaited batch
  // (counts exact or smaller, clamped to the counter's range).
  template <int KS>
  __device__ void wait_current(int sb) {
    constexpr int C0 = kPerWave, C1 = kPerWave + KS < 63 ? kPerWave + KS : 63,
                  C2 = kPerWave + 2 * KS < 63 ? kPerWave + 2 * KS : 63;
    constexpr int D1 = KS < 63 ? KS : 63, D2 = 2 * KS < 63 ? 2 * KS : 63;
    if (newer_issued) {
      if (sb == 0) wait_vmcnt<C0>();
      else if (sb == 1) wait_vmcnt<C1>();
      else wait_vmcnt<C2>();
    } else {
      if (sb == 0) wait_vmcnt<0>();
      else if (sb == 1) wait_vmcnt<D1>();
      else wait_vmcnt<D2>();
    }
  }
  __device__ void issue_ahead(const AttnArgs& a, lds_t* ring, lds_t* win, int32_t t_begin, int lw,
                              int lane, const Tile& d) {
    if (next < n) {
      issue_next(a, ring, win, t_begin, lw, lane, d);
      newer_issued = true;
    } else {
      newer_issued = false;
    }
  }
};

template <bool SP>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512))) void attend64_fp8_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[kLdsF];
  lds_t* ring = (lds_t*)smem;
  lds_t* win = ring + kRingF;                       // [2][kWin] tile descriptors
  lds_t* xbuf = win + kWinBytes;                    // [2 parity][x0, x1, rope][2 hb][4][64 lanes][16 B]
  lds_t* pbuf = xbuf + 2 * kXF;                     // [2 parity][2 hb][2 k-steps][64 lanes][16 B]
  lds_t* qrbuf = pbuf + 2 * kPF;                    // [2 hb][4 k-steps][64 lanes][16 B]
  float* s_alpha = (float*)(smem + kRingF + kWinBytes + 2 * kXF + 2 * kPF + kQrF);  // [2][2][32]
  float* s_invl = s_alpha + 2 * 2 * 32;             // [2][2][32]
  int* s_flag = (int*)(s_invl + 2 * 2 * 32);        // [2][2]
  constexpr int kXPart = 2 * 64 * 64;               // one partial of both head blocks

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g32 = lane >> 5;

  const int32_t HG = a.h / 64;
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
  select_latent_group(a, hg * 64);
  const int32_t n_total = load_ro(a.cu_tiles, a.B);
  if (n_total == 0) return;
  const int32_t t_begin = load_ro(a.split_first, g);
  const int32_t t_end = load_ro(a.split_first, g + 1);
  if (t_begin >= t_end) return;
  const int32_t n = t_end - t_begin;
  const float sm = a.sm_scale_log2;

  if (wave < 2) {
    // ================================================================ score waves
    const int kh = wave;
    const int row = lane & 31;
    i32x8 qhi[2][kBlocksHalf], qlo[2][kBlocksHalf];
    float qinv[2];
    // the absorbed query of sequence bb for both head blocks: the key half's
    // latent values as two E4M3 terms times 2^k (max |q| 2^k in [128, 256));
    // awaited here
    auto load_q = [&](int32_t bb) {
#pragma unroll
      for (int hb = 0; hb < 2; hb++) {
        const int32_t head = hg * 64 + hb * 32 + (lane & 31);
        const uint16_t* qp = static_cast<const uint16_t*>(a.q_lat) + ((int64_t)bb * a.h + head) * (kDc8 + kDr8);
        auto chunk = [&](int kb, int c) -> u32x4 {
          return *reinterpret_cast<const u32x4*>(qp + 64 * (kh * kBlocksHalf + kb) + 32 * g32 + 8 * c);
        };
        auto elem = [](const u32x4& w, int e) -> float {
          const uint32_t x = w[e >> 1];
          return __uint_as_float((e & 1) ? (x & 0xffff0000u) : (x << 16));
        };
        // (one block at a time: the query registers of both head blocks are
        // live here, so the raw chunks must not all be in flight at once)
        float mx = 0.f;
#pragma unroll 1
        for (int kb = 0; kb < kBlocksHalf; kb++) {
          u32x4 w[4];
#pragma unroll
          for (int c = 0; c < 4; c++) w[c] = chunk(kb, c);
#pragma unroll
          for (int c = 0; c < 4; c++)
#pragma unroll
            for (int e = 0; e < 8; e++) mx = fmaxf(mx, fabsf(elem(w[c], e)));
        }
        {
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
          mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        const int k = mx > 0.f ? min(max(8 - __builtin_amdgcn_frexp_expf(mx), -120), 120) : 0;
        const float qs = __builtin_amdgcn_ldexpf(1.f, k);
        qinv[hb] = __builtin_amdgcn_ldexpf(1.f, -k);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < kBlocksHalf; kb++) {
          u32x4 w[4];
#pragma unroll
          for (int c = 0; c < 4; c++) w[c] = chunk(kb, c);
          uint32_t h[8], l[8];
#pragma unroll
          for (int c = 0; c < 4; c++) {
#pragma unroll
            for (int hw = 0; hw < 2; hw++) {
              float x[4], r[4];
#pragma unroll
              for (int e = 0; e < 4; e++) x[e] = elem(w[c], 4 * hw + e) * qs;
              const uint32_t h01 = e4m3_pair(x[0], x[1]), h23 = e4m3_pair(x[2], x[3]);
              r[0] = x[0] - __builtin_amdgcn_cvt_f32_fp8((int)h01, 0);
              r[1] = x[1] - __builtin_amdgcn_cvt_f32_fp8((int)h01, 1);
              r[2] = x[2] - __builtin_amdgcn_cvt_f32_fp8((int)h23, 0);
              r[3] = x[3] - __builtin_amdgcn_cvt_f32_fp8((int)h23, 1);
              h[2 * c + hw] = h01 | (h23 << 16);
              l[2 * c + hw] = e4m3_pair(r[0], r[1]) | (e4m3_pair(r[2], r[3]) << 16);
            }
          }
          qhi[hb][kb] = i32x8{(int)h[0], (int)h[1], (int)h[2], (int)h[3], (int)h[4], (int)h[5], (int)h[6], (int)h[7]};
          qlo[hb][kb] = i32x8{(int)l[0], (int)l[1], (int)l[2], (int)l[3], (int)l[4], (int)l[5], (int)l[6], (int)l[7]};
          __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      wait_vmcnt<0>();
    };
    // the rope part of the scores of head block kh: the rope query of the
    // current sequence waits in LDS (each lane reads back what it wrote),
    // which keeps it out of the registers of the latent query
    lds_t* qrl = qrbuf + kh * kRopeKs * 1024 + lane * 16;
    auto store_qr = [&](int32_t bb) {
      const int32_t head = hg * 64 + kh * 32 + (lane & 31);
      const uint16_t* qp = static_cast<const uint16_t*>(a.q_lat) + ((int64_t)bb * a.h + head) * (kDc8 + kDr8);
#pragma unroll
      for (int kr = 0; kr < kRopeKs; kr++)
        *reinterpret_cast<bf16x8 __attribute__((address_space(3)))*>(qrl + kr * 1024) =
            *reinterpret_cast<const bf16x8*>(qp + kDc8 + 16 * kr + 8 * g32);
    };
    Tile cur = global_tile(a, t_begin);
    store_qr(cur.b);
    if (wave == 1) {
      load_window(a, win, t_begin, t_end, 0, lane);
      if (n > kWin) load_window(a, win, t_begin, t_end, 1, lane);
    }
    load_q(cur.b);
    wg_barrier();
    for (int32_t j = 0; j <= n + 1; j++) {
      wg_barrier();
      if (j < n) {
        const lds_t* st = ring + (j % kStagesF) * kStageF;
        auto ld_a = [&](int kb) -> i32x8 {  // key bytes 64 kb + 32 g32 .. +31 of row `row`
          const int c0 = 4 * (kh * kBlocksHalf + kb) + 2 * g32;
          const i32x4 x0 = *reinterpret_cast<const i32x4 __attribute__((address_space(3)))*>(
              st + row * kCRow8 + ((c0 ^ swz8(row)) << 4));
          const i32x4 x1 = *reinterpret_cast<const i32x4 __attribute__((address_space(3)))*>(
              st + row * kCRow8 + (((c0 + 1) ^ swz8(row)) << 4));
          return i32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        };
        const Tile nxt = j + 1 < n ? read_tile(win, j + 1) : Tile{};
        f32x16 s0 = f32x16{}, s1 = f32x16{};
        i32x8 av = ld_a(0);
#pragma unroll
        for (int kb = 0; kb < kBlocksHalf; kb++) {
          const i32x8 an = kb + 1 < kBlocksHalf ? ld_a(kb + 1) : av;
          s0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, qhi[0][kb], s0, 0, 0, 0, 127, 0, 127);
          s1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, qhi[1][kb], s1, 0, 0, 0, 127, 0, 127);
          s0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, qlo[0][kb], s0, 0, 0, 0, 127, 0, 127);
          s1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, qlo[1][kb], s1, 0, 0, 0, 127, 0, 127);
          av = an;
          __builtin_amdgcn_sched_barrier(0);
        }
        lds_t* xb = xbuf + (j & 1) * kXF + kh * kXPart + lane * 16;
#pragma unroll
        for (int q = 0; q < 4; q++) {
          *reinterpret_cast<f32x4 __attribute__((address_space(3)))*>(xb + 1024 * q) =
              f32x4{s0[4 * q] * qinv[0], s0[4 * q + 1] * qinv[0], s0[4 * q + 2] * qinv[0], s0[4 * q + 3] * qinv[0]};
          *reinterpret_cast<f32x4 __attribute__((address_space(3)))*>(xb + 4096 + 1024 * q) =
              f32x4{s1[4 * q] * qinv[1], s1[4 * q + 1] * qinv[1], s1[4 * q + 2] * qinv[1], s1[4 * q + 3] * qinv[1]};
        }
        {
          f32x16 r = f32x16{};
#pragma unroll
          for (int kr = 0; kr < kRopeKs; kr++) {
            const bf16x8 ar = *reinterpret_cast<const bf16x8 __attribute__((address_space(3)))*>(
                st + kStageC8 + row * kRRow8 + (((2 * kr + g32) ^ swz_r8(row)) << 4));
            const bf16x8 qk = *reinterpret_cast<const bf16x8 __attribute__((address_space(3)))*>(qrl + kr * 1024);
            r = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ar, qk, r, 0, 0, 0);
          }
          lds_t* rb = xbuf + (j & 1) * kXF + 2 * kXPart + kh * 4096 + lane * 16;
#pragma unroll
          for (int q = 0; q < 4; q++)
            *reinterpret_cast<f32x4 __attribute__((address_space(3)))*>(rb + 1024 * q) =
                f32x4{r[4 * q], r[4 * q + 1], r[4 * q + 2], r[4 * q + 3]};
        }
        // a new segment's query, read and split before the next step
        if (j + 1 < n) {
          if (cur.last) {
            load_q(nxt.b);
            store_qr(nxt.b);
          }
          cur = nxt;
        }
      }
    }
  } else if (wave == 4 || wave == 5) {
    // ================================================================ softmax waves
    const int hb = wave - 4;
    const int32_t head = hg * 64 + hb * 32 + (lane & 31);
    float sc[16];  // token scales of the step being normalised: rows 8 (jj/4) + 4 g32 + jj%4
    wg_barrier();
    float m_run = -INFINITY, l_run = 0.f;
    int32_t seg_step = 0;
    for (int32_t j = 0; j <= n + 1; j++) {
      wg_barrier();
      // the token scales of tile j (in LDS during step j), used in step j + 1;
      // the previous step's are consumed below first
      float sc_next[16] = {};
      if (j < n) {
        const lds_t* st = ring + (j % kStagesF) * kStageF;
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const f32x4 v = *reinterpret_cast<const f32x4 __attribute__((address_space(3)))*>(
              st + kStage8 + (8 * q + 4 * g32) * 4);
#pragma unroll
          for (int e = 0; e < 4; e++) sc_next[4 * q + e] = v[e];
        }
      }
      if (j >= 1 && j <= n) {
        const int par = (j - 1) & 1;
        const Tile pv = read_tile(win, j - 1);
        const bool seg_last = pv.last || j == n;
        f32x16 s;
        const lds_t* x0 = xbuf + par * kXF + hb * 4096 + lane * 16;
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const f32x4 u = *reinterpret_cast<const f32x4 __attribute__((address_space(3)))*>(x0 + 1024 * q);
          const f32x4 w = *reinterpret_cast<const f32x4 __attribute__((address_space(3)))*>(x0 + kXPart + 1024 * q);
          const f32x4 r = *reinterpret_cast<const f32x4 __attribute__((address_space(3)))*>(x0 + 2 * kXPart + 1024 * q);
#pragma unroll
          for (int e = 0; e < 4; e++) s[4 * q + e] = __builtin_fmaf(u[e] + w[e], sc[4 * q + e], r[e]);
        }
        if (pv.nv < kStep8) {
#pragma unroll
          for (int jj = 0; jj < 16; jj++)
            if (8 * (jj >> 2) + 4 * g32 + (jj & 3) >= pv.nv) s[jj] = -INFINITY;
        }
        float mx = s[0];
#pragma unroll
        for (int jj = 1; jj < 16; jj++) mx = fmaxf(mx, s[jj]);
        {
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                           false, false);
          mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        const float mt = mx * sm;
        const float thr = seg_step < kExactSteps8 ? 0.f : kLazy8;
        const bool any = __any(mt > m_run + thr);
        float alpha = 1.f;
        if (any) {
          const float m_new = fmaxf(m_run, mt);
          alpha = __builtin_amdgcn_exp2f(m_run - m_new);
          l_run *= alpha;
          m_run = m_new;
        }
        const float mref = m_run == -INFINITY ? 0.f : m_run;
        // weights p * scale_t rounded to bf16 (the value product's operand);
        // the normaliser sums the weights that product consumes, those bf16
        // values divided by scale_t (p where the scale is 0), so that their
        // rounding cancels in the normalised output as in the bf16 path
        uint32_t pk[8];
        float lsum = 0.f;
#pragma unroll
        for (int q = 0; q < 8; q++) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * q], sm, -mref));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * q + 1], sm, -mref));
          const float c0 = sc[2 * q], c1 = sc[2 * q + 1];
          const f32x2 e = {p0 * c0, p1 * c1};
          const bf16x2 pr = __builtin_convertvector(e, bf16x2);
          pk[q] = __builtin_bit_cast(uint32_t, pr);
          const f32x2 back = __builtin_convertvector(pr, f32x2);
          lsum += (c0 != 0.f ? back[0] * __builtin_amdgcn_rcpf(c0) : p0) +
                  (c1 != 0.f ? back[1] * __builtin_amdgcn_rcpf(c1) : p1);
        }
        l_run += lsum;
        lds_t* pb = pbuf + par * kPF + hb * kP8Bytes + lane * 16;
        *reinterpret_cast<u32x4 __attribute__((address_space(3)))*>(pb) = u32x4{pk[0], pk[1], pk[2], pk[3]};
        *reinterpret_cast<u32x4 __attribute__((address_space(3)))*>(pb + 64 * 16) =
            u32x4{pk[4], pk[5], pk[6], pk[7]};
        seg_step++;
        if (g32 == 0) s_alpha[(par * 2 + hb) * 32 + lane] = alpha;
        if (lane == 0) s_flag[par * 2 + hb] = any ? 1 : 0;
        if (seg_last) {
          const float ltot = l_run + __shfl_xor(l_run, 32);
          if (g32 == 0) {
            s_invl[(par * 2 + hb) * 32 + lane] = ltot > 0.f ? 1.f / ltot : 0.f;
            const int64_t slot = (int64_t)(g + pv.b);
            a.part_lse[slot * a.h + head] =
                ltot > 0.f ? (m_run + log2f(ltot)) * 0.69314718055994530942f : -INFINITY;
          }
          m_run = -INFINITY;
          l_run = 0.f;
          seg_step = 0;
        }
      }
#pragma unroll
      for (int e = 0; e < 16; e++) sc[e] = sc_next[e];
    }
  } else {
    // ================================================================ value waves
    const int v = (wave & 1) | ((wave >> 2) << 1);  // w2 -> 0, w3 -> 1, w6 -> 2, w7 -> 3
    constexpr int MD = 4;
    const int grp16 = lane >> 4, i16 = lane & 15;
    // raw fp8 fragments of two steps: slot j % 2 holds those of step j - 2
    // until its products are issued, then receives those of step j
    i32x2 cb[2][MD][2];
    // 8 tokens of latent column 32 mb + 16 (grp16 % 2) + i16 per lane, from the
    // 8-bit transposing read (lane 2 jj + h of a 16-lane group reads row jj of
    // the group's tokens, bytes 8 h .. 8 h + 7)
    auto ld_c = [&](const lds_t* st, int md, int kk) -> i32x2 {
      const int mb = v * MD + md;
      const int jj = i16 >> 1, h = i16 & 1;
      const int r = 16 * kk + 8 * (jj >> 2) + 4 * (grp16 >> 1) + (jj & 3);
      const int cc = 2 * mb + (grp16 & 1);
      return __builtin_amdgcn_ds_read_tr8_b64_v2i32(reinterpret_cast<i32x2 __attribute__((address_space(3)))*>(
          const_cast<lds_t*>(st) + r * kCRow8 + ((cc ^ swz8(r)) << 4) + 8 * h));
    };
    auto widen = [](const i32x2& w) -> bf16x8 {  // every E4M3 value is a bf16 value
      const bf16x2 b0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)w[0], 1.f, false);
      const bf16x2 b1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)w[0], 1.f, true);
      const bf16x2 b2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)w[1], 1.f, false);
      const bf16x2 b3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)w[1], 1.f, true);
      const u32x4 u = {__builtin_bit_cast(uint32_t, b0), __builtin_bit_cast(uint32_t, b1),
                       __builtin_bit_cast(uint32_t, b2), __builtin_bit_cast(uint32_t, b3)};
      return __builtin_bit_cast(bf16x8, u);
    };
    auto stage_of = [&](int32_t j) -> const lds_t* {
      int off = (j % kStagesF) * kStageF;
      asm volatile("" : "+s"(off));
      return ring + off;
    };
    constexpr int kVStores = 2 * MD * 2;  // two 16-byte stores per 32-value block and head block
    const bool loader = v < 2;
    LoaderF<2, SP> ld;
    if (loader) ld.start(a, ring, win, t_begin, n, v, lane);
    int sb1 = 0, sb2 = 0;
    wg_barrier();
    // steps 0 and 1: fragments only
    if (loader) ld.template wait_current<kVStores>(0);
    wg_barrier();
    if (loader) ld.issue_ahead(a, ring, win, t_begin, v, lane, ld.peek(win));
#pragma unroll
    for (int md = 0; md < MD; md++)
#pragma unroll
      for (int kk = 0; kk < 2; kk++) cb[0][md][kk] = ld_c(stage_of(0), md, kk);
    if (loader) ld.template wait_current<kVStores>(0);
    wg_barrier();
    if (loader) ld.issue_ahead(a, ring, win, t_begin, v, lane, ld.peek(win));
    if (n > 1) {
#pragma unroll
      for (int md = 0; md < MD; md++)
#pragma unroll
        for (int kk = 0; kk < 2; kk++) cb[1][md][kk] = ld_c(stage_of(1), md, kk);
    }
    f32x16 o[MD][2];
#pragma unroll
    for (int md = 0; md < MD; md++) o[md][0] = o[md][1] = f32x16{};
    // step j >= 2: O += C(j-2) P(j-2), then the fragments of step j
    auto step = [&](auto slot_c, int32_t j) __attribute__((always_inline)) {
      constexpr int SL = decltype(slot_c)::value;  // j % 2, also the parity of step j - 2
      if (loader) ld.template wait_current<kVStores>(sb1 + sb2);
      wg_barrier();
      const bool load = j < n;
      const lds_t* st = stage_of(j);
      bf16x8 pf[2][2];
#pragma unroll
      for (int hb = 0; hb < 2; hb++)
#pragma unroll
        for (int kk = 0; kk < 2; kk++)
          pf[hb][kk] = *reinterpret_cast<const bf16x8 __attribute__((address_space(3)))*>(
              pbuf + SL * kPF + hb * kP8Bytes + (kk * 64 + lane) * 16);
      const int flag = s_flag[SL * 2] | s_flag[SL * 2 + 1];
      const Tile nd = loader ? ld.peek(win) : Tile{};
      if (__builtin_amdgcn_readfirstlane(flag)) {
        const float a0 = s_alpha[(SL * 2) * 32 + (lane & 31)];
        const float a1 = s_alpha[(SL * 2 + 1) * 32 + (lane & 31)];
#pragma unroll
        for (int md = 0; md < MD; md++) {
          o[md][0] *= a0;
          o[md][1] *= a1;
        }
      }
#pragma unroll
      for (int md = 0; md < MD; md++) {
#pragma unroll
        for (int kk = 0; kk < 2; kk++) {
          const bf16x8 c = widen(cb[SL][md][kk]);
#pragma unroll
          for (int hb = 0; hb < 2; hb++)
            o[md][hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(c, pf[hb][kk], o[md][hb], 0, 0, 0);
        }
        if (load) {
#pragma unroll
          for (int kk = 0; kk < 2; kk++) cb[SL][md][kk] = ld_c(st, md, kk);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (loader) ld.issue_ahead(a, ring, win, t_begin, v, lane, nd);
      const Tile pv = read_tile(win, j - 2);
      int sb = 0;
      if (pv.last || j - 2 == n - 1) {
        const int64_t slot = (int64_t)(g + pv.b);
        sb = 1;
#pragma unroll
        for (int hb = 0; hb < 2; hb++) {
          const float inv = s_invl[(SL * 2 + hb) * 32 + (lane & 31)];
          uint16_t* dst = static_cast<uint16_t*>(a.part_o) + slot * a.h * kDc8 +
                          part_row(hg * 2 + hb, v * MD, lane);
#pragma unroll
          for (int md = 0; md < MD; md++) {
            store_block_bf16(dst + md * 32, o[md][hb], inv, lane);
            o[md][hb] = f32x16{};
          }
        }
      }
      sb2 = sb1;
      sb1 = sb;
    };
    for (int32_t j = 2; j <= n + 1; j += 2) {
      step(std::integral_constant<int, 0>{}, j);
      if (j + 1 > n + 1) break;
      step(std::integral_constant<int, 1>{}, j + 1);
    }
  }
}

int32_t heads_per_group8(int32_t heads) { return heads % 64 == 0 ? 64 : 32; }

}  // namespace

bool mfma_fp8_supported(const mla_decode_params& p) {
  return p.cache_dtype == MLA_FP8_E4M3 && p.rope_dtype == MLA_BF16 && p.d_latent == kDc8 &&
         p.d_rope == kDr8 && p.num_heads % 32 == 0;
}

hipError_t launch_attend_fp8(const AttnArgs& a, hipStream_t s, hipEvent_t ev_start,
                             hipEvent_t ev_stop) {
  if (a.d_c != kDc8 || a.d_r != kDr8 || a.h % 32 || !a.c_kv_scale) return hipErrorInvalidValue;
  const int32_t hpg = heads_per_group8(a.h);
  const int32_t HG = a.h / hpg;
  if (HG > 1 && a.splits % 8) return hipErrorInvalidValue;
  const dim3 grid(a.splits * HG);
  const bool sp = a.slots != nullptr;
  if (hpg == 64 && !sp)
    launch_timed(attend64_fp8_kernel<false>, grid, dim3(512), s, ev_start, ev_stop, a);
  else if (hpg == 64)
    launch_timed(attend_fp8_kernel<2, true>, grid, dim3(Shape8<2>::NW * 64), s, ev_start, ev_stop, a);
  else if (!sp)
    launch_timed(attend_fp8_kernel<1, false>, grid, dim3(Shape8<1>::NW * 64), s, ev_start, ev_stop, a);
  else
    launch_timed(attend_fp8_kernel<1, true>, grid, dim3(Shape8<1>::NW * 64), s, ev_start, ev_stop, a);
  return hipGetLastError();
}

}  // namespace mla
