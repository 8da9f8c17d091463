// Matrix-core split attention over the paged latent cache (gfx950).
//
// Shape: d_c = 512 latent values + d_r = 64 rope values per cached token,
// heads a multiple of 32, bf16 latent/rope rows, bf16 absorbed query.
//
// Work decomposition.  A token split g owns a contiguous run of 32-token tiles
// of the concatenated sequences ("split plan" in mla_common.hpp); one tile is
// one pipeline step.  Its heads are served by HG work groups of 32*HB heads
// each (HB = 2 for 64 heads, 1 for 32); the HG groups of one split get
// workgroup ids that differ by a multiple of 8 and are dispatched together, so
// they run on the same XCD and the second read of every tile is served by that
// XCD's L2.
//
// Every step is described by the tile descriptor the planning kernel wrote
// (page, sequence, first token, valid tokens, last-of-sequence flag).  The
// descriptors of a split are contiguous; they are brought into a two-buffer
// LDS window of 64 tiles by direct global->LDS loads, so the per-step
// bookkeeping of every wave is one LDS read.
//
// Inside a work group the waves specialise:
//  * 2*HB score waves.  Wave (hb, kh) holds the absorbed query of 32 heads for
//    one part of the 576-wide key (kh = 0: latent 0..255; kh = 1: latent
//    256..511 and the 64 rope values) in registers and computes, for each step,
//      S^T[t, i] = sum_d KV[t, d] Q[i, d]      (MFMA 32x32x16 bf16, M = tokens,
//                                              N = heads, K = its key part)
//    The kh = 1 wave hands its partial scores to its partner through LDS; in
//    the next step the partner adds them to its own, runs the online softmax
//    (one lane = one head) and publishes the bf16 weights P, the per-head
//    rescale factors and, at the end of a sequence segment, 1/l and the
//    log-sum-exp.  The kh = 0 part is the shorter one: its wave also runs the
//    softmax.
//  * 4*HB value waves.  Each owns a slice of 64 (HB = 2) or 128 (HB = 1)
//    latent rows of the output for all heads of the group and computes
//      O^T[d, i] += sum_t C[t, d] P[i, t]      (M = latent rows, N = heads,
//                                              K = tokens)
//    two steps behind the score waves.  It reads its latent fragments of a
//    step with the transposing LDS read in the step of that tile and keeps
//    them in registers until the weights arrive; each such read feeds HB
//    MFMAs.  The weights are in a permuted token order (slot i of lane group
//    g is token 8*(i/4) + 4*g + i%4 of the 16-token k-step) that matches the
//    score accumulator layout, and the latent tile is read in the same order.
//    The first four value waves issue the tile loads.
//
// LDS ring.  Three stages of one step: 32 latent rows of 1 KiB and 32 rope
// rows of 128 B, written by direct global->LDS 16-byte loads (one instruction
// per latent row, eight rope rows per instruction) two steps ahead of use.
// Every wave reads a stage only in the step of its tile, so a stage is free
// again one step later.  The 16-byte chunk index is XOR-swizzled with a
// permutation of the row's low four bits, which keeps both the row reads of
// the score product and the 4-row transposing reads of the value product
// free of bank conflicts (64 four-byte banks).  The partial scores, weights
// and rescale factors are double-buffered by step parity.
//
// Step j (one work-group barrier; every wave runs n + 2 steps):
//   loader waves wait for their loads of step j; barrier
//   loader waves: issue the loads of step j + 2
//   score waves kh = 0: softmax of step j - 1, publish P(j-1); partial S(j)
//   score waves kh = 1: partial S(j), hand it over
//   value waves: read P(j-2) and the latent fragments of step j;
//                O += C(j-2) P(j-2); at a segment end, store the partial.
// The barrier of step j + 1 orders what step j published before its readers.
//
// Softmax rescaling is lazy: after the first four steps of a sequence segment
// (which track the exact maximum, so an early dominant token gets weight
// exactly 1), the running maximum is only raised when a step's maximum
// exceeds it by more than 2^8 in weight, so the output accumulator is rarely
// rescaled; weights stay below 2^8.  The normaliser is the sum of the
// bf16-rounded weights that the MFMA consumes.
#include "mla_mfma_util.hpp"

#include <hip/hip_ext.h>

#include <type_traits>

namespace mla {
namespace {

constexpr int kDc = 512, kDr = 64;
constexpr int kStep = kTile;                      // tokens per pipeline step
constexpr int kCRow = kDc * 2;                    // 1024 bytes per latent row
constexpr int kRRow = kDr * 2;                    // 128 bytes per rope row
constexpr int kStageC = kStep * kCRow;            // 32768
constexpr int kStage = kStageC + kStep * kRRow;   // 36864
constexpr int kStages = 3;
constexpr int kRing = kStages * kStage;           // 110592
constexpr int kLoadsPerStep = kStep + kStep / 8;  // 32 latent rows + 4 rope groups
constexpr int kKs0 = 16, kKs1 = 20;               // score k-steps of the two key parts (36 in all)
constexpr int kNL = 4;                            // loader waves (the first value waves)
constexpr int kXBytes = 64 * 64;                  // one wave's partial scores
constexpr int kPBytes = 2 * 64 * 16;              // weights of one head block, two k-steps
constexpr float kLazy = 8.0f;                     // log2 of the largest unnormalised weight
constexpr int kExactSteps = 4;                    // steps per segment with an exact maximum
static_assert(kStep == 32, "the score and value products are laid out for 32-token steps");
static_assert(kKs0 + kKs1 == (kDc + kDr) / 16, "the key parts cover the whole key");

template <int HB>
struct Shape {
  static constexpr int NQ = 2 * HB;             // score waves
  static constexpr int NP = 4 * HB;             // value waves
  static constexpr int NW = NQ + NP;
  static constexpr int MDP = kDc / 32 / NP;     // 32-row output blocks per value wave
  static constexpr int kStores = MDP * 4 * HB;  // partial-output stores of a value wave per segment
  // ring | descriptor window | xbuf [2][HB] | pbuf [2][HB] | alpha, 1/l [2][HB][32] | flag [2][HB]
  static constexpr int LDS =
      kRing + kWinBytes + 2 * HB * (kXBytes + kPBytes) + 2 * HB * 32 * 4 * 2 + 2 * HB * 4;
};

// Chunk swizzles (LDS of 64 four-byte banks, one 256-byte bank line).  Latent
// rows: row bits (b3 b2 b1 b0) -> chunk bits (b1 b0 b3 b2), so 16 consecutive
// rows read at one chunk index hit 16 different chunks of the bank line (the
// score product's 16-byte row reads), and so do the 4-row groups of the
// transposing reads (rows 4m..4m+3 map to chunk bits b3 b2 = 0..3 and each lane
// group adds its own chunk bits b1 b0).  Rope rows share bank lines in pairs.
__device__ inline int swz_c(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ inline int swz_r(int r) { return (r >> 1) & 7; }

// Direct-to-LDS loads of one step, issued by the NL loader waves: wave lw
// loads latent rows lw, lw + NL, ... and rope groups lw, lw + NL, ...
// (kLoadsPerStep / NL loads per wave on every path).  A full step inside one
// page takes straight-line code: one scalar base per step, one offset per
// row.  Otherwise rows past the end repeat the last valid token (finite data,
// masked in the softmax) and, when a step can span pages, every lane looks up
// its own block.
template <int NL, bool SP>
__device__ __forceinline__ void issue_step(const AttnArgs& a, lds_t* stage, const Tile& d, int lw,
                                  int lane) {
  static_assert(kStep % NL == 0 && (kStep / 8) % NL == 0, "uniform row assignment");
  // recompute the per-lane offsets in every call instead of keeping them live
  // across the step loop (they would cost registers in every wave)
  asm volatile("" : "+v"(lane));
  const uint32_t st = (uint32_t)(uintptr_t)stage;
  const int64_t base = (int64_t)d.blk * a.P + d.off;
  if (d.blk >= 0 && d.nv == kStep) {
    const char* cb = static_cast<const char*>(a.c_kv) + base * kCRow;
    const char* rb = static_cast<const char*>(a.k_rope) + base * kRRow;
    const uint32_t l16 = (uint32_t)lane << 4;
#pragma unroll
    for (int m = 0; m < kStep / NL; m++) {
      const int r = lw + NL * m;
      dma16s(cb, (l16 ^ ((uint32_t)swz_c(r) << 4)) + (uint32_t)(r * kCRow), st + r * kCRow);
    }
#pragma unroll
    for (int m = 0; m < kStep / 8 / NL; m++) {
      const int j = lw + NL * m;
      const int r = 8 * j + (lane >> 3);
      dma16s(rb, (uint32_t)(r * kRRow + (((lane & 7) ^ swz_r(r)) << 4)), st + kStageC + j * 1024);
    }
    return;
  }
  const char* ckv = static_cast<const char*>(a.c_kv);
  const char* krp = static_cast<const char*>(a.k_rope);
  const int32_t rmax = d.nv - 1;
  if constexpr (SP) {
    // sparse: slots from the planner's list, read with scalar loads (one row
    // per latent load; the eight rows of a rope load picked per lane)
#pragma unroll
    for (int m = 0; m < kStep / NL; m++) {
      const int r = lw + NL * m;
      const int64_t slot = sparse_slot_uniform(a, d.b, d.t0 + min(r, rmax));
      dma16(ckv + slot * kCRow + ((lane ^ swz_c(r)) << 4), stage + r * kCRow);
    }
#pragma unroll
    for (int m = 0; m < kStep / 8 / NL; m++) {
      const int j = lw + NL * m;
      int32_t sl = 0;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const int32_t si = sparse_slot_uniform(a, d.b, d.t0 + min(8 * j + i, rmax));
        sl = (lane >> 3) == i ? si : sl;
      }
      const int r = 8 * j + (lane >> 3);
      dma16(krp + (int64_t)sl * kRRow + (((lane & 7) ^ swz_r(r)) << 4), stage + kStageC + j * 1024);
    }
    return;
  }
#pragma unroll
  for (int m = 0; m < kStep / NL; m++) {
    const int r = lw + NL * m;
    const int64_t slot = d.blk >= 0 ? base + min(r, rmax)
                                    : phys_slot(a.block_table, d.b, d.t0 + min(r, rmax), a.P,
                                                a.max_blocks, a.num_blocks);
    dma16(ckv + slot * kCRow + ((lane ^ swz_c(r)) << 4), stage + r * kCRow);
  }
#pragma unroll
  for (int m = 0; m < kStep / 8 / NL; m++) {
    const int j = lw + NL * m;
    const int r = 8 * j + (lane >> 3);
    const int64_t slot = d.blk >= 0 ? base + min(r, rmax)
                                    : phys_slot(a.block_table, d.b, d.t0 + min(r, rmax), a.P,
                                                a.max_blocks, a.num_blocks);
    dma16(krp + slot * kRRow + (((lane & 7) ^ swz_r(r)) << 4), stage + kStageC + j * 1024);
  }
}

// The load schedule of one of the NL loader waves (lane group lw): the loads
// of step i + 2 are issued in step i, into the stage that step i - 1 read.
// Loader 0 also refills the descriptor window: window w + 1 goes into the
// buffer of window w - 1 together with the loads of step kWin w + 4, issued in
// step kWin w + 2, when every wave has moved past window w - 1 (the value
// waves, the furthest behind, then consume step kWin w).  It is complete
// before step kWin w + 4 starts, long before its first use.
template <int NL, bool SP>
struct Loader {
  static_assert(kLoadsPerStep % NL == 0, "equal load counts per wave");
  static constexpr int kPerWave = kLoadsPerStep / NL;
  int32_t next;        // split-local index of the next step to load
  int32_t n;           // steps of the split
  bool newer_issued;   // the batch after the awaited one was issued

  __device__ void issue_next(const AttnArgs& a, lds_t* ring, lds_t* win, int32_t t_begin, int lw,
                             int lane, bool from_table = false) {
    if (lw == 0 && next >= kWin + 4 && next % kWin == 4 && next + kWin - 4 < n)
      load_window(a, win, t_begin, t_begin + n, next / kWin + 1, lane);
    const Tile d = from_table ? global_tile(a, t_begin + next) : read_tile(win, next);
    issue_step<NL, SP>(a, ring + (next % kStages) * kStage, d, lw, lane);
    next++;
  }
  // The first two steps, issued at kernel entry from the planner's table.
  __device__ void start(const AttnArgs& a, lds_t* ring, lds_t* win, int32_t t_begin, int32_t steps,
                        int lw, int lane) {
    next = 0;
    n = steps;
    for (int s = 0; s < 2 && next < n; s++) issue_next(a, ring, win, t_begin, lw, lane, true);
    newer_issued = next == 2;
  }
  // Wait for this wave's loads of step i.  What may stay in flight: the batch
  // of step i+1 and sb groups of KS partial-output stores issued after the
  // awaited batch (the hardware counter retires in issue order).  The counts
  // are exact or smaller, so the wait never ends early; an extra window load
  // in the newer batch only makes it longer.
  template <int KS>
  __device__ void wait_current(int sb) {
    if (newer_issued) {
      if (sb == 0) wait_vmcnt<kPerWave>();
      else if (sb == 1) wait_vmcnt<kPerWave + KS>();
      else wait_vmcnt<kPerWave + 2 * KS>();
    } else {
      if (sb == 0) wait_vmcnt<0>();
      else if (sb == 1) wait_vmcnt<KS>();
      else wait_vmcnt<2 * KS>();
    }
  }
  // In step i: issue step i+2.
  __device__ void issue_ahead(const AttnArgs& a, lds_t* ring, lds_t* win, int32_t t_begin, int lw,
                              int lane) {
    if (next < n) {
      issue_next(a, ring, win, t_begin, lw, lane);
      newer_issued = true;
    } else {
      newer_issued = false;
    }
  }
};

template <int HB, bool SP>
__global__ __attribute__((amdgpu_flat_work_group_size(Shape<HB>::NW * 64, Shape<HB>::NW * 64)))
void attend_mfma_kernel(AttnArgs a) {
  using S = Shape<HB>;
  __shared__ __attribute__((aligned(1024))) char smem[S::LDS];
  lds_t* ring = (lds_t*)smem;
  lds_t* win = ring + kRing;                        // [2][kWin] tile descriptors
  lds_t* xbuf = win + kWinBytes;                    // [2][HB][4][64 lanes][4 floats]
  lds_t* pbuf = xbuf + 2 * HB * kXBytes;            // [2][HB][2 k-steps][64 lanes][16 B]
  float* s_alpha = (float*)(smem + kRing + kWinBytes + 2 * HB * (kXBytes + kPBytes));  // [2][HB][32]
  float* s_invl = s_alpha + 2 * HB * 32;            // [2][HB][32]
  int* s_flag = (int*)(s_invl + 2 * HB * 32);       // [2][HB]

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
  select_latent_group(a, hg * 32 * HB);  // the host keeps a head group inside one latent group
  const int32_t n_total = load_ro(a.cu_tiles, a.B);
  if (n_total == 0) return;
  const int32_t t_begin = (int32_t)split_begin(n_total, a.splits, g);
  const int32_t t_end = (int32_t)split_begin(n_total, a.splits, g + 1);
  if (t_begin >= t_end) return;
  const int32_t n = t_end - t_begin;  // steps of this split

  // Descriptor windows 0 and 1, visible to every wave after the first
  // barrier; the query and the first two tiles are requested before it.
  auto load_windows = [&]() {
    load_window(a, win, t_begin, t_end, 0, lane);
    if (n > kWin) load_window(a, win, t_begin, t_end, 1, lane);
    wait_vmcnt<0>();
  };
  const float sm = a.sm_scale_log2;

  // Every wave runs n + 2 steps, each opened by one work-group barrier.
  if (wave < S::NQ) {
    // ================================================================ score waves
    const int hb = wave >> 1;
    const int32_t head = hg * 32 * HB + hb * 32 + (lane & 31);
    auto score_wave = [&](auto kh_c) {
      constexpr int KH = decltype(kh_c)::value;
      constexpr int KS = KH ? kKs1 : kKs0;  // k-steps of this key part
      constexpr int K0 = KH ? kKs0 : 0;     // its first k-step
      bf16x8 qf[KS];
      // the absorbed query of sequence bb; awaited explicitly, once per
      // segment (otherwise the compiler, unable to tell whether a segment
      // started, waits for these loads in every step)
      auto issue_q = [&](int32_t bb) {
        const bf16x8* qp = reinterpret_cast<const bf16x8*>(
            static_cast<const uint16_t*>(a.q_lat) + ((int64_t)bb * a.h + head) * (kDc + kDr));
#pragma unroll
        for (int k = 0; k < KS; k++) qf[k] = qp[2 * (K0 + k) + g32];
      };
      Tile cur = global_tile(a, t_begin), prev{};
      issue_q(cur.b);
      if (wave == 1) load_windows();
      wg_barrier();
      wait_vmcnt<0>();
      float m_run = -INFINITY, l_run = 0.f;
      int32_t seg_step = 0;  // steps of the current segment seen so far
      f32x16 s_own = f32x16{};  // KH = 0: own partial scores of the previous step
      for (int32_t j = 0; j <= n + 1; j++) {
        wg_barrier();
        // a new sequence segment starts at step j: its query was requested at
        // the end of step j - 1, before the softmax below stores the previous
        // segment's LSE
        const bool new_seg = j > 0 && j < n && prev.last;
        if (KH == 0 && j >= 1 && j <= n) {
          // ---- softmax of step j - 1: own partial + the partner's from xbuf
          const int par = (j - 1) & 1;
          const bool seg_last = prev.last || j == n;
          f32x16 s = s_own;
          const lds_t* xb = xbuf + (par * HB + hb) * kXBytes + lane * 16;
#pragma unroll
          for (int q = 0; q < 4; q++) {
            const f32x4 o = *reinterpret_cast<const f32x4 __attribute__((address_space(3)))*>(xb + 1024 * q);
            s[4 * q] += o[0];
            s[4 * q + 1] += o[1];
            s[4 * q + 2] += o[2];
            s[4 * q + 3] += o[3];
          }
          // mask the tokens past the end (only the last step of a sequence)
          const int32_t nv = prev.nv;
          if (nv < kStep) {
#pragma unroll
            for (int jj = 0; jj < 16; jj++)
              if (8 * (jj >> 2) + 4 * g32 + (jj & 3) >= nv) s[jj] = -INFINITY;
          }
          // step maximum per head: over the lane's 16 tokens, then across the
          // two lane halves that hold the same head (the scale is positive)
          float mx = s[0];
#pragma unroll
          for (int jj = 1; jj < 16; jj++) mx = fmaxf(mx, s[jj]);
          {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                             false, false);
            mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
          }
          const float mt = mx * sm;
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
          // weights as bf16 pairs (one pair per conversion: extracting elements
          // from a wider bf16 vector is not lowered correctly); the normaliser
          // sums exactly the bf16 weights the value product consumes
          const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);
          uint32_t pk[8];
          float lsum = 0.f;
#pragma unroll
          for (int q = 0; q < 8; q++) {
            const f32x2 e = {__builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * q], sm, -mref)),
                             __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * q + 1], sm, -mref))};
            const bf16x2 pr = __builtin_convertvector(e, bf16x2);
            lsum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lsum, false);
            pk[q] = __builtin_bit_cast(uint32_t, pr);
          }
          l_run += lsum;
          // publish the weights in the value product's operand layout
          lds_t* pb = pbuf + (par * HB + hb) * kPBytes + lane * 16;
          *reinterpret_cast<u32x4 __attribute__((address_space(3)))*>(pb) = u32x4{pk[0], pk[1], pk[2], pk[3]};
          *reinterpret_cast<u32x4 __attribute__((address_space(3)))*>(pb + 64 * 16) =
              u32x4{pk[4], pk[5], pk[6], pk[7]};
          seg_step++;
          if (g32 == 0) s_alpha[(par * HB + hb) * 32 + lane] = alpha;
          if (lane == 0) s_flag[par * HB + hb] = any ? 1 : 0;
          if (seg_last) {
            const float ltot = l_run + __shfl_xor(l_run, 32);
            if (g32 == 0) {
              s_invl[(par * HB + hb) * 32 + lane] = ltot > 0.f ? 1.f / ltot : 0.f;
              const int64_t slot = (int64_t)(g + prev.b);
              a.part_lse[slot * a.h + head] =
                  ltot > 0.f ? (m_run + log2f(ltot)) * 0.69314718055994530942f : -INFINITY;
            }
            m_run = -INFINITY;
            l_run = 0.f;
            seg_step = 0;
          }
        }
        if (j < n) {
          // ---- partial scores of step j over this wave's key part
          if (new_seg) {
            // the softmax stored one LSE after the query loads (KH = 0)
            if (KH == 0)
              wait_vmcnt<1>();
            else
              wait_vmcnt<0>();
          }
          const lds_t* st = ring + (j % kStages) * kStage;
          const int row = lane & 31;
          auto ld_a = [&](int k) -> bf16x8 {
            const int ks = K0 + k;
            const lds_t* p = ks < 32
                ? st + row * kCRow + (((2 * ks + g32) ^ swz_c(row)) << 4)
                : st + kStageC + row * kRRow + (((2 * (ks - 32) + g32) ^ swz_r(row)) << 4);
            return *reinterpret_cast<const bf16x8 __attribute__((address_space(3)))*>(p);
          };
          f32x16 s = f32x16{};
          constexpr int D = 4;
          bf16x8 av[D];
#pragma unroll
          for (int k = 0; k < D; k++) av[k] = ld_a(k);
#pragma unroll
          for (int k = 0; k < KS; k++) {
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[k % D], qf[k], s, 0, 0, 0);
            if (k + D < KS) av[k % D] = ld_a(k + D);
            __builtin_amdgcn_sched_barrier(0);
          }
          if (KH == 1) {
            lds_t* xb = xbuf + ((j & 1) * HB + hb) * kXBytes + lane * 16;
#pragma unroll
            for (int q = 0; q < 4; q++)
              *reinterpret_cast<f32x4 __attribute__((address_space(3)))*>(xb + 1024 * q) =
                  f32x4{s[4 * q], s[4 * q + 1], s[4 * q + 2], s[4 * q + 3]};
          } else {
            s_own = s;
          }
          prev = cur;
          if (j + 1 < n) {
            cur = read_tile(win, j + 1);
            // the products above have read the query registers: the next
            // segment's query can be requested now, a step ahead of its use
            if (prev.last) issue_q(cur.b);
          }
        }
      }
    };
    if (wave & 1)
      score_wave(std::integral_constant<int, 1>{});
    else
      score_wave(std::integral_constant<int, 0>{});
  } else {
    // ================================================================ value waves
    constexpr int MDP = S::MDP;
    const int pw_id = wave - S::NQ;
    const bool loader = pw_id < kNL;
    const int j16 = lane & 15, grp = lane >> 4, e = j16 >> 2, qd = j16 & 3;
    Loader<kNL, SP> ld;
    if (loader) ld.start(a, ring, win, t_begin, n, pw_id, lane);
    wg_barrier();
    int sb1 = 0, sb2 = 0;  // partial-store groups issued in the previous two steps
    f32x16 o[MDP][HB];
#pragma unroll
    for (int md = 0; md < MDP; md++)
#pragma unroll
      for (int hb = 0; hb < HB; hb++) o[md][hb] = f32x16{};
    // latent operand fragments of three steps: those of step j are read at
    // the start of step j and consumed in step j + 2
    bf16x8 cb[3][MDP][2];
    auto ld_c = [&](lds_t* st, int md, int kk) -> bf16x8 {
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
    // step j: issue the reads of P(j-2) and C(j), then O += C(j-2) P(j-2)
    auto step = [&](auto par_c, int32_t j) {
      constexpr int PAR = decltype(par_c)::value;  // j % 3 (also the ring stage of step j)
      constexpr int C = (PAR + 1) % 3;             // buffer of step j - 2
      if (loader) ld.template wait_current<S::kStores>(sb1 + sb2);
      wg_barrier();
      if (loader) ld.issue_ahead(a, ring, win, t_begin, pw_id, lane);
      const bool have = j >= 2;
      const int par = j & 1;  // parity of step j - 2
      bf16x8 pf[HB][2];
      if (have) {
#pragma unroll
        for (int hb = 0; hb < HB; hb++)
#pragma unroll
          for (int kk = 0; kk < 2; kk++)
            pf[hb][kk] = *reinterpret_cast<const bf16x8 __attribute__((address_space(3)))*>(
                pbuf + (par * HB + hb) * kPBytes + (kk * 64 + lane) * 16);
      }
      if (j < n) {
        // the stage offset is kept opaque so that the compiler does not keep
        // three sets of fragment addresses live across the loop
        int stage_off = PAR * kStage;
        asm volatile("" : "+s"(stage_off));
        lds_t* st = ring + stage_off;
#pragma unroll
        for (int md = 0; md < MDP; md++)
#pragma unroll
          for (int kk = 0; kk < 2; kk++) cb[PAR][md][kk] = ld_c(st, md, kk);
      }
      int sb = 0;
      if (have) {
#pragma unroll
        for (int hb = 0; hb < HB; hb++) {
          if (s_flag[par * HB + hb]) {
            const float al = s_alpha[(par * HB + hb) * 32 + (lane & 31)];
#pragma unroll
            for (int md = 0; md < MDP; md++) o[md][hb] *= al;
          }
        }
#pragma unroll
        for (int md = 0; md < MDP; md++)
#pragma unroll
          for (int kk = 0; kk < 2; kk++)
#pragma unroll
            for (int hb = 0; hb < HB; hb++)
              o[md][hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cb[C][md][kk], pf[hb][kk],
                                                                  o[md][hb], 0, 0, 0);
        // the descriptor of step j - 2, read after the fragment loads
        const Tile pv = read_tile(win, j - 2);
        if (pv.last || j - 2 == n - 1) {
          const int64_t slot = (int64_t)(g + pv.b);
#pragma unroll
          for (int hb = 0; hb < HB; hb++) {
            const float inv = s_invl[(par * HB + hb) * 32 + (lane & 31)];
            // fragment-major partial: one store instruction writes 1 KiB contiguous
            float* dst = a.part_o + slot * a.h * kDc +
                         frag_offset(hg * HB + hb, pw_id * MDP, 0, lane);
#pragma unroll
            for (int md = 0; md < MDP; md++) {
#pragma unroll
              for (int jj = 0; jj < 4; jj++) {
                const f32x4 v = {o[md][hb][4 * jj] * inv, o[md][hb][4 * jj + 1] * inv,
                                 o[md][hb][4 * jj + 2] * inv, o[md][hb][4 * jj + 3] * inv};
                *reinterpret_cast<f32x4*>(dst + (md * 4 + jj) * 256) = v;
              }
              o[md][hb] = f32x16{};
            }
          }
          sb = 1;
        }
      }
      sb2 = sb1;
      sb1 = sb;
    };
    for (int32_t j = 0; j <= n + 1; j += 3) {
      step(std::integral_constant<int, 0>{}, j);
      if (j + 1 > n + 1) break;
      step(std::integral_constant<int, 1>{}, j + 1);
      if (j + 2 > n + 1) break;
      step(std::integral_constant<int, 2>{}, j + 2);
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

int32_t mfma_heads_per_group(int32_t heads) { return heads_per_group(heads); }

hipError_t launch_attend_mfma(const AttnArgs& a, int32_t cache_dtype, hipStream_t s,
                              hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (cache_dtype != MLA_BF16 || a.d_c != kDc || a.d_r != kDr || a.h % 32) return hipErrorInvalidValue;
  const int32_t hpg = heads_per_group(a.h);
  const int32_t HG = a.h / hpg;
  if (HG > 1 && a.splits % 8) return hipErrorInvalidValue;  // XCD pairing uses whole groups of 8
  const dim3 grid(a.splits * HG);
  // sparse index lists get their own instantiations (slot-list loads)
  const bool sp = a.slots != nullptr;
  if (hpg == 64 && !sp)
    hipExtLaunchKernelGGL((attend_mfma_kernel<2, false>), grid, dim3(Shape<2>::NW * 64), 0, s,
                          ev_start, ev_stop, 0, a);
  else if (hpg == 64)
    hipExtLaunchKernelGGL((attend_mfma_kernel<2, true>), grid, dim3(Shape<2>::NW * 64), 0, s,
                          ev_start, ev_stop, 0, a);
  else if (!sp)
    hipExtLaunchKernelGGL((attend_mfma_kernel<1, false>), grid, dim3(Shape<1>::NW * 64), 0, s,
                          ev_start, ev_stop, 0, a);
  else
    hipExtLaunchKernelGGL((attend_mfma_kernel<1, true>), grid, dim3(Shape<1>::NW * 64), 0, s,
                          ev_start, ev_stop, 0, a);
  return hipGetLastError();
}

}  // namespace mla
