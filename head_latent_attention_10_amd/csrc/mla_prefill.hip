// MLA prefill in MHA mode (gfx950): a chunk of new query tokens per sequence,
// each attending causally to the cached tokens up to its own position, with
// full-width keys and values reconstructed from the latent cache.
//
// "TransMLA & Sparse Latent Attention", Chapter 7 ("DSA runs in MLA's MQA
// mode"): prefill runs MLA in its MHA-like mode (explicit reconstruction),
// decode in the absorbed mode.  "TPLA: ...", section 3.4, Eq. 4: per head i
// the key of token t is [W_UK[i] c_t ; k_rope_t] and the value W_UV[i] c_t; the
// score is sm_scale (q . k).  Query l of the L_b new tokens of sequence b sits
// at position T_b - L_b + l and sees positions 0 .. T_b - L_b + l.
//
// Two kernels:
//  * decompress: K[u, t, :] = [W_UK[i] c_t ; k_rope_t] and V^T[u, :, t] =
//    W_UV[i] c_t for every cached t < T_b of unit u = (sequence b, head i), a
//    bf16 matrix-core GEMM per (128 tokens, unit, K or V) tile, both operands
//    arriving in LDS by direct loads, the next latent chunk in flight while the
//    current one is multiplied;
//  * attention: a work group per (256 queries, unit), a wave per 32 queries;
//    per 64-key tile S^T = K Q^T (16x16x32 MFMA, keys on M), the causal mask,
//    an online softmax per query, and O^T += V^T P^T (the key order of this
//    product is the one the score fragments already hold).
// The units u = b h + i are taken in chunks of consecutive units, the two
// kernels run per chunk, and the reconstructed keys and values of one chunk
// live in the workspace at a time: its size sets the chunk, not B h T.
#include <algorithm>
#include <numeric>

#include "mla_mfma_util.hpp"

namespace mla {
namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kPDc = 512, kPDn = 128, kPDr = 64, kPDv = 128;
constexpr int kPDq = kPDn + kPDr;          // 192 query/key width
constexpr int kDecTok = 128;               // tokens per decompression tile
constexpr int kDecChunk = 64;              // latent values per LDS stage
constexpr int kDecHalf = kDecTok * kDecChunk * 2;  // 16 KB: 128 rows of 128 bytes
constexpr int kQTile = 256;                // queries per attention work group (8 waves)
constexpr int kAStages = 3;                // key/value stages in LDS
constexpr int kKTile = 64;                 // keys per attention step
constexpr int kKStage = kKTile * kPDq * 2;  // 24 KB of keys per step
constexpr int kVStage = kPDv * kKTile * 2;  // 16 KB of transposed values per step

struct PrefillArgs {
  const uint16_t* q;        // [B, Lq, h, 192]
  const int32_t* q_lens;    // [B]
  const uint16_t* c_kv;     // [nb, P, 512] bf16, or
  const uint8_t* c_kv8;     // [nb, P, 512] E4M3 codes with
  const float* c_kv_scale;  // [nb, P] per-token scales
  const uint16_t* k_rope;   // [nb, P, 64]
  const int32_t* block_table;
  const int32_t* seq_lens;
  const uint16_t* W_UK;     // [h, 128, 512]
  const uint16_t* W_UV;     // [h, 128, 512]
  uint16_t* Kn;             // [units, Tpad, 192]: reconstructed nope part, then rope
  uint16_t* Vt;             // [units, 128, Tpad]: tokens permuted within 32 (vt_pos)
  void* out;                // [B, Lq, h, 128]
  int32_t B, h, Lq, P, max_blocks, num_blocks, Tpad;
  int32_t u0;               // first unit (b h + head) of this launch's chunk
  float sm_log2;            // sm_scale * log2(e)
};

__device__ inline int32_t cached_len(const PrefillArgs& a, int32_t b) {
  const int32_t cap = a.max_blocks * a.P;
  const int32_t T = a.seq_lens[b];
  return T < 0 ? 0 : (T > cap ? cap : T);
}

__device__ inline int32_t query_len(const PrefillArgs& a, int32_t b, int32_t T) {
  const int32_t L = a.q_lens[b];
  return L < 0 ? 0 : min(L, min(a.Lq, T));
}

// Column of token t in a V^T row.  Within each block of 32 tokens, token
// 16 h + 4 q + j (h < 2, q < 4, j < 4) sits at 8 q + 4 h + j: the eight tokens a
// lane group multiplies in one value-product step (see the attention kernel)
// are then 16 contiguous bytes.
__device__ inline int32_t vt_pos(int32_t t) {
  const int32_t w = t & 31;
  return (t & ~31) + 8 * ((w >> 2) & 3) + 4 * (w >> 4) + (w & 3);
}

// LDS rows are stored in 16-byte pieces, piece p of row n at position
// p ^ swz(n): the 16 rows a quarter-wave reads then fall on distinct banks.
__device__ inline int swz(int n) { return (n >> 1) & 7; }

template <typename T>
__device__ inline T lds_read(const lds_t* p) {
  return *reinterpret_cast<const T __attribute__((address_space(3)))*>(p);
}

// ------------------------------------------------------------------ decompress
// blockIdx = (token tile, unit within the chunk); WHICH 0 reconstructs keys,
// 1 values.  Wave
// (wm, wn) computes tokens 64 wm .. +63 by outputs 64 wn .. +63 of the
// 128 x 128 tile, as outputs x tokens for keys and tokens x outputs for values,
// so that each lane holds four adjacent values of its output row (key row
// [token][output], value row [output][token]).  The finished tile is staged in
// LDS and written out in 16-byte pieces.  A stage holds 64
// latent values of the 128 tokens (rows 0..127) and of the 128 weight rows;
// the wave loads 1 KB chunks wave + 4 u of each half (8 rows of 8 pieces).
template <int WHICH, bool F8>
__global__ __launch_bounds__(256) void prefill_decompress_kernel(PrefillArgs args) {
  __shared__ __attribute__((aligned(1024))) char smem[4 * kDecHalf];  // two stages of A | B
  __shared__ float s_scale[kDecTok];  // fp8: the tile's per-token scales
  const PrefillArgs a = args;
  const int32_t ul = blockIdx.y, unit = a.u0 + ul;
  const int32_t b = unit / a.h, head = unit - b * a.h;
  const int32_t T = cached_len(a, b);
  const int32_t t0 = blockIdx.x * kDecTok;
  if (t0 >= T) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, g = lane >> 5, r = lane & 31;
  lds_t* ring = (lds_t*)smem;
  const uint16_t* W = (WHICH ? a.W_UV : a.W_UK) + (int64_t)head * kPDn * kPDc;
  // DMA sources of this lane: row 8 (wave + 4 u) + lane / 8, piece (lane & 7) ^ swz(row)
  auto src_a = [&](int u) -> const uint16_t* {
    const int row = 8 * (wave + 4 * u) + (lane >> 3);
    const int32_t t = min(t0 + row, T - 1);  // rows past T repeat the last token (finite)
    const int64_t slot = phys_slot(a.block_table, b, t, a.P, a.max_blocks, a.num_blocks);
    return a.c_kv + slot * kPDc + 8 * ((lane & 7) ^ swz(row));
  };
  auto src_b = [&](int u) -> const uint16_t* {
    const int row = 8 * (wave + 4 * u) + (lane >> 3);
    return W + (int64_t)row * kPDc + 8 * ((lane & 7) ^ swz(row));
  };
  // fp8 rows are 64 bytes a stage: row 16 (wave + 4 u) + lane / 4 (u < 2), piece
  // (lane & 3) ^ swz8(row); the codes convert to bf16 exactly, and the token's
  // scale multiplies the finished product
  auto swz8 = [](int row) { return (row >> 1) & 3; };
  auto src_a8 = [&](int u) -> const uint8_t* {
    const int row = 16 * (wave + 4 * u) + (lane >> 2);
    const int32_t t = min(t0 + row, T - 1);
    const int64_t slot = phys_slot(a.block_table, b, t, a.P, a.max_blocks, a.num_blocks);
    return a.c_kv8 + slot * kPDc + 16 * ((lane & 3) ^ swz8(row));
  };
  const uint16_t *pa0 = nullptr, *pa1 = nullptr, *pa2 = nullptr, *pa3 = nullptr;
  const uint8_t *pq0 = nullptr, *pq1 = nullptr;
  if (F8) {
    pq0 = src_a8(0);
    pq1 = src_a8(1);
    if (tid < kDecTok) {
      const int32_t t = min(t0 + tid, T - 1);
      s_scale[tid] = a.c_kv_scale[phys_slot(a.block_table, b, t, a.P, a.max_blocks, a.num_blocks)];
    }
  } else {
    pa0 = src_a(0), pa1 = src_a(1), pa2 = src_a(2), pa3 = src_a(3);
  }
  const uint16_t *pb0 = src_b(0), *pb1 = src_b(1), *pb2 = src_b(2), *pb3 = src_b(3);
  auto issue = [&](int32_t k0, lds_t* st) {
    if (F8) {
      dma16(pq0 + k0, st + (wave + 0) * 1024);
      dma16(pq1 + k0, st + (wave + 4) * 1024);
    } else {
      dma16(pa0 + k0, st + (wave + 0) * 1024);
      dma16(pa1 + k0, st + (wave + 4) * 1024);
      dma16(pa2 + k0, st + (wave + 8) * 1024);
      dma16(pa3 + k0, st + (wave + 12) * 1024);
    }
    dma16(pb0 + k0, st + kDecHalf + (wave + 0) * 1024);
    dma16(pb1 + k0, st + kDecHalf + (wave + 4) * 1024);
    dma16(pb2 + k0, st + kDecHalf + (wave + 8) * 1024);
    dma16(pb3 + k0, st + kDecHalf + (wave + 12) * 1024);
  };
  f32x16 acc[2][2] = {};
  constexpr int kChunks = kPDc / kDecChunk;
  issue(0, ring);
  for (int cc = 0; cc < kChunks; cc++) {
    if (cc + 1 < kChunks) {
      issue((cc + 1) * kDecChunk, ring + ((cc + 1) & 1) * 2 * kDecHalf);
      wait_vmcnt<F8 ? 6 : 8>();
    } else {
      wait_vmcnt<0>();
    }
    wg_barrier();  // chunk cc has landed for every wave
    const lds_t* st = ring + (cc & 1) * 2 * kDecHalf;
#pragma unroll
    for (int s = 0; s < kDecChunk / 16; s++) {
      bf16x8 av[2], bv[2];
#pragma unroll
      for (int x = 0; x < 2; x++) {
        const int ra = 64 * wm + 32 * x + r, rb = 64 * wn + 32 * x + r;
        if (F8) {
          const u32x2 w = lds_read<u32x2>(st + ra * 64 + ((s ^ swz8(ra)) << 4) + 8 * g);
          const f32x2 f0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, false);
          const f32x2 f1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, true);
          const f32x2 f2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, false);
          const f32x2 f3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, true);
          av[x] = bf16x8{(__bf16)f0[0], (__bf16)f0[1], (__bf16)f1[0], (__bf16)f1[1],
                         (__bf16)f2[0], (__bf16)f2[1], (__bf16)f3[0], (__bf16)f3[1]};
        } else {
          av[x] = lds_read<bf16x8>(st + ra * 128 + (((2 * s + g) ^ swz(ra)) << 4));
        }
        bv[x] = lds_read<bf16x8>(st + kDecHalf + rb * 128 + (((2 * s + g) ^ swz(rb)) << 4));
      }
#pragma unroll
      for (int x = 0; x < 2; x++)
#pragma unroll
        for (int y = 0; y < 2; y++)
          acc[x][y] = WHICH == 0
                          ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[y], av[x], acc[x][y], 0, 0, 0)
                          : __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[x], bv[y], acc[x][y], 0, 0, 0);
    }
    wg_barrier();  // stage cc & 1 is refilled by the next iteration (or reused below)
  }
  // Stage the tile as 128 rows of 128 bf16 (272-byte rows).  Keys: D[output]
  // [token], lane holds token 64 wm + 32 x + r and outputs 64 wn + 32 y + 8 jb +
  // 4 g + (0..3).  Values: D[token][output], lane holds output 64 wn + 32 y + r
  // and tokens 64 wm + 32 x + 8 jb + 4 g + (0..3), stored at their vt_pos.
  constexpr int kORow = 2 * kDecTok + 16;
  lds_t* ot = ring;
#pragma unroll
  for (int x = 0; x < 2; x++)
#pragma unroll
    for (int y = 0; y < 2; y++)
#pragma unroll
      for (int jb = 0; jb < 4; jb++) {
        const int quad = 8 * jb + 4 * g;
        float sc[4] = {1.f, 1.f, 1.f, 1.f};
        if (F8) {
#pragma unroll
          for (int e = 0; e < 4; e++)
            sc[e] = s_scale[WHICH == 0 ? 64 * wm + 32 * x + r : 64 * wm + 32 * x + quad + e];
        }
        const bf16x4 v = {(__bf16)(acc[x][y][4 * jb + 0] * sc[0]), (__bf16)(acc[x][y][4 * jb + 1] * sc[1]),
                          (__bf16)(acc[x][y][4 * jb + 2] * sc[2]), (__bf16)(acc[x][y][4 * jb + 3] * sc[3])};
        const int row = WHICH == 0 ? 64 * wm + 32 * x + r : 64 * wn + 32 * y + r;
        const int col = WHICH == 0 ? 64 * wn + 32 * y + quad : vt_pos(64 * wm + 32 * x + quad);
        *reinterpret_cast<bf16x4 __attribute__((address_space(3)))*>(ot + row * kORow + 2 * col) = v;
      }
  wg_barrier();
  const int64_t bh = ul;  // the unit's place in the chunk's workspace
#pragma unroll
  for (int k = 0; k < 8; k++) {
    const int pi = tid + 256 * k, row = pi >> 4, pc = pi & 15;
    const u32x4 v = lds_read<u32x4>(ot + row * kORow + 16 * pc);
    if (WHICH == 0)  // key row t0 + row, reconstructed part
      *reinterpret_cast<u32x4*>(a.Kn + (bh * a.Tpad + t0 + row) * kPDq + 8 * pc) = v;
    else  // value row `row`, tokens t0 .. t0 + 127
      *reinterpret_cast<u32x4*>(a.Vt + (bh * kPDv + row) * a.Tpad + t0 + 8 * pc) = v;
  }
  if (WHICH == 0) {
    // the key's rope part, copied beside the reconstructed part (rows past T
    // repeat the last token, as above)
#pragma unroll
    for (int k = 0; k < 4; k++) {
      const int32_t idx = tid + 256 * k, row = idx >> 3, pc = idx & 7;
      const int32_t t = min(t0 + row, T - 1);
      const int64_t slot = phys_slot(a.block_table, b, t, a.P, a.max_blocks, a.num_blocks);
      *reinterpret_cast<uint4*>(a.Kn + (bh * a.Tpad + t0 + row) * kPDq + kPDn + 8 * pc) =
          *reinterpret_cast<const uint4*>(a.k_rope + slot * kPDr + 8 * pc);
    }
  }
}

// ------------------------------------------------------------------ attention
// One work group per (256 queries, unit) on a 1-D grid, a wave per
// 32 queries (two 16-query MFMA column blocks sharing every key fragment).
// Key and value tiles arrive by direct-to-LDS loads into three stages, the
// tiles of steps n + 1 and n + 2 in flight while step n is multiplied, one
// barrier per step.  A stage holds 64 keys x 192 (rows of 384 bytes) and then
// 128 value rows x 64 tokens (128 bytes), 40 chunks of 1 KB; wave w loads key
// chunks w + 8 u (u < 3) and value chunks w + 8 u (u < 2).  Waves skip steps
// wholly after their queries; only steps on a wave's diagonal are masked.
// Element offsets of this lane's DMA sources within a step's key rows and
// value rows; the same for every step.
struct AttnSrc {
  int32_t k0, k1, k2;
  int64_t v0, v1;  // value rows are Tpad apart: 127 Tpad can pass 2^31
};

__device__ inline int32_t attn_koff(int wave, int lane, int u) {
  const int o = (wave + 8 * u) * 1024 + 16 * lane;
  const int key = o / (kPDq * 2), pos = (o % (kPDq * 2)) >> 4;
  return key * kPDq + 8 * (pos ^ swz(key));
}

__device__ inline int64_t attn_voff(int wave, int lane, int u, int32_t Tpad) {
  const int o = (wave + 8 * u) * 1024 + 16 * lane;
  const int row = o >> 7, pos = (o >> 4) & 7;
  return (int64_t)row * Tpad + 8 * (pos ^ swz(row));
}

__device__ inline void attn_issue(const uint16_t* kbase, const uint16_t* vbase, const AttnSrc& f,
                                  lds_t* st, int wave) {
  lds_t* sk = st + wave * 1024;
  lds_t* sv = st + kKStage + wave * 1024;
  dma16(kbase + f.k0, sk);
  dma16(kbase + f.k1, sk + 8192);
  dma16(kbase + f.k2, sk + 16384);
  dma16(vbase + f.v0, sv);
  dma16(vbase + f.v1, sv + 8192);
}

template <int OT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_attn_kernel(
    PrefillArgs args, int32_t n_qtiles) {
  __shared__ __attribute__((aligned(1024))) char smem[kAStages * (kKStage + kVStage)];
  const PrefillArgs a = args;
  // Block order: the 8 XCDs take block ids round-robin; regroup so that each
  // XCD runs a contiguous range of (q-tile, unit) work, the q-tiles of one
  // unit (which read the same keys and values) sharing its L2, and the
  // causally heaviest q-tile of each unit first.
  const uint32_t nwg = gridDim.x, per = nwg / 8;
  uint32_t id = blockIdx.x;
  if (id < per * 8) id = (id % 8) * per + id / 8;
  const int32_t qt = n_qtiles - 1 - (int32_t)(id % n_qtiles);
  const int32_t ul = (int32_t)(id / n_qtiles), unit = a.u0 + ul;
  const int32_t b = unit / a.h, head = unit - b * a.h;
  const int32_t T = cached_len(a, b);
  const int32_t Lb = query_len(a, b, T);
  const int32_t q0 = qt * kQTile;
  if (q0 >= Lb) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int64_t bh = ul;  // the unit's place in the chunk's workspace
  lds_t* ring = (lds_t*)smem;
  constexpr int kStage = kKStage + kVStage;
  const int32_t t_end = T - Lb + min(q0 + kQTile, Lb);  // keys this work group needs
  const int32_t n_tiles = (t_end + kKTile - 1) / kKTile;
  const AttnSrc src{attn_koff(wave, lane, 0), attn_koff(wave, lane, 1), attn_koff(wave, lane, 2),
                    attn_voff(wave, lane, 0, a.Tpad), attn_voff(wave, lane, 1, a.Tpad)};
  const uint16_t* kseq = a.Kn + bh * a.Tpad * kPDq;
  const uint16_t* vseq = a.Vt + bh * kPDv * a.Tpad;
  // this lane's queries: column c of the wave's two 16-query blocks
  int32_t qpos[2];
  bf16x8 qv[2][kPDq / 32];
#pragma unroll
  for (int qb = 0; qb < 2; qb++) {
    const int32_t ql = min(q0 + 32 * wave + 16 * qb + c, Lb - 1);
    qpos[qb] = T - Lb + ql;
    const uint16_t* qrow = a.q + (((int64_t)b * a.Lq + ql) * a.h + head) * kPDq + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kPDq / 32; ks++)
      qv[qb][ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks);
  }
  attn_issue(kseq, vseq, src, ring, wave);
  if (n_tiles > 1) attn_issue(kseq + kKTile * kPDq, vseq + kKTile, src, ring + kStage, wave);
  // the wave's first and last query positions (wave-uniform)
  const int32_t wave_lo = T - Lb + min(q0 + 32 * wave, Lb - 1);
  const int32_t wave_hi = T - Lb + min(q0 + 32 * wave + 31, Lb - 1);
  const float cs = a.sm_log2;   // > 0: the max commutes with it
  const float lazy = 8.f / cs;  // the running maximum moves only by more than 2^8 in weight
  const int sw = (c >> 1) & 7;  // swz() of every row this lane reads
  const bf16x8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
  f32x4v o[2][kPDv / 16] = {};
  f32x4v lsum[2] = {};  // every element: the weights' sum for this lane's query
  float m[2] = {-INFINITY, -INFINITY};
  int stage = 0;  // n % kAStages
  for (int32_t n = 0; n < n_tiles; n++) {
    const int32_t t0 = n * kKTile;
    if (n + 1 < n_tiles)
      wait_vmcnt<5>();  // tile n + 1 may stay in flight
    else
      wait_vmcnt<0>();
    // tile n has landed for every wave, and every wave is done with tile n - 1,
    // whose stage tile n + 2 refills
    wg_barrier();
    if (n + 2 < n_tiles) {
      const int st2 = stage == 0 ? 2 : stage - 1;  // (n + 2) % 3
      attn_issue(kseq + (int64_t)(t0 + 2 * kKTile) * kPDq, vseq + t0 + 2 * kKTile, src,
                 ring + st2 * kStage, wave);
    }
    const lds_t* sk = ring + stage * kStage;
    stage = stage == kAStages - 1 ? 0 : stage + 1;
    const lds_t* sv = sk + kKStage;
    if (t0 <= wave_hi) {  // else every key of the tile comes after every query of the wave
      // S^T[key][query]: lane holds query c of block qb, keys 16 kb + 4 g + j
      f32x4v s[2][4];
#pragma unroll
      for (int qb = 0; qb < 2; qb++)
#pragma unroll
        for (int kb = 0; kb < 4; kb++) s[qb][kb] = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kPDq / 32; ks++) {
#pragma unroll
        for (int kb = 0; kb < 4; kb++) {
          const bf16x8 kv = lds_read<bf16x8>(sk + (16 * kb + c) * (kPDq * 2) + (((4 * ks + g) ^ sw) << 4));
          s[0][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qv[0][ks], s[0][kb], 0, 0, 0);
          s[1][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qv[1][ks], s[1][kb], 0, 0, 0);
        }
      }
      const bool diag = t0 + kKTile - 1 > wave_lo;
      bf16x8 pb[2][2];
      bool moved = false;
      float alpha[2];
#pragma unroll
      for (int qb = 0; qb < 2; qb++) {
        if (diag) {
          // causal mask: key t0 + 16 kb + 4 g + j is visible while it is <= qpos
          const int32_t lim = qpos[qb] - t0 - 4 * g;
#pragma unroll
          for (int kb = 0; kb < 4; kb++)
#pragma unroll
            for (int j = 0; j < 4; j++)
              if (16 * kb + j > lim) s[qb][kb][j] = -INFINITY;
        }
        float tmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; kb++)
#pragma unroll
          for (int j = 0; j < 4; j++) tmax = fmaxf(tmax, s[qb][kb][j]);
        // The running maximum is raised only when the tile's exceeds it by more
        // than `lazy` (weights stay <= 2^8); the same maximum cancels in O / l.
        // The four lanes of a query must agree on it, so the maximum over them
        // is taken only when some lane of the wave would raise it.  Key 0 is
        // visible to every query, so m is finite from the first tile on.
        if (__builtin_amdgcn_ballot_w64(tmax > m[qb] + lazy)) {
          tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
          tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        }
        const float m_new = tmax > m[qb] + lazy ? tmax : m[qb];
        moved |= m_new != m[qb];
        alpha[qb] = __builtin_amdgcn_exp2f((m[qb] - m_new) * cs);
        m[qb] = m_new;
        const float mc = m_new * cs;
#pragma unroll
        for (int kb = 0; kb < 4; kb++)
#pragma unroll
          for (int j = 0; j < 4; j++)  // rounded to nearest even
            pb[qb][kb >> 1][4 * (kb & 1) + j] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[qb][kb][j], cs, -mc));
      }
      if (__builtin_amdgcn_ballot_w64(moved)) {
#pragma unroll
        for (int qb = 0; qb < 2; qb++) {
          lsum[qb] *= alpha[qb];
#pragma unroll
          for (int mb = 0; mb < kPDv / 16; mb++) o[qb][mb] *= alpha[qb];
        }
      }
      // O^T[d][query] += V^T[d][keys] P^T[keys][query]: in step k2 lane group g
      // multiplies keys 32 k2 + 16 h + 4 g + j (element 4 h + j of its weight
      // fragment), which vt_pos stores as the 16 bytes at 32 k2 + 8 g.  A row
      // of ones in place of V^T sums the same bf16 weights for the normaliser.
#pragma unroll
      for (int k2 = 0; k2 < 2; k2++) {
#pragma unroll
        for (int mb = 0; mb < kPDv / 16; mb++) {
          const bf16x8 vv = lds_read<bf16x8>(sv + (16 * mb + c) * (kKTile * 2) + (((4 * k2 + g) ^ sw) << 4));
          o[0][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, pb[0][k2], o[0][mb], 0, 0, 0);
          o[1][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, pb[1][k2], o[1][mb], 0, 0, 0);
        }
        lsum[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[0][k2], lsum[0], 0, 0, 0);
        lsum[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[1][k2], lsum[1], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int qb = 0; qb < 2; qb++) {
    const float l_tot = lsum[qb][0];
    const int32_t ql = q0 + 32 * wave + 16 * qb + c;
    if (ql >= Lb) continue;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int64_t orow = (((int64_t)b * a.Lq + ql) * a.h + head) * kPDv;
    // lane holds query c, value rows 16 mb + 4 g + j
#pragma unroll
    for (int mb = 0; mb < kPDv / 16; mb++)
#pragma unroll
      for (int j = 0; j < 4; j++) store_elem<OT>(a.out, orow + 16 * mb + 4 * g + j, o[qb][mb][j] * inv);
  }
}

}  // namespace

bool prefill_supported(const mla_decode_params& p) {
  return p.q_dtype == MLA_BF16 && (p.cache_dtype == MLA_BF16 || p.cache_dtype == MLA_FP8_E4M3) &&
         p.rope_dtype == MLA_BF16 &&
         p.weight_dtype == MLA_BF16 && p.d_latent == kPDc && p.d_nope == kPDn &&
         p.d_rope == kPDr && p.d_v == kPDv;
}

int32_t prefill_tpad(const mla_decode_params& p) {
  const int64_t cap = (int64_t)p.max_blocks_per_seq * p.page_size;
  return (int32_t)((cap + kDecTok - 1) / kDecTok * kDecTok);
}

size_t prefill_unit_bytes(const mla_decode_params& p) {
  // keys [Tpad, 192] and transposed values [128, Tpad], bf16; a multiple of 256
  return (size_t)prefill_tpad(p) * (kPDq + kPDv) * sizeof(uint16_t);
}

int64_t prefill_chunk_units(const mla_decode_params& p, int32_t max_q_len, size_t workspace_bytes) {
  const int64_t units = (int64_t)p.batch * p.num_heads;
  const int64_t fit = std::min<int64_t>((int64_t)(workspace_bytes / prefill_unit_bytes(p)), 65535);
  if (units == 0 || fit < 1) return 0;
  if (fit >= units) return units;
  // The fewest chunks the workspace allows.  An attention work group fills a
  // compute unit (its LDS ring), so a chunk's (256 queries, unit) work groups
  // are taken as whole rounds of the compute units where the workspace
  // allows: the unit count of a chunk a multiple of m.
  constexpr int64_t kComputeUnits = 256;  // MI355X
  const int64_t n_qtiles = (max_q_len + kQTile - 1) / kQTile;
  int64_t m = kComputeUnits / std::gcd(kComputeUnits, n_qtiles);
  if (fit < m) m = 1;
  const int64_t cap = fit / m * m;
  const int64_t chunks = (units + cap - 1) / cap;
  const int64_t even = (units + chunks - 1) / chunks;
  return (even + m - 1) / m * m;  // <= cap, since cap is a multiple of m
}

hipError_t launch_prefill(const mla_decode_params& p, int32_t max_q_len, const void* q,
                          const int32_t* q_lens, const void* c_kv, const float* c_kv_scale,
                          const void* k_rope, const int32_t* block_table, const int32_t* seq_lens,
                          const void* W_UK, const void* W_UV, void* out, void* workspace,
                          size_t workspace_bytes, hipStream_t s) {
  PrefillArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.q_lens = q_lens;
  a.c_kv = static_cast<const uint16_t*>(c_kv);
  a.c_kv8 = static_cast<const uint8_t*>(c_kv);
  a.c_kv_scale = c_kv_scale;
  a.k_rope = static_cast<const uint16_t*>(k_rope);
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.W_UK = static_cast<const uint16_t*>(W_UK);
  a.W_UV = static_cast<const uint16_t*>(W_UV);
  a.out = out;
  a.B = p.batch;
  a.h = p.num_heads;
  a.Lq = max_q_len;
  a.P = p.page_size;
  a.max_blocks = p.max_blocks_per_seq;
  a.num_blocks = p.num_blocks;
  a.Tpad = prefill_tpad(p);
  const float sm = p.sm_scale > 0.f ? p.sm_scale : 1.0f / sqrtf((float)(p.d_nope + p.d_rope));
  a.sm_log2 = sm * 1.4426950408889634f;
  const int64_t units = (int64_t)p.batch * p.num_heads;
  const int64_t per = prefill_chunk_units(p, max_q_len, workspace_bytes);
  if (per < 1) return hipErrorInvalidValue;
  a.Kn = static_cast<uint16_t*>(workspace);
  a.Vt = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) +
                                     (size_t)per * a.Tpad * kPDq * sizeof(uint16_t));
  const int32_t n_qtiles = (max_q_len + kQTile - 1) / kQTile;
  for (int64_t u0 = 0; u0 < units; u0 += per) {
    const int32_t n = (int32_t)std::min(per, units - u0);
    a.u0 = (int32_t)u0;
    const dim3 dgrid(a.Tpad / kDecTok, n);
    if (p.cache_dtype == MLA_FP8_E4M3) {
      hipLaunchKernelGGL((prefill_decompress_kernel<0, true>), dgrid, dim3(256), 0, s, a);
      hipLaunchKernelGGL((prefill_decompress_kernel<1, true>), dgrid, dim3(256), 0, s, a);
    } else {
      hipLaunchKernelGGL((prefill_decompress_kernel<0, false>), dgrid, dim3(256), 0, s, a);
      hipLaunchKernelGGL((prefill_decompress_kernel<1, false>), dgrid, dim3(256), 0, s, a);
    }
    const dim3 grid((uint32_t)((int64_t)n_qtiles * n));
    if (p.out_dtype == MLA_BF16)
      hipLaunchKernelGGL(prefill_attn_kernel<MLA_BF16>, grid, dim3(512), 0, s, a, n_qtiles);
    else
      hipLaunchKernelGGL(prefill_attn_kernel<MLA_F32>, grid, dim3(512), 0, s, a, n_qtiles);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace mla
