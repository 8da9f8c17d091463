// Shared device helpers for the MLA decode kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla.h"

namespace mla {

constexpr int kTile = 32;  // tokens per planning tile (one step of the attention kernels)

// Planning: kPlanGroups work groups of kPlanThreads threads (see plan_block).
constexpr int kPlanThreads = 256;
constexpr int kPlanGroups = 8;

// Per-tile descriptor written by the planning kernel, tiles numbered across
// the sequences in order (four int32):
//   x: block id of the page holding the whole tile (clamped to the pool), or
//      -1 when a tile can span pages (page size not a multiple of kTile)
//   y: sequence b
//   z: first token t0 of the tile within the sequence
//   w: valid tokens nv (1..kTile) | last tile of the sequence << 6 |
//      offset of t0 within its page << 7
__host__ __device__ inline int32_t tile_word(int32_t nv, bool last, int32_t off) {
  return nv | ((int32_t)last << 6) | (off << 7);
}

// Fragment-major layout of one slot's partial output, used by the matrix-core
// kernel (512 latent values, heads a multiple of 32): the slot's [h, 512] fp32
// block is stored as [h/32][16][4][64][4] = (head block, 32-value latent block
// mdg, 8-value group jj, lane, 4 values), where lane = 32*g + r holds head
// 32*hblk + r and latent values 32*mdg + 8*jj + 4*g + (0..3).  This is the
// matrix-core accumulator layout, so each 64-lane store covers 1 KiB.
__host__ __device__ inline int64_t frag_offset(int32_t hblk, int32_t mdg, int32_t jj, int32_t lane) {
  return (((int64_t)hblk * 16 + mdg) * 4 + jj) * 256 + lane * 4;
}

// ---------------------------------------------------------------- split plan
// Tiles of all sequences are numbered in order; split g owns a contiguous run.
__host__ __device__ inline int64_t split_begin(int64_t n_tiles, int32_t splits, int32_t g) {
  return (n_tiles * (int64_t)g) / (int64_t)splits;
}
// The largest g whose run starts at or before `tile`; that run contains it.
__host__ __device__ inline int32_t split_owner(int64_t n_tiles, int32_t splits, int64_t tile) {
  return (int32_t)(((tile + 1) * (int64_t)splits - 1) / n_tiles);
}

// Everything the attention kernels need to know about the problem.
struct AttnArgs {
  const void* q_lat;         // [B, h, d_c + d_r] (fp32 or bf16)
  const void* c_kv;          // [nb, P, d_c]
  const float* c_kv_scale;   // [nb, P] or null
  const void* k_rope;        // [nb, P, d_r]
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* cu_tiles;   // [B + 1] prefix sums of ceil(T_b / kTile) (workspace)
  const int32_t* tiles;      // [n_tiles][4] tile descriptors (workspace)
  float* part_o;             // [slots, h, d_c]
  float* part_lse;           // [slots, h]
  int32_t B, h, d_c, d_r, P, max_blocks, num_blocks;
  int32_t log2P;             // log2(P) when P is a power of two, else -1
  int32_t splits;            // work groups along tokens (gridDim.x)
  int32_t streams;           // partial slots per (split, sequence)
  int32_t frag_layout;       // part_o in fragment-major layout (frag_offset), else row-major
  float sm_scale_log2;       // sm_scale * log2(e)
  // Sparse mode (slots != null): sequence b attends to seq_lens[b] entries
  // (at most idx_stride) whose physical slots (block * P + offset) the planner
  // wrote to slots[b * idx_stride + n]; tiles number those entries.
  const int32_t* slots;
  int32_t idx_stride;
  // Grouped latent (group_heads > 0): heads [g group_heads, (g + 1) group_heads)
  // read latent pool g, which starts c_group_bytes after pool g - 1 (and its
  // fp8 scales c_group_scales floats after), all sharing one rope pool.
  int32_t group_heads;
  int64_t c_group_bytes;
  int64_t c_group_scales;
};

// Point a's latent pool (and scales) at the group of the heads starting at
// head0 (no change without groups).
__device__ inline void select_latent_group(AttnArgs& a, int32_t head0) {
  if (a.group_heads > 0) {
    const int32_t grp = head0 / a.group_heads;
    a.c_kv = static_cast<const char*>(a.c_kv) + grp * a.c_group_bytes;
    if (a.c_kv_scale) a.c_kv_scale += grp * a.c_group_scales;
  }
}

// Read of a table that no kernel of the launch writes (sequence lengths, block
// table, tile prefix sums).  The constant address space lets the compiler use
// scalar loads for wave-uniform indices, whose waits do not depend on the
// vector-memory traffic in flight.
__device__ inline int32_t load_ro(const int32_t* p, int64_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}

// Tokens of sequence b, clamped to what its table row can address.
__device__ inline int32_t seq_len_clamped(const int32_t* seq_lens, int32_t b, int32_t max_blocks,
                                          int32_t P) {
  int32_t t = seq_lens[b];
  int32_t cap = max_blocks * P;
  return t < 0 ? 0 : (t > cap ? cap : t);
}

// Physical slot (block * P + offset) of logical token t of sequence b.
__device__ inline int64_t phys_slot(const int32_t* block_table, int32_t b, int32_t t, int32_t P,
                                    int32_t max_blocks, int32_t num_blocks) {
  int32_t blk = block_table[(int64_t)b * max_blocks + t / P];
  blk = blk < 0 ? 0 : (blk >= num_blocks ? num_blocks - 1 : blk);
  return (int64_t)blk * P + (t % P);
}

// Entries sequence b attends to: its tokens (dense) or its index list (sparse).
__device__ inline int32_t attn_len(const AttnArgs& a, int32_t b) {
  if (!a.slots) return seq_len_clamped(a.seq_lens, b, a.max_blocks, a.P);
  const int32_t n = a.seq_lens[b];
  return n < 0 ? 0 : (n > a.idx_stride ? a.idx_stride : n);
}

// Physical slot of entry n of sequence b (any lane may differ).
__device__ inline int64_t entry_slot(const AttnArgs& a, int32_t b, int32_t n) {
  if (a.slots) return a.slots[(int64_t)b * a.idx_stride + n];
  return phys_slot(a.block_table, b, n, a.P, a.max_blocks, a.num_blocks);
}

// Physical slot of entry n of sequence b in sparse mode, for a wave-uniform
// (b, n): a scalar load, which the vector-memory counter does not track.
__device__ inline int32_t sparse_slot_uniform(const AttnArgs& a, int32_t b, int32_t n) {
  return load_ro(a.slots, __builtin_amdgcn_readfirstlane(b * a.idx_stride + n));
}

// ---------------------------------------------------------------- planner
// What the planner reads and writes.  Sparse mode (indices != null): sequence
// b attends to the first seq_lens[b] (clamped to [0, idx_stride]) entries of
// its row of indices [B, idx_stride], token positions that are clamped into
// the table row [0, max_blocks * P) and resolved through the block table into
// slots[b * idx_stride + n].
struct PlanInput {
  const int32_t* seq_lens;
  const int32_t* block_table;
  int32_t B, max_blocks, P, num_blocks;
  const int32_t* indices;
  int32_t idx_stride;
  int32_t* slots;
  int32_t* cu_tiles;
  int32_t* tiles;
};

// LDS of one planning work group.
struct PlanShared {
  int32_t scan[kPlanThreads];
  int32_t cu[kPlanThreads + 1];  // tile prefix sums of the current chunk of sequences
  int32_t len[kPlanThreads];
};

// Work group `wg` of `nwg` (kPlanThreads threads each) of the planner.  The
// sequences are taken in chunks of kPlanThreads; every planning group scans
// each chunk (cu_tiles[b] = sum_{j<b} ceil(T_j / kTile), written by group 0),
// and the groups share out the chunk's tiles, writing one descriptor per tile
// (tile_word).  The tile's page is resolved here when no tile can span two
// pages (P a multiple of kTile).
__device__ inline void plan_block(const PlanInput& in, int32_t wg, int32_t nwg, PlanShared& sh) {
  const int32_t* __restrict__ seq_lens = in.seq_lens;
  const int32_t* __restrict__ block_table = in.block_table;
  const int32_t B = in.B, max_blocks = in.max_blocks, P = in.P, num_blocks = in.num_blocks;
  int32_t* __restrict__ cu_tiles = in.cu_tiles;
  int32_t* __restrict__ tiles = in.tiles;
  const bool sparse = in.indices != nullptr;
  const int tid = threadIdx.x;
  const bool one_page = !sparse && P % kTile == 0;
  int32_t carry = 0;
  if (wg == 0 && tid == 0) cu_tiles[0] = 0;
  for (int32_t base = 0; base < B; base += kPlanThreads) {
    const int32_t cnt = min(kPlanThreads, B - base);
    const int32_t b = base + tid;
    int32_t n = 0;
    if (tid < cnt) {
      int32_t T;
      if (sparse) {
        T = seq_lens[b];
        T = T < 0 ? 0 : (T > in.idx_stride ? in.idx_stride : T);
      } else {
        T = seq_len_clamped(seq_lens, b, max_blocks, P);
      }
      sh.len[tid] = T;
      n = (T + kTile - 1) / kTile;
    }
    sh.scan[tid] = n;
    __syncthreads();
    for (int off = 1; off < kPlanThreads; off <<= 1) {  // inclusive Hillis-Steele scan
      const int32_t v = tid >= off ? sh.scan[tid - off] : 0;
      __syncthreads();
      sh.scan[tid] += v;
      __syncthreads();
    }
    sh.cu[tid + 1] = carry + sh.scan[tid];
    if (tid == 0) sh.cu[0] = carry;
    if (wg == 0 && tid < cnt) cu_tiles[b + 1] = carry + sh.scan[tid];
    __syncthreads();
    // tile t of this chunk belongs to the last local sequence j with cu[j] <= t
    // (sequences without tiles share their start with the next one)
    const int32_t t_end = sh.cu[cnt];
#pragma unroll 4
    for (int32_t t = sh.cu[0] + wg * kPlanThreads + tid; t < t_end; t += nwg * kPlanThreads) {
      int32_t lo = 0, hi = cnt - 1;
      while (lo < hi) {
        const int32_t mid = (lo + hi + 1) >> 1;
        if (sh.cu[mid] <= t) lo = mid; else hi = mid - 1;
      }
      const int32_t T = sh.len[lo];
      const int32_t t0 = (t - sh.cu[lo]) * kTile;
      const int32_t nv = min(kTile, T - t0);
      int32_t blk = -1, off = 0;
      if (one_page) {
        const int32_t raw = block_table[(int64_t)(base + lo) * max_blocks + t0 / P];
        blk = raw < 0 ? 0 : (raw >= num_blocks ? num_blocks - 1 : raw);
        off = t0 % P;
      }
      reinterpret_cast<int4*>(tiles)[t] =
          make_int4(blk, base + lo, t0, tile_word(nv, t0 + kTile >= T, off));
    }
    carry = t_end;
    __syncthreads();
  }
  if (!sparse) return;
  // slot list: entries e = b * idx_stride + n, eight per thread at a time so
  // that their index and table loads are in flight together
  const int32_t cap = max_blocks * P;
  const int32_t total = B * in.idx_stride;  // < 2^31 (checked on the host)
  const int32_t nthr = nwg * kPlanThreads;
  for (int32_t e0 = wg * kPlanThreads + tid; e0 < total; e0 += 8 * nthr) {
    int32_t t[8], bb[8];
    bool ok[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const int32_t e = e0 + j * nthr;
      bb[j] = e < total ? e / in.idx_stride : 0;
      ok[j] = e < total && e - bb[j] * in.idx_stride < seq_lens[bb[j]];
      t[j] = in.indices[e < total ? e : 0];
    }
    int32_t sl[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {  // unconditional (valid addresses), so they overlap
      const int32_t tc = t[j] < 0 ? 0 : (t[j] >= cap ? cap - 1 : t[j]);
      sl[j] = (int32_t)phys_slot(block_table, bb[j], tc, P, max_blocks, num_blocks);
    }
#pragma unroll
    for (int j = 0; j < 8; j++)
      if (ok[j]) in.slots[e0 + j * nthr] = sl[j];
  }
}

// ---------------------------------------------------------------- storage types
__device__ inline float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ inline uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// OCP E4M3FN byte -> fp32 using the gfx950 hardware conversion.
__device__ inline float e4m3_to_f32(uint8_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
}

template <int DT>
__device__ inline float load_elem(const void* base, int64_t idx);
template <>
__device__ inline float load_elem<MLA_F32>(const void* base, int64_t idx) {
  return static_cast<const float*>(base)[idx];
}
template <>
__device__ inline float load_elem<MLA_BF16>(const void* base, int64_t idx) {
  return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[idx]);
}
template <>
__device__ inline float load_elem<MLA_FP8_E4M3>(const void* base, int64_t idx) {
  return e4m3_to_f32(static_cast<const uint8_t*>(base)[idx]);
}

template <int DT>
__device__ inline void store_elem(void* base, int64_t idx, float v);
template <>
__device__ inline void store_elem<MLA_F32>(void* base, int64_t idx, float v) {
  static_cast<float*>(base)[idx] = v;
}
template <>
__device__ inline void store_elem<MLA_BF16>(void* base, int64_t idx, float v) {
  static_cast<uint16_t*>(base)[idx] = f32_to_bf16_bits(v);
}

}  // namespace mla
