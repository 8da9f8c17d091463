// Shared device helpers for the MLA decode kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla.h"

namespace mla {

constexpr int kTile = 32;  // tokens per planning tile (one step of the attention kernels)

// Planning limit: the planning kernel keeps the tile prefix sums in LDS.
constexpr int kPlanMaxBatch = 16384;

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
  float sm_scale_log2;       // sm_scale * log2(e)
};

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
