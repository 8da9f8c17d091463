// Shared device helpers for the MLA decode kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla.h"

namespace mla {

constexpr int kTile = 32;  // tokens per planning tile (one step of the attention kernels)

// Planning: kPlanGroups work groups of kPlanThreads threads (see plan_block).
constexpr int kPlanThreads = 256;
constexpr int kPlanGroups = 32;

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

// bf16 partial outputs of the shapes the matrix-core kernels serve (512
// latent values, heads a multiple of 32): slot k's [h, 512] block is
// row-major, value (head i, latent x) at k h 512 + 512 i + x, so that one
// head's partial is 1 KiB contiguous for the merge.  part_row: where the
// 32-value latent block mdg of head 32 hblk + (lane % 32) starts in a slot.
__host__ __device__ inline int64_t part_row(int32_t hblk, int32_t mdg, int32_t lane) {
  return (int64_t)(32 * hblk + (lane & 31)) * 512 + 32 * mdg;
}

// ---------------------------------------------------------------- split plan
// Tiles of all sequences are numbered in order, and every split owns a
// contiguous run of them: split g owns [split_first[g], split_first[g + 1]).
// Two rules, chosen by the batch size:
//  * sequence-aligned (batch <= splits and batch <= kAlignedMaxBatch): no split
//    crosses a sequence.  With
//    n_b tiles in sequence b, L is the least bound such that
//    sum_b ceil(n_b / L) <= splits, sequence b gets k_b = ceil(n_b / L)
//    splits in order, and its i-th split owns tiles [n_b i / k_b,
//    n_b (i + 1) / k_b) of it; splits left over own nothing.  A work group
//    then serves one sequence, and the longest split is as short as it can be
//    without crossing one.
//  * contiguous (otherwise): split g owns [n g / splits, n (g + 1) /
//    splits) of all n tiles, whatever sequences they belong to.
// seq_splits[2 b], seq_splits[2 b + 1] are the first and last split holding
// a tile of sequence b (last < first when it has none).
__host__ __device__ inline int64_t split_begin(int64_t n_tiles, int32_t splits, int32_t g) {
  return (n_tiles * (int64_t)g) / (int64_t)splits;
}
// The largest g whose run starts at or before `tile`; that run contains it.
__host__ __device__ inline int32_t split_owner(int64_t n_tiles, int32_t splits, int64_t tile) {
  return (int32_t)(((tile + 1) * (int64_t)splits - 1) / n_tiles);
}
// Split count of a sequence of n tiles under the sequence-aligned rule with bound L.
// (The aligned rule applies when the batch is at most the split count and at
// most kAlignedMaxBatch, defined with the planner below.)
__host__ __device__ inline int32_t aligned_splits(int32_t n, int32_t L) {
  return n > 0 ? (n + L - 1) / L : 0;
}
// First tile (within its sequence of n tiles split k ways) of split i.
__host__ __device__ inline int32_t aligned_first(int32_t n, int32_t k, int32_t i) {
  return (int32_t)(((int64_t)n * i) / k);
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
  const int32_t* split_first;  // [splits + 1] first tile of each split (workspace)
  const int32_t* seq_splits;   // [B][2] first and last split of each sequence (workspace)
  void* part_o;              // [slots, h, d_c] row-major: bf16 when part_bf16, else fp32
  float* part_lse;           // [slots, h]
  int32_t B, h, d_c, d_r, P, max_blocks, num_blocks;
  int32_t log2P;             // log2(P) when P is a power of two, else -1
  int32_t splits;            // work groups along tokens (gridDim.x)
  int32_t streams;           // partial slots per (split, sequence)
  int32_t part_bf16;         // part_o bf16 (the matrix-core shapes, part_piece), else fp32
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
  // TPLA (shards > 1): the h heads are the shard heads of h / shards heads in
  // shard-major order (head j h / shards + i: head i, shard j), whose queries
  // are zero outside their shard's d_c / shards latent columns.  Kernels may
  // then leave a shard head's other latent columns of its partials unwritten;
  // the combine merges each head's own shard columns into an [B, h / shards,
  // d_c] output.
  int32_t shards;
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
  int32_t splits;
  int32_t* split_first;  // [splits + 1]
  int32_t* seq_splits;   // [B][2]
};

// Sequences the sequence-aligned split rule serves (above it, and above the
// split count, the contiguous rule applies).
constexpr int kAlignedMaxBatch = 2048;

// LDS of one planning work group.
struct PlanShared {
  int32_t red[8];                // per-wave partial results of the reductions
  int32_t cu[kPlanThreads + 1];  // tile prefix sums of the current chunk of sequences
  int32_t len[kPlanThreads];
  int32_t ntile[kAlignedMaxBatch];      // tiles per sequence (split table, aligned rule)
  int32_t gfirst[kAlignedMaxBatch + 1];  // first split of each sequence, then the total
  int32_t tfirst[kAlignedMaxBatch];      // first tile of each sequence
};

// Tiles of sequence b as the planner counts them.
__device__ inline int32_t plan_tiles(const PlanInput& in, int32_t b) {
  int32_t T;
  if (in.indices) {
    T = in.seq_lens[b];
    T = T < 0 ? 0 : (T > in.idx_stride ? in.idx_stride : T);
  } else {
    T = seq_len_clamped(in.seq_lens, b, in.max_blocks, in.P);
  }
  return (T + kTile - 1) / kTile;
}

// Work-group reductions of the planner: across each wave by lane exchanges,
// then across the four waves through LDS (two barriers each).
__device__ inline int2 plan_sum_max(int32_t s, int32_t m, PlanShared& sh) {
  const int tid = threadIdx.x, w = tid >> 6;
  for (int off = 32; off > 0; off >>= 1) {
    s += __shfl_xor(s, off);
    const int32_t o = __shfl_xor(m, off);
    m = o > m ? o : m;
  }
  __syncthreads();
  if ((tid & 63) == 0) {
    sh.red[w] = s;
    sh.red[4 + w] = m;
  }
  __syncthreads();
  int2 r = make_int2(sh.red[0], sh.red[4]);
  for (int i = 1; i < kPlanThreads / 64; i++) {
    r.x += sh.red[i];
    r.y = sh.red[4 + i] > r.y ? sh.red[4 + i] : r.y;
  }
  return r;
}

// Number of threads of the work group whose `pred` holds.
__device__ inline int32_t plan_count(bool pred, PlanShared& sh) {
  const int tid = threadIdx.x, w = tid >> 6;
  const int32_t c = __popcll(__ballot(pred));
  __syncthreads();
  if ((tid & 63) == 0) sh.red[w] = c;
  __syncthreads();
  int32_t r = 0;
  for (int i = 0; i < kPlanThreads / 64; i++) r += sh.red[i];
  return r;
}

// Inclusive prefix sums of two values per thread over the work group, and
// their totals.
__device__ inline void plan_scan2(int32_t& a, int32_t& b, int32_t* tot_a, int32_t* tot_b,
                                  PlanShared& sh) {
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t oa = __shfl_up(a, off), ob = __shfl_up(b, off);
    if (l >= off) {
      a += oa;
      b += ob;
    }
  }
  __syncthreads();
  if (l == 63) {
    sh.red[w] = a;
    sh.red[4 + w] = b;
  }
  __syncthreads();
  int32_t ta = 0, tb = 0;
  for (int i = 0; i < kPlanThreads / 64; i++) {
    if (i < w) {
      a += sh.red[i];
      b += sh.red[4 + i];
    }
    ta += sh.red[i];
    tb += sh.red[4 + i];
  }
  *tot_a = ta;
  *tot_b = tb;
}

// Least L in [lo, hi] with sum_b ceil(ntile[b] / L) <= S, given that hi
// qualifies (the count does not grow with L).  Each round tests up to
// kPlanThreads / T evenly spaced candidates at once, T threads sharing the
// sequences of one candidate; the candidates that fail form a prefix, whose
// length narrows [lo, hi] to one step.
__device__ inline int32_t plan_least_bound(int32_t B, int32_t S, int32_t lo, int32_t hi,
                                           PlanShared& sh) {
  const int tid = threadIdx.x;
  // threads per candidate: at most 16 sequences each, or more threads when
  // few candidates are left
  int32_t tb = 1;
  while (tb < 64 && B > 16 * tb) tb *= 2;
  while (lo < hi) {
    const int32_t span = hi - lo;  // candidates lo .. hi - 1; hi qualifies
    int32_t T = 1;
    while (T < 64 && (int64_t)span * (2 * T) <= kPlanThreads) T *= 2;
    if (T < tb) T = tb;
    const int32_t ncand = kPlanThreads / T;
    const int32_t step = (span + ncand - 1) / ncand;
    const int32_t sub = tid & (T - 1);
    const int32_t c = lo + (tid / T) * step;
    int32_t cnt = 0;
    if (c < hi)
      for (int32_t b = sub; b < B; b += T) cnt += aligned_splits(sh.ntile[b], c);
    for (int off = 1; off < T; off <<= 1) cnt += __shfl_xor(cnt, off);
    const int32_t nf = plan_count(c < hi && sub == 0 && cnt > S, sh);
    const int32_t first_ok = lo + nf * step;  // first candidate that qualifies (or past hi)
    if (first_ok < hi) hi = first_ok;
    if (nf > 0) lo = lo + (nf - 1) * step + 1;
  }
  return lo;
}

// The split table (split rules above), written by one planning work group.
__device__ inline void plan_splits(const PlanInput& in, PlanShared& sh) {
  const int32_t B = in.B, S = in.splits;
  const int tid = threadIdx.x;
  const bool aligned = B <= S && B <= kAlignedMaxBatch;
  int32_t tot = 0, mx = 0;
  for (int32_t b = tid; b < B; b += kPlanThreads) {
    const int32_t n = plan_tiles(in, b);
    if (aligned) sh.ntile[b] = n;
    tot += n;
    mx = n > mx ? n : mx;
  }
  const int2 tm = plan_sum_max(tot, mx, sh);  // its barriers also publish ntile
  tot = tm.x;
  mx = tm.y;
  if (aligned) {
    // L = max n_b qualifies, and so does any L >= tot / (S - B), since
    // sum_b ceil(n_b / L) < tot / L + B
    int32_t L = 1;
    if (tot > 0) {
      const int32_t lo = (tot + S - 1) / S;
      int32_t hi = mx;
      if (S > B) {
        const int32_t ub = (int32_t)(((int64_t)tot + (S - B) - 1) / (S - B));
        if (ub < hi) hi = ub;
      }
      L = plan_least_bound(B, S, lo, hi < lo ? lo : hi, sh);
    }
    // split counts k_b and their exclusive prefix sums (first split, first
    // tile of each sequence) in LDS, a chunk of kPlanThreads sequences at a time
    int32_t gcarry = 0, tcarry = 0;
    for (int32_t base = 0; base < B; base += kPlanThreads) {
      const int32_t b = base + tid;
      const int32_t n = b < B ? sh.ntile[b] : 0;
      const int32_t k = aligned_splits(n, L);
      int32_t sk = k, sn = n, tk, tn;
      plan_scan2(sk, sn, &tk, &tn, sh);
      if (b < B) {
        sh.gfirst[b] = gcarry + sk - k;
        sh.tfirst[b] = tcarry + sn - n;
        in.seq_splits[2 * b] = gcarry + sk - k;
        in.seq_splits[2 * b + 1] = gcarry + sk - 1;
      }
      gcarry += tk;
      tcarry += tn;
    }
    if (tid == 0) sh.gfirst[B] = gcarry;
    __syncthreads();
    // one split per thread: its sequence by binary search over the first splits
    for (int32_t g = tid; g <= S; g += kPlanThreads) {
      int32_t first = tot;
      if (g < gcarry) {
        int32_t lo = 0, hi = B - 1;  // last b with gfirst[b] <= g
        while (lo < hi) {
          const int32_t mid = (lo + hi + 1) >> 1;
          if (sh.gfirst[mid] <= g) lo = mid; else hi = mid - 1;
        }
        const int32_t n = sh.ntile[lo], k = sh.gfirst[lo + 1] - sh.gfirst[lo];
        first = sh.tfirst[lo] + aligned_first(n, k, g - sh.gfirst[lo]);
      }
      in.split_first[g] = first;
    }
    return;
  }
  for (int32_t g = tid; g <= S; g += kPlanThreads) in.split_first[g] = (int32_t)split_begin(tot, S, g);
  int32_t tcarry = 0;
  for (int32_t base = 0; base < B; base += kPlanThreads) {
    const int32_t b = base + tid;
    const int32_t n = b < B ? plan_tiles(in, b) : 0;
    int32_t sn = n, unused = 0, tn, tu;
    plan_scan2(sn, unused, &tn, &tu, sh);
    if (b < B) {
      const int32_t C = tcarry + sn - n;
      in.seq_splits[2 * b] = n == 0 ? 0 : split_owner(tot, S, C);
      in.seq_splits[2 * b + 1] = n == 0 ? -1 : split_owner(tot, S, C + n - 1);
    }
    tcarry += tn;
  }
}

// Work group `wg` of `nwg` (kPlanThreads threads each) of the planner.  The
// sequences are taken in chunks of kPlanThreads; every planning group scans
// each chunk (cu_tiles[b] = sum_{j<b} ceil(T_j / kTile), written by group 0),
// and the groups share out the chunk's tiles, writing one descriptor per tile
// (tile_word).  The tile's page is resolved here when no tile can span two
// pages (P a multiple of kTile).  A thread takes four tiles at a time: their
// sequences first (LDS), then all four table loads, then the stores, so the
// loads are in flight together.
__device__ inline void plan_block(const PlanInput& in, int32_t wg, int32_t nwg, PlanShared& sh) {
  const int32_t* __restrict__ seq_lens = in.seq_lens;
  const int32_t* __restrict__ block_table = in.block_table;
  const int32_t B = in.B, max_blocks = in.max_blocks, P = in.P, num_blocks = in.num_blocks;
  int32_t* __restrict__ cu_tiles = in.cu_tiles;
  int32_t* __restrict__ tiles = in.tiles;
  const bool sparse = in.indices != nullptr;
  const int tid = threadIdx.x;
  const bool one_page = !sparse && P % kTile == 0;
  // with more than one planning group, the last one writes the split table
  // and the others the tile descriptors, at the same time
  if (nwg > 1 && wg == nwg - 1) {
    plan_splits(in, sh);
    return;
  }
  const int32_t ntile_groups = nwg > 1 ? nwg - 1 : 1;
  const int32_t stride = ntile_groups * kPlanThreads;
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
    int32_t inc = n, unused = 0, tot, tu;
    plan_scan2(inc, unused, &tot, &tu, sh);
    sh.cu[tid + 1] = carry + inc;
    if (tid == 0) sh.cu[0] = carry;
    if (wg == 0 && tid < cnt) cu_tiles[b + 1] = carry + inc;
    __syncthreads();
    // tile t of this chunk belongs to the last local sequence j with cu[j] <= t
    // (sequences without tiles share their start with the next one)
    const int32_t t_end = carry + tot;
    for (int32_t t4 = carry + wg * kPlanThreads + tid; t4 < t_end; t4 += 4 * stride) {
      int32_t seq[4], tok[4], raw[4];
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const int32_t t = t4 + u * stride;
        int32_t lo = 0;
        if (t < t_end) {
          int32_t hi = cnt - 1;
          while (lo < hi) {
            const int32_t mid = (lo + hi + 1) >> 1;
            if (sh.cu[mid] <= t) lo = mid; else hi = mid - 1;
          }
        }
        seq[u] = lo;
        tok[u] = (t - sh.cu[lo]) * kTile;
      }
#pragma unroll
      for (int u = 0; u < 4; u++)
        raw[u] = one_page && t4 + u * stride < t_end
                     ? block_table[(int64_t)(base + seq[u]) * max_blocks + tok[u] / P]
                     : 0;
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const int32_t t = t4 + u * stride;
        if (t < t_end) {
          const int32_t T = sh.len[seq[u]], t0 = tok[u];
          const int32_t nv = min(kTile, T - t0);
          int32_t blk = -1, off = 0;
          if (one_page) {
            blk = raw[u] < 0 ? 0 : (raw[u] >= num_blocks ? num_blocks - 1 : raw[u]);
            off = t0 % P;
          }
          reinterpret_cast<int4*>(tiles)[t] =
              make_int4(blk, base + seq[u], t0, tile_word(nv, t0 + kTile >= T, off));
        }
      }
    }
    carry = t_end;
    __syncthreads();
  }
  if (nwg == 1) plan_splits(in, sh);
  if (!sparse) return;
  // slot list: entries e = b * idx_stride + n, eight per thread at a time so
  // that their index and table loads are in flight together
  const int32_t cap = max_blocks * P;
  const int32_t total = B * in.idx_stride;  // < 2^31 (checked on the host)
  const int32_t nthr = ntile_groups * kPlanThreads;
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

// Four fp32 values -> four bf16 (round to nearest even) in 8 bytes, the first
// in the low half of the first word: two packed conversions (v_cvt_pk_bf16_f32).
__device__ inline uint2 pack_bf16x4(float a, float b, float c, float d) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t lo = __builtin_convertvector((f32x2_t{a, b}), bf16x2_t);
  const bf16x2_t hi = __builtin_convertvector((f32x2_t{c, d}), bf16x2_t);
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

// One 32-value latent block of a matrix-core accumulator (32 latent values x
// 32 heads; lane 32 g + r holds head r, values 8 jj + 4 g + 0..3 in elements
// 4 jj .. 4 jj + 3), times s, stored as bf16 into the heads' partial rows
// (dst: lane r's row at the block's first value).  Lanes r and 32 + r swap
// halves (v_permlane32_swap) so that each lane stores 8 consecutive values,
// 16 bytes: lane r values 16 p + 0..7 and lane 32 + r values 16 p + 8..15 of
// each half p of the block.
template <typename V>
__device__ inline void store_block_bf16(uint16_t* dst, const V& o, float s, int lane) {
#pragma unroll
  for (int p = 0; p < 2; p++) {
    const uint2 x = pack_bf16x4(o[8 * p] * s, o[8 * p + 1] * s, o[8 * p + 2] * s, o[8 * p + 3] * s);
    const uint2 y = pack_bf16x4(o[8 * p + 4] * s, o[8 * p + 5] * s, o[8 * p + 6] * s, o[8 * p + 7] * s);
    // lanes 0..31 keep x and take the upper lanes' x; lanes 32..63 take the
    // lower lanes' y and keep their own
    const auto s0 = __builtin_amdgcn_permlane32_swap(x.x, y.x, false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(x.y, y.y, false, false);
    typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
    *reinterpret_cast<u32x4_t*>(dst + 16 * p + 8 * (lane >> 5)) = u32x4_t{s0[0], s1[0], s0[1], s1[1]};
  }
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
