// Host-side launchers of the MLA decode kernels (one translation unit each).
#pragma once

#include "mla_common.hpp"

namespace mla {

// Prefix sums of ceil(T_b / kTile) over the batch -> cu_tiles[B + 1], the
// descriptor of every tile -> tiles[n][4], and in sparse mode the slot list.
hipError_t launch_plan(const PlanInput& in, hipStream_t s);

// Where the split planner writes when it shares the absorption's launch
// (the PlanInput fields that do not come from the decode parameters).
struct PlanRequest {
  const int32_t* seq_lens;
  const int32_t* block_table;
  int32_t* cu_tiles;
  int32_t* tiles;
  int32_t splits;
  int32_t* split_first;
  int32_t* seq_splits;
  const int32_t* indices = nullptr;  // sparse mode
  int32_t idx_stride = 0;
  int32_t* slots = nullptr;
};

inline PlanInput plan_input(const mla_decode_params& p, const PlanRequest& r) {
  return PlanInput{r.seq_lens, r.block_table, p.batch, p.max_blocks_per_seq, p.page_size,
                   p.num_blocks, r.indices, r.idx_stride, r.slots, r.cu_tiles, r.tiles,
                   r.splits, r.split_first, r.seq_splits};
}

// The split table on the host (the planner's rules, for tests): tiles[b] =
// tiles of sequence b; writes split_first[splits + 1] and seq_splits[2 B].
void split_plan_host(const int32_t* tiles, int32_t B, int32_t splits, int32_t* split_first,
                     int32_t* seq_splits);

// q_lat[b,i,:d_c] = W_UK[i]^T q_nope[b,i,:]; q_lat[b,i,d_c:] = q_rope[b,i,:].
// With plan != null the matrix-core absorption also runs the split planner in
// the same launch and sets *planned; otherwise the caller launches the plan.
hipError_t launch_absorb(const mla_decode_params& p, const void* q, const void* W_UK, void* q_lat,
                         int32_t q_lat_dtype, const PlanRequest* plan, bool* planned,
                         hipStream_t s);

// Generic (any shape, any storage type) split attention -> partials.
hipError_t launch_attend_simt(const AttnArgs& a, int32_t cache_dtype, int32_t rope_dtype,
                              int32_t q_lat_dtype, hipStream_t s);

// Matrix-core split attention for d_c = 512, d_r = 64, h % 32 == 0, bf16 or fp8 latent,
// bf16 rope and bf16 absorbed query.
bool mfma_supported(const mla_decode_params& p);
int32_t mfma_streams(int32_t heads);
// Work groups that share one token split (head groups of 64 or 32 heads); with
// more than one, the split count must be a multiple of 8 (XCD pairing).
int32_t mfma_head_groups(int32_t heads);
// Heads one matrix-core work group serves (64, or 32 when heads is not a multiple of 64).
int32_t mfma_heads_per_group(int32_t heads);
// The optional events are stamped by the kernel's own dispatch (start and end
// of execution), not by separate markers queued around it.
hipError_t launch_attend_mfma(const AttnArgs& a, int32_t cache_dtype, hipStream_t s,
                              hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);

// Matrix-core split attention for an fp8 (E4M3) latent with per-token scales,
// d_c = 512, d_r = 64 bf16, h % 32 == 0, bf16 absorbed query; same head groups
// and partial layout as launch_attend_mfma.
bool mfma_fp8_supported(const mla_decode_params& p);
hipError_t launch_attend_fp8(const AttnArgs& a, hipStream_t s, hipEvent_t ev_start = nullptr,
                             hipEvent_t ev_stop = nullptr);

// Either matrix-core attention kernel serves this shape.
inline bool mfma_any_supported(const mla_decode_params& p) {
  return mfma_supported(p) || mfma_fp8_supported(p);
}

// Matrix-core absorb / up-projection for bf16 q and weights, d_c = 512
// (d_nope <= 128, multiple of 16; d_v multiple of 32).
bool proj_mfma_supported(const mla_decode_params& p);
// With plan != null the launch also runs the planner (as launch_plan would).
// With ex (TPLA, ex->g of at most 4 equal shards of the latent columns): q_lat receives the ex->g h shard heads' queries instead,
// shard-major (shard head j h + i: head i's query times ex->mu[j] on shard j's
// columns, 0 on the others, its rope part copied), the same values as
// absorption followed by launch_tpla_expand.
struct ShardExpand {
  int32_t g;
  float mu[4];
};
hipError_t launch_absorb_mfma(const mla_decode_params& p, const void* q, const void* W_UK,
                              void* q_lat, int32_t q_lat_dtype, const PlanRequest* plan,
                              hipStream_t s, const ShardExpand* ex = nullptr);
// Whether launch_absorb takes the matrix-core kernel for these pointers.
bool absorb_mfma_ok(const mla_decode_params& p, const void* q, const void* W_UK, const void* q_lat);
hipError_t launch_up_project_mfma(const mla_decode_params& p, const float* o_lat,
                                  const void* W_UV, void* out, hipStream_t s);

// Log-sum-exp merge of the token splits -> o_lat [B, h, d_c] fp32.
hipError_t launch_combine(const AttnArgs& a, float* o_lat, hipStream_t s);

// The merge and the up-projection in one launch, from the bf16 partials of a
// (a.shards 1): the same bits as launch_combine, then launch_up_project.
// Matrix-core shapes with bf16 weights, d_v = 128 and at most 16 sequences.
bool merge_up_supported(const mla_decode_params& p);
hipError_t launch_merge_up(const mla_decode_params& p, const AttnArgs& a, const void* W_UV,
                           void* out, hipStream_t s);

// out[b,i,:] = W_UV[i] o_lat[b,i,:].
hipError_t launch_up_project(const mla_decode_params& p, const float* o_lat, const void* W_UV,
                             void* out, hipStream_t s);

// Paged -> contiguous copy of the cache (storage bits).
hipError_t launch_gather(const mla_decode_params& p, const void* c_kv, const float* c_kv_scale,
                         const void* k_rope, const int32_t* block_table, const int32_t* seq_lens,
                         int32_t max_tokens, void* c_out, float* scale_out, void* rope_out,
                         hipStream_t s);

inline int32_t dtype_size(int32_t dt) { return dt == MLA_F32 ? 4 : (dt == MLA_BF16 ? 2 : 1); }

// Latent-cache writer (mla_cache_write.hip).
bool writer_mfma_ok(const mla_cache_write_params& p);
int32_t writer_chunks(const mla_cache_write_params& p);
hipError_t launch_cache_write(const mla_cache_write_params& p, const void* x, const void* W_DKV,
                              const void* gamma, const void* W_KR, const int32_t* positions,
                              const int32_t* block_table, void* c_kv, float* c_kv_scale,
                              void* k_rope, float* part, hipStream_t s);
hipError_t launch_quantize_rows(const float* x, int64_t rows, int32_t d, uint8_t* codes,
                                float* scales, hipStream_t s);

// TPLA decode (mla_tpla.hip): per-shard content factors, and the kernels that
// turn h heads into h g shard heads and back.
struct TplaMu {
  float v[4];
};
hipError_t launch_tpla_expand(const void* q1, void* q2, int32_t q_dtype, int32_t B, int32_t h,
                              int32_t g, int32_t d_c, int32_t d_r, const TplaMu& mu,
                              hipStream_t s);
hipError_t launch_tpla_gather(const float* o2, float* o1, int32_t B, int32_t h, int32_t g,
                              int32_t d_c, hipStream_t s);

// MHA-mode prefill (mla_prefill.hip): bf16 or fp8 cache, d_c 512, d_nope 128, d_rope 64, d_v 128.
bool prefill_supported(const mla_decode_params& p);
int32_t prefill_tpad(const mla_decode_params& p);  // token stride of the K / V^T workspace
// workspace bytes of one unit (sequence, head): its reconstructed keys and values
size_t prefill_unit_bytes(const mla_decode_params& p);
// units per chunk for a workspace of that size (0: not even one unit fits)
int64_t prefill_chunk_units(const mla_decode_params& p, int32_t max_q_len, size_t workspace_bytes);
hipError_t launch_prefill(const mla_decode_params& p, int32_t max_q_len, const void* q,
                          const int32_t* q_lens, const void* c_kv, const float* c_kv_scale,
                          const void* k_rope, const int32_t* block_table, const int32_t* seq_lens,
                          const void* W_UK, const void* W_UV, void* out, void* workspace,
                          size_t workspace_bytes, hipStream_t s);

// DSA indexer and top-k (mla_dsa.hip).
bool indexer_mfma_ok(int32_t heads, int32_t dim);
hipError_t launch_indexer(const uint8_t* q, const float* q_scale, const float* w, const uint8_t* k,
                          const float* k_scale, const int32_t* block_table,
                          const int32_t* seq_lens, float* scores, int32_t B, int32_t H, int32_t d,
                          int32_t P, int32_t max_blocks, int32_t num_blocks, int32_t stride,
                          hipStream_t s);
hipError_t launch_topk(const float* scores, int32_t score_stride, const int32_t* seq_lens,
                       int32_t B, int32_t k, int32_t* indices, int32_t index_stride,
                       int32_t* counts, hipStream_t s);
// The same selection with the candidate pass spread over several work groups
// per sequence; workspace of topk_split_ws_bytes(B, score_stride) bytes,
// 4-byte aligned.
size_t topk_split_ws_bytes(int32_t B, int32_t score_stride);
hipError_t launch_topk_split(const float* scores, int32_t score_stride, const int32_t* seq_lens,
                             int32_t B, int32_t k, int32_t* indices, int32_t index_stride,
                             int32_t* counts, void* workspace, hipStream_t s);

}  // namespace mla
