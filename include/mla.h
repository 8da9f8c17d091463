/*
 * mla.h -- C ABI of the MLA decode library for MI355X (gfx950).
 *
 * One decode step of multi-head latent attention over a paged, compressed
 * latent KV cache, run in absorbed form.  The operation is defined in
 * "TPLA: Tensor Parallel Latent Attention for Efficient Disaggregated Prefill
 * and Decode Inference", section 3.4 ("MLA Matrix Absorption": the key
 * absorption of Eq. 5 and "The RoPE handling"):
 *
 *   q_lat[b,i,:]  = W_UK[i]^T q_nope[b,i,:]                       (absorb)
 *   s[b,i,t]      = sm_scale * (q_lat[b,i,:] . c_KV[b,t,:]
 *                               + q_rope[b,i,:] . k_rope[b,t,:])
 *   p[b,i,:]      = softmax_t(s[b,i,:])
 *   o_lat[b,i,:]  = sum_t p[b,i,t] c_KV[b,t,:]
 *   out[b,i,:]    = W_UV[i] o_lat[b,i,:]                           (up-projection)
 *
 * which equals softmax((q_nope.(W_UK c) + q_rope.k_rope) * sm_scale) (W_UV c),
 * the unabsorbed form, by associativity.
 *
 * Beside the decode step the library holds the latent-cache writer, DSA
 * sparse decode (indexer, top-k, sparse step), TPLA decode, grouped-MLA
 * decode and MHA-mode prefill; each entry point's comment below cites the
 * passage that defines it.
 *
 * Conventions shared by every entry point:
 *   - All tensor arguments are DEVICE pointers owned by the caller; the
 *     library never allocates, frees or retains them.  Scratch memory is the
 *     caller's workspace.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream).  No entry point synchronises the host.
 *   - Host-side validation runs before any launch; on error a negative
 *     mla_status is returned, nothing is enqueued, and mla_last_error() gives
 *     a message (thread-local).  Launch failures return MLA_ERR_HIP.
 *   - Layouts are dense, row-major, innermost dimension last.  Indices are
 *     0-based.  bf16 is IEEE binary32's top 16 bits; fp8 is OCP E4M3FN.
 *   - The library is stateless and re-entrant; concurrent calls on different
 *     streams need separate workspaces and outputs.
 *
 * Cache layout (the paged latent cache):
 *   c_kv       [num_blocks, page_size, d_latent]   cache_dtype (bf16, fp8, f32)
 *   c_kv_scale [num_blocks, page_size] fp32        per-token scale, fp8 only:
 *              the latent row's value is scale * e4m3(byte)
 *   k_rope     [num_blocks, page_size, d_rope]     rope_dtype, already rotated
 *   block_table[batch, max_blocks_per_seq] int32   physical block of logical
 *              block j of sequence b
 *   seq_lens   [batch] int32                       cached tokens per sequence,
 *              including the current one
 *   Logical token t of sequence b lives in block block_table[b][t / page_size]
 *   at slot t % page_size.  Table entries at or past ceil(T_b / page_size) are
 *   never read, nor are slots at or past T_b.  Lengths are clamped on the
 *   device to [0, max_blocks_per_seq * page_size] and block ids to
 *   [0, num_blocks - 1], so malformed tables give wrong answers, not faults.
 *   A sequence with T_b = 0 produces a zero output.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = -1, /* bad shape, null pointer, inconsistent params */
  MLA_ERR_UNSUPPORTED = -2, /* valid but not implemented combination        */
  MLA_ERR_WORKSPACE = -3,   /* workspace null or smaller than required      */
  MLA_ERR_HIP = -4          /* a HIP runtime call or launch failed           */
} mla_status;

typedef enum { MLA_F32 = 0, MLA_BF16 = 1, MLA_FP8_E4M3 = 2 } mla_dtype;

typedef struct {
  int32_t batch;              /* B >= 1, with B x ceil(max_blocks_per_seq x
                               * page_size / 32) below 2^31                  */
  int32_t num_heads;          /* h  >= 1                                     */
  int32_t d_nope;             /* width of q_nope, rows of W_UK[i]            */
  int32_t d_rope;             /* width of q_rope and k_rope (may be 0)       */
  int32_t d_latent;           /* d_c, width of c_KV                          */
  int32_t d_v;                /* rows of W_UV[i], width of out               */
  int32_t page_size;          /* tokens per cache block, 1..4096             */
  int32_t max_blocks_per_seq; /* block_table row stride                      */
  int32_t num_blocks;         /* blocks in the pool                          */
  int32_t q_dtype;            /* mla_dtype of q: F32 or BF16                 */
  int32_t cache_dtype;        /* mla_dtype of c_kv: F32, BF16 or FP8_E4M3    */
  int32_t rope_dtype;         /* mla_dtype of k_rope: F32 or BF16            */
  int32_t weight_dtype;       /* mla_dtype of W_UK and W_UV: F32 or BF16     */
  int32_t out_dtype;          /* mla_dtype of out: F32 or BF16               */
  float sm_scale;             /* softmax scale; <= 0 means 1/sqrt(d_nope+d_rope) */
  int32_t num_splits;         /* token-split work groups; 0 = one per compute unit */
} mla_decode_params;

/* Static description of a status code. */
const char* mla_status_string(int32_t status);

/* Message for the last error returned on this thread ("" if none). */
const char* mla_last_error(void);

/* Bytes of workspace mla_decode and mla_attend_latent need for *p.  With
 * num_splits == 0 the count depends on the current device's compute units
 * (a HIP call); with num_splits > 0 no HIP call is made. */
mla_status mla_decode_workspace_size(const mla_decode_params* p, size_t* bytes);

/* Number of token-split work groups the kernels use for *p (resolves
 * num_splits == 0 against the current device). */
mla_status mla_decode_num_splits(const mla_decode_params* p, int32_t* splits);

/* Element type of the absorbed query that mla_absorb_q writes: MLA_F32 when
 * cache_dtype is F32, else MLA_BF16 (the matrix-core operand type). */
mla_status mla_absorbed_dtype(const mla_decode_params* p, int32_t* dtype);

/* The whole decode step (absorb, attention over the paged latent cache with
 * token splits and their log-sum-exp merge, W_UV up-projection).
 *   q           [B, h, d_nope + d_rope] q_dtype; q_rope (last d_rope) pre-rotated
 *   W_UK        [h, d_nope, d_latent]   weight_dtype
 *   W_UV        [h, d_v, d_latent]      weight_dtype
 *   out         [B, h, d_v]             out_dtype (written)
 *   c_kv_scale  must be non-NULL iff cache_dtype is FP8_E4M3
 *   workspace   >= mla_decode_workspace_size bytes, 256-byte aligned
 * Cache arguments as described at the top of this header.  For a fixed
 * split count the result is bitwise deterministic run to run. */
mla_status mla_decode(const mla_decode_params* p, const void* q, const void* c_kv,
                      const float* c_kv_scale, const void* k_rope,
                      const int32_t* block_table, const int32_t* seq_lens,
                      const void* W_UK, const void* W_UV, void* out,
                      void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): mla_decode
 * with the workspace taken from a fixed array of MLA_NO_ALLOC_SCRATCH_BYTES
 * bytes of device memory that the library holds on each device it runs on
 * (from its first use there until the process ends).  The call makes no
 * allocation of its own.  Arguments, results and errors as for mla_decode,
 * less the workspace; MLA_ERR_WORKSPACE when mla_decode_workspace_size(p)
 * exceeds MLA_NO_ALLOC_SCRATCH_BYTES (checked before any HIP call when
 * num_splits > 0; fewer splits or a smaller batch fit).  Every call on one
 * device shares that device's array and nothing in it needs to start at zero
 * (each call writes what it reads), so calls that overlap on one device --
 * on two streams, or from two threads -- race and must be ordered by the
 * caller.  Devices 0..63. */
#define MLA_NO_ALLOC_SCRATCH_BYTES (128u << 20)
mla_status mla_decode_no_alloc(const mla_decode_params* p, const void* q, const void* c_kv,
                               const float* c_kv_scale, const void* k_rope,
                               const int32_t* block_table, const int32_t* seq_lens,
                               const void* W_UK, const void* W_UV, void* out, void* stream);

/* mla_decode that also records two caller-created hipEvent_t (may be NULL)
 * at the start and end of the split-attention kernel, so the caller can time
 * that kernel alone (hipEventElapsedTime).  The matrix-core kernels take the
 * events into their own dispatch, so the interval is the kernel's execution;
 * the generic kernel is bracketed by event records on `stream`.  Same
 * arguments, results and errors as mla_decode otherwise. */
mla_status mla_decode_timed(const mla_decode_params* p, const void* q, const void* c_kv,
                            const float* c_kv_scale, const void* k_rope,
                            const int32_t* block_table, const int32_t* seq_lens,
                            const void* W_UK, const void* W_UV, void* out, void* workspace,
                            size_t workspace_bytes, void* stream, void* ev_before,
                            void* ev_after);

/* Stage: query absorption ("MLA Matrix Absorption", Eq. 5).
 *   q_lat [B, h, d_latent + d_rope] of mla_absorbed_dtype: the first d_latent
 *   values are W_UK[i]^T q_nope[b,i,:] (fp32 accumulation, then rounded),
 *   the last d_rope are q_rope copied. */
mla_status mla_absorb_q(const mla_decode_params* p, const void* q, const void* W_UK,
                        void* q_lat, void* stream);

/* Stage: attention in the latent space over the paged cache, split along
 * tokens, partial results merged by their log-sum-exp ("The RoPE handling"
 * score, softmax, p . c_KV): mla_attend_partial followed by mla_combine.
 *   q_lat [B, h, d_latent + d_rope] as written by mla_absorb_q
 *   o_lat [B, h, d_latent] fp32 (written)
 *   workspace as for mla_decode. */
mla_status mla_attend_latent(const mla_decode_params* p, const void* q_lat, const void* c_kv,
                             const float* c_kv_scale, const void* k_rope,
                             const int32_t* block_table, const int32_t* seq_lens,
                             float* o_lat, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Stage: the split attention alone ("The RoPE handling" score, the softmax
 * over each split's tokens and p . c_KV over them; TPLA section 3.4, Eq. 5):
 * plans the token splits (split rules above) and writes, for every
 * (split, sequence) pair that shares tokens, the split's normalised partial
 * output o_s = sum_t p_t c_t / sum_t p_t and its log-sum-exp
 * lse_s = m + ln sum_t exp(s_t - m) into the workspace.  q_lat, the cache
 * arguments and the workspace as for mla_attend_latent; the partials stay in
 * the workspace for mla_combine (mla_partials_layout says where). */
mla_status mla_attend_partial(const mla_decode_params* p, const void* q_lat, const void* c_kv,
                              const float* c_kv_scale, const void* k_rope,
                              const int32_t* block_table, const int32_t* seq_lens,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Stage: the log-sum-exp merge of the partials that mla_attend_partial left
 * in `workspace` (same *p, enqueued after it):
 *   o_lat[b,i,:] = sum_s e^(lse_s - M) o_s / sum_s e^(lse_s - M),  M = max_s lse_s
 * over the splits s holding tokens of sequence b -- the exact merge of
 * softmax partials over disjoint token ranges.  A sequence with one split gets
 * its partial back unchanged; one with no tokens gets zeros.
 *   o_lat [B, h, d_latent] fp32 (written). */
mla_status mla_combine(const mla_decode_params* p, float* o_lat, void* workspace,
                       size_t workspace_bytes, void* stream);

/* Where mla_attend_partial keeps the partials of *p in the workspace; slots =
 * splits + batch, and the pair (split g, sequence b) uses slot g + b.  Slot
 * k's o_s block is row-major [h][d_latent], head i's row starting at element
 * (k h + i) d_latent from part_o_offset:
 *  - bf16_rows = 1 for the shapes the matrix-core kernels serve (d_latent
 *    512, heads a multiple of 32, bf16 or fp8 cache): o_s is bf16;
 *  - otherwise o_s is fp32.
 * lse_s of slot k and head i is fp32 at part_lse_offset + (k h + i) 4. */
mla_status mla_partials_layout(const mla_decode_params* p, size_t* part_o_offset,
                               size_t* part_lse_offset, int32_t* slots, int32_t* bf16_rows);

/* Stage: value up-projection, kept apart from W_O ("MLA Matrix Absorption":
 * W_UV is in practice not folded into the output projection).
 *   o_lat [B, h, d_latent] fp32;  out [B, h, d_v] out_dtype (written). */
mla_status mla_up_project(const mla_decode_params* p, const float* o_lat, const void* W_UV,
                          void* out, void* stream);

/* Debug/test: copy the paged cache to contiguous per-sequence rows, bit for
 * bit in the storage type.
 *   c_out     [B, max_tokens, d_latent] cache_dtype
 *   scale_out [B, max_tokens] fp32 (fp8 only; else may be NULL)
 *   rope_out  [B, max_tokens, d_rope]   rope_dtype
 * Rows at or past min(T_b, max_tokens) are zero-filled. */
mla_status mla_gather_cache(const mla_decode_params* p, const void* c_kv, const float* c_kv_scale,
                            const void* k_rope, const int32_t* block_table,
                            const int32_t* seq_lens, int32_t max_tokens, void* c_out,
                            float* scale_out, void* rope_out, void* stream);

/* Host-side split arithmetic (no HIP call; the kernels' planner follows the
 * same rules on the device).  The cache of all sequences is cut into 32-token
 * tiles, numbered across sequences in order, and every split (token-split work
 * group) owns a contiguous run of them.  Two rules, chosen by the batch size:
 *  - batch <= splits and batch <= 2048: no split crosses a sequence.  With n_b tiles in
 *    sequence b, L is the least bound with sum_b ceil(n_b / L) <= splits;
 *    sequence b gets k_b = ceil(n_b / L) splits in order, its i-th owning its
 *    tiles [n_b i / k_b, n_b (i + 1) / k_b); splits left over own nothing.
 *  - otherwise: split g owns tiles [n g / splits, n (g + 1) / splits) of
 *    all n tiles (mla_split_begin); mla_split_owner returns the split owning
 *    a tile under this rule.
 * mla_split_plan applies the rule to tiles[batch] (tiles per sequence, >= 0,
 * summing below 2^31) and writes split_first[splits + 1] (split g owns
 * [split_first[g], split_first[g + 1])) and seq_splits[2 batch] (first and
 * last split holding a tile of sequence b; last < first when it has none).
 * Errors: MLA_ERR_INVALID_ARG for batch < 1, splits < 1, a null array or a
 * negative count; MLA_ERR_UNSUPPORTED for 2^31 tiles or more. */
int64_t mla_split_begin(int64_t n_tiles, int32_t splits, int32_t g);
int32_t mla_split_owner(int64_t n_tiles, int32_t splits, int64_t tile);
mla_status mla_split_plan(const int32_t* tiles, int32_t batch, int32_t splits,
                          int32_t* split_first, int32_t* seq_splits);

/* ------------------------------------------------------------------------
 * Latent-cache writer: appends one new token per sequence to the paged cache
 * above ("TransMLA: Multi-Head Latent Attention Is All You Need", the MLA
 * structure after conversion: the cached latent is a down projection of the
 * hidden state, the decoupled RoPE key a second projection rotated to the
 * token's position; "TPLA: ...", "RMSNorm Slicing", Eqs. 8-9: the latent is
 * RMS-normalised).  For each sequence b with t = positions[b]:
 *   y      = W_DKV x[b]            (d_latent; fp32 accumulation)
 *   c      = y / sqrt(mean(y^2) + rms_eps) * gamma
 *   r      = W_KR x[b]             (d_rope)
 *   k      = r with pair i (dims 2i, 2i+1) turned by t * rope_base^(-2i/d_rope):
 *            (u, v) -> (u cos a - v sin a, u sin a + v cos a)
 *   c_kv[blk][t % P] = c, k_rope[blk][t % P] = k, blk = block_table[b][t / P].
 * An fp8 latent row is stored as the OCP E4M3FN codes of c / s, s = max|c| / 448
 * (fp32, round to nearest even, values clamped to +-448; an all-zero row has
 * s = 0 and zero codes), with s in c_kv_scale[blk][t % P].
 * A sequence whose position is negative, or whose table entry is past the row
 * or outside [0, num_blocks), is skipped (nothing written).  Two sequences
 * naming the same slot race; the caller keeps slots distinct.
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t batch;              /* sequences (one new token each); 0 = no-op   */
  int32_t d_model;            /* hidden size of x                            */
  int32_t d_latent;           /* latent width (rows of W_DKV)                */
  int32_t d_rope;             /* rope key width (rows of W_KR), even; d_latent
                                 + d_rope <= 8192                             */
  int32_t page_size;          /* tokens per block                            */
  int32_t max_blocks_per_seq; /* block_table row stride                      */
  int32_t num_blocks;         /* pool size                                   */
  int32_t x_dtype;            /* F32 or BF16                                 */
  int32_t weight_dtype;       /* W_DKV, W_KR and gamma: F32 or BF16          */
  int32_t cache_dtype;        /* c_kv: F32, BF16 or FP8_E4M3                 */
  int32_t rope_dtype;         /* k_rope: F32 or BF16                         */
  float rms_eps;              /* >= 0                                        */
  float rope_base;            /* > 0, e.g. 10000                             */
} mla_cache_write_params;

/* Workspace bytes mla_cache_write needs (fp32 partial projections). */
mla_status mla_cache_write_workspace_size(const mla_cache_write_params* p, size_t* bytes);

/* The writer.
 *   x           [batch, d_model]            x_dtype
 *   W_DKV       [d_latent, d_model]         weight_dtype
 *   gamma       [d_latent]                  weight_dtype
 *   W_KR        [d_rope, d_model]           weight_dtype
 *   positions   [batch] int32 (device)      0-based position of the new token
 *   block_table [batch, max_blocks_per_seq] int32 (device)
 *   c_kv, c_kv_scale, k_rope                the pools, as at the top of this
 *               header; c_kv_scale must be non-NULL iff cache_dtype is FP8
 *   workspace   >= mla_cache_write_workspace_size bytes, 256-byte aligned
 * For fixed parameters the result is bitwise deterministic run to run. */
mla_status mla_cache_write(const mla_cache_write_params* p, const void* x, const void* W_DKV,
                           const void* gamma, const void* W_KR, const int32_t* positions,
                           const int32_t* block_table, void* c_kv, float* c_kv_scale,
                           void* k_rope, void* workspace, size_t workspace_bytes, void* stream);

/* The writer's fp8 row encoding on its own: rows x [rows, d] fp32 ->
 * codes [rows, d] (E4M3FN) and scales [rows], by the rule above.
 * 1 <= d <= 8192; rows >= 0 (0 = no-op). */
mla_status mla_quantize_e4m3_rows(const float* x, int64_t rows, int32_t d, uint8_t* codes,
                                  float* scales, void* stream);

/* ------------------------------------------------------------------------
 * DeepSeek Sparse Attention (DSA) at decode time ("TransMLA & Sparse Latent
 * Attention", Chapter 6 "DeepSeek's Second Wall": "The lightning indexer",
 * "Fine-grained token selection"; Chapter 7: DSA runs on MLA's absorbed
 * (MQA-mode) decode path, one selection per token shared by all heads, and
 * every cached position keeps an indexer key beside its latent).
 *
 *   I[b, s] = sum_j w[b, j] * ReLU(q_I[b, j, :] . k_I[b, s, :])  (no softmax)
 *   S_b     = the k positions s < T_b with the largest I[b, s]; equal scores
 *             go to the earlier position; every position when T_b <= k
 *   out     = the decode step above with the softmax over S_b only.
 *
 * Indexer storage (fp8, as the chapter runs it):
 *   q_I       [batch, index_heads, index_dim]  E4M3FN codes
 *   q_I_scale [batch, index_heads] fp32        value = scale * e4m3(code), > 0
 *   w_I       [batch, index_heads] fp32        head weights (any sign)
 *   k_I       [num_blocks, page_size, index_dim] E4M3FN codes, paged through
 *             the same block table as c_kv
 *   k_I_scale [num_blocks, page_size] fp32     per-slot scale, >= 0
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t index_heads;  /* H_I >= 1 (64 in DeepSeek-V3.2; the matrix-core
                           indexer serves 64 heads of width 128)           */
  int32_t index_dim;    /* d_I, 1..1024 (128 in DeepSeek-V3.2)              */
  int32_t topk;         /* k >= 1 (2048 in DeepSeek-V3.2)                   */
} mla_dsa_params;

/* Index scores of every cached position of every sequence.  Uses batch,
 * page_size, max_blocks_per_seq and num_blocks of *p.
 *   scores [batch, score_stride] fp32: scores[b][s] for s < min(T_b,
 *   max_blocks_per_seq * page_size, score_stride); other entries untouched.
 * The matrix-core path (64 heads, width 128) needs q_I and k_I 16-byte
 * aligned.  fp32 accumulation; the head sum is in a fixed order, so results
 * are bitwise reproducible. */
mla_status mla_indexer_scores(const mla_decode_params* p, const mla_dsa_params* d,
                              const uint8_t* q_I, const float* q_I_scale, const float* w_I,
                              const uint8_t* k_I, const float* k_I_scale,
                              const int32_t* block_table, const int32_t* seq_lens, float* scores,
                              int32_t score_stride, void* stream);

/* Top-k selection per sequence: with T_b = clamp(seq_lens[b], 0,
 * score_stride), writes min(T_b, k) positions, increasing, to
 * indices[b][0 ..) (row stride index_stride >= k) and that count to
 * counts[b].  Scores are ordered as floats (-0 equals +0; NaN by its bits);
 * equal scores go to the earlier position.  Integer-exact: the same scores
 * always give the same selection. */
mla_status mla_topk_select(const float* scores, int32_t score_stride, const int32_t* seq_lens,
                           int32_t batch, int32_t k, int32_t* indices, int32_t index_stride,
                           int32_t* counts, void* stream);

/* The same selection (same results bit for bit) with each sequence's
 * candidate pass spread over work groups of 2048 positions, for batches too
 * small to fill the GPU with one work group per sequence ("TransMLA & Sparse
 * Latent Attention", Chapter 6, "Fine-grained token selection": the k
 * highest-scoring positions).  batch <= 65535.  The workspace (device memory,
 * caller-owned, 256-byte aligned, contents on entry irrelevant) holds the
 * candidate positions and keys: mla_topk_select_split_workspace_size bytes,
 * about 8 x min(score_stride, 262144) bytes per sequence. */
mla_status mla_topk_select_split_workspace_size(int32_t batch, int32_t score_stride, size_t* bytes);

mla_status mla_topk_select_split(const float* scores, int32_t score_stride,
                                 const int32_t* seq_lens, int32_t batch, int32_t k,
                                 int32_t* indices, int32_t index_stride, int32_t* counts,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace mla_decode_sparse needs for index lists of row stride
 * index_stride (>= 1). */
mla_status mla_decode_sparse_workspace_size(const mla_decode_params* p, int32_t index_stride,
                                            size_t* bytes);

/* The decode step over index lists: sequence b attends to the counts[b]
 * (clamped to [0, index_stride]) cached positions indices[b][0 .. counts[b])
 * instead of all its tokens.  Positions are clamped into
 * [0, max_blocks_per_seq * page_size) and resolved through block_table; a
 * position past T_b reads whatever its slot holds.  A repeated position
 * counts twice.  Other arguments and rules as for mla_decode. */
mla_status mla_decode_sparse(const mla_decode_params* p, const void* q, const void* c_kv,
                             const float* c_kv_scale, const void* k_rope,
                             const int32_t* block_table, const int32_t* indices,
                             int32_t index_stride, const int32_t* counts, const void* W_UK,
                             const void* W_UV, void* out, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Bytes of workspace mla_dsa_decode needs. */
mla_status mla_dsa_decode_workspace_size(const mla_decode_params* p, const mla_dsa_params* d,
                                         size_t* bytes);

/* The whole DSA decode step: index scores, top-k, and the decode over the
 * selection (mla_indexer_scores, mla_topk_select, mla_decode_sparse on the
 * workspace).  indices_out [batch, topk] int32 may be NULL; when given it
 * receives the selection (min(T_b, topk) positions per row, increasing; the
 * rest of the row is untouched). */
mla_status mla_dsa_decode(const mla_decode_params* p, const mla_dsa_params* d, const void* q,
                          const void* c_kv, const float* c_kv_scale, const void* k_rope,
                          const int32_t* block_table, const int32_t* seq_lens,
                          const uint8_t* q_I, const float* q_I_scale, const float* w_I,
                          const uint8_t* k_I, const float* k_I_scale, const void* W_UK,
                          const void* W_UV, void* out, int32_t* indices_out, void* workspace,
                          size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Prefill in MHA mode ("TransMLA & Sparse Latent Attention", Chapter 7: MLA
 * runs in its MHA-like mode for prefill, reconstructing full-width keys and
 * values; "TPLA: ...", section 3.4, Eq. 4).  For sequence b with T_b cached
 * tokens (seq_lens; the new tokens already written to the cache) and
 * L_b = clamp(q_lens[b], 0, min(max_q_len, T_b)) new query tokens, query l sits
 * at position T_b - L_b + l and, per head i,
 *   out[b, l, i] = softmax_{t <= T_b - L_b + l}(sm_scale (q_nope . W_UK[i] c_t
 *                  + q_rope . k_rope_t)) (W_UV[i] c_t)
 *   q   [B, max_q_len, h, d_nope + d_rope]   bf16, q_rope pre-rotated
 *   out [B, max_q_len, h, d_v]               out_dtype (rows l >= L_b untouched)
 * Supported: bf16 q, rope and weights, a bf16 or fp8 (E4M3 with c_kv_scale,
 * which must be NULL otherwise) cache, with d_latent 512, d_nope 128, d_rope
 * 64, d_v 128 (else MLA_ERR_UNSUPPORTED); q, c_kv, k_rope, W_UK and W_UV
 * 16-byte aligned.  The work is taken in chunks of consecutive units (b, i),
 * unit b h + i; for each chunk the workspace (256-byte aligned, caller-owned)
 * holds the reconstructed keys (nope and rope parts) and values of every
 * cached token of the chunk's units: Tpad x (192 + 128) bf16 values a unit,
 * Tpad = max_blocks_per_seq x page_size rounded up to 128.  Any workspace of
 * at least one unit works (MLA_ERR_WORKSPACE below that); a larger one means
 * fewer, larger chunks (at most 65535 units each, split evenly).
 * mla_prefill_workspace_size returns every unit's size when that is at most
 * MLA_PREFILL_DEFAULT_WORKSPACE_BYTES, else the most units that fit in it (at
 * least one).  Chunks run in order on the stream; the workspace is free once
 * the call's work on the stream has completed.
 * ------------------------------------------------------------------------ */
#define MLA_PREFILL_DEFAULT_WORKSPACE_BYTES ((size_t)1 << 30)

mla_status mla_prefill_workspace_size(const mla_decode_params* p, size_t* bytes);

mla_status mla_prefill(const mla_decode_params* p, int32_t max_q_len, const void* q,
                       const int32_t* q_lens, const void* c_kv, const float* c_kv_scale,
                       const void* k_rope,
                       const int32_t* block_table, const int32_t* seq_lens, const void* W_UK,
                       const void* W_UV, void* out, void* workspace, size_t workspace_bytes,
                       void* stream);

/* ------------------------------------------------------------------------
 * Grouped MLA decode (the TransMLA OpenReview discussion, reply A2 to the
 * FlashMLA question: a kv_rank of 1088 held as two 512-wide latent groups plus
 * one 64-wide positional part, each group served like an ordinary 576-wide MLA
 * cache).  The heads are split evenly over latent_groups groups; head i reads
 * latent group g = i / (num_heads / latent_groups) and the shared rope key:
 *   c_kv       [latent_groups][num_blocks, page_size, d_latent]  group-major pools
 *   c_kv_scale [latent_groups][num_blocks, page_size] fp32       (fp8 only)
 *   k_rope     [num_blocks, page_size, d_rope]                    shared
 * W_UK[i] and W_UV[i] act on head i's group (shapes as for mla_decode).  Every
 * other argument, the workspace size (mla_decode_workspace_size) and the rules
 * are mla_decode's; latent_groups = 1 is mla_decode.  The matrix-core kernels
 * serve it when num_heads / latent_groups is a multiple of 64 (32 when
 * num_heads is not a multiple of 64); other splits use the generic kernel.
 * ------------------------------------------------------------------------ */
mla_status mla_grouped_decode(const mla_decode_params* p, int32_t latent_groups, const void* q,
                              const void* c_kv, const float* c_kv_scale, const void* k_rope,
                              const int32_t* block_table, const int32_t* seq_lens,
                              const void* W_UK, const void* W_UV, void* out, void* workspace,
                              size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * TPLA decode ("TPLA: Tensor Parallel Latent Attention for Efficient
 * Disaggregated Prefill and Decode Inference", "The Core TPLA Computation and
 * Structural Differences from GLA", Eqs. 6-7; "TPLA as a special case of GLA",
 * Section 4.4), emulated on one GPU: the latent dimension is cut into
 * `shards` contiguous equal slices S_j; for every head
 *   o_j = softmax_t(sm_scale (mu_j q_lat[S_j] . c_t[S_j] + q_rope . k_rope_t)) c[:, S_j]
 *   out = sum_j W_UV[i][:, S_j] o_j
 * (each shard its own softmax; the rope key replicated on every shard).  With
 * shards = 1 and mu_0 = 1 this is mla_decode.  The cache and weights are used
 * as given: a change of latent basis (the page's Hadamard or PCA
 * reparameterisation) is applied to them beforehand by the caller.
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t shards;  /* g: 1, 2 or 4; d_latent must divide by it              */
  float mu[4];     /* content-score factor of each shard (finite; 1 = none) */
} mla_tpla_params;

/* Bytes of workspace mla_tpla_decode needs. */
mla_status mla_tpla_decode_workspace_size(const mla_decode_params* p, const mla_tpla_params* t,
                                          size_t* bytes);

/* The TPLA decode step above; arguments and rules as for mla_decode.
 * Runs as: absorption, expansion to shards x num_heads shard heads (zero
 * outside their shard), the split attention and merge over those heads, the
 * gather of each head's shard columns, and the up-projection. */
mla_status mla_tpla_decode(const mla_decode_params* p, const mla_tpla_params* t, const void* q,
                           const void* c_kv, const float* c_kv_scale, const void* k_rope,
                           const int32_t* block_table, const int32_t* seq_lens, const void* W_UK,
                           const void* W_UV, void* out, void* workspace, size_t workspace_bytes,
                           void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MLA_H_ */
