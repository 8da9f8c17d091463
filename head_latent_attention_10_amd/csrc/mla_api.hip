// C ABI: host-side validation, workspace layout and launch sequencing.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "mla_kernels.hpp"

// Workspace of mla_decode_no_alloc: a fixed array of device memory that comes
// with the code object, so that call allocates nothing.  Each device holds its
// own copy at its own address, from the library's first use of the array on
// it until the process ends.  In host code this name is a stand-in, never a
// device address: host code uses the per-device address that
// hipGetSymbolAddress returns (no_alloc_scratch below).
static __device__ __align__(256) unsigned char scratch[MLA_NO_ALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

mla_status fail(mla_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
mla_status fail(mla_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

mla_status hip_fail(hipError_t e, const char* what) {
  return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool is_dtype(int32_t d, bool allow_fp8) {
  return d == MLA_F32 || d == MLA_BF16 || (allow_fp8 && d == MLA_FP8_E4M3);
}

mla_status validate(const mla_decode_params* p) {
  if (!p) return fail(MLA_ERR_INVALID_ARG, "params is NULL");
  if (p->batch < 1 || p->num_heads < 1 || p->d_nope < 1 || p->d_rope < 0 || p->d_latent < 1 ||
      p->d_v < 1)
    return fail(MLA_ERR_INVALID_ARG,
                "shape out of range (batch=%d heads=%d d_nope=%d d_rope=%d d_latent=%d d_v=%d)",
                p->batch, p->num_heads, p->d_nope, p->d_rope, p->d_latent, p->d_v);
  if (p->page_size < 1 || p->page_size > 4096)
    return fail(MLA_ERR_INVALID_ARG, "page_size %d outside [1, 4096]", p->page_size);
  if (p->max_blocks_per_seq < 1 || p->num_blocks < 1)
    return fail(MLA_ERR_INVALID_ARG, "max_blocks_per_seq=%d num_blocks=%d must be >= 1",
                p->max_blocks_per_seq, p->num_blocks);
  if ((int64_t)p->max_blocks_per_seq * p->page_size > (int64_t)1 << 30)
    return fail(MLA_ERR_INVALID_ARG, "table capacity above 2^30 tokens per sequence");
  if ((int64_t)p->batch * (((int64_t)p->max_blocks_per_seq * p->page_size + mla::kTile - 1) /
                           mla::kTile) >= ((int64_t)1 << 31))
    return fail(MLA_ERR_UNSUPPORTED, "batch x table capacity above 2^31 tiles of %d tokens",
                mla::kTile);
  if (p->num_splits < 0 || p->num_splits > 65535)
    return fail(MLA_ERR_INVALID_ARG, "num_splits %d outside [0, 65535]", p->num_splits);
  if (!std::isfinite(p->sm_scale)) return fail(MLA_ERR_INVALID_ARG, "sm_scale not finite");
  if (!is_dtype(p->q_dtype, false) || !is_dtype(p->cache_dtype, true) ||
      !is_dtype(p->rope_dtype, false) || !is_dtype(p->weight_dtype, false) ||
      !is_dtype(p->out_dtype, false))
    return fail(MLA_ERR_INVALID_ARG, "unknown dtype code (q=%d cache=%d rope=%d weight=%d out=%d)",
                p->q_dtype, p->cache_dtype, p->rope_dtype, p->weight_dtype, p->out_dtype);
  if (p->d_nope > 1024 || p->d_rope > 1024 || p->d_v > 4096)
    return fail(MLA_ERR_UNSUPPORTED, "d_nope <= 1024, d_rope <= 1024 and d_v <= 4096 required");
  if (!mla::mfma_any_supported(*p) && p->d_latent > 1024)
    return fail(MLA_ERR_UNSUPPORTED, "d_latent %d above 1024 outside the matrix-core shape",
                p->d_latent);
  return MLA_OK;
}

int32_t absorbed_dtype(const mla_decode_params& p) {
  return p.cache_dtype == MLA_F32 ? MLA_F32 : MLA_BF16;
}

struct Layout {
  size_t q_lat, cu_tiles, split_first, seq_splits, tiles, part_o, part_lse, o_lat, entry_slots,
      total;
  int32_t splits, streams;
  int64_t slots;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Token splits.  The matrix-core kernel serves a split's heads with HG work
// groups that must share an XCD, which needs the split count to be a multiple
// of 8 when HG > 1; by default one work group runs per compute unit.
mla_status resolve_splits(const mla_decode_params& p, int32_t* splits) {
  const int32_t hg = mla::mfma_any_supported(p) ? mla::mfma_head_groups(p.num_heads) : 1;
  int32_t n = p.num_splits;
  if (n <= 0) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(multiProcessorCount)");
    n = cus / hg;
  }
  if (n < 1) n = 1;
  if (hg > 1) n = (n + 7) / 8 * 8;
  *splits = n;
  return MLA_OK;
}

// sparse_stride > 0: the sparse decode (index lists of that stride) -- tiles
// cover at most sparse_stride entries per sequence, plus the slot list.
mla_status layout(const mla_decode_params& p, Layout* L, int32_t sparse_stride = 0) {
  mla_status st = resolve_splits(p, &L->splits);
  if (st != MLA_OK) return st;
  L->streams = mla::mfma_any_supported(p) ? mla::mfma_streams(p.num_heads) : 1;
  L->slots = ((int64_t)L->splits + p.batch) * L->streams;
  const size_t B = p.batch, h = p.num_heads, dc = p.d_latent, dr = p.d_rope;
  size_t off = 0;
  L->q_lat = off;
  off = align256(off + B * h * (dc + dr) * mla::dtype_size(absorbed_dtype(p)));
  L->cu_tiles = off;
  off = align256(off + (B + 1) * sizeof(int32_t));
  L->split_first = off;
  off = align256(off + ((size_t)L->splits + 1) * sizeof(int32_t));
  L->seq_splits = off;
  off = align256(off + 2 * B * sizeof(int32_t));
  L->tiles = off;
  const size_t cap = sparse_stride > 0 ? (size_t)sparse_stride
                                        : (size_t)p.max_blocks_per_seq * p.page_size;
  const size_t tiles_per_seq = (cap + mla::kTile - 1) / mla::kTile;
  off = align256(off + B * tiles_per_seq * 4 * sizeof(int32_t));
  L->part_o = off;
  // partials of the matrix-core shapes are bf16, others fp32
  off = align256(off + (size_t)L->slots * h * dc * (mla::mfma_any_supported(p) ? 2 : 4));
  L->part_lse = off;
  off = align256(off + (size_t)L->slots * h * sizeof(float));
  L->o_lat = off;
  off = align256(off + B * h * dc * sizeof(float));
  L->entry_slots = off;
  if (sparse_stride > 0) off = align256(off + B * (size_t)sparse_stride * sizeof(int32_t));
  L->total = off;
  return MLA_OK;
}

mla_status validate_sparse(const mla_decode_params& p, int32_t stride) {
  if (stride < 1) return fail(MLA_ERR_INVALID_ARG, "index_stride %d must be >= 1", stride);
  if ((int64_t)p.batch * stride >= ((int64_t)1 << 31))
    return fail(MLA_ERR_UNSUPPORTED, "batch x index_stride at or above 2^31");
  if ((int64_t)p.num_blocks * p.page_size >= ((int64_t)1 << 31))
    return fail(MLA_ERR_UNSUPPORTED, "pool of 2^31 slots or more (slot list is int32)");
  return MLA_OK;
}

float resolved_scale(const mla_decode_params& p) {
  return p.sm_scale > 0.f ? p.sm_scale : 1.0f / std::sqrt((float)(p.d_nope + p.d_rope));
}

mla_status check_cache_ptrs(const mla_decode_params* p, const void* c_kv, const float* c_kv_scale,
                            const void* k_rope, const int32_t* block_table,
                            const int32_t* seq_lens) {
  if (!c_kv || !block_table || !seq_lens || (p->d_rope > 0 && !k_rope))
    return fail(MLA_ERR_INVALID_ARG, "null cache, table or length pointer");
  if ((p->cache_dtype == MLA_FP8_E4M3) != (c_kv_scale != nullptr))
    return fail(MLA_ERR_INVALID_ARG, "c_kv_scale must be given exactly when the cache is fp8");
  return MLA_OK;
}

mla_status check_workspace(const Layout& L, void* ws, size_t bytes) {
  if (!ws) return fail(MLA_ERR_WORKSPACE, "workspace is NULL");
  if (bytes < L.total)
    return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes, %zu required", bytes, L.total);
  if (reinterpret_cast<uintptr_t>(ws) & 255)
    return fail(MLA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return MLA_OK;
}

// The planner's inputs and outputs for this layout (dense, or sparse when
// indices is given).
mla::PlanRequest plan_request(const Layout& L, char* ws, const int32_t* block_table,
                              const int32_t* seq_lens, const int32_t* indices = nullptr,
                              int32_t stride = 0) {
  mla::PlanRequest r{seq_lens, block_table, reinterpret_cast<int32_t*>(ws + L.cu_tiles),
                     reinterpret_cast<int32_t*>(ws + L.tiles), L.splits,
                     reinterpret_cast<int32_t*>(ws + L.split_first),
                     reinterpret_cast<int32_t*>(ws + L.seq_splits)};
  if (indices) {
    r.indices = indices;
    r.idx_stride = stride;
    r.slots = reinterpret_cast<int32_t*>(ws + L.entry_slots);
  }
  return r;
}

// Everything the attention and combine kernels need to know about the problem
// and the workspace, but the cache pointers.
mla::AttnArgs attn_args(const mla_decode_params& p, const Layout& L, char* ws,
                        const int32_t* block_table, const int32_t* seq_lens) {
  mla::AttnArgs a{};
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.cu_tiles = reinterpret_cast<int32_t*>(ws + L.cu_tiles);
  a.tiles = reinterpret_cast<int32_t*>(ws + L.tiles);
  a.split_first = reinterpret_cast<int32_t*>(ws + L.split_first);
  a.seq_splits = reinterpret_cast<int32_t*>(ws + L.seq_splits);
  a.part_o = ws + L.part_o;
  a.part_lse = reinterpret_cast<float*>(ws + L.part_lse);
  a.B = p.batch;
  a.h = p.num_heads;
  a.d_c = p.d_latent;
  a.d_r = p.d_rope;
  a.P = p.page_size;
  a.log2P = (p.page_size & (p.page_size - 1)) == 0 ? __builtin_ctz(p.page_size) : -1;
  a.max_blocks = p.max_blocks_per_seq;
  a.num_blocks = p.num_blocks;
  a.splits = L.splits;
  a.streams = L.streams;
  // the partial type follows the shape: bf16 for the shapes the matrix-core
  // kernels serve (whichever kernel runs), fp32 otherwise
  a.part_bf16 = mla::mfma_any_supported(p) ? 1 : 0;
  a.sm_scale_log2 = resolved_scale(p) * 1.4426950408889634f;
  return a;
}

// The split attention into the workspace's partials (a2..a6).
// `groups` > 1: grouped latent, group-major pools (mla_grouped_decode).
mla_status attend_partial(const mla_decode_params& p, const Layout& L, const void* q_lat,
                          const void* c_kv, const float* c_kv_scale, const void* k_rope,
                          const mla::PlanRequest& req, char* ws, hipStream_t s,
                          bool planned = false, hipEvent_t ev_before = nullptr,
                          hipEvent_t ev_after = nullptr, int32_t groups = 1,
                          int32_t shards = 1) {
  mla::AttnArgs a = attn_args(p, L, ws, req.block_table, req.seq_lens);
  a.shards = shards;
  a.q_lat = q_lat;
  a.c_kv = c_kv;
  a.c_kv_scale = c_kv_scale;
  a.k_rope = k_rope;
  a.slots = req.indices ? req.slots : nullptr;
  a.idx_stride = req.indices ? req.idx_stride : 0;
  a.group_heads = groups > 1 ? p.num_heads / groups : 0;
  const int64_t pool_slots = (int64_t)p.num_blocks * p.page_size;
  a.c_group_bytes = groups > 1 ? pool_slots * p.d_latent * mla::dtype_size(p.cache_dtype) : 0;
  a.c_group_scales = groups > 1 ? pool_slots : 0;
  // matrix-core kernels read 16-byte pieces of the pools; other pointers go
  // to the generic kernel (same workspace layout, row-major partials)
  const bool aligned = aligned16(c_kv) && aligned16(k_rope) && aligned16(c_kv_scale);
  // a matrix-core work group serves 64 (or 32) heads, which must share a latent group
  const bool groups_fit = groups <= 1 || (p.num_heads / groups) % mla::mfma_heads_per_group(p.num_heads) == 0;
  const bool use_bf16 = aligned && groups_fit && mla::mfma_supported(p);
  const bool use_fp8 = aligned && groups_fit && mla::mfma_fp8_supported(p);

  hipError_t e = hipSuccess;
  if (!planned) {
    e = mla::launch_plan(mla::plan_input(p, req), s);
    if (e != hipSuccess) return hip_fail(e, "plan launch");
  }
  // matrix-core kernels take the events into their dispatch (start/end of the
  // kernel itself); the generic one is bracketed by event records
  if (use_bf16) {
    e = mla::launch_attend_mfma(a, p.cache_dtype, s, ev_before, ev_after);
  } else if (use_fp8) {
    e = mla::launch_attend_fp8(a, s, ev_before, ev_after);
  } else {
    if (ev_before && (e = hipEventRecord(ev_before, s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    e = mla::launch_attend_simt(a, p.cache_dtype, p.rope_dtype, absorbed_dtype(p), s);
    if (e == hipSuccess && ev_after) e = hipEventRecord(ev_after, s);
  }
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return MLA_OK;
}

// The log-sum-exp merge of the workspace's partials into o_lat (a7).
// shards > 1: TPLA shard heads, merged into the h / shards heads' output.
mla_status combine(const mla_decode_params& p, const Layout& L, char* ws, float* o_lat,
                   hipStream_t s, int32_t shards = 1) {
  mla::AttnArgs a = attn_args(p, L, ws, nullptr, nullptr);
  a.shards = shards;
  const hipError_t e = mla::launch_combine(a, o_lat, s);
  return e == hipSuccess ? MLA_OK : hip_fail(e, "combine launch");
}

// Split attention and merge (a2..a7).
mla_status attend(const mla_decode_params& p, const Layout& L, const void* q_lat, const void* c_kv,
                  const float* c_kv_scale, const void* k_rope, const mla::PlanRequest& req,
                  float* o_lat, char* ws, hipStream_t s, bool planned = false,
                  hipEvent_t ev_before = nullptr, hipEvent_t ev_after = nullptr,
                  int32_t groups = 1, int32_t shards = 1) {
  mla_status st = attend_partial(p, L, q_lat, c_kv, c_kv_scale, k_rope, req, ws, s, planned,
                                 ev_before, ev_after, groups, shards);
  if (st != MLA_OK) return st;
  return combine(p, L, ws, o_lat, s, shards);
}

}  // namespace

namespace {

// ---------------------------------------------------------------- writer
mla_status validate_writer(const mla_cache_write_params* p) {
  if (!p) return fail(MLA_ERR_INVALID_ARG, "params is NULL");
  if (p->batch < 0 || p->d_model < 1 || p->d_latent < 1 || p->d_rope < 0 || p->d_rope % 2)
    return fail(MLA_ERR_INVALID_ARG,
                "shape out of range (batch=%d d_model=%d d_latent=%d d_rope=%d, d_rope even)",
                p->batch, p->d_model, p->d_latent, p->d_rope);
  if (p->page_size < 1 || p->page_size > 4096 || p->max_blocks_per_seq < 1 || p->num_blocks < 1)
    return fail(MLA_ERR_INVALID_ARG, "page_size=%d max_blocks_per_seq=%d num_blocks=%d",
                p->page_size, p->max_blocks_per_seq, p->num_blocks);
  if (!is_dtype(p->x_dtype, false) || !is_dtype(p->weight_dtype, false) ||
      !is_dtype(p->cache_dtype, true) || !is_dtype(p->rope_dtype, false))
    return fail(MLA_ERR_INVALID_ARG, "unknown dtype code (x=%d weight=%d cache=%d rope=%d)",
                p->x_dtype, p->weight_dtype, p->cache_dtype, p->rope_dtype);
  if (!std::isfinite(p->rms_eps) || p->rms_eps < 0.f)
    return fail(MLA_ERR_INVALID_ARG, "rms_eps must be finite and >= 0");
  if (!std::isfinite(p->rope_base) || p->rope_base <= 0.f)
    return fail(MLA_ERR_INVALID_ARG, "rope_base must be finite and > 0");
  if (p->d_latent + p->d_rope > 8192)
    return fail(MLA_ERR_UNSUPPORTED, "d_latent + d_rope above 8192");
  if ((int64_t)p->batch * p->d_model >= ((int64_t)1 << 31))
    return fail(MLA_ERR_UNSUPPORTED, "batch x d_model at or above 2^31");
  return MLA_OK;
}

// The decode step, dense (indices == null) or over index lists.
mla_status decode_impl(const mla_decode_params* p, const void* q, const void* c_kv,
                       const float* c_kv_scale, const void* k_rope, const int32_t* block_table,
                       const int32_t* lens, const int32_t* indices, int32_t stride,
                       const void* W_UK, const void* W_UV, void* out, void* workspace,
                       size_t workspace_bytes, void* stream, void* ev_before, void* ev_after,
                       int32_t groups = 1) {
  g_last_error.clear();
  mla_status st = validate(p);
  if (st != MLA_OK) return st;
  st = check_cache_ptrs(p, c_kv, c_kv_scale, k_rope, block_table, lens);
  if (st != MLA_OK) return st;
  if (!q || !W_UK || !W_UV || !out) return fail(MLA_ERR_INVALID_ARG, "null q, W_UK, W_UV or out");
  if (indices) {
    st = validate_sparse(*p, stride);
    if (st != MLA_OK) return st;
  }
  Layout L;
  st = layout(*p, &L, indices ? stride : 0);
  if (st != MLA_OK) return st;
  st = check_workspace(L, workspace, workspace_bytes);
  if (st != MLA_OK) return st;
  char* ws = static_cast<char*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const mla::PlanRequest plan = plan_request(L, ws, block_table, lens, indices, stride);
  bool planned = false;
  hipError_t e =
      mla::launch_absorb(*p, q, W_UK, ws + L.q_lat, absorbed_dtype(*p), &plan, &planned, s);
  if (e != hipSuccess) return hip_fail(e, "absorb launch");
  st = attend_partial(*p, L, ws + L.q_lat, c_kv, c_kv_scale, k_rope, plan, ws, s, planned,
                      static_cast<hipEvent_t>(ev_before), static_cast<hipEvent_t>(ev_after),
                      groups);
  if (st != MLA_OK) return st;
  if (mla::merge_up_supported(*p) && aligned16(W_UV)) {
    // merge and up-projection in one launch (the same bits as the two stages)
    e = mla::launch_merge_up(*p, attn_args(*p, L, ws, nullptr, nullptr), W_UV, out, s);
    return e == hipSuccess ? MLA_OK : hip_fail(e, "merge + up-projection launch");
  }
  float* o_lat = reinterpret_cast<float*>(ws + L.o_lat);
  st = combine(*p, L, ws, o_lat, s);
  if (st != MLA_OK) return st;
  e = mla::launch_up_project(*p, o_lat, W_UV, out, s);
  return e == hipSuccess ? MLA_OK : hip_fail(e, "up-projection launch");
}

// ---------------------------------------------------------------- no-allocation decode
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};

// Device address of `scratch` on the current device, looked up once per device
// with that device current.
mla_status no_alloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kScratchDevices)
    return fail(MLA_ERR_UNSUPPORTED, "device %d: the scratch table holds devices 0..%d", dev,
                kScratchDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr || (reinterpret_cast<uintptr_t>(ptr) & 255))
      return fail(MLA_ERR_HIP, "scratch array at %p is not 256-byte aligned", ptr);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MLA_OK;
}

// ---------------------------------------------------------------- DSA
mla_status validate_dsa(const mla_dsa_params* d, bool need_topk) {
  if (!d) return fail(MLA_ERR_INVALID_ARG, "dsa params is NULL");
  if (d->index_heads < 1 || d->index_heads > 1024 || d->index_dim < 1 || d->index_dim > 1024)
    return fail(MLA_ERR_INVALID_ARG, "index_heads=%d index_dim=%d outside [1, 1024]",
                d->index_heads, d->index_dim);
  if (need_topk && (d->topk < 1 || d->topk > (1 << 24)))
    return fail(MLA_ERR_INVALID_ARG, "topk %d outside [1, 2^24]", d->topk);
  return MLA_OK;
}

mla_status check_indexer_ptrs(const mla_decode_params& p, const mla_dsa_params& d,
                              const uint8_t* q_I, const float* q_I_scale, const float* w_I,
                              const uint8_t* k_I, const float* k_I_scale) {
  if (!q_I || !q_I_scale || !w_I || !k_I || !k_I_scale)
    return fail(MLA_ERR_INVALID_ARG, "null indexer pointer");
  if (mla::indexer_mfma_ok(d.index_heads, d.index_dim) && !(aligned16(q_I) && aligned16(k_I)))
    return fail(MLA_ERR_INVALID_ARG, "q_I and k_I must be 16-byte aligned");
  (void)p;
  return MLA_OK;
}

int32_t score_cap(const mla_decode_params& p) { return p.max_blocks_per_seq * p.page_size; }

// Batches up to this size take the top-k with its candidate pass spread over
// several work groups per sequence (one work group per sequence above).
constexpr int32_t kTopkSplitMaxBatch = 64;

struct DsaLayout {
  size_t scores, indices, counts, topk, decode, total;
  Layout dec;
};

mla_status dsa_layout(const mla_decode_params& p, const mla_dsa_params& d, DsaLayout* L) {
  const size_t B = p.batch;
  size_t off = 0;
  L->scores = off;
  off = align256(off + B * (size_t)score_cap(p) * sizeof(float));
  L->indices = off;
  off = align256(off + B * (size_t)d.topk * sizeof(int32_t));
  L->counts = off;
  off = align256(off + B * sizeof(int32_t));
  L->topk = off;  // the split top-k's candidate lists
  if (p.batch <= kTopkSplitMaxBatch) off = align256(off + mla::topk_split_ws_bytes(p.batch, score_cap(p)));
  L->decode = off;
  mla_status st = layout(p, &L->dec, d.topk);
  if (st != MLA_OK) return st;
  L->total = off + L->dec.total;
  return MLA_OK;
}

// ---------------------------------------------------------------- TPLA
mla_status validate_tpla(const mla_decode_params& p, const mla_tpla_params* t,
                         mla_decode_params* p2) {
  if (!t) return fail(MLA_ERR_INVALID_ARG, "tpla params is NULL");
  if (t->shards != 1 && t->shards != 2 && t->shards != 4)
    return fail(MLA_ERR_INVALID_ARG, "shards %d not 1, 2 or 4", t->shards);
  if (p.d_latent % t->shards)
    return fail(MLA_ERR_INVALID_ARG, "d_latent %d does not divide into %d shards", p.d_latent,
                t->shards);
  for (int j = 0; j < t->shards; j++)
    if (!std::isfinite(t->mu[j])) return fail(MLA_ERR_INVALID_ARG, "mu[%d] not finite", j);
  if ((int64_t)p.num_heads * t->shards > 65536)
    return fail(MLA_ERR_UNSUPPORTED, "num_heads x shards above 65536");
  *p2 = p;
  p2->num_heads = p.num_heads * t->shards;
  return validate(p2);
}

struct TplaLayout {
  Layout dec;       // the shard heads' decode workspace
  size_t q_lat1;    // absorbed queries of the num_heads heads
  size_t o_lat1;    // gathered latent outputs of the num_heads heads
  size_t total;
};

mla_status tpla_layout(const mla_decode_params& p, const mla_decode_params& p2, TplaLayout* L) {
  mla_status st = layout(p2, &L->dec);
  if (st != MLA_OK) return st;
  size_t off = L->dec.total;
  L->q_lat1 = off;
  off = align256(off + (size_t)p.batch * p.num_heads * (p.d_latent + p.d_rope) *
                           mla::dtype_size(absorbed_dtype(p)));
  L->o_lat1 = off;
  off = align256(off + (size_t)p.batch * p.num_heads * p.d_latent * sizeof(float));
  L->total = off;
  return MLA_OK;
}

size_t writer_ws_bytes(const mla_cache_write_params& p) {
  return align256((size_t)mla::writer_chunks(p) * (size_t)p.batch *
                  (size_t)(p.d_latent + p.d_rope) * sizeof(float));
}

}  // namespace

namespace mla {

void split_plan_host(const int32_t* tiles, int32_t B, int32_t S, int32_t* split_first,
                     int32_t* seq_splits) {
  int32_t tot = 0, mx = 0;
  for (int32_t b = 0; b < B; b++) {
    tot += tiles[b];
    mx = tiles[b] > mx ? tiles[b] : mx;
  }
  const bool aligned = B <= S && B <= kAlignedMaxBatch;
  int32_t L = 1;
  if (aligned && tot > 0) {
    int32_t lo = (tot + S - 1) / S, hi = mx;
    while (lo < hi) {
      const int32_t mid = lo + (hi - lo) / 2;
      int64_t cnt = 0;
      for (int32_t b = 0; b < B; b++) cnt += aligned_splits(tiles[b], mid);
      if (cnt <= S) hi = mid; else lo = mid + 1;
    }
    L = lo;
  }
  int32_t G = 0, C = 0;
  for (int32_t b = 0; b < B; b++) {
    const int32_t n = tiles[b];
    if (aligned) {
      const int32_t k = aligned_splits(n, L);
      for (int32_t i = 0; i < k; i++) split_first[G + i] = C + aligned_first(n, k, i);
      seq_splits[2 * b] = G;
      seq_splits[2 * b + 1] = G + k - 1;
      G += k;
    } else if (n == 0) {
      seq_splits[2 * b] = 0;
      seq_splits[2 * b + 1] = -1;
    } else {
      seq_splits[2 * b] = split_owner(tot, S, C);
      seq_splits[2 * b + 1] = split_owner(tot, S, C + n - 1);
    }
    C += n;
  }
  if (aligned) {
    for (int32_t g = G; g <= S; g++) split_first[g] = tot;
  } else {
    for (int32_t g = 0; g <= S; g++) split_first[g] = (int32_t)split_begin(tot, S, g);
  }
}

}  // namespace mla

extern "C" {

const char* mla_status_string(int32_t st) {
  switch (st) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported combination";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small";
    case MLA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* mla_last_error(void) { return g_last_error.c_str(); }

mla_status mla_decode_workspace_size(const mla_decode_params* p, size_t* bytes) {
  g_last_error.clear();
  mla_status st = validate(p);
  if (st != MLA_OK) return st;
  if (!bytes) return fail(MLA_ERR_INVALID_ARG, "bytes is NULL");
  Layout L;
  st = layout(*p, &L);
  if (st != MLA_OK) return st;
  *bytes = L.total;
  return MLA_OK;
}

mla_status mla_decode_num_splits(const mla_decode_params* p, int32_t* splits) {
  g_last_error.clear();
  mla_status st = validate(p);
  if (st != MLA_OK) return st;
  if (!splits) return fail(MLA_ERR_INVALID_ARG, "splits is NULL");
  return resolve_splits(*p, splits);
}

mla_status mla_absorbed_dtype(const mla_decode_params* p, int32_t* dtype) {
  g_last_error.clear();
  mla_status st = validate(p);
  if (st != MLA_OK) return st;
  if (!dtype) return fail(MLA_ERR_INVALID_ARG, "dtype is NULL");
  *dtype = absorbed_dtype(*p);
  return MLA_OK;
}

mla_status mla_absorb_q(const mla_decode_params* p, const void* q, const void* W_UK, void* q_lat,
                        void* stream) {
  g_last_error.clear();
  mla_status st = validate(p);
  if (st != MLA_OK) return st;
  if (!q || !W_UK || !q_lat) return fail(MLA_ERR_INVALID_ARG, "null q, W_UK or q_lat");
  hipError_t e = mla::launch_absorb(*p, q, W_UK, q_lat, absorbed_dtype(*p), nullptr, nullptr,
                                    static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLA_OK : hip_fail(e, "absorb launch");
}

mla_status mla_attend_latent(const mla_decode_params* p, const void* q_lat, const void* c_kv,
                             const float* c_kv_scale, const void* k_rope,
                             const int32_t* block_table, const int32_t* seq_lens, float* o_lat,
                             void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  mla_status st = validate(p);
  if (st != MLA_OK) return st;
  st = check_cache_ptrs(p, c_kv, c_kv_scale, k_rope, block_table, seq_lens);
  if (st != MLA_OK) return st;
  if (!q_lat || !o_lat) return fail(MLA_ERR_INVALID_ARG, "null q_lat or o_lat");
  Layout L;
  st = layout(*p, &L);
  if (st != MLA_OK) return st;
  st = check_workspace(L, workspace, workspace_bytes);
  if (st != MLA_OK) return st;
  char* ws = static_cast<char*>(workspace);
  return attend(*p, L, q_lat, c_kv, c_kv_scale, k_rope, plan_request(L, ws, block_table, seq_lens),
                o_lat, ws, static_cast<hipStream_t>(stream));
}

mla_status mla_attend_partial(const mla_decode_params* p, const void* q_lat, const void* c_kv,
                              const float* c_kv_scale, const void* k_rope,
                              const int32_t* block_table, const int32_t* seq_lens,
                              void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  mla_status st = validate(p);
  if (st != MLA_OK) return st;
  st = check_cache_ptrs(p, c_kv, c_kv_scale, k_rope, block_table, seq_lens);
  if (st != MLA_OK) return st;
  if (!q_lat) return fail(MLA_ERR_INVALID_ARG, "null q_lat");
  Layout L;
  st = layout(*p, &L);
  if (st != MLA_OK) return st;
  st = check_workspace(L, workspace, workspace_bytes);
  if (st != MLA_OK) return st;
  char* ws = static_cast<char*>(workspace);
  return attend_partial(*p, L, q_lat, c_kv, c_kv_scale, k_rope,
                        plan_request(L, ws, block_table, seq_lens), ws,
                        static_cast<hipStream_t>(stream));
}

mla_status mla_combine(const mla_decode_params* p, float* o_lat, void* workspace,
                       size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  mla_status st = validate(p);
  if (st != MLA_OK) return st;
  if (!o_lat) return fail(MLA_ERR_INVALID_ARG, "null o_lat");
  Layout L;
  st = layout(*p, &L);
  if (st != MLA_OK) return st;
  st = check_workspace(L, workspace, workspace_bytes);
  if (st != MLA_OK) return st;
  return combine(*p, L, static_cast<char*>(workspace), o_lat, static_cast<hipStream_t>(stream));
}

mla_status mla_partials_layout(const mla_decode_params* p, size_t* part_o_offset,
                               size_t* part_lse_offset, int32_t* slots, int32_t* bf16_rows) {
  g_last_error.clear();
  mla_status st = validate(p);
  if (st != MLA_OK) return st;
  if (!part_o_offset || !part_lse_offset || !slots || !bf16_rows)
    return fail(MLA_ERR_INVALID_ARG, "null output pointer");
  Layout L;
  st = layout(*p, &L);
  if (st != MLA_OK) return st;
  *part_o_offset = L.part_o;
  *part_lse_offset = L.part_lse;
  *slots = (int32_t)L.slots;
  *bf16_rows = mla::mfma_any_supported(*p) ? 1 : 0;
  return MLA_OK;
}

mla_status mla_up_project(const mla_decode_params* p, const float* o_lat, const void* W_UV,
                          void* out, void* stream) {
  g_last_error.clear();
  mla_status st = validate(p);
  if (st != MLA_OK) return st;
  if (!o_lat || !W_UV || !out) return fail(MLA_ERR_INVALID_ARG, "null o_lat, W_UV or out");
  hipError_t e = mla::launch_up_project(*p, o_lat, W_UV, out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLA_OK : hip_fail(e, "up-projection launch");
}

mla_status mla_decode_timed(const mla_decode_params* p, const void* q, const void* c_kv,
                            const float* c_kv_scale, const void* k_rope,
                            const int32_t* block_table, const int32_t* seq_lens,
                            const void* W_UK, const void* W_UV, void* out, void* workspace,
                            size_t workspace_bytes, void* stream, void* ev_before,
                            void* ev_after) {
  return decode_impl(p, q, c_kv, c_kv_scale, k_rope, block_table, seq_lens, nullptr, 0, W_UK,
                     W_UV, out, workspace, workspace_bytes, stream, ev_before, ev_after);
}

mla_status mla_decode(const mla_decode_params* p, const void* q, const void* c_kv,
                      const float* c_kv_scale, const void* k_rope, const int32_t* block_table,
                      const int32_t* seq_lens, const void* W_UK, const void* W_UV, void* out,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return mla_decode_timed(p, q, c_kv, c_kv_scale, k_rope, block_table, seq_lens, W_UK, W_UV, out,
                          workspace, workspace_bytes, stream, nullptr, nullptr);
}

mla_status mla_decode_no_alloc(const mla_decode_params* p, const void* q, const void* c_kv,
                               const float* c_kv_scale, const void* k_rope,
                               const int32_t* block_table, const int32_t* seq_lens,
                               const void* W_UK, const void* W_UV, void* out, void* stream) {
  g_last_error.clear();
  mla_status st = validate(p);
  if (st != MLA_OK) return st;
  st = check_cache_ptrs(p, c_kv, c_kv_scale, k_rope, block_table, seq_lens);
  if (st != MLA_OK) return st;
  if (!q || !W_UK || !W_UV || !out) return fail(MLA_ERR_INVALID_ARG, "null q, W_UK, W_UV or out");
  Layout L;
  st = layout(*p, &L);
  if (st != MLA_OK) return st;
  if (L.total > (size_t)MLA_NO_ALLOC_SCRATCH_BYTES)
    return fail(MLA_ERR_WORKSPACE,
                "the step needs %zu bytes of workspace; the fixed scratch holds %zu "
                "(fewer splits or a smaller batch fit)",
                L.total, (size_t)MLA_NO_ALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  st = no_alloc_scratch(&ws);
  if (st != MLA_OK) return st;
  return decode_impl(p, q, c_kv, c_kv_scale, k_rope, block_table, seq_lens, nullptr, 0, W_UK,
                     W_UV, out, ws, (size_t)MLA_NO_ALLOC_SCRATCH_BYTES, stream, nullptr, nullptr);
}

mla_status mla_decode_sparse_workspace_size(const mla_decode_params* p, int32_t index_stride,
                                            size_t* bytes) {
  g_last_error.clear();
  mla_status st = validate(p);
  if (st != MLA_OK) return st;
  st = validate_sparse(*p, index_stride);
  if (st != MLA_OK) return st;
  if (!bytes) return fail(MLA_ERR_INVALID_ARG, "bytes is NULL");
  Layout L;
  st = layout(*p, &L, index_stride);
  if (st != MLA_OK) return st;
  *bytes = L.total;
  return MLA_OK;
}

mla_status mla_decode_sparse(const mla_decode_params* p, const void* q, const void* c_kv,
                             const float* c_kv_scale, const void* k_rope,
                             const int32_t* block_table, const int32_t* indices,
                             int32_t index_stride, const int32_t* counts, const void* W_UK,
                             const void* W_UV, void* out, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (!indices) return fail(MLA_ERR_INVALID_ARG, "indices is NULL");
  return decode_impl(p, q, c_kv, c_kv_scale, k_rope, block_table, counts, indices, index_stride,
                     W_UK, W_UV, out, workspace, workspace_bytes, stream, nullptr, nullptr);
}

mla_status mla_grouped_decode(const mla_decode_params* p, int32_t latent_groups, const void* q,
                              const void* c_kv, const float* c_kv_scale, const void* k_rope,
                              const int32_t* block_table, const int32_t* seq_lens,
                              const void* W_UK, const void* W_UV, void* out, void* workspace,
                              size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (!p) return fail(MLA_ERR_INVALID_ARG, "params is NULL");
  if (latent_groups < 1 || p->num_heads % latent_groups)
    return fail(MLA_ERR_INVALID_ARG, "latent_groups %d must be >= 1 and divide num_heads %d",
                latent_groups, p->num_heads);
  if ((int64_t)latent_groups * p->num_blocks * p->page_size * p->d_latent >= ((int64_t)1 << 40))
    return fail(MLA_ERR_UNSUPPORTED, "grouped pools above 2^40 values");
  return decode_impl(p, q, c_kv, c_kv_scale, k_rope, block_table, seq_lens, nullptr, 0, W_UK,
                     W_UV, out, workspace, workspace_bytes, stream, nullptr, nullptr,
                     latent_groups);
}

mla_status mla_gather_cache(const mla_decode_params* p, const void* c_kv, const float* c_kv_scale,
                            const void* k_rope, const int32_t* block_table,
                            const int32_t* seq_lens, int32_t max_tokens, void* c_out,
                            float* scale_out, void* rope_out, void* stream) {
  g_last_error.clear();
  mla_status st = validate(p);
  if (st != MLA_OK) return st;
  st = check_cache_ptrs(p, c_kv, c_kv_scale, k_rope, block_table, seq_lens);
  if (st != MLA_OK) return st;
  if (max_tokens < 0) return fail(MLA_ERR_INVALID_ARG, "max_tokens < 0");
  if (!c_out || (p->d_rope > 0 && !rope_out) || (p->cache_dtype == MLA_FP8_E4M3 && !scale_out))
    return fail(MLA_ERR_INVALID_ARG, "null output pointer");
  hipError_t e = mla::launch_gather(*p, c_kv, c_kv_scale, k_rope, block_table, seq_lens,
                                    max_tokens, c_out, scale_out, rope_out,
                                    static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLA_OK : hip_fail(e, "gather launch");
}

mla_status mla_cache_write_workspace_size(const mla_cache_write_params* p, size_t* bytes) {
  const mla_status st = validate_writer(p);
  if (st != MLA_OK) return st;
  if (!bytes) return fail(MLA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = writer_ws_bytes(*p);
  return MLA_OK;
}

mla_status mla_cache_write(const mla_cache_write_params* p, const void* x, const void* W_DKV,
                           const void* gamma, const void* W_KR, const int32_t* positions,
                           const int32_t* block_table, void* c_kv, float* c_kv_scale,
                           void* k_rope, void* workspace, size_t workspace_bytes, void* stream) {
  mla_status st = validate_writer(p);
  if (st != MLA_OK) return st;
  if (p->batch == 0) return MLA_OK;
  if (!x || !W_DKV || !gamma || !positions || !block_table || !c_kv ||
      (p->d_rope > 0 && (!W_KR || !k_rope)))
    return fail(MLA_ERR_INVALID_ARG, "a required pointer is NULL");
  if ((p->cache_dtype == MLA_FP8_E4M3) != (c_kv_scale != nullptr))
    return fail(MLA_ERR_INVALID_ARG, "c_kv_scale must be given exactly for an fp8 cache");
  const size_t need = writer_ws_bytes(*p);
  if (!workspace || workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "workspace of %zu bytes needed", need);
  if (reinterpret_cast<uintptr_t>(workspace) & 255)
    return fail(MLA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (mla::writer_mfma_ok(*p) && !(aligned16(x) && aligned16(W_DKV) && aligned16(W_KR)))
    return fail(MLA_ERR_INVALID_ARG, "bf16 x, W_DKV and W_KR must be 16-byte aligned");
  const hipError_t e = mla::launch_cache_write(*p, x, W_DKV, gamma, W_KR, positions, block_table,
                                               c_kv, c_kv_scale, k_rope,
                                               static_cast<float*>(workspace),
                                               static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "cache writer launch");
  return MLA_OK;
}

mla_status mla_quantize_e4m3_rows(const float* x, int64_t rows, int32_t d, uint8_t* codes,
                                  float* scales, void* stream) {
  if (rows < 0 || rows >= ((int64_t)1 << 31) || d < 1 || d > 8192)
    return fail(MLA_ERR_INVALID_ARG, "rows=%lld d=%d (1 <= d <= 8192)", (long long)rows, d);
  if (rows == 0) return MLA_OK;
  if (!x || !codes || !scales) return fail(MLA_ERR_INVALID_ARG, "a required pointer is NULL");
  const hipError_t e =
      mla::launch_quantize_rows(x, rows, d, codes, scales, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "quantiser launch");
  return MLA_OK;
}

mla_status mla_indexer_scores(const mla_decode_params* p, const mla_dsa_params* d,
                              const uint8_t* q_I, const float* q_I_scale, const float* w_I,
                              const uint8_t* k_I, const float* k_I_scale,
                              const int32_t* block_table, const int32_t* seq_lens, float* scores,
                              int32_t score_stride, void* stream) {
  g_last_error.clear();
  mla_status st = validate(p);
  if (st != MLA_OK) return st;
  st = validate_dsa(d, false);
  if (st != MLA_OK) return st;
  st = check_indexer_ptrs(*p, *d, q_I, q_I_scale, w_I, k_I, k_I_scale);
  if (st != MLA_OK) return st;
  if (!block_table || !seq_lens || !scores)
    return fail(MLA_ERR_INVALID_ARG, "null table, length or score pointer");
  if (score_stride < 1) return fail(MLA_ERR_INVALID_ARG, "score_stride %d < 1", score_stride);
  const hipError_t e = mla::launch_indexer(
      q_I, q_I_scale, w_I, k_I, k_I_scale, block_table, seq_lens, scores, p->batch,
      d->index_heads, d->index_dim, p->page_size, p->max_blocks_per_seq, p->num_blocks,
      score_stride, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLA_OK : hip_fail(e, "indexer launch");
}

static mla_status check_topk_args(const float* scores, int32_t score_stride,
                                  const int32_t* seq_lens, int32_t batch, int32_t k,
                                  int32_t* indices, int32_t index_stride, int32_t* counts) {
  if (batch < 0 || batch > (1 << 24) || k < 1 || k > (1 << 24) || score_stride < 1 ||
      index_stride < k)
    return fail(MLA_ERR_INVALID_ARG,
                "batch=%d k=%d score_stride=%d index_stride=%d (need k >= 1, index_stride >= k)",
                batch, k, score_stride, index_stride);
  if (batch > 0 && (!scores || !seq_lens || !indices || !counts))
    return fail(MLA_ERR_INVALID_ARG, "a required pointer is NULL");
  return MLA_OK;
}

mla_status mla_topk_select(const float* scores, int32_t score_stride, const int32_t* seq_lens,
                           int32_t batch, int32_t k, int32_t* indices, int32_t index_stride,
                           int32_t* counts, void* stream) {
  g_last_error.clear();
  mla_status st = check_topk_args(scores, score_stride, seq_lens, batch, k, indices, index_stride,
                                  counts);
  if (st != MLA_OK) return st;
  if (batch == 0) return MLA_OK;
  const hipError_t e = mla::launch_topk(scores, score_stride, seq_lens, batch, k, indices,
                                        index_stride, counts, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLA_OK : hip_fail(e, "top-k launch");
}

mla_status mla_topk_select_split_workspace_size(int32_t batch, int32_t score_stride, size_t* bytes) {
  g_last_error.clear();
  if (batch < 0 || batch > 65535 || score_stride < 1)
    return fail(MLA_ERR_INVALID_ARG, "batch=%d (0..65535) score_stride=%d (>= 1)", batch,
                score_stride);
  if (!bytes) return fail(MLA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = mla::topk_split_ws_bytes(batch, score_stride);
  return MLA_OK;
}

mla_status mla_topk_select_split(const float* scores, int32_t score_stride,
                                 const int32_t* seq_lens, int32_t batch, int32_t k,
                                 int32_t* indices, int32_t index_stride, int32_t* counts,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  mla_status st = check_topk_args(scores, score_stride, seq_lens, batch, k, indices, index_stride,
                                  counts);
  if (st != MLA_OK) return st;
  if (batch > 65535) return fail(MLA_ERR_INVALID_ARG, "batch %d above 65535", batch);
  if (batch == 0) return MLA_OK;
  const size_t need = mla::topk_split_ws_bytes(batch, score_stride);
  if (!workspace || workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes, %zu required", workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) & 255)
    return fail(MLA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const hipError_t e = mla::launch_topk_split(scores, score_stride, seq_lens, batch, k, indices,
                                              index_stride, counts, workspace,
                                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLA_OK : hip_fail(e, "top-k launch");
}

mla_status mla_dsa_decode_workspace_size(const mla_decode_params* p, const mla_dsa_params* d,
                                         size_t* bytes) {
  g_last_error.clear();
  mla_status st = validate(p);
  if (st != MLA_OK) return st;
  st = validate_dsa(d, true);
  if (st != MLA_OK) return st;
  st = validate_sparse(*p, d->topk);
  if (st != MLA_OK) return st;
  if (!bytes) return fail(MLA_ERR_INVALID_ARG, "bytes is NULL");
  DsaLayout L;
  st = dsa_layout(*p, *d, &L);
  if (st != MLA_OK) return st;
  *bytes = L.total;
  return MLA_OK;
}

mla_status mla_dsa_decode(const mla_decode_params* p, const mla_dsa_params* d, const void* q,
                          const void* c_kv, const float* c_kv_scale, const void* k_rope,
                          const int32_t* block_table, const int32_t* seq_lens,
                          const uint8_t* q_I, const float* q_I_scale, const float* w_I,
                          const uint8_t* k_I, const float* k_I_scale, const void* W_UK,
                          const void* W_UV, void* out, int32_t* indices_out, void* workspace,
                          size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  mla_status st = validate(p);
  if (st != MLA_OK) return st;
  st = validate_dsa(d, true);
  if (st != MLA_OK) return st;
  st = validate_sparse(*p, d->topk);
  if (st != MLA_OK) return st;
  st = check_cache_ptrs(p, c_kv, c_kv_scale, k_rope, block_table, seq_lens);
  if (st != MLA_OK) return st;
  st = check_indexer_ptrs(*p, *d, q_I, q_I_scale, w_I, k_I, k_I_scale);
  if (st != MLA_OK) return st;
  DsaLayout L;
  st = dsa_layout(*p, *d, &L);
  if (st != MLA_OK) return st;
  if (!workspace || workspace_bytes < L.total)
    return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes, %zu required", workspace_bytes, L.total);
  if (reinterpret_cast<uintptr_t>(workspace) & 255)
    return fail(MLA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  char* ws = static_cast<char*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* scores = reinterpret_cast<float*>(ws + L.scores);
  int32_t* idx = indices_out ? indices_out : reinterpret_cast<int32_t*>(ws + L.indices);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
  const int32_t cap = score_cap(*p);
  hipError_t e = mla::launch_indexer(q_I, q_I_scale, w_I, k_I, k_I_scale, block_table, seq_lens,
                                     scores, p->batch, d->index_heads, d->index_dim,
                                     p->page_size, p->max_blocks_per_seq, p->num_blocks, cap, s);
  if (e != hipSuccess) return hip_fail(e, "indexer launch");
  e = p->batch <= kTopkSplitMaxBatch
          ? mla::launch_topk_split(scores, cap, seq_lens, p->batch, d->topk, idx, d->topk, counts,
                                   ws + L.topk, s)
          : mla::launch_topk(scores, cap, seq_lens, p->batch, d->topk, idx, d->topk, counts, s);
  if (e != hipSuccess) return hip_fail(e, "top-k launch");
  return decode_impl(p, q, c_kv, c_kv_scale, k_rope, block_table, counts, idx, d->topk, W_UK,
                     W_UV, out, ws + L.decode, workspace_bytes - L.decode, stream, nullptr,
                     nullptr);
}

mla_status mla_tpla_decode_workspace_size(const mla_decode_params* p, const mla_tpla_params* t,
                                          size_t* bytes) {
  g_last_error.clear();
  mla_status st = validate(p);
  if (st != MLA_OK) return st;
  mla_decode_params p2;
  st = validate_tpla(*p, t, &p2);
  if (st != MLA_OK) return st;
  if (!bytes) return fail(MLA_ERR_INVALID_ARG, "bytes is NULL");
  TplaLayout L;
  st = tpla_layout(*p, p2, &L);
  if (st != MLA_OK) return st;
  *bytes = L.total;
  return MLA_OK;
}

mla_status mla_tpla_decode(const mla_decode_params* p, const mla_tpla_params* t, const void* q,
                           const void* c_kv, const float* c_kv_scale, const void* k_rope,
                           const int32_t* block_table, const int32_t* seq_lens, const void* W_UK,
                           const void* W_UV, void* out, void* workspace, size_t workspace_bytes,
                           void* stream) {
  g_last_error.clear();
  mla_status st = validate(p);
  if (st != MLA_OK) return st;
  mla_decode_params p2;
  st = validate_tpla(*p, t, &p2);
  if (st != MLA_OK) return st;
  st = check_cache_ptrs(p, c_kv, c_kv_scale, k_rope, block_table, seq_lens);
  if (st != MLA_OK) return st;
  if (!q || !W_UK || !W_UV || !out) return fail(MLA_ERR_INVALID_ARG, "null q, W_UK, W_UV or out");
  TplaLayout L;
  st = tpla_layout(*p, p2, &L);
  if (st != MLA_OK) return st;
  st = check_workspace(L.dec, workspace, workspace_bytes);  // alignment
  if (st != MLA_OK) return st;
  if (workspace_bytes < L.total)
    return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes, %zu required", workspace_bytes, L.total);
  char* ws = static_cast<char*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t qt = absorbed_dtype(*p);
  // absorption of the num_heads heads (its planner groups plan the split)
  const mla::PlanRequest plan = plan_request(L.dec, ws, block_table, seq_lens);
  bool planned = false;
  hipError_t e;
  if (mla::absorb_mfma_ok(*p, q, W_UK, ws + L.dec.q_lat)) {
    // the matrix-core absorption writes the shard heads' queries itself
    mla::ShardExpand ex{t->shards, {1.f, 1.f, 1.f, 1.f}};
    for (int j = 0; j < t->shards; j++) ex.mu[j] = t->mu[j];
    e = mla::launch_absorb_mfma(*p, q, W_UK, ws + L.dec.q_lat, qt, &plan, s, &ex);
    if (e != hipSuccess) return hip_fail(e, "absorb launch");
    planned = true;
  } else {
    e = mla::launch_absorb(*p, q, W_UK, ws + L.q_lat1, qt, &plan, &planned, s);
    if (e != hipSuccess) return hip_fail(e, "absorb launch");
    mla::TplaMu mu{};
    for (int j = 0; j < t->shards; j++) mu.v[j] = t->mu[j];
    e = mla::launch_tpla_expand(ws + L.q_lat1, ws + L.dec.q_lat, qt, p->batch, p->num_heads,
                                t->shards, p->d_latent, p->d_rope, mu, s);
    if (e != hipSuccess) return hip_fail(e, "expand launch");
  }
  float* o2 = reinterpret_cast<float*>(ws + L.dec.o_lat);
  float* o1 = reinterpret_cast<float*>(ws + L.o_lat1);
  // With bf16 partials and whole 32-head blocks the merge takes
  // each head's own shard columns straight into o1 (and the 64-head attention
  // reads only its shard); otherwise every shard head is merged whole and the
  // gather picks the columns.
  const bool by_shard = t->shards > 1 && mla::mfma_any_supported(p2) && p->num_heads % 32 == 0;
  st = attend(p2, L.dec, ws + L.dec.q_lat, c_kv, c_kv_scale, k_rope, plan, by_shard ? o1 : o2, ws,
              s, planned, nullptr, nullptr, 1, by_shard ? t->shards : 1);
  if (st != MLA_OK) return st;
  if (!by_shard) {
    e = mla::launch_tpla_gather(o2, o1, p->batch, p->num_heads, t->shards, p->d_latent, s);
    if (e != hipSuccess) return hip_fail(e, "gather launch");
  }
  e = mla::launch_up_project(*p, o1, W_UV, out, s);
  return e == hipSuccess ? MLA_OK : hip_fail(e, "up-projection launch");
}

// The workspace size asked for by default: every (sequence, head) unit's keys
// and values when they fit in MLA_PREFILL_DEFAULT_WORKSPACE_BYTES, else as many
// units as fit there (at least one); the call then runs in chunks of units.
static size_t prefill_ws_bytes(const mla_decode_params& p) {
  const size_t unit = mla::prefill_unit_bytes(p);
  const size_t units = (size_t)p.batch * p.num_heads;
  const size_t fit = std::max<size_t>(1, MLA_PREFILL_DEFAULT_WORKSPACE_BYTES / unit);
  return unit * std::max<size_t>(1, std::min(units, fit));
}

mla_status mla_prefill_workspace_size(const mla_decode_params* p, size_t* bytes) {
  g_last_error.clear();
  mla_status st = validate(p);
  if (st != MLA_OK) return st;
  if (!mla::prefill_supported(*p))
    return fail(MLA_ERR_UNSUPPORTED, "prefill needs bf16 (cache bf16 or fp8) and d_latent 512, d_nope 128, d_rope 64, d_v 128");
  if (!bytes) return fail(MLA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = prefill_ws_bytes(*p);
  return MLA_OK;
}

mla_status mla_prefill(const mla_decode_params* p, int32_t max_q_len, const void* q,
                       const int32_t* q_lens, const void* c_kv, const float* c_kv_scale,
                       const void* k_rope,
                       const int32_t* block_table, const int32_t* seq_lens, const void* W_UK,
                       const void* W_UV, void* out, void* workspace, size_t workspace_bytes,
                       void* stream) {
  g_last_error.clear();
  mla_status st = validate(p);
  if (st != MLA_OK) return st;
  if (!mla::prefill_supported(*p))
    return fail(MLA_ERR_UNSUPPORTED, "prefill needs bf16 (cache bf16 or fp8) and d_latent 512, d_nope 128, d_rope 64, d_v 128");
  if (max_q_len < 1 || max_q_len > (1 << 24))
    return fail(MLA_ERR_INVALID_ARG, "max_q_len %d outside [1, 2^24]", max_q_len);
  if ((int64_t)p->batch * max_q_len * p->num_heads * 192 >= ((int64_t)1 << 40))
    return fail(MLA_ERR_UNSUPPORTED, "query tensor too large");
  if ((int64_t)p->batch * p->num_heads * ((max_q_len + 127) / 128) >= ((int64_t)1 << 31))
    return fail(MLA_ERR_UNSUPPORTED, "prefill grid too large (batch %d, heads %d, max_q_len %d)",
                p->batch, p->num_heads, max_q_len);
  if (!q || !q_lens || !c_kv || !k_rope || !block_table || !seq_lens || !W_UK || !W_UV || !out)
    return fail(MLA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!(aligned16(q) && aligned16(c_kv) && aligned16(k_rope) && aligned16(W_UK) && aligned16(W_UV)))
    return fail(MLA_ERR_INVALID_ARG, "q, c_kv, k_rope, W_UK and W_UV must be 16-byte aligned");
  if ((p->cache_dtype == MLA_FP8_E4M3) != (c_kv_scale != nullptr))
    return fail(MLA_ERR_INVALID_ARG, "c_kv_scale is required for an fp8 cache and only then");
  if (reinterpret_cast<uintptr_t>(c_kv_scale) & 3)
    return fail(MLA_ERR_INVALID_ARG, "c_kv_scale must be 4-byte aligned");
  const size_t need = mla::prefill_unit_bytes(*p);
  if (!workspace || workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "workspace of at least %zu bytes (one sequence and head) needed",
                need);
  if (reinterpret_cast<uintptr_t>(workspace) & 255)
    return fail(MLA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const hipError_t e = mla::launch_prefill(*p, max_q_len, q, q_lens, c_kv, c_kv_scale, k_rope,
                                           block_table, seq_lens, W_UK, W_UV, out, workspace,
                                           workspace_bytes, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLA_OK : hip_fail(e, "prefill launch");
}

int64_t mla_split_begin(int64_t n_tiles, int32_t splits, int32_t g) {
  if (splits < 1) return 0;
  return mla::split_begin(n_tiles, splits, g);
}

int32_t mla_split_owner(int64_t n_tiles, int32_t splits, int64_t tile) {
  if (n_tiles < 1 || splits < 1) return -1;
  return mla::split_owner(n_tiles, splits, tile);
}

mla_status mla_split_plan(const int32_t* tiles, int32_t batch, int32_t splits,
                          int32_t* split_first, int32_t* seq_splits) {
  g_last_error.clear();
  if (batch < 1 || splits < 1 || !tiles || !split_first || !seq_splits)
    return fail(MLA_ERR_INVALID_ARG, "batch=%d splits=%d and three non-null arrays required",
                batch, splits);
  int64_t tot = 0;
  for (int32_t b = 0; b < batch; b++) {
    if (tiles[b] < 0) return fail(MLA_ERR_INVALID_ARG, "tiles[%d] < 0", b);
    tot += tiles[b];
  }
  if (tot >= ((int64_t)1 << 31)) return fail(MLA_ERR_UNSUPPORTED, "2^31 tiles or more");
  mla::split_plan_host(tiles, batch, splits, split_first, seq_splits);
  return MLA_OK;
}

}  // extern "C"
