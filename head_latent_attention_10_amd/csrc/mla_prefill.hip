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
//  * decompress: K[b, i, t, :] = W_UK[i] c_t and V^T[b, i, :, t] = W_UV[i] c_t
//    for every cached t < T_b, a bf16 matrix-core GEMM per (128 tokens, head,
//    K or V) tile with both operands staged in LDS;
//  * attention: a work group per (64 queries, head, sequence), a wave per 16
//    queries; per 64-key tile S^T = K Q^T (16x16x32 MFMA, keys on M), the
//    causal mask, an online softmax per query, and O^T += V^T P^T (the key
//    order of this product is the one the score fragments already hold).
#include "mla_mfma_util.hpp"

namespace mla {
namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kPDc = 512, kPDn = 128, kPDr = 64, kPDv = 128;
constexpr int kPDq = kPDn + kPDr;          // 192 query/key width
constexpr int kDecTok = 128;               // tokens per decompression tile
constexpr int kDecChunk = 64;              // latent values per LDS stage
constexpr int kDecRow = kDecChunk * 2 + 16;  // LDS bytes per staged row
constexpr int kQTile = 64;                 // queries per attention work group
constexpr int kKTile = 64;                 // keys per attention step
constexpr int kKRow = kPDq * 2 + 16;       // LDS bytes per key row (400)
constexpr int kVRow = kKTile * 2 + 16;     // LDS bytes per V^T row (144)

struct PrefillArgs {
  const uint16_t* q;        // [B, Lq, h, 192]
  const int32_t* q_lens;    // [B]
  const uint16_t* c_kv;     // [nb, P, 512]
  const uint16_t* k_rope;   // [nb, P, 64]
  const int32_t* block_table;
  const int32_t* seq_lens;
  const uint16_t* W_UK;     // [h, 128, 512]
  const uint16_t* W_UV;     // [h, 128, 512]
  uint16_t* Kn;             // [B, h, Tpad, 128]
  uint16_t* Vt;             // [B, h, 128, Tpad]
  void* out;                // [B, Lq, h, 128]
  int32_t B, h, Lq, P, max_blocks, num_blocks, Tpad;
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

// ------------------------------------------------------------------ decompress
// blockIdx = (token tile, 2 i + which, b); wave (wm, wn) computes tokens
// 64 wm .. +63 by outputs 64 wn .. +63 of the 128 x 128 tile.
__global__ __launch_bounds__(256) void prefill_decompress_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char s_a[kDecTok * kDecRow];
  __shared__ __attribute__((aligned(16))) char s_b[kPDn * kDecRow];
  const int32_t b = blockIdx.z, head = blockIdx.y >> 1, which = blockIdx.y & 1;
  const int32_t T = cached_len(a, b);
  const int32_t t0 = blockIdx.x * kDecTok;
  if (t0 >= T) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, g = lane >> 5, r = lane & 31;
  const uint16_t* W = (which ? a.W_UV : a.W_UK) + (int64_t)head * kPDn * kPDc;
  // this thread's staged pieces: rows idx / 8, 16-byte piece idx % 8
  int64_t arow[4];
#pragma unroll
  for (int u = 0; u < 4; u++) {
    const int32_t idx = tid + 256 * u, row = idx >> 3;
    const int32_t t = min(t0 + row, T - 1);  // rows past T repeat the last token (finite)
    arow[u] = phys_slot(a.block_table, b, t, a.P, a.max_blocks, a.num_blocks) * kPDc;
  }
  f32x16 acc[2][2] = {};
  for (int32_t k0 = 0; k0 < kPDc; k0 += kDecChunk) {
    uint4 va[4], vb[4];
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int32_t idx = tid + 256 * u, row = idx >> 3, pc = idx & 7;
      va[u] = *reinterpret_cast<const uint4*>(a.c_kv + arow[u] + k0 + 8 * pc);
      vb[u] = *reinterpret_cast<const uint4*>(W + (int64_t)row * kPDc + k0 + 8 * pc);
    }
    __syncthreads();  // the previous chunk's products are done
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int32_t idx = tid + 256 * u, row = idx >> 3, pc = idx & 7;
      *reinterpret_cast<uint4*>(s_a + row * kDecRow + 16 * pc) = va[u];
      *reinterpret_cast<uint4*>(s_b + row * kDecRow + 16 * pc) = vb[u];
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kDecChunk / 16; s++) {
      bf16x8 av[2], bv[2];
#pragma unroll
      for (int x = 0; x < 2; x++) {
        av[x] = *reinterpret_cast<const bf16x8*>(s_a + (64 * wm + 32 * x + r) * kDecRow + 32 * s + 16 * g);
        bv[x] = *reinterpret_cast<const bf16x8*>(s_b + (64 * wn + 32 * x + r) * kDecRow + 32 * s + 16 * g);
      }
#pragma unroll
      for (int x = 0; x < 2; x++)
#pragma unroll
        for (int y = 0; y < 2; y++)
          acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[x], bv[y], acc[x][y], 0, 0, 0);
    }
  }
  // D[token][output]: lane holds output column r, tokens 8 (j / 4) + 4 g + j % 4
  const int64_t bh = (int64_t)b * a.h + head;
#pragma unroll
  for (int x = 0; x < 2; x++) {
#pragma unroll
    for (int y = 0; y < 2; y++) {
      const int32_t col = 64 * wn + 32 * y + r;
#pragma unroll
      for (int jb = 0; jb < 4; jb++) {
        const int32_t tok = t0 + 64 * wm + 32 * x + 8 * jb + 4 * g;  // 4 consecutive tokens
        if (which == 0) {
#pragma unroll
          for (int e = 0; e < 4; e++)
            a.Kn[(bh * a.Tpad + tok + e) * kPDn + col] = f32_to_bf16_bits(acc[x][y][4 * jb + e]);
        } else {
          const uint32_t lo = f32_to_bf16_bits(acc[x][y][4 * jb + 0]) |
                              ((uint32_t)f32_to_bf16_bits(acc[x][y][4 * jb + 1]) << 16);
          const uint32_t hi = f32_to_bf16_bits(acc[x][y][4 * jb + 2]) |
                              ((uint32_t)f32_to_bf16_bits(acc[x][y][4 * jb + 3]) << 16);
          *reinterpret_cast<uint2*>(a.Vt + (bh * kPDv + col) * a.Tpad + tok) = uint2{lo, hi};
        }
      }
    }
  }
}

// ------------------------------------------------------------------ attention
template <int OT>
__global__ __launch_bounds__(256) void prefill_attn_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char s_k[kKTile * kKRow];
  __shared__ __attribute__((aligned(16))) char s_v[kPDv * kVRow];
  const int32_t b = blockIdx.z, head = blockIdx.y, q0 = blockIdx.x * kQTile;
  const int32_t T = cached_len(a, b);
  const int32_t Lb = query_len(a, b, T);
  if (q0 >= Lb) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int64_t bh = (int64_t)b * a.h + head;
  // this lane's query (column c of the wave's 16) and its position
  const int32_t ql = q0 + 16 * wave + c;
  const bool q_live = ql < Lb;
  const int32_t qpos = T - Lb + min(ql, Lb - 1);
  bf16x8 qv[kPDq / 32];
  {
    const uint16_t* qrow = a.q + (((int64_t)b * a.Lq + min(ql, Lb - 1)) * a.h + head) * kPDq + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kPDq / 32; ks++) qv[ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks);
  }
  const int32_t last_q = min(q0 + kQTile, Lb) - 1;
  const int32_t t_end = T - Lb + last_q + 1;  // keys this work group needs
  f32x4v o[kPDv / 16] = {};
  float m = -INFINITY, l_part = 0.f;
  for (int32_t t0 = 0; t0 < t_end; t0 += kKTile) {
    __syncthreads();  // previous tile consumed
    // K tile: 64 keys x (128 reconstructed + 64 rope); V^T tile: 128 x 64 keys
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int32_t idx = tid + 256 * u, key = idx >> 4, pc = idx & 15;
      const uint4 v = *reinterpret_cast<const uint4*>(a.Kn + (bh * a.Tpad + t0 + key) * kPDn + 8 * pc);
      *reinterpret_cast<uint4*>(s_k + key * kKRow + 16 * pc) = v;
    }
#pragma unroll
    for (int u = 0; u < 2; u++) {
      const int32_t idx = tid + 256 * u, key = idx >> 3, pc = idx & 7;
      const int32_t t = min(t0 + key, T - 1);
      const int64_t slot = phys_slot(a.block_table, b, t, a.P, a.max_blocks, a.num_blocks);
      const uint4 v = *reinterpret_cast<const uint4*>(a.k_rope + slot * kPDr + 8 * pc);
      *reinterpret_cast<uint4*>(s_k + key * kKRow + 2 * kPDn + 16 * pc) = v;
    }
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int32_t idx = tid + 256 * u, row = idx >> 3, pc = idx & 7;
      const uint4 v = *reinterpret_cast<const uint4*>(a.Vt + (bh * kPDv + row) * a.Tpad + t0 + 8 * pc);
      *reinterpret_cast<uint4*>(s_v + row * kVRow + 16 * pc) = v;
    }
    __syncthreads();
    // S^T[key][query]: lane holds query c, keys 16 kb + 4 g + j
    f32x4v s[4];
#pragma unroll
    for (int kb = 0; kb < 4; kb++) {
      s[kb] = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kPDq / 32; ks++) {
        const bf16x8 kv = *reinterpret_cast<const bf16x8*>(s_k + (16 * kb + c) * kKRow + 64 * ks + 16 * g);
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qv[ks], s[kb], 0, 0, 0);
      }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; kb++)
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int32_t t = t0 + 16 * kb + 4 * g + j;
        s[kb][j] = t <= qpos ? s[kb][j] * a.sm_log2 : -INFINITY;
        tmax = fmaxf(tmax, s[kb][j]);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m, tmax);
    const float alpha = m == -INFINITY ? 0.f : exp2f(m - m_new);
    m = m_new;
    // weights in bf16 (the product's operand); the normaliser adds the same values
    bf16x8 pb[2];
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; kb++)
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const float p = m_new == -INFINITY ? 0.f : exp2f(s[kb][j] - m_new);
        const uint16_t pbits = f32_to_bf16_bits(p);
        psum += bf16_bits_to_f32(pbits);
        pb[kb >> 1][4 * (kb & 1) + j] = __builtin_bit_cast(__bf16, pbits);
      }
    l_part = l_part * alpha + psum;
    // O^T[d][query] += V^T[d][keys] P^T[keys][query], keys in the fragments' order:
    // lane group g takes keys 16 (2 k2) + 4 g + (0..3) and 16 (2 k2 + 1) + 4 g + (0..3)
#pragma unroll
    for (int mb = 0; mb < kPDv / 16; mb++) {
      o[mb] *= alpha;
#pragma unroll
      for (int k2 = 0; k2 < 2; k2++) {
        const char* vrow = s_v + (16 * mb + c) * kVRow;
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow + 2 * (32 * k2 + 4 * g));
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 2 * (32 * k2 + 16 + 4 * g));
        const bf16x8 vv = __builtin_bit_cast(bf16x8, uint4{lo.x, lo.y, hi.x, hi.y});
        o[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, pb[k2], o[mb], 0, 0, 0);
      }
    }
  }
  float l_tot = l_part + __shfl_xor(l_part, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (!q_live) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int64_t orow = (((int64_t)b * a.Lq + ql) * a.h + head) * kPDv;
  // lane holds query c, value rows 16 mb + 4 g + j
#pragma unroll
  for (int mb = 0; mb < kPDv / 16; mb++)
#pragma unroll
    for (int j = 0; j < 4; j++) store_elem<OT>(a.out, orow + 16 * mb + 4 * g + j, o[mb][j] * inv);
}

}  // namespace

bool prefill_supported(const mla_decode_params& p) {
  return p.q_dtype == MLA_BF16 && p.cache_dtype == MLA_BF16 && p.rope_dtype == MLA_BF16 &&
         p.weight_dtype == MLA_BF16 && p.d_latent == kPDc && p.d_nope == kPDn &&
         p.d_rope == kPDr && p.d_v == kPDv;
}

int32_t prefill_tpad(const mla_decode_params& p) {
  const int64_t cap = (int64_t)p.max_blocks_per_seq * p.page_size;
  return (int32_t)((cap + kDecTok - 1) / kDecTok * kDecTok);
}

hipError_t launch_prefill(const mla_decode_params& p, int32_t max_q_len, const void* q,
                          const int32_t* q_lens, const void* c_kv, const void* k_rope,
                          const int32_t* block_table, const int32_t* seq_lens, const void* W_UK,
                          const void* W_UV, void* out, void* Kn, void* Vt, hipStream_t s) {
  PrefillArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.q_lens = q_lens;
  a.c_kv = static_cast<const uint16_t*>(c_kv);
  a.k_rope = static_cast<const uint16_t*>(k_rope);
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.W_UK = static_cast<const uint16_t*>(W_UK);
  a.W_UV = static_cast<const uint16_t*>(W_UV);
  a.Kn = static_cast<uint16_t*>(Kn);
  a.Vt = static_cast<uint16_t*>(Vt);
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
  hipLaunchKernelGGL(prefill_decompress_kernel, dim3(a.Tpad / kDecTok, 2 * p.num_heads, p.batch),
                     dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((max_q_len + kQTile - 1) / kQTile, p.num_heads, p.batch);
  if (p.out_dtype == MLA_BF16)
    hipLaunchKernelGGL(prefill_attn_kernel<MLA_BF16>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(prefill_attn_kernel<MLA_F32>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
