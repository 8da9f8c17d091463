// Matrix-core query absorption and value up-projection (bf16 weights, gfx950).
//
// Both are per-head products with a short sequence dimension:
//   absorb:  q_lat[b, i, c] = sum_n q[b, i, n] W_UK[i, n, c]   (K = d_nope)
//   up-proj: out[b, i, v]   = sum_c o_lat[b, i, c] W_UV[i, v, c] (K = d_latent)
// computed with MFMA 32x32x16 bf16 (fp32 accumulation), sequences on M
// (padded to 32 with zero rows).
#include "mla_kernels.hpp"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) char lds_t;

constexpr int kLat = 512;             // latent width of the fast path
constexpr int kUpKs = kLat / 16;      // k-steps of the up-projection

// ------------------------------------------------------------------ up-projection
// Work group = one wave = (head, 32 rows of W_UV).  The wave keeps its 32 W_UV
// rows (32 KiB) in registers as the MFMA B operand and sweeps the sequences in
// blocks of 32.  o_lat is fp32; it is split into a bf16 high part and a bf16
// remainder, multiplied separately and summed in fp32, which keeps about 16
// significant bits of o_lat in the product.
template <int OT>
__global__ __launch_bounds__(64) void up_project_mfma_kernel(const float* __restrict__ o_lat,
                                                             const uint16_t* __restrict__ W_UV,
                                                             void* __restrict__ out, int32_t B,
                                                             int32_t h, int32_t d_v) {
  const int32_t head = blockIdx.x;
  const int32_t v0 = blockIdx.y * 32;
  const int lane = threadIdx.x, g = lane >> 5, r = lane & 31;
  bf16x8 wf[kUpKs];
  const uint16_t* wrow = W_UV + ((int64_t)head * d_v + v0 + r) * kLat + 8 * g;
#pragma unroll
  for (int ks = 0; ks < kUpKs; ks++) wf[ks] = *reinterpret_cast<const bf16x8*>(wrow + 16 * ks);
  for (int32_t b0 = 0; b0 < B; b0 += 32) {
    const int32_t b = b0 + r;
    const bool live = b < B;
    const float* orow = o_lat + ((int64_t)(live ? b : 0) * h + head) * kLat + 8 * g;
    f32x16 acc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < kUpKs; ks++) {
      f32x8 x = *reinterpret_cast<const f32x8*>(orow + 16 * ks);
      if (!live) x = f32x8{};
      const bf16x8 hi = __builtin_convertvector(x, bf16x8);
      const bf16x8 lo = __builtin_convertvector(x - __builtin_convertvector(hi, f32x8), bf16x8);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hi, wf[ks], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lo, wf[ks], acc, 0, 0, 0);
    }
    // D[m = sequence][n = row]: lane holds row v0 + r, sequences 8(j/4) + 4g + j%4
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const int32_t bb = b0 + 8 * (j >> 2) + 4 * g + (j & 3);
      if (bb < B) store_elem<OT>(out, ((int64_t)bb * h + head) * d_v + v0 + r, acc[j]);
    }
  }
}

// ------------------------------------------------------------------ absorb
// Work group = (head, 128 latent columns), four waves of 32 columns each.  The
// W_UK rows of the group (d_nope x 128 bf16) are staged in LDS with the
// 16-byte chunk index XOR-swizzled by the row; the MFMA B operand (8
// consecutive rows n of one column) comes from the transposing LDS read.
constexpr int kAbsCols = 128;
constexpr int kAbsMaxN = 128;         // d_nope of the fast path (LDS 32 KiB)

__device__ inline int abs_swz(int row) { return row & 15; }

template <int OT>
__global__ __launch_bounds__(256) void absorb_mfma_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ W_UK,
                                                          void* __restrict__ q_lat, int32_t B,
                                                          int32_t h, int32_t d_n, int32_t d_r) {
  __shared__ __attribute__((aligned(16))) char ws[kAbsMaxN * kAbsCols * 2];
  const int32_t head = blockIdx.x;
  const int32_t c0 = blockIdx.y * kAbsCols;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int32_t dq = d_n + d_r, dl = kLat + d_r;
  // stage W_UK[head][0:d_n][c0:c0+128]: rows of 256 B, 16 chunks of 16 B
  for (int idx = tid; idx < d_n * 16; idx += 256) {
    const int row = idx >> 4, ch = idx & 15;
    const uint4 v = *reinterpret_cast<const uint4*>(W_UK + ((int64_t)head * d_n + row) * kLat + c0 + 8 * ch);
    *reinterpret_cast<uint4*>(ws + row * 256 + ((ch ^ abs_swz(row)) << 4)) = v;
  }
  // the rope part of the absorbed query is q_rope copied (once per head)
  if (blockIdx.y == 0) {
    for (int32_t i = tid; i < B * d_r; i += 256) {
      const int32_t b = i / d_r, k = i % d_r;
      store_elem<OT>(q_lat, ((int64_t)b * h + head) * dl + kLat + k,
                     load_elem<MLA_BF16>(q, ((int64_t)b * h + head) * dq + d_n + k));
    }
  }
  __syncthreads();
  const int g = lane >> 5, r = lane & 31;
  const int j16 = lane & 15, grp = lane >> 4, e = j16 >> 2, qd = j16 & 3;
  const int cw = 32 * wave;                      // this wave's columns within the group
  const int col_in = cw + 16 * (grp & 1) + 4 * qd;
  const int chunk = col_in >> 3, hoff = (col_in & 7) * 2;
  const int nks = d_n / 16;
  for (int32_t b0 = 0; b0 < B; b0 += 32) {
    const int32_t b = b0 + r;
    const bool live = b < B;
    const uint16_t* qrow = q + ((int64_t)(live ? b : 0) * h + head) * dq + 8 * g;
    f32x16 acc = f32x16{};
    for (int ks = 0; ks < nks; ks++) {
      bf16x8 a = *reinterpret_cast<const bf16x8*>(qrow + 16 * ks);
      if (!live) a = __builtin_bit_cast(bf16x8, i16x8{});
      const int row0 = 16 * ks + 8 * g + e, row1 = row0 + 4;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<i16x4 __attribute__((address_space(3)))*>(
          (lds_t*)ws + row0 * 256 + ((chunk ^ abs_swz(row0)) << 4) + hoff));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<i16x4 __attribute__((address_space(3)))*>(
          (lds_t*)ws + row1 * 256 + ((chunk ^ abs_swz(row1)) << 4) + hoff));
      const bf16x8 bw = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bw, acc, 0, 0, 0);
    }
    // D[m = sequence][n = column]: lane holds column c0 + cw + r
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const int32_t bb = b0 + 8 * (j >> 2) + 4 * g + (j & 3);
      if (bb < B) store_elem<OT>(q_lat, ((int64_t)bb * h + head) * dl + c0 + cw + r, acc[j]);
    }
  }
}

}  // namespace

bool proj_mfma_supported(const mla_decode_params& p) {
  return p.q_dtype == MLA_BF16 && p.weight_dtype == MLA_BF16 && p.d_latent == kLat &&
         p.d_nope % 16 == 0 && p.d_nope <= kAbsMaxN && p.d_v % 32 == 0;
}

hipError_t launch_absorb_mfma(const mla_decode_params& p, const void* q, const void* W_UK,
                              void* q_lat, int32_t ot, hipStream_t s) {
  const dim3 grid(p.num_heads, kLat / kAbsCols);
  if (ot == MLA_BF16)
    hipLaunchKernelGGL((absorb_mfma_kernel<MLA_BF16>), grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(W_UK), q_lat,
                       p.batch, p.num_heads, p.d_nope, p.d_rope);
  else
    hipLaunchKernelGGL((absorb_mfma_kernel<MLA_F32>), grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(W_UK), q_lat,
                       p.batch, p.num_heads, p.d_nope, p.d_rope);
  return hipGetLastError();
}

hipError_t launch_up_project_mfma(const mla_decode_params& p, const float* o_lat,
                                  const void* W_UV, void* out, hipStream_t s) {
  const dim3 grid(p.num_heads, p.d_v / 32);
  if (p.out_dtype == MLA_BF16)
    hipLaunchKernelGGL((up_project_mfma_kernel<MLA_BF16>), grid, dim3(64), 0, s, o_lat,
                       static_cast<const uint16_t*>(W_UV), out, p.batch, p.num_heads, p.d_v);
  else
    hipLaunchKernelGGL((up_project_mfma_kernel<MLA_F32>), grid, dim3(64), 0, s, o_lat,
                       static_cast<const uint16_t*>(W_UV), out, p.batch, p.num_heads, p.d_v);
  return hipGetLastError();
}

}  // namespace mla
