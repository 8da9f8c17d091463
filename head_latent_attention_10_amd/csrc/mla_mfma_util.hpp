// Helpers shared by the matrix-core attention kernels (gfx950): vector types,
// work-group barriers that leave direct-to-LDS loads in flight, the
// direct-to-LDS load itself, and the per-step tile descriptors.
#pragma once

#include "mla_kernels.hpp"

#include <hip/hip_ext.h>

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_t;

constexpr int kWin = 64;                  // tile descriptors per window buffer
constexpr int kWinBytes = 2 * kWin * 16;  // two window buffers

// Work-group barrier that only waits for this wave's LDS traffic.  Unlike
// __syncthreads() it does not drain the vector-memory counter, so the
// direct-to-LDS loads of later steps stay in flight across it; each batch of
// those loads is awaited explicitly by the waves that issued it before the
// barrier that starts the step using it.
__device__ inline void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt left at their maxima
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Work-group barrier for a wave that has no LDS writes to publish: it does
// not wait for its own outstanding LDS or scalar-memory operations.
__device__ inline void wg_barrier_nowait() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One 16-byte-per-lane direct global->LDS load (lane l writes lds + 16 l).
// Issued from inline assembly so that the compiler does not track it: the
// compiler cannot tell which ring stage a load targets, and for a load it
// tracks it waits for completion (vmcnt(0)) before the issuing wave's next
// LDS read of the ring, which would serialise the two-step prefetch.  Every
// stage is instead awaited explicitly (wait_vmcnt in the issuing waves, then a
// work-group barrier) before any wave reads it.  The load has no register
// results, so nothing the compiler allocates is written behind its back; M0 is
// a reserved register that the compiler sets before each of its own uses.
__device__ inline void dma16(const void* g, lds_t* l) {
  // the LDS base is wave-uniform at every call; readfirstlane keeps it in a
  // scalar register where the compiler cannot prove that itself
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)l);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m0)
               : "memory");
}

// The same load with a wave-uniform 64-bit base and a 32-bit per-lane offset.
__device__ inline void dma16s(const void* sbase, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
               "s"(m0)
               : "memory");
}

// One 4-byte-per-lane direct global->LDS load (lane l writes lds + 4 l), for
// the lanes active at the call.
__device__ inline void dma4(const void* g, lds_t* l) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)l);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(m0)
               : "memory");
}

template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");  // LDS written by the awaited loads is read after this
}

// Launch with the two optional events stamped by the dispatch itself (start
// and end of the kernel's execution); without events, a plain launch, which
// adds no packets around the kernel.
template <typename... KArgs, typename... Args>
inline void launch_timed(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t s,
                         hipEvent_t ev_start, hipEvent_t ev_stop, Args... args) {
  if (!ev_start && !ev_stop)
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
  else
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ev_start, ev_stop, 0, args...);
}

// ------------------------------------------------------------------ tiles
// A step's descriptor, read from the LDS window (wave-uniform).
struct Tile {
  int32_t blk, b, t0, nv, off;
  bool last;  // last tile of its sequence
};

__device__ inline Tile decode_tile(int32_t blk, int32_t b, int32_t t0, int32_t w) {
  Tile t;
  t.blk = blk;
  t.b = b;
  t.t0 = t0;
  t.nv = w & 63;
  t.last = (w >> 6) & 1;
  t.off = w >> 7;
  return t;
}

__device__ inline Tile read_tile(const lds_t* win, int32_t local) {
  const i32x4 v = *reinterpret_cast<const i32x4 __attribute__((address_space(3)))*>(
      win + (((local / kWin) & 1) * kWin + (local % kWin)) * 16);
  return decode_tile(__builtin_amdgcn_readfirstlane(v[0]), __builtin_amdgcn_readfirstlane(v[1]),
                     __builtin_amdgcn_readfirstlane(v[2]), __builtin_amdgcn_readfirstlane(v[3]));
}

// The descriptor of tile t straight from the planner's table (scalar loads),
// for the first steps, before the LDS window has arrived.
__device__ inline Tile global_tile(const AttnArgs& a, int32_t t) {
  return decode_tile(load_ro(a.tiles, 4 * (int64_t)t), load_ro(a.tiles, 4 * (int64_t)t + 1),
                     load_ro(a.tiles, 4 * (int64_t)t + 2), load_ro(a.tiles, 4 * (int64_t)t + 3));
}

// Descriptors of tiles [t_begin + kWin w, +kWin) of the split ending at t_end
// into window buffer w % 2 (one direct load, lane l = tile l).
__device__ inline void load_window(const AttnArgs& a, lds_t* win, int32_t t_begin, int32_t t_end,
                                   int32_t w, int lane) {
  const int32_t first = t_begin + kWin * w;
  if (first + lane < t_end)
    dma16(a.tiles + 4 * (int64_t)(first + lane), win + (w & 1) * kWin * 16);
}

}  // namespace
}  // namespace mla
