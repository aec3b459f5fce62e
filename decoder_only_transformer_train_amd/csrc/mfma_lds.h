// gfx950 building blocks for kernels that stream operand blocks into LDS with
// direct-to-LDS buffer loads and multiply them on 32x32x16 bf16 MFMAs.
#pragma once
#include "common.h"

namespace gk {
namespace mx {

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(3))) void lds_void;

constexpr float NEG_INF = -__builtin_huge_valf();

// buffer descriptor over [p, p + bytes); loads past the range return zeros
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, int64_t bytes) {
  const uint32_t n = bytes > 0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, 0x00020000);
}
// one wave instruction: lane i's 16 (4) bytes at byte offset voff land at lds + 16 i (4 i)
__device__ __forceinline__ void dma16(rsrc_t r, char* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void dma4(rsrc_t r, char* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, voff, 0, 0, 0);
}
// wait until at most N of this wave's vector-memory instructions are outstanding
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // s_waitcnt simm16 on gfx9: vmcnt bits [3:0] and [15:14]; expcnt and lgkmcnt at their maxima
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for data exchanged through LDS: this wave's LDS reads and
// writes are complete, then s_barrier.  Unlike __syncthreads() it does not wait
// for outstanding direct-to-LDS loads (vmcnt), so blocks prefetched into other
// stages stay in flight; the empty asm statements keep the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt at their maxima (gfx9 encoding)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void mma32(f32x16& c, const uint4& a, const uint4& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bitcast<bf16x8>(a), bitcast<bf16x8>(b), c, 0, 0, 0);
}
__device__ __forceinline__ void zero16(f32x16& c) {
#pragma unroll
  for (int e = 0; e < 16; ++e) c[e] = 0.f;
}
// A 32x32 C tile: lane l holds column l % 32 and rows crow(e, l / 32), e = 0..15
__device__ __forceinline__ int crow(int e, int g) { return (e >> 2) * 8 + g * 4 + (e & 3); }
// the 8 accumulators 8 hh .. 8 hh + 7 of a C tile (its rows 16 hh .. 16 hh + 15)
// as the bf16 B fragment of a 32x32x16 product whose k runs over those rows
__device__ __forceinline__ uint4 pack_half(const f32x16& c, int hh) {
  bf16x8 v;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = (bf16)c[8 * hh + j];
  return bitcast<uint4>(v);
}
// the two lane halves' values of v, summed (lane l and lane l ^ 32)
__device__ __forceinline__ float halves_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float halves_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

}  // namespace mx
}  // namespace gk
