// gfx950 device helpers shared by the bf16 fold kernels (forward and
// backward): vector types, XCD-aware workgroup order, lane-pair reductions,
// bf16 packing, LDS transpose reads, the LDS swizzle, direct-to-LDS loads and
// the LDS barrier.
#pragma once

#include <hip/hip_runtime.h>

namespace ra {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Workgroups are dispatched round-robin over the 8 XCDs.  Return the logical
// tile id such that each XCD walks a contiguous range of logical tiles.
__device__ __forceinline__ int xcd_remap(int wg, int total) {
  const int xcd = wg & 7;
  const int idx = wg >> 3;
  const int per = total >> 3;
  const int rem = total & 7;
  return xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

// max / sum of a value over the lane pair (l, l ^ 32).
__device__ __forceinline__ float pair_max(float x) {
  auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// max / sum of a value over the four lanes l, l ^ 16, l ^ 32, l ^ 48
// (v_permlane16_swap pairs rows 0-1 and 2-3 of 16 lanes, then the 32-lane swap).
__device__ __forceinline__ float quad_max(float x) {
  auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return pair_max(fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])));
}
__device__ __forceinline__ float quad_sum(float x) {
  auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return pair_sum(__uint_as_float(sw[0]) + __uint_as_float(sw[1]));
}

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(unsigned, v);
}

__device__ __forceinline__ float sum_bf16_pair(unsigned pr, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pr), one, acc, false);
}

__device__ __forceinline__ s16x4 lds_tr16(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

// XOR swizzle of the 16-byte units of LDS row r.  K is read as 16-byte
// units of 16 consecutive rows and V as 8-byte transposed reads of 4 rows x 4
// units; with the 64-bank LDS both patterns are conflict-free when f is a
// bijection on 16 consecutive rows whose bits 2..3 differ across 4 consecutive
// rows (rows of 128 B for d = 64 pair up within one 256-byte bank row, hence
// the separate form).
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D >= 128)
    return ((r & 3) << 2) | ((r >> 2) & 3);
  else
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Direct-to-LDS loads, issued from inline assembly so that the compiler does
// not track them: it neither counts them in its own vmcnt waits nor makes
// later LDS reads wait for them (it cannot tell which LDS bytes such a load
// writes, and so made the value product of every other tile wait for the
// next tile's loads).  The tile loops wait for them themselves (s_waitcnt
// vmcnt, then lds_barrier), and wait for every load issued before a loop
// once before it.  M0 is an operand of the statement, so the compiler writes
// it and knows it is taken; the s_nop is the wait state between an SALU write
// of M0 and the load that reads it.  Lane l's bytes land at LDS address
// lds + 16 l (lds + 4 l for the dword form).
//  * global_load_lds_dwordx4 / _dword from a 64-bit address per lane;
//  * buffer_load_dwordx4 ... lds from byte offset voff of the buffer whose
//    resource words are rs (the 64-bit base in scalar registers, so a tile
//    costs no vector address arithmetic).
__device__ __forceinline__ void gload_lds16(const void* g, unsigned lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void gload_lds4(const void* g, unsigned lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" : : "v"(g), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void bload_lds16(u32x4 rs, int voff, unsigned lds) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voff), "s"(rs), "{m0}"(lds) : "memory");
}
// The LDS address of a __shared__ object.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(size_t)(const __attribute__((address_space(3))) void*)p;
}
// Resource words of a buffer over `base` with no effective range limit (every
// access is computed in bounds by the kernel).
__device__ __forceinline__ u32x4 rsrc_words(const void* base) {
  const size_t a = (size_t)base;
  return u32x4{(unsigned)a, (unsigned)(a >> 32) & 0xffffu, 0x7fffffffu, 0x00020000u};
}
// Workgroup barrier that orders LDS only: the tile loops call it right after
// their own vmcnt wait, with no global access of theirs left to order
// (__syncthreads would add a wait for every vector memory access in flight).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace dev
}  // namespace ra
