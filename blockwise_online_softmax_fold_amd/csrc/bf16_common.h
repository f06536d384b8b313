// gfx950 device helpers shared by the bf16 fold kernels (forward and
// backward): vector types, XCD-aware workgroup order, lane-pair reductions,
// bf16 packing, LDS transpose reads, the LDS swizzle and direct-to-LDS loads.
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

// 16 bytes from global memory straight into LDS (global_load_lds_dwordx4):
// lane i's bytes land at lds_wave_base + 16 i.
__device__ __forceinline__ void gload_lds16(const __bf16* g, __bf16* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(g),
                                   (__attribute__((address_space(3))) void*)(lds_wave_base), 16, 0, 0);
}

// Buffer resource over `base` with no effective range limit (every access is
// computed in bounds by the kernel) for the raw buffer loads below.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}

// 16 bytes at byte offset voff of the buffer straight into LDS
// (buffer_load_dwordx4 ... lds): lane i's bytes land at lds_wave_base + 16 i.
// The 64-bit base lives in scalar registers, so a tile costs no vector
// address arithmetic.
__device__ __forceinline__ void bload_lds16(__amdgpu_buffer_rsrc_t rs, int voff, __bf16* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(lds_wave_base), 16, voff, 0,
                                           0, 0);
}

}  // namespace dev
}  // namespace ra
