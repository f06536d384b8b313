// State set-up and finalisation kernels.
//  * init: (m, l, o) = (-inf, 0, 0)  -- aicassindra.com "Ring Attention, math",
//    "Accumulation math, step by step", the state before the first block.
//  * finalize: O = o / l -- same passage, after the last block.  A row that
//    never saw a key (l == 0) is written as 0.
// Both are plain HBM-bound elementwise passes with 16-byte accesses.
//  * backward set-up: per query row, the negated log-sum-exp in base 2 and
//    D = rowsum(dO * O) (the softmax derivative's row term); scaled cast of
//    the fp32 gradient accumulators; zero fill.
#include <math.h>

#include "kernels.h"

namespace ra {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void state_init_kernel(float* m, float* l, float* o, int64_t rows, int64_t o_vec4) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < o_vec4; i += stride)
    ((f32x4*)o)[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < rows; i += stride) {
    m[i] = -INFINITY;
    l[i] = 0.0f;
  }
}

template <bool kBf16>
__global__ __launch_bounds__(256) void finalize_kernel(const float* l, const float* o, void* out, int64_t out_sb,
                                                       int64_t out_sh, int64_t out_sr, int H, int64_t rows, int d,
                                                       int64_t n_vec4) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int per_row = d / 4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_vec4; i += stride) {
    const int64_t row_all = i / per_row;  // (bi * H + hi) * rows + row
    const int c = (int)(i % per_row) * 4;
    const int64_t bh = row_all / rows;
    const int64_t row = row_all % rows;
    const int64_t bi = bh / H;
    const int64_t hi = bh % H;
    const float lv = l[row_all];
    const float inv = lv > 0.0f ? 1.0f / lv : 0.0f;
    const f32x4 t = ((const f32x4*)o)[i];
    const int64_t off = bi * out_sb + hi * out_sh + row * out_sr + c;
    if (kBf16) {
      bf16x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = (__bf16)(t[e] * inv);
      *(bf16x4*)((__bf16*)out + off) = r;
    } else {
      f32x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = t[e] * inv;
      *(f32x4*)((float*)out + off) = r;
    }
  }
}

// One wave per row: nl2 = -lse log2(e) (-inf stays -inf), dd = sum_c dO O.
template <bool kBf16>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const float* lse, const void* dout, int64_t do_sb,
                                                       int64_t do_sh, int64_t do_sr, const void* out, int64_t o_sb,
                                                       int64_t o_sh, int64_t o_sr, int H, int64_t rows, int d,
                                                       int64_t n_rows, float* nl2, float* dd) {
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * 4;
  for (int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); i < n_rows; i += waves) {
    const int64_t bh = i / rows, row = i % rows;
    const int64_t bi = bh / H, hi = bh % H;
    float acc = 0.0f;
    for (int c = lane; c < d; c += 64) {
      const int64_t od = bi * do_sb + hi * do_sh + row * do_sr + c;
      const int64_t oo = bi * o_sb + hi * o_sh + row * o_sr + c;
      if (kBf16)
        acc = fmaf((float)((const __bf16*)dout)[od], (float)((const __bf16*)out)[oo], acc);
      else
        acc = fmaf(((const float*)dout)[od], ((const float*)out)[oo], acc);
    }
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) acc += __shfl_xor(acc, x);
    if (lane == 0) {
      const float L = lse[i];
      nl2[i] = L == -INFINITY ? -INFINITY : -L * 1.4426950408889634f;
      dd[i] = acc;
    }
  }
}

template <bool kBf16>
__global__ __launch_bounds__(256) void scale_cast_kernel(const float* acc, float alpha, void* dst, int64_t sb,
                                                         int64_t sh, int64_t sr, int H, int64_t rows, int d,
                                                         int64_t n_vec4) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int per_row = d / 4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_vec4; i += stride) {
    const int64_t row_all = i / per_row;
    const int c = (int)(i % per_row) * 4;
    const int64_t bh = row_all / rows, row = row_all % rows;
    const int64_t bi = bh / H, hi = bh % H;
    const f32x4 t = ((const f32x4*)acc)[i];
    const int64_t off = bi * sb + hi * sh + row * sr + c;
    if (kBf16) {
      bf16x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = (__bf16)(t[e] * alpha);
      *(bf16x4*)((__bf16*)dst + off) = r;
    } else {
      f32x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = t[e] * alpha;
      *(f32x4*)((float*)dst + off) = r;
    }
  }
}

__global__ __launch_bounds__(256) void zero_kernel(float* x, int64_t n_vec4) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_vec4; i += stride)
    ((f32x4*)x)[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
}

__global__ __launch_bounds__(256) void fill_kernel(unsigned* x, int64_t n_vec4, unsigned value) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_vec4; i += stride)
    ((u32x4*)x)[i] = u32x4{value, value, value, value};
}

inline unsigned grid_for(int64_t n) {
  const int64_t g = (n + 255) / 256;
  return (unsigned)(g < 1 ? 1 : (g > 65536 ? 65536 : g));
}

}  // namespace

hipError_t launch_state_init(float* m, float* l, float* o, int64_t rows_total, int d, hipStream_t s) {
  const int64_t o_vec4 = rows_total * d / 4;
  if (rows_total <= 0) return hipSuccess;
  state_init_kernel<<<grid_for(o_vec4), 256, 0, s>>>(m, l, o, rows_total, o_vec4);
  return hipGetLastError();
}

hipError_t launch_finalize(const float* l, const float* o, void* out, bool out_bf16, int64_t out_sb,
                           int64_t out_sh, int64_t out_sr, int B, int H, int64_t rows, int d, hipStream_t s) {
  const int64_t n_vec4 = (int64_t)B * H * rows * d / 4;
  if (n_vec4 <= 0) return hipSuccess;
  if (out_bf16)
    finalize_kernel<true><<<grid_for(n_vec4), 256, 0, s>>>(l, o, out, out_sb, out_sh, out_sr, H, rows, d, n_vec4);
  else
    finalize_kernel<false><<<grid_for(n_vec4), 256, 0, s>>>(l, o, out, out_sb, out_sh, out_sr, H, rows, d, n_vec4);
  return hipGetLastError();
}

hipError_t launch_bwd_prep(const float* lse, const void* dout, int64_t do_sb, int64_t do_sh, int64_t do_sr,
                           const void* out, int64_t o_sb, int64_t o_sh, int64_t o_sr, bool bf16, int B, int H,
                           int64_t rows, int d, float* nl2, float* dd, hipStream_t s) {
  const int64_t n_rows = (int64_t)B * H * rows;
  if (n_rows <= 0) return hipSuccess;
  const int64_t g = (n_rows + 3) / 4;
  const unsigned grid = (unsigned)(g > 65536 ? 65536 : g);
  if (bf16)
    bwd_prep_kernel<true><<<grid, 256, 0, s>>>(lse, dout, do_sb, do_sh, do_sr, out, o_sb, o_sh, o_sr, H, rows, d,
                                               n_rows, nl2, dd);
  else
    bwd_prep_kernel<false><<<grid, 256, 0, s>>>(lse, dout, do_sb, do_sh, do_sr, out, o_sb, o_sh, o_sr, H, rows, d,
                                                n_rows, nl2, dd);
  return hipGetLastError();
}

hipError_t launch_scale_cast(const float* acc, float alpha, void* dst, int64_t sb, int64_t sh, int64_t sr, bool bf16,
                             int B, int H, int64_t rows, int d, hipStream_t s) {
  const int64_t n_vec4 = (int64_t)B * H * rows * d / 4;
  if (n_vec4 <= 0) return hipSuccess;
  if (bf16)
    scale_cast_kernel<true><<<grid_for(n_vec4), 256, 0, s>>>(acc, alpha, dst, sb, sh, sr, H, rows, d, n_vec4);
  else
    scale_cast_kernel<false><<<grid_for(n_vec4), 256, 0, s>>>(acc, alpha, dst, sb, sh, sr, H, rows, d, n_vec4);
  return hipGetLastError();
}

hipError_t launch_fill_u32(void* x, size_t bytes, unsigned value, hipStream_t s) {
  if (bytes % 16 != 0 || ((uintptr_t)x & 15) != 0) return hipErrorInvalidValue;
  const int64_t n_vec4 = (int64_t)(bytes / 16);
  if (n_vec4 <= 0) return hipSuccess;
  fill_kernel<<<grid_for(n_vec4), 256, 0, s>>>((unsigned*)x, n_vec4, value);
  return hipGetLastError();
}

hipError_t launch_zero(float* x, int64_t n, hipStream_t s) {
  const int64_t n_vec4 = n / 4;
  if (n_vec4 <= 0) return hipSuccess;
  zero_kernel<<<grid_for(n_vec4), 256, 0, s>>>(x, n_vec4);
  return hipGetLastError();
}

}  // namespace ra
