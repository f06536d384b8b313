// fp32 backward fold kernels: the same step as the bf16 backward kernels with
// true fp32 products on the vector ALUs (no reduced-precision matrix path).
//
// Math (the softmax derivative, vibeengines.com "Ring attention, explained",
// method step 6 for the ring): P = exp(s q.k - L), dP = dO.v,
// dS = P (dP - D), dQ += s dS k, dK += s dS q, dV += P dO.
//
//  * bwd_dq_f32_kernel: D/32 lanes share one query row (32 columns of q, dO
//    and dQ each); the visiting K and V stream through LDS in 32-key tiles
//    read as broadcasts; partial dot products combine with xor shuffles.
//  * bwd_dkdv_f32_kernel: D/32 lanes share one key (32 columns of k, v, dK,
//    dV each); the resident block's Q, dO, L and D rows stream through LDS.
#include <math.h>

#include "kernels.h"

namespace ra {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int last_row(const BwdParams& p, int blk_id, int x) {
  return last_key_at_or_before(p.mask, p.P, p.blk, p.rem, blk_id, x);
}
__device__ __forceinline__ int pos_of(const BwdParams& p, int blk_id, int row) {
  return token_pos(p.mask, p.P, p.blk, p.rem, blk_id, row);
}

template <int D>
__global__ __launch_bounds__(256) void bwd_dq_f32_kernel(const BwdParams p) {
  constexpr int TPR = D / 32;
  constexpr int ROWS = 256 / TPR;
  constexpr int TK = 32;
  constexpr int C4 = D / 4;
  __shared__ __attribute__((aligned(16))) float ks[TK * D];
  __shared__ __attribute__((aligned(16))) float vs[TK * D];

  const int tiles_q = (p.q_rows + ROWS - 1) / ROWS;
  int w = blockIdx.x;
  const int qt = w % tiles_q;
  w /= tiles_q;
  const int r = w % p.n_res;
  w /= p.n_res;
  const int hi = w % p.H;
  const int bi = w / p.H;

  const int tid = threadIdx.x;
  const int sub = tid % TPR;
  const int row = qt * ROWS + tid / TPR;
  const int q_len = p.q_len[r], kv_len = p.kv_len[r];
  if (qt * ROWS >= q_len) return;
  const bool row_ok = row < q_len;
  const int64_t srow = p.q_row0[r] + (row_ok ? row : q_len - 1);
  const int64_t st_row = ((int64_t)bi * p.H + hi) * p.st_bh + srow;
  const int col0 = 32 * sub;

  int kv_vis = kv_len, lim = kv_len - 1;
  if (p.mask != kMaskNone) {
    const int qb = p.q_blk[r], kb = p.kv_blk[r];
    kv_vis = last_row(p, kb, pos_of(p, qb, min(qt * ROWS + ROWS, q_len) - 1)) + 1;
    lim = min(lim, last_row(p, kb, pos_of(p, qb, min(row, q_len - 1))));
    if (kv_vis == 0 && p.flags == (kLoadState | kStoreState)) return;
  }

  float qv[32], dov[32], acc[32];
  {
    const float* qp = (const float*)p.q + bi * p.q_sb + hi * p.q_sh + srow * p.q_sr + col0;
    const float* dp = (const float*)p.dout + bi * p.do_sb + hi * p.do_sh + srow * p.do_sr + col0;
    const float* ap = p.dq_acc + st_row * D + col0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const f32x4 a = *(const f32x4*)(qp + 4 * c);
      const f32x4 b = *(const f32x4*)(dp + 4 * c);
      f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
      if (p.flags & kLoadState) z = *(const f32x4*)(ap + 4 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qv[4 * c + e] = a[e];
        dov[4 * c + e] = b[e];
        acc[4 * c + e] = z[e];
      }
    }
  }
  const float nl2 = p.nl2[st_row];
  const float ddv = p.dd[st_row];
  const float c2 = p.scale_log2;

  const float* kbase = (const float*)p.k + bi * p.k_sb + hi * p.k_sh + p.k_off[r];
  const float* vbase = (const float*)p.v + bi * p.v_sb + hi * p.v_sh + p.v_off[r];
  const int n_kt = (kv_vis + TK - 1) / TK;
  for (int kt = 0; kt < n_kt; ++kt) {
    const int key0 = kt * TK;
    __syncthreads();
    for (int ch = tid; ch < TK * C4; ch += 256) {
      const int rr = ch / C4;
      const int cc = (ch % C4) * 4;
      const int64_t g = min(key0 + rr, kv_len - 1);
      *(f32x4*)(ks + rr * D + cc) = *(const f32x4*)(kbase + g * p.k_sr + cc);
      *(f32x4*)(vs + rr * D + cc) = *(const f32x4*)(vbase + g * p.v_sr + cc);
    }
    __syncthreads();
#pragma unroll 2
    for (int j = 0; j < TK; ++j) {
      const float* kr = ks + j * D + col0;
      const float* vr = vs + j * D + col0;
      float s = 0.0f, dpv = 0.0f;
#pragma unroll
      for (int c = 0; c < 32; ++c) {
        s = fmaf(qv[c], kr[c], s);
        dpv = fmaf(dov[c], vr[c], dpv);
      }
#pragma unroll
      for (int x = 1; x < TPR; x <<= 1) {
        s += __shfl_xor(s, x);
        dpv += __shfl_xor(dpv, x);
      }
      const float pw = key0 + j <= lim ? __builtin_amdgcn_exp2f(fmaf(s, c2, nl2)) : 0.0f;
      const float ds = pw * (dpv - ddv);
#pragma unroll
      for (int c = 0; c < 32; ++c) acc[c] = fmaf(ds, kr[c], acc[c]);
    }
  }

  if (!row_ok) return;
  if (p.flags & kWriteOut) {
    float* op = (float*)p.dq + bi * p.dq_sb + hi * p.dq_sh + srow * p.dq_sr + col0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      f32x4 t;
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] = acc[4 * c + e] * p.scale;
      *(f32x4*)(op + 4 * c) = t;
    }
  } else if (p.flags & kStoreState) {
    float* ap = p.dq_acc + st_row * D + col0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      f32x4 t;
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] = acc[4 * c + e];
      *(f32x4*)(ap + 4 * c) = t;
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void bwd_dkdv_f32_kernel(const BwdParams p) {
  constexpr int TPK = D / 32;       // threads per key
  constexpr int KEYS = 256 / TPK;   // keys per workgroup
  constexpr int TQ = 32;
  constexpr int C4 = D / 4;
  __shared__ __attribute__((aligned(16))) float qs[TQ * D];
  __shared__ __attribute__((aligned(16))) float ds_[TQ * D];
  __shared__ float nls[TQ], dds[TQ];

  const int tiles_k = (p.kv_rows + KEYS - 1) / KEYS;
  int w = blockIdx.x;
  const int kt = w % tiles_k;
  w /= tiles_k;
  const int r = w % p.n_res;
  w /= p.n_res;
  const int hi = w % p.H;
  const int bi = w / p.H;

  const int tid = threadIdx.x;
  const int sub = tid % TPK;
  const int q_len = p.q_len[r], kv_len = p.kv_len[r];
  if (kt * KEYS >= kv_len) return;
  const int key = kt * KEYS + tid / TPK;
  const bool key_ok = key < kv_len;
  const int ck = key_ok ? key : kv_len - 1;
  const int col0 = 32 * sub;

  int q_from = 0, fr = 0;
  if (p.mask != kMaskNone) {
    const int qb = p.q_blk[r], kb = p.kv_blk[r];
    auto first_row = [&](int krow) { return last_row(p, qb, pos_of(p, kb, krow) - 1) + 1; };
    q_from = first_row(kt * KEYS);
    fr = first_row(ck);
    if (q_from >= q_len) return;
  }

  float kv[32], vv[32], dk[32], dv[32];
  const int64_t arow = ((int64_t)bi * p.H + hi) * p.acc_bh + p.acc_row0[r] + ck;
  {
    const float* kp = (const float*)p.k + bi * p.k_sb + hi * p.k_sh + p.k_off[r] + (int64_t)ck * p.k_sr + col0;
    const float* vp = (const float*)p.v + bi * p.v_sb + hi * p.v_sh + p.v_off[r] + (int64_t)ck * p.v_sr + col0;
    const float* dkp = p.dk_acc + arow * D + col0;
    const float* dvp = p.dv_acc + arow * D + col0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const f32x4 a = *(const f32x4*)(kp + 4 * c);
      const f32x4 b = *(const f32x4*)(vp + 4 * c);
      const f32x4 x = *(const f32x4*)(dkp + 4 * c);
      const f32x4 y = *(const f32x4*)(dvp + 4 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kv[4 * c + e] = a[e];
        vv[4 * c + e] = b[e];
        dk[4 * c + e] = x[e];
        dv[4 * c + e] = y[e];
      }
    }
  }

  const int64_t row0 = p.q_row0[r];
  const float* qbase = (const float*)p.q + bi * p.q_sb + hi * p.q_sh + row0 * p.q_sr;
  const float* dbase = (const float*)p.dout + bi * p.do_sb + hi * p.do_sh + row0 * p.do_sr;
  const int64_t rbase = ((int64_t)bi * p.H + hi) * p.st_bh + row0;
  const float c2 = p.scale_log2;
  const int n_qt = (q_len + TQ - 1) / TQ;
  for (int qt = q_from / TQ; qt < n_qt; ++qt) {
    const int q0 = qt * TQ;
    __syncthreads();
    for (int ch = tid; ch < TQ * C4; ch += 256) {
      const int rr = ch / C4;
      const int cc = (ch % C4) * 4;
      const int64_t g = min(q0 + rr, q_len - 1);
      *(f32x4*)(qs + rr * D + cc) = *(const f32x4*)(qbase + g * p.q_sr + cc);
      *(f32x4*)(ds_ + rr * D + cc) = *(const f32x4*)(dbase + g * p.do_sr + cc);
    }
    if (tid < TQ) {
      const int64_t g = min(q0 + tid, q_len - 1);
      nls[tid] = p.nl2[rbase + g];
      dds[tid] = p.dd[rbase + g];
    }
    __syncthreads();
#pragma unroll 2
    for (int i = 0; i < TQ; ++i) {
      const float* qr = qs + i * D + col0;
      const float* dr = ds_ + i * D + col0;
      float s = 0.0f, dpv = 0.0f;
#pragma unroll
      for (int c = 0; c < 32; ++c) {
        s = fmaf(kv[c], qr[c], s);
        dpv = fmaf(vv[c], dr[c], dpv);
      }
#pragma unroll
      for (int x = 1; x < TPK; x <<= 1) {
        s += __shfl_xor(s, x);
        dpv += __shfl_xor(dpv, x);
      }
      const int rq = q0 + i;
      const float pw = (rq >= fr && rq < q_len) ? __builtin_amdgcn_exp2f(fmaf(s, c2, nls[i])) : 0.0f;
      const float dsv = pw * (dpv - dds[i]);
#pragma unroll
      for (int c = 0; c < 32; ++c) {
        dv[c] = fmaf(pw, dr[c], dv[c]);
        dk[c] = fmaf(dsv, qr[c], dk[c]);
      }
    }
  }

  if (!key_ok) return;
  float* dkp = p.dk_acc + arow * D + col0;
  float* dvp = p.dv_acc + arow * D + col0;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    f32x4 x, y;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = dk[4 * c + e];
      y[e] = dv[4 * c + e];
    }
    *(f32x4*)(dkp + 4 * c) = x;
    *(f32x4*)(dvp + 4 * c) = y;
  }
}

}  // namespace

hipError_t launch_bwd_dq_f32(const BwdParams& p, int d, hipStream_t s) {
  const int rows = 256 / (d / 32);
  const int64_t grid = (int64_t)((p.q_rows + rows - 1) / rows) * p.n_res * p.H * p.B;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  switch (d) {
    case 64:
      bwd_dq_f32_kernel<64><<<dim3((unsigned)grid), dim3(256), 0, s>>>(p);
      break;
    case 128:
      bwd_dq_f32_kernel<128><<<dim3((unsigned)grid), dim3(256), 0, s>>>(p);
      break;
    case 256:
      bwd_dq_f32_kernel<256><<<dim3((unsigned)grid), dim3(256), 0, s>>>(p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_f32(const BwdParams& p, int d, hipStream_t s) {
  const int keys = 256 / (d / 32);
  const int64_t grid = (int64_t)((p.kv_rows + keys - 1) / keys) * p.n_res * p.H * p.B;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  switch (d) {
    case 64:
      bwd_dkdv_f32_kernel<64><<<dim3((unsigned)grid), dim3(256), 0, s>>>(p);
      break;
    case 128:
      bwd_dkdv_f32_kernel<128><<<dim3((unsigned)grid), dim3(256), 0, s>>>(p);
      break;
    case 256:
      bwd_dkdv_f32_kernel<256><<<dim3((unsigned)grid), dim3(256), 0, s>>>(p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ra
