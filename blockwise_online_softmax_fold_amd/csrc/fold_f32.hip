// fp32 fold kernel: the same recurrence as the bf16 kernel with true fp32
// products (plain VALU FMAs, no reduced-precision matrix path) and fp32
// weights, for inputs given in fp32.
//
// Math: aicassindra.com "Ring Attention, math", the per-query pseudo-code under
// the online-softmax identity (m' = max(m, max s), alpha = exp(m - m'),
// l' = alpha l + sum exp(s - m'), o' = alpha o + sum exp(s - m') v).
//
// Layout: TPR = d / CPL threads share one query row, each holding CPL of its
// q and o columns in registers; partial dot products are combined across
// those lanes with xor shuffles.  A small CPL (8 for d = 64, 16 above) keeps
// the serial work per lane short and the workgroup count up on small rings.  K and V stream through LDS in 32-key tiles, which
// every row of the workgroup reads as broadcasts.
//
// Causal masking (math page, "Causal masking, load balance, and other
// wrinkles"): the keys a row sees form a prefix of the visiting block in every
// token layout, so the tile loop stops after the last key any row of the
// workgroup sees and each row masks keys past its own last visible key.
#include <math.h>

#include "kernels.h"

namespace ra {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTileK = 32;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D, int CPL>
__global__ __launch_bounds__(256) void fold_f32_kernel(const FoldParams p) {
  constexpr int TPR = D / CPL;    // threads per query row
  constexpr int ROWS = 256 / TPR; // query rows per workgroup
  constexpr int C4 = D / 4;       // float4 chunks per K/V row
  __shared__ __attribute__((aligned(16))) float ks[kTileK * D];
  __shared__ __attribute__((aligned(16))) float vs[kTileK * D];

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
  // This resident's block lengths; a query tile past its end has nothing to do.
  const int q_len = p.q_len[r], kv_len = p.kv_len[r];
  if (qt * ROWS >= q_len) return;
  const bool row_ok = row < q_len;

  // Keys [0, kv_vis) are visible to some row of this workgroup; key c is
  // visible to this thread's row iff c <= lim.
  int kv_vis = kv_len;
  int lim = kv_len - 1;
  if (p.mask != kMaskNone) {
    const int qb = p.q_blk[r], kb = p.kv_blk[r];
    auto last_key = [&](int qrow) {
      return last_key_at_or_before(p.mask, p.P, p.blk, p.rem, kb, token_pos(p.mask, p.P, p.blk, p.rem, qb, qrow));
    };
    kv_vis = last_key(min(qt * ROWS + ROWS, q_len) - 1) + 1;
    lim = min(lim, last_key(min(row, q_len - 1)));
    // Nothing visible and nothing to initialise or write: the state stays as it is.
    if (kv_vis == 0 && (p.flags & ~kRefState) == (kLoadState | kStoreState)) return;
  }
  const int64_t srow = (int64_t)p.q_row0[r] + (row_ok ? row : q_len - 1);
  const int col0 = CPL * sub;

  float qv[CPL];
  {
    const float* qp = (const float*)p.q + bi * p.q_sb + hi * p.q_sh + srow * p.q_sr + col0;
#pragma unroll
    for (int c = 0; c < CPL / 4; ++c) {
      const f32x4 t = *(const f32x4*)(qp + 4 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) qv[4 * c + e] = t[e];
    }
  }

  const int64_t st_row = ((int64_t)bi * p.H + hi) * p.st_bh + srow;
  float mc, l, m_in;
  float ov[CPL];
  if (p.flags & kLoadState) {
    m_in = p.m[st_row];
    mc = m_in * kLog2e;
    l = p.l[st_row];
    const float* op = p.o + st_row * D + col0;
#pragma unroll
    for (int c = 0; c < CPL / 4; ++c) {
      const f32x4 t = *(const f32x4*)(op + 4 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) ov[4 * c + e] = t[e];
    }
  } else {
    m_in = -INFINITY;
    mc = -INFINITY;
    l = 0.0f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) ov[c] = 0.0f;
  }

  const float* kbase = (const float*)p.k + bi * p.k_sb + hi * p.k_sh + p.k_off[r];
  const float* vbase = (const float*)p.v + bi * p.v_sb + hi * p.v_sh + p.v_off[r];
  const int n_kt = (kv_vis + kTileK - 1) / kTileK;
  const float c2 = p.scale_log2;

  for (int kt = 0; kt < n_kt; ++kt) {
    const int key0 = kt * kTileK;
    __syncthreads();
    for (int ch = tid; ch < kTileK * C4; ch += 256) {
      const int rr = ch / C4;
      const int cc = (ch % C4) * 4;
      const int64_t g = min(key0 + rr, kv_len - 1);
      *(f32x4*)(ks + rr * D + cc) = *(const f32x4*)(kbase + g * p.k_sr + cc);
      *(f32x4*)(vs + rr * D + cc) = *(const f32x4*)(vbase + g * p.v_sr + cc);
    }
    __syncthreads();

    float s[kTileK];
#pragma unroll
    for (int j = 0; j < kTileK; ++j) {
      const float* kr = ks + j * D + col0;
      float acc = 0.0f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc = fmaf(qv[c], kr[c], acc);
#pragma unroll
      for (int x = 1; x < TPR; x <<= 1) acc += __shfl_xor(acc, x);
      s[j] = key0 + j <= lim ? acc : -INFINITY;
    }
    float mx = s[0];
#pragma unroll
    for (int j = 1; j < kTileK; ++j) mx = fmaxf(mx, s[j]);
    const float m_new = fmaxf(mc, mx * c2);
    // A row that has seen no visible key yet keeps (-inf, 0, 0): exponents are
    // taken against 0 instead of -inf, so every weight is exp2(-inf) = 0.
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(mc - m_use);
    mc = m_new;
    float lsum = 0.0f;
#pragma unroll
    for (int j = 0; j < kTileK; ++j) {
      s[j] = __builtin_amdgcn_exp2f(fmaf(s[j], c2, -m_use));
      lsum += s[j];
    }
    l = fmaf(l, alpha, lsum);
#pragma unroll
    for (int c = 0; c < CPL; ++c) ov[c] *= alpha;
#pragma unroll
    for (int j = 0; j < kTileK; ++j) {
      const float* vr = vs + j * D + col0;
#pragma unroll
      for (int c = 0; c < CPL; ++c) ov[c] = fmaf(s[j], vr[c], ov[c]);
    }
  }

  if (!row_ok) return;
  if (p.flags & kWriteOut) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    if (p.lse != nullptr && sub == 0) p.lse[st_row] = l > 0.0f ? (mc + log2f(l)) * kLn2 : -INFINITY;
    float* op = (float*)p.out + bi * p.out_sb + hi * p.out_sh + srow * p.out_sr + col0;
#pragma unroll
    for (int c = 0; c < CPL / 4; ++c) {
      f32x4 t;
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] = ov[4 * c + e] * inv;
      *(f32x4*)(op + 4 * c) = t;
    }
  }
  if (p.flags & kStoreState) {
    if (sub == 0) {
      // A maximum that did not rise is stored exactly as it was loaded.
      p.m[st_row] = mc == m_in * kLog2e ? m_in : mc * kLn2;
      p.l[st_row] = l;
    }
    float* op = p.o + st_row * D + col0;
#pragma unroll
    for (int c = 0; c < CPL / 4; ++c) {
      f32x4 t;
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] = ov[4 * c + e];
      *(f32x4*)(op + 4 * c) = t;
    }
  }
}

}  // namespace

// Columns of q and o per lane.
constexpr int cols_per_lane(int d) { return d == 64 ? 8 : 16; }

hipError_t launch_fold_f32(const FoldParams& p, int d, hipStream_t s) {
  const int rows_per_wg = 256 / (d / cols_per_lane(d));
  const int64_t tiles_q = (p.q_rows + rows_per_wg - 1) / rows_per_wg;
  const int64_t grid = tiles_q * p.n_res * p.H * p.B;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  switch (d) {
    case 64:
      fold_f32_kernel<64, cols_per_lane(64)><<<dim3((unsigned)grid), dim3(256), 0, s>>>(p);
      break;
    case 128:
      fold_f32_kernel<128, cols_per_lane(128)><<<dim3((unsigned)grid), dim3(256), 0, s>>>(p);
      break;
    case 256:
      fold_f32_kernel<256, cols_per_lane(256)><<<dim3((unsigned)grid), dim3(256), 0, s>>>(p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ra
