// bf16 fold kernel for gfx950: one launch folds one visiting K/V block into the
// running (m, l, o) state of every resident query row.
//
// Math (aicassindra.com "Ring Attention, math", the per-query pseudo-code under
// the online-softmax identity; bembew.net "Conceptual Algorithm"): per query row,
// s = q.k * scale, m' = max(m, max s), alpha = exp(m - m'),
// l' = alpha l + sum exp(s - m'), o' = alpha o + sum exp(s - m') v.
//
// Mapping onto CDNA4:
//  * A workgroup is 4 waves; each wave owns 32 query rows, so a workgroup owns
//    a 128-row query tile.  Q stays in registers as MFMA operands for the whole
//    launch; the state (m, l, o) is loaded once, kept in registers while the
//    visiting block streams past, and stored once (or normalised and written as
//    the output on the last ring step).
//  * The visiting block streams through LDS in 64-key tiles (K and V row-major,
//    rows padded so both access patterns below are free of bank conflicts).
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    in the accumulator layout a lane then holds 16 scores of ONE query row
//    (lane % 32) and the other 16 of the 32 keys sit in lane ^ 32, so the row
//    max and row sum need one v_permlane32_swap instead of a 32-lane reduction.
//  * The same accumulator registers, rounded to bf16 with v_cvt_pk_bf16_f32,
//    are directly the B operand of O^T += V^T P^T (v_mfma_f32_32x32x16_bf16):
//    the contraction runs over keys in the order the score layout holds them,
//    and the matching V^T operand comes from row-major V in LDS with
//    ds_read_b64_tr_b16 (two 4-key runs per operand), so V is never transposed
//    in memory.
//  * exp is one v_exp_f32 (base 2): log2(e) is folded into the scale.  The row
//    sum l adds the same bf16-rounded weights that enter the value product
//    (v_dot2_f32_bf16 against (1, 1)), so numerator and denominator agree.
//  * Workgroup ids are remapped so that consecutive query tiles of one
//    (batch, head, resident block) -- which read the same K/V -- land on the
//    same XCD and share its L2.
#include <math.h>

#include "kernels.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kTileQ = kWaves * 32;  // query rows per workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Workgroups are dispatched round-robin over the 8 XCDs.  Return the logical
// tile id such that each XCD walks a contiguous range of logical tiles.
__device__ inline int xcd_remap(int wg, int total) {
  const int xcd = wg & 7;
  const int idx = wg >> 3;
  const int per = total >> 3;
  const int rem = total & 7;
  return xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

// max / sum of a value over the lane pair (l, l ^ 32).
__device__ inline float pair_max(float x) {
  auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ inline float pair_sum(float x) {
  auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

__device__ inline unsigned pack_bf16(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(unsigned, v);
}

__device__ inline float sum_bf16_pair(unsigned pr, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pr), one, acc, false);
}

__device__ inline s16x4 lds_tr16(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

// Keys per LDS tile for each head dim.
template <int D>
struct TileCfg {
  static constexpr int TK = D >= 256 ? 32 : 64;
};

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

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D >= 256 ? 1 : 2)))
void fold_bf16_kernel(const FoldParams p) {
  constexpr int TK = TileCfg<D>::TK;
  constexpr int NKB = TK / 32;          // 32-key blocks per tile
  constexpr int NC = D / 16;            // 16-wide d chunks of the score contraction
  constexpr int NDB = D / 32;           // 32-wide d blocks of the output
  constexpr int UPR = D / 8;            // 16-byte units per K/V row
  constexpr int TE = TK * D;            // elements of one K (or V) tile
  constexpr int CPW = TE / 512 / 4;     // 1 KB direct-load chunks per wave per tensor
  static_assert(CPW >= 1 && TE % 2048 == 0, "tile must split into whole 1 KB chunks per wave");
  // Two buffers, each a K tile followed by a V tile, rows unpadded, units swizzled.
  __shared__ __attribute__((aligned(1024))) __bf16 lds[2 * 2 * TE];

  const int tiles_q = (p.q_rows + kTileQ - 1) / kTileQ;
  const int total = tiles_q * p.n_res * p.H * p.B;
  int w = xcd_remap(blockIdx.x, total);
  const int qt = w % tiles_q;
  w /= tiles_q;
  const int r = w % p.n_res;
  w /= p.n_res;
  const int hi = w % p.H;
  const int bi = w / p.H;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lr = lane & 31;
  const int lg = lane >> 5;

  const int row = qt * kTileQ + wave * 32 + lr;
  const bool row_ok = row < p.q_rows;
  const int64_t srow = (int64_t)r * p.q_rows + (row_ok ? row : p.q_rows - 1);

  // Q fragments: B operand of S^T = K Q^T; lane holds Q[row][16c + 8lg .. +8].
  bf16x8 qf[NC];
  {
    const __bf16* qp = (const __bf16*)p.q + bi * p.q_sb + hi * p.q_sh + srow * p.q_sr + 8 * lg;
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[c] = *(const bf16x8*)(qp + 16 * c);
  }

  // Running state.  O^T accumulator layout: oacc[db][4j + e] holds
  // o[row][32 db + 8 j + 4 lg + e].  l is kept as two partial sums, one per
  // lane half, added at the end.
  const int64_t st_row = ((int64_t)bi * p.H + hi) * p.st_bh + srow;
  float mc;  // running max in base-2 units of the scaled score
  float lpart;
  f32x16 oacc[NDB];
  if (p.flags & kLoadState) {
    mc = p.m[st_row] * kLog2e;
    lpart = lg == 0 ? p.l[st_row] : 0.0f;
    const float* orow = p.o + st_row * D + 4 * lg;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 t = *(const f32x4*)(orow + 32 * db + 8 * j);
#pragma unroll
        for (int e = 0; e < 4; ++e) oacc[db][4 * j + e] = t[e];
      }
  } else {
    mc = -INFINITY;
    lpart = 0.0f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] = 0.0f;
  }

  const __bf16* kbase = (const __bf16*)p.k + bi * p.k_sb + hi * p.k_sh + p.k_off[r];
  const __bf16* vbase = (const __bf16*)p.v + bi * p.v_sb + hi * p.v_sh + p.v_off[r];
  const int n_kt = (p.kv_rows + TK - 1) / TK;
  const float c2 = p.scale_log2;

  // Direct-load addressing: chunk c of a tile is LDS units [64c, 64c + 64);
  // lane i writes unit 64c + i = (row, pos) and so fetches global unit
  // pos ^ swz(row) of that row.
  // (The host guarantees row strides below 2^24 elements, so these fit in 32 bits.)
  const int k_sr = (int)p.k_sr, v_sr = (int)p.v_sr;
  int ld_koff[CPW], ld_voff[CPW];
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const int u = (wave * CPW + j) * 64 + lane;
    const int lrow = u / UPR;
    const int gunit = (u % UPR) ^ swz<D>(lrow);
    ld_koff[j] = lrow * k_sr + gunit * 8;
    ld_voff[j] = lrow * v_sr + gunit * 8;
  }
  auto issue_tile = [&](int kt, int buf) {
    const int key0 = kt * TK;
    __bf16* kl = lds + buf * 2 * TE + wave * CPW * 512;
    __bf16* vl = kl + TE;
    if (key0 + TK <= p.kv_rows) {
      const __bf16* kg = kbase + (int64_t)key0 * k_sr;
      const __bf16* vg = vbase + (int64_t)key0 * v_sr;
#pragma unroll
      for (int j = 0; j < CPW; ++j) {
        gload_lds16(kg + ld_koff[j], kl + j * 512);
        gload_lds16(vg + ld_voff[j], vl + j * 512);
      }
    } else {  // ragged last tile: rows past the end re-read the last row
#pragma unroll
      for (int j = 0; j < CPW; ++j) {
        const int u = (wave * CPW + j) * 64 + lane;
        const int lrow = u / UPR;
        const int gunit = (u % UPR) ^ swz<D>(lrow);
        const int64_t g = min(key0 + lrow, p.kv_rows - 1);
        gload_lds16(kbase + g * k_sr + gunit * 8, kl + j * 512);
        gload_lds16(vbase + g * v_sr + gunit * 8, vl + j * 512);
      }
    }
  };

  // LDS read addressing (element offsets inside a K or V tile).
  // K (A operand of S^T): row 32kb + lr, unit 2c + lg  -> ((2c) ^ gk) with gk = lg ^ swz(lr).
  const int gk = lg ^ swz<D>(lr);
  int k_rd[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) k_rd[c] = lr * D + (((2 * c) ^ gk) << 3);
  // V (A operand of O^T, transposed reads): row 32kb + 16c + vr (+8), column
  // 32db + 16h + 4(lane & 3), i.e. unit (4db + x) with x = 2h + ((lane & 3) >> 1).
  const int vr = 4 * lg + ((lane & 15) >> 2);
  const int vx = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  int v_rd[2][NDB];
#pragma unroll
  for (int run = 0; run < 2; ++run) {
    const int rr = vr + 8 * run;
    const int y = vx ^ swz<D>(rr);
#pragma unroll
    for (int db = 0; db < NDB; ++db) v_rd[run][db] = rr * D + (((4 * db) ^ y) << 3) + 4 * (lane & 1);
  }

  if (n_kt > 0) issue_tile(0, 0);
  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt & 1;
    const int key0 = kt * TK;
    // Tile kt landed (this wave's loads), then every wave's loads and every
    // wave's reads of the other buffer (previous iteration) are complete.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (kt + 1 < n_kt) issue_tile(kt + 1, buf ^ 1);
    const __bf16* kl = lds + buf * 2 * TE;
    const __bf16* vl = kl + TE;

    // S^T for the 32-key blocks: sacc[kb][i] is the score of query row `row`
    // against key key0 + 32 kb + 8 (i / 4) + 4 lg + i % 4.
    f32x16 sacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.0f;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const bf16x8 a = *(const bf16x8*)(kl + 32 * kb * D + k_rd[c]);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], sacc[kb], 0, 0, 0);
      }
    }
    if (key0 + TK > p.kv_rows) {  // ragged last tile: keys past the end get -inf
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + 32 * kb + 8 * (i >> 2) + 4 * lg + (i & 3);
          if (key >= p.kv_rows) sacc[kb][i] = -INFINITY;
        }
    }

    float mx = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
    mx = pair_max(mx);
    // Every tile holds at least one real key, so mx and m_new are finite and
    // alpha = exp2(-inf) = 0 on the first tile of a fresh state.
    const float m_new = fmaxf(mc, mx * c2);
    const float alpha = __builtin_amdgcn_exp2f(mc - m_new);
    mc = m_new;

    unsigned pk[NKB][8];
    float lsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][2 * j], c2, -m_new));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][2 * j + 1], c2, -m_new));
        pk[kb][j] = pack_bf16(p0, p1);
        lsum = sum_bf16_pair(pk[kb][j], lsum);
      }
    lpart = fmaf(lpart, alpha, lsum);
    // o is rescaled only when some row of this wave raised its maximum
    // (alpha == 1 exactly otherwise).
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    }

    // O^T += V^T P^T.  For key chunk (kb, c) the lane's B operand is its
    // weights i = 8c .. 8c+7 of block kb, i.e. keys 32kb+16c+4lg+{0..3} and
    // 32kb+16c+8+4lg+{0..3}; the A operand holds V at the same keys, column d.
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const u32x4 bw = {pk[kb][4 * c], pk[kb][4 * c + 1], pk[kb][4 * c + 2], pk[kb][4 * c + 3]};
        const bf16x8 b = __builtin_bit_cast(bf16x8, bw);
        const __bf16* vrow = vl + (32 * kb + 16 * c) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const s16x4 t0 = lds_tr16(vrow + v_rd[0][db]);
          const s16x4 t1 = lds_tr16(vrow + v_rd[1][db]);
          const u32x2 w0 = __builtin_bit_cast(u32x2, t0);
          const u32x2 w1 = __builtin_bit_cast(u32x2, t1);
          const u32x4 aw = {w0[0], w0[1], w1[0], w1[1]};
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, aw), b, oacc[db], 0, 0, 0);
        }
      }
  }

  const float l_tot = pair_sum(lpart);
  if (!row_ok) return;
  if (p.flags & kWriteOut) {
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    __bf16* orow = (__bf16*)p.out + bi * p.out_sb + hi * p.out_sh + srow * p.out_sr + 4 * lg;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 t;
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = (__bf16)(oacc[db][4 * j + e] * inv);
        *(bf16x4*)(orow + 32 * db + 8 * j) = t;
      }
  }
  if (p.flags & kStoreState) {
    if (lg == 0) {
      p.m[st_row] = mc * kLn2;
      p.l[st_row] = l_tot;
    }
    float* orow = p.o + st_row * D + 4 * lg;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 t;
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = oacc[db][4 * j + e];
        *(f32x4*)(orow + 32 * db + 8 * j) = t;
      }
  }
}

}  // namespace

hipError_t launch_fold_bf16(const FoldParams& p, int d, hipStream_t s) {
  const int64_t tiles_q = (p.q_rows + kTileQ - 1) / kTileQ;
  const int64_t grid = tiles_q * p.n_res * p.H * p.B;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  switch (d) {
    case 64:
      fold_bf16_kernel<64><<<dim3((unsigned)grid), dim3(256), 0, s>>>(p);
      break;
    case 128:
      fold_bf16_kernel<128><<<dim3((unsigned)grid), dim3(256), 0, s>>>(p);
      break;
    case 256:
      fold_bf16_kernel<256><<<dim3((unsigned)grid), dim3(256), 0, s>>>(p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ra
