// bf16 backward fold kernels for gfx950: one ring step of the backward pass.
//
// Math: the gradients of O = softmax(s Q K^T) V written out with the softmax
// derivative, P = exp(s Q K^T - L) with L = m + ln l the row log-sum-exp the
// forward kept, dP = dO V^T, D = rowsum(dO * O), dS = P * (dP - D),
// dQ = s dS K, dK = s dS^T Q, dV = P^T dO.  On the ring (vibeengines.com "Ring
// attention, explained", method step 6) device i keeps dQ_i and adds its share
// to the visiting block's dK_j, dV_j, which travel with the block.
//
// Two kernels per step, no atomics:
// Both run NW waves per workgroup (8 for d = 128, 4 for d = 64 and 256), so a
// tile streamed through L2 into LDS serves 32 NW rows (keys).
//  * bwd_dq_kernel: like the forward fold -- NW waves x 32 query rows, Q and dO
//    in registers as MFMA B operands, the visiting K and V streamed through
//    double-buffered swizzled LDS in 32-key tiles.  S^T = K Q^T and
//    dP^T = V dO^T put one query row in each lane (lane ^ 32 holds the other
//    keys), so L and D are one register each; dS is rounded to bf16 in the
//    accumulator layout and is directly the B operand of dQ^T += K^T dS^T,
//    with the K^T operand read from row-major K by ds_read_b64_tr_b16.
//  * bwd_dkdv_kernel: the transpose of the same pattern -- each wave owns 32
//    keys (K in registers, the workgroup's V rows in LDS, both as B operands)
//    and streams the resident block's Q and dO rows (plus their L and D)
//    through LDS in 32-row tiles; S = Q K^T and dP = dO V^T put one key in
//    each lane, and
//    dV^T += dO^T P, dK^T += Q^T dS read dO^T and Q^T by transposed LDS
//    reads.  The dK, dV accumulators (fp32, unscaled by s) are loaded and
//    stored once per launch; one workgroup owns each 32 NW-key tile, so no two
//    workgroups touch the same rows.  Keeping V in LDS rather than registers
//    leaves the d <= 128 kernel within 256 VGPRs: two waves per SIMD, and the
//    MFMA accumulators stay in VGPRs where the VALU reads them directly.
// Causal masking uses the same prefix argument as the forward: the keys a
// query sees are a prefix of the visiting block, so the queries a key is seen
// by are a suffix of the resident block; tiles outside are skipped.
#include <math.h>

#include "bf16_common.h"
#include "kernels.h"

namespace ra {
namespace {

using namespace dev;

__device__ __forceinline__ int last_row_at_or_before(const BwdParams& p, int blk_id, int x) {
  return last_key_at_or_before(p.mask, p.P, p.blk, p.rem, blk_id, x);
}
__device__ __forceinline__ int pos_of(const BwdParams& p, int blk_id, int row) {
  return token_pos(p.mask, p.P, p.blk, p.rem, blk_id, row);
}

// Per-lane byte offsets for the direct loads of one [rows][D] LDS tile of
// CPW 1 KB chunks per wave: chunk c covers LDS units [64c, 64c + 64); lane i
// writes unit 64c + i = (row, pos) and fetches global unit pos ^ swz(row).
// Matrix products by which an LDS operand read runs ahead of its use (the
// products of each phase are issued in a fixed order).
constexpr int kReadAhead = 3;

template <int D, int CPW>
__device__ __forceinline__ void tile_offsets(int wave, int lane, int row_stride, int (&off)[CPW]) {
  constexpr int UPR = D / 8;
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const int u = (wave * CPW + j) * 64 + lane;
    const int lrow = u / UPR;
    const int gunit = (u % UPR) ^ swz<D>(lrow);
    off[j] = (lrow * row_stride + gunit * 8) * 2;
  }
}

// Request rows [row0, row0 + R) of a row-major matrix (rows of D bf16, stride
// sr elements) into an LDS tile; rows past n re-read row n - 1.
template <int D, int CPW, int R>
__device__ __forceinline__ void issue_rows(const __bf16* base, int sr, const int (&off)[CPW], int row0, int n,
                                           __bf16* tile, int wave, int lane) {
  constexpr int UPR = D / 8;
  __bf16* dst = tile + wave * CPW * 512;
  if (row0 + R <= n) {
    const u32x4 rs = rsrc_words(base + (int64_t)row0 * sr);
#pragma unroll
    for (int j = 0; j < CPW; ++j) bload_lds16(rs, off[j], lds_addr(dst + j * 512));
  } else {
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      const int u = (wave * CPW + j) * 64 + lane;
      const int lrow = u / UPR;
      const int gunit = (u % UPR) ^ swz<D>(lrow);
      const int64_t g = min(row0 + lrow, n - 1);
      gload_lds16(base + g * sr + gunit * 8, lds_addr(dst + j * 512));
    }
  }
}

// LDS element offsets of the transposed (A-operand) reads of a [rows][D] tile:
// two 4-row runs per operand, in the key order the accumulator layout holds.
template <int D>
__device__ __forceinline__ void tr_offsets(int lane, int (&rd)[2][D / 32]) {
  const int lg = lane >> 5;
  const int vr = 4 * lg + ((lane & 15) >> 2);
  const int vx = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
  for (int run = 0; run < 2; ++run) {
    const int rr = vr + 8 * run;
    const int y = vx ^ swz<D>(rr);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) rd[run][db] = rr * D + (((4 * db) ^ y) << 3) + 4 * (lane & 1);
  }
}

// The transposed A operand for rows [16c, 16c + 16) of a tile and d block db.
__device__ __forceinline__ bf16x8 tr_operand(const __bf16* rows16, int off0, int off1) {
  const s16x4 t0 = lds_tr16(rows16 + off0);
  const s16x4 t1 = lds_tr16(rows16 + off1);
  const u32x2 w0 = __builtin_bit_cast(u32x2, t0);
  const u32x2 w1 = __builtin_bit_cast(u32x2, t1);
  const u32x4 aw = {w0[0], w0[1], w1[0], w1[1]};
  return __builtin_bit_cast(bf16x8, aw);
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per 32 NW query rows of one resident block.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(D >= 256 ? 1 : 2)))
void bwd_dq_kernel(const BwdParams p) {
  constexpr int TK = 32;
  constexpr int NC = D / 16;
  constexpr int NDB = D / 32;
  constexpr int TE = TK * D;
  constexpr int CPW = TE / 512 / NW;
  constexpr int QT = NW * 32;
  static_assert(CPW >= 1 && TE % (512 * NW) == 0, "tile must split into whole 1 KB chunks per wave");
  __shared__ __attribute__((aligned(1024))) __bf16 lds[2 * 2 * TE];  // [buffer][K | V][TK][D]

  const int tiles_q = (p.q_rows + QT - 1) / QT;
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

  const int q_len = p.q_len[r], kv_len = p.kv_len[r];
  if (qt * QT >= q_len) return;

  // Keys [0, kv_vis) are visible to some row of the workgroup, [0, kv_all) to
  // all of them; key c is visible to this lane's row iff c <= lim.
  int kv_vis = kv_len, kv_all = kv_len;
  int lim = kv_len - 1;
  if (p.mask != kMaskNone) {
    const int qb = p.q_blk[r], kb = p.kv_blk[r];
    const int q_first = qt * QT, q_last = min(q_first + QT, q_len) - 1;
    kv_vis = last_row_at_or_before(p, kb, pos_of(p, qb, q_last)) + 1;
    kv_all = last_row_at_or_before(p, kb, pos_of(p, qb, q_first)) + 1;
    lim = min(lim, last_row_at_or_before(p, kb, pos_of(p, qb, min(q_first + wave * 32 + lr, q_len - 1))));
    if (kv_vis == 0 && p.flags == (kLoadState | kStoreState)) return;  // nothing to add
  }

  const int row = qt * QT + wave * 32 + lr;
  const bool row_ok = row < q_len;
  const int64_t srow = p.q_row0[r] + (row_ok ? row : q_len - 1);
  const int64_t st_row = ((int64_t)bi * p.H + hi) * p.st_bh + srow;

  bf16x8 qf[NC], df[NC];
  {
    const __bf16* qp = (const __bf16*)p.q + bi * p.q_sb + hi * p.q_sh + srow * p.q_sr + 8 * lg;
    const __bf16* dp = (const __bf16*)p.dout + bi * p.do_sb + hi * p.do_sh + srow * p.do_sr + 8 * lg;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      qf[c] = *(const bf16x8*)(qp + 16 * c);
      df[c] = *(const bf16x8*)(dp + 16 * c);
    }
  }
  const float nl2 = p.nl2[st_row];
  const float ddv = p.dd[st_row];

  // dQ^T / s of this wave's 32 rows: lane (row, half) holds d columns
  // 32 db + 8 (e / 4) + 4 half + e % 4.
  f32x16 acc[NDB];
  if (p.flags & kLoadState) {
    const float* arow = p.dq_acc + st_row * D + 4 * lg;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 t = *(const f32x4*)(arow + 32 * db + 8 * j);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[db][4 * j + e] = t[e];
      }
  } else {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[db][i] = 0.0f;
  }

  const __bf16* kbase = (const __bf16*)p.k + bi * p.k_sb + hi * p.k_sh + p.k_off[r];
  const __bf16* vbase = (const __bf16*)p.v + bi * p.v_sb + hi * p.v_sh + p.v_off[r];
  const int k_sr = (int)p.k_sr, v_sr = (int)p.v_sr;
  const int n_plain = min(kv_all, kv_len) / TK;
  const int n_kt = (kv_vis + TK - 1) / TK;
  const float c2 = p.scale_log2;

  int ld_koff[CPW], ld_voff[CPW];
  tile_offsets<D, CPW>(wave, lane, k_sr, ld_koff);
  tile_offsets<D, CPW>(wave, lane, v_sr, ld_voff);
  auto issue_tile = [&](int kt, int buf) {
    __bf16* kl = lds + buf * 2 * TE;
    issue_rows<D, CPW, TK>(kbase, k_sr, ld_koff, kt * TK, kv_len, kl, wave, lane);
    issue_rows<D, CPW, TK>(vbase, v_sr, ld_voff, kt * TK, kv_len, kl + TE, wave, lane);
  };

  const int gk = lg ^ swz<D>(lr);
  int row_rd[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) row_rd[c] = lr * D + (((2 * c) ^ gk) << 3);
  int tr_rd[2][NDB];
  tr_offsets<D>(lane, tr_rd);

  auto tile = [&](int kt, int buf, bool masked) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile kt landed for this wave
    lds_barrier();                       // ... for every wave; the other buffer is free
    if (kt + 1 < n_kt) issue_tile(kt + 1, buf ^ 1);
    const __bf16* kl = lds + buf * 2 * TE;
    const __bf16* vl = kl + TE;
    f32x16 s = {}, dp = {};
    {  // S^T and dP^T chains interleaved; product i reads its K (even i) or V
       // (odd i) operand kReadAhead products ahead, in a fixed order
      constexpr int N = 2 * NC;
      auto rd = [&](int i) { return *(const bf16x8*)((i % 2 ? vl : kl) + row_rd[i / 2]); };
      bf16x8 a[kReadAhead];
#pragma unroll
      for (int i = 0; i < kReadAhead; ++i) a[i] = rd(i);
#pragma unroll
      for (int i = 0; i < N; ++i) {
        if (i % 2)
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i % kReadAhead], df[i / 2], dp, 0, 0, 0);
        else
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i % kReadAhead], qf[i / 2], s, 0, 0, 0);
        if (i + kReadAhead < N) a[i % kReadAhead] = rd(i + kReadAhead);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (masked) {
      const int lim_t = lim - kt * TK - 4 * lg;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (8 * (i >> 2) + (i & 3) > lim_t) s[i] = -INFINITY;
    }
    unsigned dsk[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s[2 * j], c2, nl2));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(s[2 * j + 1], c2, nl2));
      dsk[j] = pack_bf16(p0 * (dp[2 * j] - ddv), p1 * (dp[2 * j + 1] - ddv));
    }
    {  // dQ^T += K^T dS^T, transposed K operands read ahead in a fixed order
      constexpr int N = 2 * NDB;
      bf16x8 b[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) b[c] = __builtin_bit_cast(bf16x8, u32x4{dsk[4 * c], dsk[4 * c + 1], dsk[4 * c + 2], dsk[4 * c + 3]});
      auto rd = [&](int i) { return tr_operand(kl + 16 * (i / NDB) * D, tr_rd[0][i % NDB], tr_rd[1][i % NDB]); };
      bf16x8 a[kReadAhead];
#pragma unroll
      for (int i = 0; i < kReadAhead; ++i) a[i] = rd(i);
#pragma unroll
      for (int i = 0; i < N; ++i) {
        acc[i % NDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i % kReadAhead], b[i / NDB], acc[i % NDB], 0, 0, 0);
        if (i + kReadAhead < N) a[i % kReadAhead] = rd(i + kReadAhead);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  if (n_kt > 0) {
    issue_tile(0, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // Q, dO, the row statistics and tile 0, before the loop
    int kt = 0;
    for (; kt + 2 <= n_plain; kt += 2) {
      tile(kt, 0, false);
      tile(kt + 1, 1, false);
    }
    if (kt < n_plain) {
      tile(kt, 0, false);
      ++kt;
    }
    for (; kt < n_kt; ++kt) tile(kt, kt & 1, true);
  }

  if (!row_ok) return;
  if (p.flags & kWriteOut) {
    __bf16* orow = (__bf16*)p.dq + bi * p.dq_sb + hi * p.dq_sh + srow * p.dq_sr + 4 * lg;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 t;
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = (__bf16)(acc[db][4 * j + e] * p.scale);
        *(bf16x4*)(orow + 32 * db + 8 * j) = t;
      }
  } else if (p.flags & kStoreState) {
    float* arow = p.dq_acc + st_row * D + 4 * lg;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 t;
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = acc[db][4 * j + e];
        *(f32x4*)(arow + 32 * db + 8 * j) = t;
      }
  }
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per 32 NW keys of one visiting block.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(D >= 256 ? 1 : 2)))
void bwd_dkdv_kernel(const BwdParams p) {
  constexpr int TQ = 32;
  constexpr int NC = D / 16;
  constexpr int NDB = D / 32;
  constexpr int TE = TQ * D;
  constexpr int CPW = TE / 512 / NW;
  constexpr int KT = NW * 32;
  static_assert(CPW >= 1 && TE % (512 * NW) == 0, "tile must split into whole 1 KB chunks per wave");
  __shared__ __attribute__((aligned(1024))) __bf16 lds[2 * 2 * TE];  // [buffer][Q | dO][TQ][D]
  __shared__ __attribute__((aligned(16))) float lrow[2][2 * TQ];     // [buffer][nl2 of TQ rows | dd of TQ rows]
  __shared__ __attribute__((aligned(1024))) __bf16 vlds[KT * D];     // V rows of the workgroup's keys

  const int tiles_k = (p.kv_rows + KT - 1) / KT;
  const int total = tiles_k * p.n_res * p.H * p.B;
  int w = xcd_remap(blockIdx.x, total);
  const int kt = w % tiles_k;
  w /= tiles_k;
  const int r = w % p.n_res;
  w /= p.n_res;
  const int hi = w % p.H;
  const int bi = w / p.H;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lr = lane & 31;
  const int lg = lane >> 5;

  const int q_len = p.q_len[r], kv_len = p.kv_len[r];
  if (kt * KT >= kv_len) return;
  const int key = kt * KT + wave * 32 + lr;
  const bool key_ok = key < kv_len;
  const int ck = key_ok ? key : kv_len - 1;

  // Query rows [q_from, q_len) see some key of the workgroup, rows from q_all
  // on see all of them; this lane's key is seen by rows from fr on.
  int q_from = 0, q_all = 0, fr = 0;
  if (p.mask != kMaskNone) {
    const int qb = p.q_blk[r], kb = p.kv_blk[r];
    auto first_row = [&](int krow) { return last_row_at_or_before(p, qb, pos_of(p, kb, krow) - 1) + 1; };
    q_from = first_row(kt * KT);
    q_all = first_row(min(kt * KT + KT, kv_len) - 1);
    fr = first_row(ck);
    if (q_from >= q_len) return;  // no query of this block sees these keys
  }

  bf16x8 kf[NC];
  {
    const __bf16* kp = (const __bf16*)p.k + bi * p.k_sb + hi * p.k_sh + p.k_off[r] + (int64_t)ck * p.k_sr + 8 * lg;
#pragma unroll
    for (int c = 0; c < NC; ++c) kf[c] = *(const bf16x8*)(kp + 16 * c);
  }

  // dK^T / s and dV^T of this wave's 32 keys: lane (key, half) holds d
  // columns 32 db + 8 (e / 4) + 4 half + e % 4.
  const int64_t arow_i = ((int64_t)bi * p.H + hi) * p.acc_bh + p.acc_row0[r] + ck;
  f32x16 dk[NDB], dv[NDB];
  {
    const float* krow = p.dk_acc + arow_i * D + 4 * lg;
    const float* vrow = p.dv_acc + arow_i * D + 4 * lg;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 a = *(const f32x4*)(krow + 32 * db + 8 * j);
        const f32x4 b = *(const f32x4*)(vrow + 32 * db + 8 * j);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dk[db][4 * j + e] = a[e];
          dv[db][4 * j + e] = b[e];
        }
      }
  }

  const int64_t row0 = p.q_row0[r];
  const __bf16* qbase = (const __bf16*)p.q + bi * p.q_sb + hi * p.q_sh + row0 * p.q_sr;
  const __bf16* dbase = (const __bf16*)p.dout + bi * p.do_sb + hi * p.do_sh + row0 * p.do_sr;
  const int64_t rbase = ((int64_t)bi * p.H + hi) * p.st_bh + row0;
  const int q_sr = (int)p.q_sr, do_sr = (int)p.do_sr;
  const float c2 = p.scale_log2;

  int ld_qoff[CPW], ld_doff[CPW];
  tile_offsets<D, CPW>(wave, lane, q_sr, ld_qoff);
  tile_offsets<D, CPW>(wave, lane, do_sr, ld_doff);
  // nl2 (lanes 0-31) or dd (lanes 32-63) of this lane's row, chosen once here:
  // chosen inside the loop, the pointer was re-read from the kernel arguments
  // on every tile.
  const float* lrow_src = (lg == 0 ? p.nl2 : p.dd) + rbase;
  asm volatile("" : "+v"(lrow_src));
  auto issue_tile = [&](int qt, int buf) {
    __bf16* ql = lds + buf * 2 * TE;
    issue_rows<D, CPW, TQ>(qbase, q_sr, ld_qoff, qt * TQ, q_len, ql, wave, lane);
    issue_rows<D, CPW, TQ>(dbase, do_sr, ld_doff, qt * TQ, q_len, ql + TE, wave, lane);
    if (wave == 0)  // nl2 of the tile's rows into lrow[buf][0, TQ), dd into [TQ, 2 TQ)
      gload_lds4(lrow_src + min(qt * TQ + lr, q_len - 1), lds_addr(&lrow[buf][0]));
  };

  const int gq = lg ^ swz<D>(lr);
  int row_rd[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) row_rd[c] = lr * D + (((2 * c) ^ gq) << 3);
  int tr_rd[2][NDB];
  tr_offsets<D>(lane, tr_rd);

  const int n_qt = (q_len + TQ - 1) / TQ;
  const int qt0 = q_from / TQ;
  const int qt_plain = (q_all + TQ - 1) / TQ;  // tiles from here on are seen by every key ...
  const int n_full = q_len / TQ;               // ... up to the last whole tile

  auto tile = [&](int qt, int buf, bool masked) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile qt landed for this wave
    lds_barrier();                       // ... for every wave; the other buffer is free
    if (qt + 1 < n_qt) issue_tile(qt + 1, buf ^ 1);
    const __bf16* ql = lds + buf * 2 * TE;
    const __bf16* dl = ql + TE;
    f32x16 s = {}, dp = {};
    {  // S^T and dP^T chains interleaved in a fixed order, operands (Q for even
       // products; dO and the wave's V rows for odd ones) read kReadAhead ahead
      constexpr int N = 2 * NC;
      auto rd = [&](int i) { return *(const bf16x8*)((i % 2 ? dl : ql) + row_rd[i / 2]); };
      auto rdv = [&](int i) { return *(const bf16x8*)(vlds + wave * 32 * D + row_rd[i / 2]); };
      bf16x8 a[kReadAhead], bv[kReadAhead];
#pragma unroll
      for (int i = 0; i < kReadAhead; ++i) {
        a[i] = rd(i);
        if (i % 2) bv[i] = rdv(i);
      }
#pragma unroll
      for (int i = 0; i < N; ++i) {
        if (i % 2)
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i % kReadAhead], bv[i % kReadAhead], dp, 0, 0, 0);
        else
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i % kReadAhead], kf[i / 2], s, 0, 0, 0);
        if (i + kReadAhead < N) {
          a[i % kReadAhead] = rd(i + kReadAhead);
          if ((i + kReadAhead) % 2) bv[i % kReadAhead] = rdv(i + kReadAhead);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (masked) {
      const int rbase_t = qt * TQ + 4 * lg;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rq = rbase_t + 8 * (i >> 2) + (i & 3);
        if (rq < fr || rq >= q_len) s[i] = -INFINITY;
      }
    }
    // lane (key, half) holds query rows 8 (e / 4) + 4 half + e % 4 of the
    // tile: group j of 4 elements reads those rows' L and D as one float4.
    unsigned pk[8], dsk[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 nl = *(const f32x4*)(&lrow[buf][8 * j + 4 * lg]);
      const f32x4 dd = *(const f32x4*)(&lrow[buf][TQ + 8 * j + 4 * lg]);
      float pe[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) pe[e] = __builtin_amdgcn_exp2f(fmaf(s[4 * j + e], c2, nl[e]));
      pk[2 * j] = pack_bf16(pe[0], pe[1]);
      pk[2 * j + 1] = pack_bf16(pe[2], pe[3]);
      dsk[2 * j] = pack_bf16(pe[0] * (dp[4 * j] - dd[0]), pe[1] * (dp[4 * j + 1] - dd[1]));
      dsk[2 * j + 1] = pack_bf16(pe[2] * (dp[4 * j + 2] - dd[2]), pe[3] * (dp[4 * j + 3] - dd[3]));
    }
    {  // dV^T += dO^T P^T and dK^T += Q^T dS^T interleaved, transposed
       // operands read ahead in a fixed order
      constexpr int N = 4 * NDB;
      bf16x8 pw[2], sw[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        pw[c] = __builtin_bit_cast(bf16x8, u32x4{pk[4 * c], pk[4 * c + 1], pk[4 * c + 2], pk[4 * c + 3]});
        sw[c] = __builtin_bit_cast(bf16x8, u32x4{dsk[4 * c], dsk[4 * c + 1], dsk[4 * c + 2], dsk[4 * c + 3]});
      }
      // product i: rows 16 c (c = i / (2 NDB)), d block (i / 2) % NDB, dV (even) or dK (odd)
      auto rd = [&](int i) {
        const int c = i / (2 * NDB), db = (i / 2) % NDB;
        return tr_operand((i % 2 ? ql : dl) + 16 * c * D, tr_rd[0][db], tr_rd[1][db]);
      };
      bf16x8 a[kReadAhead];
#pragma unroll
      for (int i = 0; i < kReadAhead; ++i) a[i] = rd(i);
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int c = i / (2 * NDB), db = (i / 2) % NDB;
        if (i % 2)
          dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i % kReadAhead], sw[c], dk[db], 0, 0, 0);
        else
          dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i % kReadAhead], pw[c], dv[db], 0, 0, 0);
        if (i + kReadAhead < N) a[i % kReadAhead] = rd(i + kReadAhead);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  if (qt0 < n_qt) {
    {  // the workgroup's V rows, swizzled like the tiles, in 32-row pieces (so the
       // byte offsets from each piece's first row stay below 2^31); they land
       // with the first tile
      const __bf16* vb = (const __bf16*)p.v + bi * p.v_sb + hi * p.v_sh + p.v_off[r];
      const int v_sr = (int)p.v_sr;
      int ld_voff[CPW];
      tile_offsets<D, CPW>(wave, lane, v_sr, ld_voff);
#pragma unroll
      for (int i = 0; i < KT / TQ; ++i)
        issue_rows<D, CPW, TQ>(vb, v_sr, ld_voff, kt * KT + i * TQ, kv_len, vlds + i * TE, wave, lane);
    }
    issue_tile(qt0, qt0 & 1);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // K, V, the V rows and tile qt0, before the loop
    for (int qt = qt0; qt < n_qt; ++qt) tile(qt, qt & 1, qt < qt_plain || qt >= n_full);
  }

  if (!key_ok) return;
  float* krow = p.dk_acc + arow_i * D + 4 * lg;
  float* vrow = p.dv_acc + arow_i * D + 4 * lg;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x4 a, b;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[e] = dk[db][4 * j + e];
        b[e] = dv[db][4 * j + e];
      }
      *(f32x4*)(krow + 32 * db + 8 * j) = a;
      *(f32x4*)(vrow + 32 * db + 8 * j) = b;
    }
}

}  // namespace

// Waves per workgroup of the d-specialised backward kernels.
constexpr int bwd_waves(int d) { return d == 128 ? 8 : 4; }

hipError_t launch_bwd_dq_bf16(const BwdParams& p, int d, hipStream_t s) {
  const int64_t grid = (int64_t)((p.q_rows + bwd_waves(d) * 32 - 1) / (bwd_waves(d) * 32)) * p.n_res * p.H * p.B;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 gd((unsigned)grid), bd(bwd_waves(d) * 64);
  switch (d) {
    case 64:
      bwd_dq_kernel<64, bwd_waves(64)><<<gd, bd, 0, s>>>(p);
      break;
    case 128:
      bwd_dq_kernel<128, bwd_waves(128)><<<gd, bd, 0, s>>>(p);
      break;
    case 256:
      bwd_dq_kernel<256, bwd_waves(256)><<<gd, bd, 0, s>>>(p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_bf16(const BwdParams& p, int d, hipStream_t s) {
  const int64_t grid = (int64_t)((p.kv_rows + bwd_waves(d) * 32 - 1) / (bwd_waves(d) * 32)) * p.n_res * p.H * p.B;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 gd((unsigned)grid), bd(bwd_waves(d) * 64);
  switch (d) {
    case 64:
      bwd_dkdv_kernel<64, bwd_waves(64)><<<gd, bd, 0, s>>>(p);
      break;
    case 128:
      bwd_dkdv_kernel<128, bwd_waves(128)><<<gd, bd, 0, s>>>(p);
      break;
    case 256:
      bwd_dkdv_kernel<256, bwd_waves(256)><<<gd, bd, 0, s>>>(p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ra
