// bf16 fold kernel for wide heads (d = 256) on gfx950: 16 query rows per wave.
//
// Math as in the 32-row kernel (aicassindra.com "Ring Attention, math", the
// per-query pseudo-code under the online-softmax identity): per query row,
// s = q.k * scale, m' = max(m, max s), alpha = exp(m - m'),
// l' = alpha l + sum exp(s - m'), o' = alpha o + sum exp(s - m') v.
//
// Why a second kernel: with 32 rows per wave and d = 256 the wave's Q operand
// (64 registers) and o accumulators (128) leave no room for two waves per
// SIMD, so the matrix cores idle whenever the one wave does its softmax.  With
// 16 rows per wave on v_mfma_f32_16x16x32_bf16 the same state takes half the
// registers and two waves share each SIMD.  The price is one 1 KB operand read
// from LDS per 16 K-FLOP product instead of per 32 K-FLOP; at d = 256 every
// score carries twice the products of d = 128, so the softmax work per product
// is half that of the d = 128 kernel.
//
// Mapping (lane l, row lr = l % 16 of the wave's 16, lane group lg = l / 16):
//  * Scores transposed, S^T = K Q^T: the accumulator of a 16-key block holds
//    in lane l the scores of keys 4 lg .. 4 lg + 3 against query row lr; the
//    other 12 keys of the block sit in lanes l ^ 16, l ^ 32, l ^ 48, so the row
//    max and row sum take one v_permlane16_swap and one v_permlane32_swap.
//  * Q is the B operand: lane l holds q[lr][32 c + 8 lg .. + 7] for d chunk c.
//  * Two 16-key score blocks, rounded to bf16, are directly the B operand of
//    O^T += V^T P^T over 32 keys, with the contraction running over the keys
//    in the order the accumulators hold them; the matching V^T operand is two
//    ds_read_b64_tr_b16 of four consecutive keys each from row-major V.
//  * K and V tiles stream through a ring of NB LDS buffers, filled straight
//    from global memory (buffer_load ... lds) NB - 1 tiles ahead; the 16-byte
//    units of each row are XOR swizzled so that neither the transposed V reads
//    (8 rows of two adjacent units per 32 lanes, swz16 below) nor the K reads
//    (16 rows of one unit per 16 lanes, swz16_k below) meet a bank conflict.
//  * Within a tile the matrix products run in a fixed order, each LDS operand
//    read a few products ahead of its use; a wave's two phases (scores, then
//    softmax and value products) overlap the other wave of its SIMD.
//  * exp2 with log2(e) folded into the scale, l from the bf16-rounded weights,
//    the lazy reference maximum, causal tile skipping and masking, and the
//    XCD-aware workgroup order are those of the 32-row kernel.
#include <math.h>

#include "bf16_common.h"
#include "kernels.h"

namespace ra {
namespace {

using namespace dev;

constexpr float kLazy = 8.0f;
// Matrix products by which an LDS operand read runs ahead of its use.
constexpr int kReadAhead = 4;

// XOR swizzle of the low four bits of a 16-byte unit index in row r: a
// bijection on 16 consecutive rows, and for 8 consecutive rows aligned to 8 it
// keeps bit 0 constant while bits 1..3 run through all values, so two adjacent
// units of those rows land on 16 distinct bank groups (the V^T reads).
__device__ __forceinline__ int swz16(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

// Row swizzle of the K tile.  gfx950 serves a ds_read_b128 in four groups of
// 16 lanes, lanes l and l' sharing a group when bit 5 and the parity of bits
// 2..4 of l and l' agree (measured: a read costs one pass per group exactly
// when no two lanes of a group touch the same 16-byte bank group).  A K read
// puts row lr = l % 16 and unit 4 e + l / 16 on lane l, so a group holds
// every row once, with bit 0 of its unit index flipped by bits 2 ^ 3 of the
// row; XORing that parity into swz16 makes the group's 16 bank groups distinct
// (with swz16 alone they pair up: two passes per group).
__device__ __forceinline__ int swz16_k(int r) { return swz16(r) ^ (((r >> 2) ^ (r >> 3)) & 1); }

// Buffer resource words over `base` (no effective range limit; every access is
// computed in bounds by the kernel), held in scalar registers.
__device__ __forceinline__ u32x4 rsrc_words(const void* base) {
  const uint64_t a = (uint64_t)base;
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)a);
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)(a >> 32) & 0xffffu);
  return u32x4{lo, hi, 0x7fffffffu, 0x00020000u};
}

// 16 bytes per lane at byte offset voff of the buffer straight into LDS at
// byte address lds_addr + 16 lane (buffer_load_dwordx4 ... lds; M0 holds the
// LDS address).  Issued from inline assembly so that the compiler, which cannot
// tell which LDS bytes such a load writes, does not make every later LDS read
// wait for it; the tile loop waits for the loads itself (s_waitcnt vmcnt, then
// a barrier) before any wave reads them.  The instruction has no destination
// registers.  M0 is an operand of the statement ("{m0}"), so the compiler
// writes it and knows it is taken; the s_nop is the wait state the hardware
// needs between an SALU write of M0 and an LDS-direct load that reads it.
__device__ __forceinline__ void dma16(u32x4 rsrc, int voff, unsigned lds_addr) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "{m0}"(lds_addr)
               : "memory");
}

// s_waitcnt immediate that waits until at most n vector memory loads are
// outstanding (the other counters unconstrained).
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

template <int D, int NW, int TK, int NB>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void fold_bf16_r16_kernel(const FoldParams p) {
  constexpr int NKB = TK / 16;  // 16-key score blocks per tile
  constexpr int NPV = TK / 32;  // 32-key value products per tile
  constexpr int NC = D / 32;    // 32-wide d chunks of the score product
  constexpr int NDB = D / 16;   // 16-wide d blocks of o
  constexpr int UPR = D / 8;    // 16-byte units per K / V row
  constexpr int TE = TK * D;    // elements of one K (or V) tile
  constexpr int CPW = TE / 512 / NW;
  constexpr int QT = NW * 16;  // query rows per workgroup
  static_assert(D >= 128 && D % 128 == 0, "swizzle and unit split assume rows of 16 units or more");
  static_assert(CPW >= 1 && TE % (512 * NW) == 0, "tile must split into whole 1 KB chunks per wave");
  static_assert(NKB % 2 == 0, "value products take two score blocks");
  static_assert(NB >= 2 && (NB - 2) * 2 * CPW < 64, "buffer ring depth");
  __shared__ __attribute__((aligned(1024))) __bf16 lds[NB * 2 * TE];

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
  const int lr = lane & 15;
  const int lg = lane >> 4;

  const int q_len = p.q_len[r], kv_len = p.kv_len[r];
  if (qt * QT >= q_len) return;

  // Keys [0, kv_vis) are visible to some row of this workgroup, keys
  // [0, kv_all) to every row; key c is visible to this lane's row iff c <= lim.
  int kv_vis = kv_len, kv_all = kv_len;
  int lim = kv_len - 1;
  if (p.mask != kMaskNone) {
    const int qb = p.q_blk[r], kb = p.kv_blk[r];
    const int q_first = qt * QT, q_last = min(q_first + QT, q_len) - 1;
    auto last_key = [&](int qrow) {
      return last_key_at_or_before(p.mask, p.P, p.blk, p.rem, kb, token_pos(p.mask, p.P, p.blk, p.rem, qb, qrow));
    };
    kv_vis = last_key(q_last) + 1;
    kv_all = last_key(q_first) + 1;
    lim = min(lim, last_key(min(q_first + wave * 16 + lr, q_len - 1)));
    if (kv_vis == 0 && (p.flags & ~kRefState) == (kLoadState | kStoreState)) return;
  }

  const int row = qt * QT + wave * 16 + lr;
  const bool row_ok = row < q_len;
  const int64_t srow = (int64_t)p.q_row0[r] + (row_ok ? row : q_len - 1);
  const int64_t st_row = ((int64_t)bi * p.H + hi) * p.st_bh + srow;

  const __bf16* kbase = (const __bf16*)p.k + bi * p.k_sb + hi * p.k_sh + p.k_off[r];
  const __bf16* vbase = (const __bf16*)p.v + bi * p.v_sb + hi * p.v_sh + p.v_off[r];
  const int n_plain = min(kv_all, kv_len) / TK;
  const int n_kt = (kv_vis + TK - 1) / TK;
  const float c2 = p.scale_log2;

  // Direct loads: chunk j of this wave is LDS units [64 (wave CPW + j), +64);
  // lane i writes unit u = (row, pos) and fetches global unit pos ^ swz16_k(row)
  // of K, pos ^ swz16(row) of V.
  const int k_sr = (int)p.k_sr, v_sr = (int)p.v_sr;
  int ld_koff[CPW], ld_voff[CPW];
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const int u = (wave * CPW + j) * 64 + lane;
    const int lrow = u / UPR;
    ld_koff[j] = (lrow * k_sr + ((u % UPR) ^ swz16_k(lrow)) * 8) * 2;
    ld_voff[j] = (lrow * v_sr + ((u % UPR) ^ swz16(lrow)) * 8) * 2;
  }
  // LDS byte address of this wave's first chunk in buffer 0 (wave-uniform).
  const unsigned lds_wave = (unsigned)__builtin_amdgcn_readfirstlane(
      (unsigned)(size_t)(__attribute__((address_space(3))) __bf16*)lds + wave * CPW * 1024);
  auto issue_tile = [&](int kt, int buf) {
    const int key0 = kt * TK;
    const unsigned kl = lds_wave + buf * 4 * TE;  // bytes
    const unsigned vl = kl + 2 * TE;
    const u32x4 kr = rsrc_words(kbase + (int64_t)key0 * k_sr);
    const u32x4 vr = rsrc_words(vbase + (int64_t)key0 * v_sr);
    if (key0 + TK <= kv_len) {
#pragma unroll
      for (int j = 0; j < CPW; ++j) {
        dma16(kr, ld_koff[j], kl + j * 1024);
        dma16(vr, ld_voff[j], vl + j * 1024);
      }
    } else {  // ragged last tile: rows past the end re-read the last row
#pragma unroll
      for (int j = 0; j < CPW; ++j) {
        const int u = (wave * CPW + j) * 64 + lane;
        const int lrow = u / UPR;
        const int rr = min(lrow, kv_len - 1 - key0);
        dma16(kr, (rr * k_sr + ((u % UPR) ^ swz16_k(lrow)) * 8) * 2, kl + j * 1024);
        dma16(vr, (rr * v_sr + ((u % UPR) ^ swz16(lrow)) * 8) * 2, vl + j * 1024);
      }
    }
  };

  // Tile 0 is requested before Q and the state, so the three loads' latencies
  // overlap.
  if (n_kt > 0) issue_tile(0, 0);

  bf16x8 qf[NC];
  {
    const __bf16* qp = (const __bf16*)p.q + bi * p.q_sb + hi * p.q_sh + srow * p.q_sr + 8 * lg;
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[c] = *(const bf16x8*)(qp + 32 * c);
  }

  // mref: the reference maximum the weights are taken against (base-2 units
  // of the scaled score), trailing the true running maximum mtrue by less than
  // kLazy; o and l are brought to mtrue once, before they are stored.
  float mref, mtrue, lpart, m_in;
  f32x4 oacc[NDB];
  if (p.flags & kLoadState) {
    m_in = p.m[st_row];
    mref = m_in * kLog2e;
    lpart = lg == 0 ? p.l[st_row] : 0.0f;
    const float* orow = p.o + st_row * D + 4 * lg;
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = *(const f32x4*)(orow + 16 * db);
  } else {
    m_in = -INFINITY;
    mref = -INFINITY;
    lpart = 0.0f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  mtrue = mref;

  // K operand of chunk c = 4 h + e (global unit 16 h + 4 e + lg of row lr):
  // LDS element lr D + 128 h + (((4 e + lg) ^ swz16_k(lr)) << 3).
  const int ks = swz16_k(lr);
  int k_rd[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) k_rd[e] = lr * D + (((4 * e + lg) ^ ks) << 3);
  // V^T operand of d block db = 8 h + e: lane 4 r0 + cc of its 16-lane group
  // reads key 4 lg + r0 (plus the run's offset), elements 16 db + 4 cc .. + 3,
  // i.e. half cc & 1 of global unit 2 db + (cc >> 1).
  const int vrow = 4 * lg + ((lane & 15) >> 2);
  const int cc = lane & 3;
  const int vs = swz16(vrow);
  int v_rd[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v_rd[e] = vrow * D + (((2 * e + (cc >> 1)) ^ vs) << 3) + 4 * (cc & 1);

  // Products are issued in a fixed order (scheduling barriers), each K
  // operand read kReadAhead products before its use.
  auto scores = [&](f32x4 (&s)[NKB], const __bf16* kl) {
    constexpr int N = NC * NKB;
    auto rd = [&](int i) {  // product i: d chunk i / NKB, key block i % NKB
      const int c = i / NKB, kb = i % NKB;
      return *(const bf16x8*)(kl + 16 * kb * D + 128 * (c >> 2) + k_rd[c & 3]);
    };
    bf16x8 a[kReadAhead];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < kReadAhead; ++i) a[i] = rd(i);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      s[i % NKB] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i % kReadAhead], qf[i / NKB], s[i % NKB], 0, 0, 0);
      if (i + kReadAhead < N) a[i % kReadAhead] = rd(i + kReadAhead);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Keys past this row's last visible key score -inf.
  auto mask = [&](f32x4 (&s)[NKB], int key0) {
    const int lim_t = lim - key0 - 4 * lg;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (16 * kb + i > lim_t) s[kb][i] = -INFINITY;
  };
  // Row maximum of the tile; raises mtrue, and mref when it falls more than
  // kLazy below the new maximum (then o and l are rescaled here).
  auto track_max = [&](const f32x4 (&s)[NKB]) {
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[kb][i]);
    const float mt = quad_max(mx) * c2;
    mtrue = fmaxf(mtrue, mt);
    const bool fresh = mref == -INFINITY;
    const bool raise = !fresh && mt > mref + kLazy;
    if (fresh) mref = mt;
    if (__builtin_amdgcn_ballot_w64(raise)) {
      const float alpha = raise ? __builtin_amdgcn_exp2f(mref - mt) : 1.0f;
      if (raise) mref = mt;
      lpart *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
    }
  };
  auto weights = [&](const f32x4 (&s)[NKB], unsigned (&pk)[NKB][2]) {
    const float mr = mref == -INFINITY ? 0.0f : mref;
    float lsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][2 * j], c2, -mr));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][2 * j + 1], c2, -mr));
        pk[kb][j] = pack_bf16(p0, p1);
        lsum = sum_bf16_pair(pk[kb][j], lsum);
      }
    lpart += lsum;
  };
  // Same fixed order for the value products, each V^T operand (two
  // transposed reads) read kReadAhead products ahead.
  auto values = [&](const unsigned (&pk)[NKB][2], const __bf16* vl) {
    constexpr int N = NPV * NDB;
    auto rd = [&](int i) {  // product i: key run pair i / NDB, d block i % NDB
      const int m = i / NDB, db = i % NDB;
      const __bf16* v0 = vl + 32 * m * D + 128 * (db >> 3) + v_rd[db & 7];
      const u32x2 w0 = __builtin_bit_cast(u32x2, lds_tr16(v0));
      const u32x2 w1 = __builtin_bit_cast(u32x2, lds_tr16(v0 + 16 * D));
      return __builtin_bit_cast(bf16x8, u32x4{w0[0], w0[1], w1[0], w1[1]});
    };
    bf16x8 b[NPV];
#pragma unroll
    for (int m = 0; m < NPV; ++m)
      b[m] = __builtin_bit_cast(bf16x8, u32x4{pk[2 * m][0], pk[2 * m][1], pk[2 * m + 1][0], pk[2 * m + 1][1]});
    bf16x8 a[kReadAhead];
#pragma unroll
    for (int i = 0; i < kReadAhead; ++i) a[i] = rd(i);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      oacc[i % NDB] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i % kReadAhead], b[i / NDB], oacc[i % NDB], 0, 0, 0);
      if (i + kReadAhead < N) a[i % kReadAhead] = rd(i + kReadAhead);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Tile kt sits in buffer buf; tiles up to kt + NB - 2 have been requested.
  // With `deep`, tiles kt + 1 .. kt + NB - 2 are all in flight behind it, so
  // waiting until that many tiles' loads remain outstanding means tile kt has
  // landed; near the end of the block everything is waited for.  The barrier
  // then makes the tile visible to every wave and frees the buffer of tile
  // kt - 1, which receives tile kt + NB - 1.
  auto tile = [&](int kt, int buf, bool masked, bool deep) {
    if (deep)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm((NB - 2) * 2 * CPW));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    if (kt + NB - 1 < n_kt) issue_tile(kt + NB - 1, buf == 0 ? NB - 1 : buf - 1);
    const __bf16* kc = lds + buf * 2 * TE;
    const __bf16* vc = kc + TE;
    f32x4 sa[NKB];
    unsigned pa[NKB][2];
    scores(sa, kc);
    if (masked) mask(sa, kt * TK);
    track_max(sa);
    weights(sa, pa);
    values(pa, vc);
  };

  // Q, the state and tile 0 land before the tile loop, so the compiler's own
  // waits for Q and the state stay outside it (inside, they would also wait
  // for the tile loads the compiler does not see).  Tile 0 was issued before
  // them, so those waits are never too short.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  if (n_kt > 0) {
#pragma unroll
    for (int t = 1; t < NB - 1; ++t)
      if (t < n_kt) issue_tile(t, t);
    // Full-depth, unmasked tiles in groups of NB (compile-time buffers), then
    // the rest one by one.
    int kt = 0;
    for (; kt + NB <= n_plain && kt + 2 * NB - 2 <= n_kt; kt += NB) {
#pragma unroll
      for (int u = 0; u < NB; ++u) tile(kt + u, u, false, true);
    }
    for (; kt < n_kt; ++kt) tile(kt, kt % NB, kt >= n_plain, kt + NB - 1 <= n_kt);
  }

  // Bring (l, o) from the reference maximum to the true running maximum.
  const float fix = mref == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(mref - mtrue);
  const float l_tot = quad_sum(lpart) * fix;
  if (!row_ok) return;
  if (p.flags & kWriteOut) {
    // (o fix) (1 / l): the stored state, then ra_finalize's normalisation
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    if (p.lse != nullptr && lg == 0) p.lse[st_row] = l_tot > 0.0f ? (mtrue + __log2f(l_tot)) * kLn2 : -INFINITY;
    __bf16* orow = (__bf16*)p.out + bi * p.out_sb + hi * p.out_sh + srow * p.out_sr + 4 * lg;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      bf16x4 t;
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] = (__bf16)((oacc[db][e] * fix) * inv);
      *(bf16x4*)(orow + 16 * db) = t;
    }
  }
  if (p.flags & kStoreState) {
    if (lg == 0) {
      // A maximum that did not rise is stored exactly as it was loaded.
      p.m[st_row] = mtrue == m_in * kLog2e ? m_in : mtrue * kLn2;
      p.l[st_row] = l_tot;
    }
    float* orow = p.o + st_row * D + 4 * lg;
#pragma unroll
    for (int db = 0; db < NDB; ++db) *(f32x4*)(orow + 16 * db) = oacc[db] * fix;
  }
}

// Workgroup shape of the 16-row kernel: 8 waves (128 query rows, two waves per
// SIMD), 32-key tiles, three K/V buffers (96 KB of LDS).  The shape leaves
// registers and LDS on each CU for the hand-off copies that run beside the
// fold; four buffers or 64-key tiles fold slightly faster but crowd them out.
constexpr int kR16Waves = 8;
constexpr int kR16Keys = 32;
constexpr int kR16Bufs = 3;

}  // namespace

hipError_t launch_fold_bf16_r16(const FoldParams& p, int d, hipStream_t s) {
  const int64_t tiles_q = (p.q_rows + kR16Waves * 16 - 1) / (kR16Waves * 16);
  const int64_t grid = tiles_q * p.n_res * p.H * p.B;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 gd((unsigned)grid), bd(kR16Waves * 64);
  switch (d) {
    case 256:
      fold_bf16_r16_kernel<256, kR16Waves, kR16Keys, kR16Bufs><<<gd, bd, 0, s>>>(p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ra
