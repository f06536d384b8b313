// bf16 fold kernel for gfx950: one launch folds one visiting K/V block into the
// running (m, l, o) state of every resident query row.
//
// Math (aicassindra.com "Ring Attention, math", the per-query pseudo-code under
// the online-softmax identity; bembew.net "Conceptual Algorithm"): per query row,
// s = q.k * scale, m' = max(m, max s), alpha = exp(m - m'),
// l' = alpha l + sum exp(s - m'), o' = alpha o + sum exp(s - m') v.
//
// Mapping onto CDNA4:
//  * A workgroup is NW waves (8 for d = 128, 4 for d = 64 and 256); each wave
//    owns 32 query rows, so a workgroup owns a 32 NW-row query tile, and every
//    K/V tile brought into LDS (and through L2) serves all of them.  With 8
//    waves one workgroup fills a CU at two waves per SIMD; at d = 256 the 32
//    rows' Q and o take 192 registers, so two 4-wave workgroups share a CU
//    (measured faster on a 1024-key visiting block than one 8-wave workgroup:
//    while one loads or stores its state the other computes).  Q stays in
//    registers as MFMA operands for the whole launch; the state (m, l, o) is
//    loaded once, kept in registers while the visiting block streams past, and
//    stored once (or normalised and written as the output on the last ring
//    step).
//  * The visiting block streams through two LDS buffers in 64-key tiles (32
//    at d = 256): K and V row-major, the 16-byte units of each row
//    XOR-swizzled (d = 256: rows padded) so both read patterns below are free
//    of bank conflicts, filled straight from global memory by
//    buffer_load ... lds while the other buffer is in use.
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
//  * The weights are taken against a reference maximum that is raised only
//    when a tile's maximum exceeds it by more than kLazy (base 2; the identity holds
//    for any constant), so o is almost never rescaled inside the loop; the true
//    running maximum is tracked alongside and (l, o) are brought to it before
//    they are stored.
//  * Workgroup ids are remapped so that consecutive query tiles of one
//    (batch, head, resident block) -- which read the same K/V -- land on the
//    same XCD and share its L2.
//  * The ring's hand-off (math page, "The ring schedule": a device passes the
//    block it holds on to the next device) can ride on the fold: with
//    p.send_k set, each workgroup of a resident writes every n_qt-th tile of
//    the visiting block back out of LDS into the slot the next resident
//    reads at the next step, so the block moves without being read again.
//  * Causal masking (math page, "Causal masking, load balance, and other
//    wrinkles"): positions rise with the row index in every token layout, so
//    the keys a query tile can see are a prefix of the visiting block.  Tiles
//    past that prefix are never loaded, tiles every row of the workgroup sees
//    run unmasked, and only the few tiles in between compare each key with the
//    row's last visible key.
#include <math.h>

#include "bf16_common.h"
#include "kernels.h"

namespace ra {
namespace {

using namespace dev;

// Lazy rescaling threshold (base-2 units): weights stay below 2^kLazy.
constexpr float kLazy = 8.0f;
// With the reference state (kRefState), a tile's weights are first taken
// against the current reference without looking at the tile's maximum.  A
// lane's 32 weights summing to at most 2^kLazy bounds each of them by 2^kLazy,
// as the maximum test would; a larger sum (some weight above 2^kLazy / 32 =
// 2^(kLazy - 5)) sends the wave through the maximum, a raise of the reference
// for the rows whose maximum exceeds it by more than kLazy - 5, and the
// weights again.
constexpr float kRefSum = 256.0f;  // 2^kLazy
constexpr float kRefRaise = 3.0f;  // kLazy - 5

// Matrix products by which an LDS operand read runs ahead of its use.
constexpr int kReadAhead = 2;

// LDS layout of one K/V tile (K region, then V region; two such buffers).
//  * d = 64, 128: 64-key tiles, rows of d elements, the 16-byte units of each
//    row XOR-swizzled (swz); every read pattern is conflict-free and each
//    operand read has its own per-lane offset.
//  * d = 256: 32-key tiles (the o accumulators and Q of 32 rows take 192
//    registers, so the scores of one 32-key block are all that fit beside
//    them), rows padded instead of swizzled: a K row is 33 units, so a
//    16-lane group of a K read (16 rows, one unit each) meets 16 bank groups;
//    a V row is 36 units (four units of padding shift each row by a quarter
//    of the 64 banks), so the 32 lanes of a transposed V read (4 rows x 4
//    units x 2 halves) meet all 64 banks once.  Every operand read of a wave
//    is then one per-lane address plus an immediate offset, which keeps the
//    kernel within 256 registers.
//  Tiles are filled in whole 1 KB chunks (64 lanes x 16 bytes); in the padded
//  layout the lanes that land on padding, or past the last row, fetch a copy
//  of a valid unit.
template <int D>
struct TileLayout {
  static constexpr bool kPad = D == 256;
  static constexpr int kKeys = kPad ? 32 : 64;
  static constexpr int kKRow = kPad ? D + 8 : D;   // K row stride (elements)
  static constexpr int kVRow = kPad ? D + 32 : D;  // V row stride (elements)
  static constexpr int kKChunks = (kKeys * kKRow + 511) / 512;
  static constexpr int kVChunks = (kKeys * kVRow + 511) / 512;
  static constexpr int kKElems = kKChunks * 512;
  static constexpr int kBufElems = kKElems + kVChunks * 512;
};

// ---------------------------------------------------------------------------
// Per tile: wait for it, request the next one into the other buffer, scores,
// maximum tracking, bf16 weights and their sum, value product.  Full tiles run
// in a loop unrolled by two, so both LDS buffers have compile-time offsets; a
// ragged last tile runs once after it, with key masking.  The per-wave state
// is written for G groups of 32 query rows; one group per wave is used.
// REF: the state is kept relative to the reference maximum (kRefState): no
// per-tile maximum unless the weights' sums call for one, no true maximum.
template <int D, int NW, bool REF>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void fold_bf16_kernel(const FoldParams p) {
  using L = TileLayout<D>;
  constexpr int G = 1;  // query groups of 32 rows per wave
  constexpr int TK = L::kKeys;
  constexpr int NKB = TK / 32;
  constexpr int NC = D / 16;
  constexpr int NDB = D / 32;
  constexpr int UPR = D / 8;
  // 1 KB chunks each wave fills per tile and tensor: chunk wave + NW j (a
  // wave-uniform test skips those past the last); unpadded tiles split evenly.
  constexpr int KPW = (L::kKChunks + NW - 1) / NW;
  constexpr int VPW = (L::kVChunks + NW - 1) / NW;
  constexpr int QT = NW * 32 * G;  // query rows per workgroup
  static_assert(L::kPad || (L::kKChunks % NW == 0 && L::kVChunks % NW == 0),
                "unpadded tiles split into whole 1 KB chunks per wave");
  __shared__ __attribute__((aligned(1024))) __bf16 lds[2 * L::kBufElems];

  // The launch-wide arguments every path reads, loaded here in one round of
  // scalar loads: left to itself the compiler loads each at its first use,
  // behind the branches below, one round trip after another.
  asm volatile("" ::"s"(p.B), "s"(p.H), "s"(p.n_res), "s"(p.q_rows), "s"(p.flags), "s"(p.mask), "s"(p.scale_log2),
               "s"(p.q), "s"(p.k), "s"(p.v), "s"(p.o), "s"(p.m), "s"(p.l), "s"(p.q_sb), "s"(p.q_sh), "s"(p.q_sr),
               "s"(p.k_sb), "s"(p.k_sh), "s"(p.k_sr), "s"(p.v_sb), "s"(p.v_sh), "s"(p.v_sr), "s"(p.st_bh), "s"(p.P),
               "s"(p.blk), "s"(p.rem));

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

  // This resident's block lengths and offsets, all read here, before any
  // branch, so their scalar loads go out together; a query tile past the
  // block's end has nothing to do.
  const int q_len = p.q_len[r], kv_len = p.kv_len[r];
  const int64_t q_row0 = p.q_row0[r], k_off = p.k_off[r], v_off = p.v_off[r];
  const int q_blk = p.q_blk[r], kv_blk = p.kv_blk[r];
  asm volatile("" ::"s"(q_len), "s"(kv_len), "s"(q_row0), "s"(k_off), "s"(v_off), "s"(q_blk), "s"(kv_blk));
  if (qt * QT >= q_len) return;

  // Keys [0, kv_vis) are visible to some row of this workgroup, keys
  // [0, kv_all) to every row; key c is visible to this lane's row iff c <= lim.
  int kv_vis = kv_len, kv_all = kv_len;
  int lim = kv_len - 1;
  if (p.mask != kMaskNone) {
    const int qb = q_blk, kb = kv_blk;
    const int q_first = qt * QT, q_last = min(q_first + QT, q_len) - 1;
    auto last_key = [&](int qrow) {
      return last_key_at_or_before(p.mask, p.P, p.blk, p.rem, kb, token_pos(p.mask, p.P, p.blk, p.rem, qb, qrow));
    };
    kv_vis = last_key(q_last) + 1;
    kv_all = last_key(q_first) + 1;
    lim = min(lim, last_key(min(q_first + wave * 32 * G + lr, q_len - 1)));
    // Nothing visible and nothing to initialise or write: the state stays as it is.
    if (kv_vis == 0 && (p.flags & ~kRefState) == (kLoadState | kStoreState)) return;
  }

  int64_t srow[G], st_row[G];
  bool row_ok[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int row = qt * QT + wave * 32 * G + g * 32 + lr;
    row_ok[g] = row < q_len;
    srow[g] = q_row0 + (row_ok[g] ? row : q_len - 1);
    st_row[g] = ((int64_t)bi * p.H + hi) * p.st_bh + srow[g];
  }

  bf16x8 qf[G][NC];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const __bf16* qp = (const __bf16*)p.q + bi * p.q_sb + hi * p.q_sh + srow[g] * p.q_sr + 8 * lg;
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[g][c] = *(const bf16x8*)(qp + 16 * c);
  }

  // mref: the reference maximum the weights are taken against (base-2 units
  // of the scaled score); it trails the true running maximum mtrue by less
  // than kLazy, which keeps every weight below 2^kLazy.  o and l are rescaled
  // to mtrue once, before they are stored; with REF they stay relative to
  // mref, which is stored as it is (base 2) and mtrue is not tracked.
  float mref[G], mtrue[G], lpart[G], m_in[G];
  f32x16 oacc[G][NDB];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (p.flags & kLoadState) {
      m_in[g] = p.m[st_row[g]];
      mref[g] = REF ? m_in[g] : m_in[g] * kLog2e;
      lpart[g] = lg == 0 ? p.l[st_row[g]] : 0.0f;
      const float* orow = p.o + st_row[g] * D + 4 * lg;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 t = *(const f32x4*)(orow + 32 * db + 8 * j);
#pragma unroll
          for (int e = 0; e < 4; ++e) oacc[g][db][4 * j + e] = t[e];
        }
    } else {
      m_in[g] = -INFINITY;
      mref[g] = -INFINITY;
      lpart[g] = 0.0f;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[g][db][i] = 0.0f;
    }
    mtrue[g] = mref[g];
  }

  const __bf16* kbase = (const __bf16*)p.k + bi * p.k_sb + hi * p.k_sh + k_off;
  const __bf16* vbase = (const __bf16*)p.v + bi * p.v_sb + hi * p.v_sh + v_off;
  // Tiles [0, n_plain) need no mask; tiles [n_plain, n_kt) compare keys with lim.
  const int n_plain = min(kv_all, kv_len) / TK;
  const int n_kt = (kv_vis + TK - 1) / TK;
  const float c2 = p.scale_log2;

  // Direct loads: chunk c of a tile is LDS units [64c, 64c + 64); lane i
  // writes unit 64c + i, the (row, unit) of the tile that LDS unit holds.
  // Unpadded: unit u of row r sits at u ^ swz(r); padded: rows of kKRow / 8
  // (K) or kVRow / 8 (V) units, the units past D / 8 and the rows past the
  // tile fetch unit D / 8 - 1 of the last row they reach.
  const int k_sr = (int)p.k_sr, v_sr = (int)p.v_sr;
  auto chunk = [&](int j) { return L::kPad ? wave + NW * j : wave * KPW + j; };
  auto k_chunk_ok = [&](int j) { return !L::kPad || chunk(j) < L::kKChunks; };
  auto v_chunk_ok = [&](int j) { return !L::kPad || chunk(j) < L::kVChunks; };
  auto unit_src = [&](int c, int ln, int row_units, int& row, int& col) {
    const int u = c * 64 + ln;
    if constexpr (L::kPad) {
      row = min(u / row_units, TK - 1);
      col = min(u % row_units, UPR - 1);
    } else {
      row = u / UPR;
      col = (u % UPR) ^ swz<D>(row);
    }
  };
  // A copy of the lane id the compiler cannot see through: what is computed
  // from it is computed where it is used, not hoisted out of the tile loop
  // into registers held for the whole launch.
  auto opaque_lane = [&]() {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    return ln;
  };
  // Byte offsets inside a tile: chunks j < KRES (VRES) of a wave keep theirs
  // in registers; the padded layout's last chunks, which only the first waves
  // fill, compute theirs when issued.
  constexpr int KRES = L::kPad ? L::kKChunks / NW : KPW;
  constexpr int VRES = L::kPad ? L::kVChunks / NW : VPW;
  static_assert(KRES >= 1 && VRES >= 1, "every wave fills a chunk of each tile");
  int ld_koff[KRES], ld_voff[VRES];
#pragma unroll
  for (int j = 0; j < (KRES > VRES ? KRES : VRES); ++j) {
    int row, col;
    if (j < KRES) {
      unit_src(chunk(j), lane, L::kKRow / 8, row, col);
      ld_koff[j] = (row * k_sr + col * 8) * 2;
    }
    if (j < VRES) {
      if constexpr (L::kPad) unit_src(chunk(j), lane, L::kVRow / 8, row, col);
      ld_voff[j] = (row * v_sr + col * 8) * 2;
    }
  }
  auto koff = [&](int j) {
    if (j < KRES) return ld_koff[j < KRES ? j : 0];
    int row, col;
    unit_src(chunk(j), opaque_lane(), L::kKRow / 8, row, col);
    return (row * k_sr + col * 8) * 2;
  };
  auto voff = [&](int j) {
    if (j < VRES) return ld_voff[j < VRES ? j : 0];
    int row, col;
    unit_src(chunk(j), opaque_lane(), L::kVRow / 8, row, col);
    return (row * v_sr + col * 8) * 2;
  };
  auto issue_tile = [&](int kt, int buf) {
    const int key0 = kt * TK;
    __bf16* kl = lds + buf * L::kBufElems;
    __bf16* vl = kl + L::kKElems;
    if (key0 + TK <= kv_len) {
      const u32x4 kr = rsrc_words(kbase + (int64_t)key0 * k_sr);
      const u32x4 vr = rsrc_words(vbase + (int64_t)key0 * v_sr);
#pragma unroll
      for (int j = 0; j < KPW; ++j)
        if (k_chunk_ok(j)) bload_lds16(kr, koff(j), lds_addr(kl + chunk(j) * 512));
#pragma unroll
      for (int j = 0; j < VPW; ++j)
        if (v_chunk_ok(j)) bload_lds16(vr, voff(j), lds_addr(vl + chunk(j) * 512));
    } else {  // ragged last tile: rows past the end re-read the last row
      const int ln = L::kPad ? opaque_lane() : lane;
#pragma unroll
      for (int j = 0; j < KPW; ++j)
        if (k_chunk_ok(j)) {
          int row, col;
          unit_src(chunk(j), ln, L::kKRow / 8, row, col);
          const int64_t g = min(key0 + row, kv_len - 1);
          gload_lds16(kbase + g * k_sr + col * 8, lds_addr(kl + chunk(j) * 512));
        }
#pragma unroll
      for (int j = 0; j < VPW; ++j)
        if (v_chunk_ok(j)) {
          int row, col;
          unit_src(chunk(j), ln, L::kVRow / 8, row, col);
          const int64_t g = min(key0 + row, kv_len - 1);
          gload_lds16(vbase + g * v_sr + col * 8, lds_addr(vl + chunk(j) * 512));
        }
    }
  };

  // The ring hand-off fused into the fold (p.send_k set): this workgroup
  // writes tiles qt, qt + n_qt, qt + 2 n_qt, ... of the visiting block from
  // LDS to the slot the next ring step reads, the resident's other workgroups
  // the rest.  LDS unit 64 c + l holds the block's (row, unit) that lane l
  // loaded into it, so each lane writes its own unit back out (the padded
  // layout's extra units hold copies and write the same bytes twice).
  __bf16* const send_k =
      p.send_k == nullptr ? nullptr : (__bf16*)p.send_k + bi * p.send_sb + hi * p.send_sh + p.send_off[r];
  __bf16* const send_v =
      p.send_v == nullptr ? nullptr : (__bf16*)p.send_v + bi * p.send_sb + hi * p.send_sh + p.send_off[r];
  const int n_qt = (q_len + QT - 1) / QT;
  int send_at = send_k != nullptr ? qt : 0x7fffffff;  // the next tile this workgroup writes
  auto send_tile = [&](int kt, int buf) {
    const int key0 = kt * TK;
    const __bf16* kl = lds + buf * L::kBufElems;
    const __bf16* vl = kl + L::kKElems;
    const int ln = opaque_lane();
#pragma unroll
    for (int j = 0; j < KPW; ++j)
      if (k_chunk_ok(j)) {
        int row, col;
        unit_src(chunk(j), ln, L::kKRow / 8, row, col);
        const bf16x8 x = *(const bf16x8*)(kl + chunk(j) * 512 + 8 * ln);
        if (key0 + row < kv_len) *(bf16x8*)(send_k + (int64_t)(key0 + row) * D + col * 8) = x;
      }
#pragma unroll
    for (int j = 0; j < VPW; ++j)
      if (v_chunk_ok(j)) {
        int row, col;
        unit_src(chunk(j), ln, L::kVRow / 8, row, col);
        const bf16x8 x = *(const bf16x8*)(vl + chunk(j) * 512 + 8 * ln);
        if (key0 + row < kv_len) *(bf16x8*)(send_v + (int64_t)(key0 + row) * D + col * 8) = x;
      }
  };

  // Operand read offsets (elements).  K: row lr, unit 2 c + lg for d chunk c.
  // V^T (two transposed 8-byte reads per operand, 4 keys x 4 units x 2 halves
  // per 32 lanes): key vr + 8 run, unit 4 db + vx, half lane & 1.
  const int vr = 4 * lg + ((lane & 15) >> 2);
  const int vx = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  constexpr int NKO = L::kPad ? 1 : NC;
  constexpr int NVO = L::kPad ? 1 : NDB;
  int k_rd[NKO];
  int v_rd[2][NVO];
  if constexpr (L::kPad) {
    k_rd[0] = lr * L::kKRow + 8 * lg;
    v_rd[0][0] = vr * L::kVRow + 8 * vx + 4 * (lane & 1);
  } else {
    const int gk = lg ^ swz<D>(lr);
#pragma unroll
    for (int c = 0; c < NC; ++c) k_rd[c] = lr * D + (((2 * c) ^ gk) << 3);
#pragma unroll
    for (int run = 0; run < 2; ++run) {
      const int rr = vr + 8 * run;
      const int y = vx ^ swz<D>(rr);
#pragma unroll
      for (int db = 0; db < NDB; ++db) v_rd[run][db] = rr * D + (((4 * db) ^ y) << 3) + 4 * (lane & 1);
    }
  }
  auto k_at = [&](int c) { return L::kPad ? k_rd[0] + 16 * c : k_rd[c]; };
  auto v_at = [&](int run, int db) { return L::kPad ? v_rd[0][0] + 8 * L::kVRow * run + 32 * db : v_rd[run][db]; };

  // S^T of group g against the K tile at kl; the 32-key blocks are
  // independent accumulation chains, interleaved.  The products are issued in
  // a fixed order (a scheduling barrier after each), each K operand read
  // kReadAhead products before its use; left to itself the compiler reads
  // operands earlier and holds more registers, which measured slower.
  auto scores = [&](f32x16 (&s)[NKB], const __bf16* kl, int g) {
    constexpr int N = NC * NKB;
    auto rd = [&](int i) {  // product i: d chunk i / NKB, key block i % NKB
      return *(const bf16x8*)(kl + 32 * (i % NKB) * L::kKRow + k_at(i / NKB));
    };
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.0f;
    bf16x8 a[kReadAhead];
#pragma unroll
    for (int i = 0; i < kReadAhead; ++i) a[i] = rd(i);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      s[i % NKB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i % kReadAhead], qf[g][i / NKB], s[i % NKB], 0, 0, 0);
      if (i + kReadAhead < N) a[i % kReadAhead] = rd(i + kReadAhead);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Keys past this row's last visible key (the block's end, or the causal
  // boundary) score -inf.
  auto mask = [&](f32x16 (&s)[NKB], int key0) {
    const int lim_t = lim - key0 - 4 * lg;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (32 * kb + 8 * (i >> 2) + (i & 3) > lim_t) s[kb][i] = -INFINITY;
  };
  // Row maximum of the tile; raises mtrue, and mref when it falls more than
  // kLazy below the new maximum (rare: then o and l are rescaled here).  A
  // row that has seen no key yet (mref = -inf, o = 0, l = 0) just takes the
  // new maximum as its reference.
  auto track_max = [&](const f32x16 (&s)[NKB], int g) {
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    const float mt = pair_max(mx) * c2;
    mtrue[g] = fmaxf(mtrue[g], mt);
    const bool fresh = mref[g] == -INFINITY;
    const bool raise = !fresh && mt > mref[g] + kLazy;
    if (fresh) mref[g] = mt;
    if (__builtin_amdgcn_ballot_w64(raise)) {
      const float alpha = raise ? __builtin_amdgcn_exp2f(mref[g] - mt) : 1.0f;
      if (raise) mref[g] = mt;
      lpart[g] *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[g][db][i] *= alpha;
    }
  };
  // bf16 weights exp2(s c - mref) as packed pairs, and their sum into l.  A
  // row that has seen no visible key yet (mref = -inf, every score -inf) gets
  // weights exp2(-inf) = 0.
  auto weights = [&](const f32x16 (&s)[NKB], unsigned (&pk)[NKB][8], int g) -> float {
    const float mr = mref[g] == -INFINITY ? 0.0f : mref[g];
    float lsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][2 * j], c2, -mr));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][2 * j + 1], c2, -mr));
        pk[kb][j] = pack_bf16(p0, p1);
        lsum = sum_bf16_pair(pk[kb][j], lsum);
      }
    return lsum;
  };
  // REF: the slow path of a tile.  Row maximum of the tile; a row that has
  // seen no key yet takes it as its reference, a row whose maximum exceeds
  // the reference by more than kRefRaise raises it (o and l rescaled here).
  auto settle_ref = [&](const f32x16 (&s)[NKB], int g) {
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    const float mt = pair_max(mx) * c2;
    const bool fresh = mref[g] == -INFINITY;
    const bool raise = !fresh && mt > mref[g] + kRefRaise;
    if (fresh) mref[g] = mt;
    if (__builtin_amdgcn_ballot_w64(raise)) {
      const float alpha = raise ? __builtin_amdgcn_exp2f(mref[g] - mt) : 1.0f;
      if (raise) mref[g] = mt;
      lpart[g] *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[g][db][i] *= alpha;
    }
  };
  // O^T += V^T P^T over the tile, 16 keys per product, in the same fixed
  // order with each V^T operand (two transposed reads) read ahead.
  auto values = [&](const unsigned (&pk)[NKB][8], const __bf16* vl, int g) {
    constexpr int N = NKB * 2 * NDB;
    bf16x8 b[NKB * 2];  // weights of keys 16 h .. 16 h + 15 of the tile
#pragma unroll
    for (int h = 0; h < NKB * 2; ++h) {
      const int kb = h / 2, c = h % 2;
      b[h] = __builtin_bit_cast(bf16x8, u32x4{pk[kb][4 * c], pk[kb][4 * c + 1], pk[kb][4 * c + 2], pk[kb][4 * c + 3]});
    }
    auto rd = [&](int i) {  // product i: key run pair i / NDB, d block i % NDB
      const __bf16* vrow = vl + 16 * (i / NDB) * L::kVRow;
      const u32x2 w0 = __builtin_bit_cast(u32x2, lds_tr16(vrow + v_at(0, i % NDB)));
      const u32x2 w1 = __builtin_bit_cast(u32x2, lds_tr16(vrow + v_at(1, i % NDB)));
      return __builtin_bit_cast(bf16x8, u32x4{w0[0], w0[1], w1[0], w1[1]});
    };
    bf16x8 a[kReadAhead];
#pragma unroll
    for (int i = 0; i < kReadAhead; ++i) a[i] = rd(i);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      oacc[g][i % NDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i % kReadAhead], b[i / NDB], oacc[g][i % NDB], 0, 0, 0);
      if (i + kReadAhead < N) a[i % kReadAhead] = rd(i + kReadAhead);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // One tile whose K/V sit in LDS buffer `buf`; `masked` applies lim.
  auto tile = [&](int kt, int buf, bool masked) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile kt landed for this wave
    lds_barrier();                       // ... for every wave; the other buffer is free
    if (kt + 1 < n_kt) issue_tile(kt + 1, buf ^ 1);
    if (kt == send_at) {
      send_at += n_qt;
      send_tile(kt, buf);
    }
    const __bf16* kc = lds + buf * L::kBufElems;
    const __bf16* vc = kc + L::kKElems;
    f32x16 sa[NKB];
    unsigned pa[NKB][8];
    scores(sa, kc, 0);
    if (masked) mask(sa, kt * TK);
    if constexpr (REF) {
      // The weights against the current reference; the wave settles the
      // maximum first only if a lane's sum exceeds 2^kLazy (or is not a
      // number) or a row that has seen no key yet sees one in this tile.
      float ls = weights(sa, pa, 0);
      const bool fresh_vis = mref[0] == -INFINITY && lim >= kt * TK;
      if (__builtin_amdgcn_ballot_w64(fresh_vis || !(ls <= kRefSum))) {
        settle_ref(sa, 0);
        ls = weights(sa, pa, 0);
      }
      lpart[0] += ls;
    } else {
      track_max(sa, 0);
      lpart[0] += weights(sa, pa, 0);
    }
    values(pa, vc, 0);
  };

  if (n_kt > 0) {
    issue_tile(0, 0);
    // Q, the state and tile 0 in registers and LDS before the loop: with the
    // tile loads out of its sight, the compiler would otherwise wait for Q at
    // its first use, inside the loop, on every tile.
    __builtin_amdgcn_s_waitcnt(0x0F70);
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

#pragma unroll
  for (int g = 0; g < G; ++g) {
    // Bring (l, o) from the reference maximum to the true running maximum
    // (REF: they stay relative to the reference).
    const float fix = REF || mref[g] == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(mref[g] - mtrue[g]);
    const float mrow = REF ? mref[g] : mtrue[g];  // the maximum (l, o) are relative to
    const float l_tot = pair_sum(lpart[g]) * fix;
    if (!row_ok[g]) continue;
    if (p.flags & kWriteOut) {
      // (o fix) (1 / l): the state the step would store, then ra_finalize's
      // normalisation, so a ring equals the same folds followed by ra_finalize
      // bit for bit
      const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
      if (p.lse != nullptr && lg == 0)
        p.lse[st_row[g]] = l_tot > 0.0f ? (mrow + __log2f(l_tot)) * kLn2 : -INFINITY;
      __bf16* orow = (__bf16*)p.out + bi * p.out_sb + hi * p.out_sh + srow[g] * p.out_sr + 4 * lg;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bf16x4 t;
#pragma unroll
          for (int e = 0; e < 4; ++e) t[e] = (__bf16)((oacc[g][db][4 * j + e] * fix) * inv);
          *(bf16x4*)(orow + 32 * db + 8 * j) = t;
        }
    }
    if (p.flags & kStoreState) {
      if (lg == 0) {
        // A maximum that did not rise is stored exactly as it was loaded; the
        // reference (REF) is stored in base 2 as it is.
        p.m[st_row[g]] = REF ? mref[g] : mtrue[g] == m_in[g] * kLog2e ? m_in[g] : mtrue[g] * kLn2;
        p.l[st_row[g]] = l_tot;
      }
      float* orow = p.o + st_row[g] * D + 4 * lg;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4 t;
#pragma unroll
          for (int e = 0; e < 4; ++e) t[e] = oacc[g][db][4 * j + e] * fix;
          *(f32x4*)(orow + 32 * db + 8 * j) = t;
        }
    }
  }
}

}  // namespace

// Waves per workgroup of the d-specialised kernel.
constexpr int waves_for(int d) { return d == 128 ? 8 : 4; }

hipError_t launch_fold_bf16(const FoldParams& p, int d, hipStream_t s) {
  const int rows_per_wg = waves_for(d) * 32;
  const int64_t tiles_q = (p.q_rows + rows_per_wg - 1) / rows_per_wg;
  const int64_t grid = tiles_q * p.n_res * p.H * p.B;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 gd((unsigned)grid), bd(waves_for(d) * 64);
  const bool ref = (p.flags & kRefState) != 0;
  switch (d) {
    case 64:
      if (ref)
        fold_bf16_kernel<64, waves_for(64), true><<<gd, bd, 0, s>>>(p);
      else
        fold_bf16_kernel<64, waves_for(64), false><<<gd, bd, 0, s>>>(p);
      break;
    case 128:
      if (ref)
        fold_bf16_kernel<128, waves_for(128), true><<<gd, bd, 0, s>>>(p);
      else
        fold_bf16_kernel<128, waves_for(128), false><<<gd, bd, 0, s>>>(p);
      break;
    case 256:
      if (ref)
        fold_bf16_kernel<256, waves_for(256), true><<<gd, bd, 0, s>>>(p);
      else
        fold_bf16_kernel<256, waves_for(256), false><<<gd, bd, 0, s>>>(p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ra
