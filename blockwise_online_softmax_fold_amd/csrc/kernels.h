// Internal interface between the host driver (ra_api.hip) and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

// At most this many resident query blocks are folded by one launch; the host
// splits larger sets into several launches.
constexpr int kMaxResident = 64;

// Flags of one fold launch.
enum FoldFlags : int {
  kLoadState = 1,   // read (m, l, o) from the state arrays; else start from (-inf, 0, 0)
  kStoreState = 2,  // write (m, l, o) back (the spill between ring steps)
  kWriteOut = 4,    // write O = o / l to `out` instead (the last step of the ring)
  // The spilled state is internal to a ring: m may hold the reference maximum
  // the weights were taken against (base 2, at most the running maximum) with
  // l and o relative to it, instead of the running maximum itself.  O and the
  // log-sum-exp are the same either way.  fold_bf16_kernel (d = 64, 128, 256)
  // keeps the reference; the fp32 kernel ignores the flag and keeps the
  // running maximum, which is one such state too.
  kRefState = 8,
};

// One fold launch: n_res resident query blocks; resident r has q_len[r] query
// rows and folds its own visiting block of kv_len[r] rows (q_rows is the
// largest q_len, which sizes the grid).  Offsets and strides are in elements.
// Resident r's query rows start at row q_row0[r] of q and of out; its state
// row `row` is (bi * H + hi) * st_bh + q_row0[r] + row of m and l (times d
// for o); its visiting block starts at k + k_off[r] / v + v_off[r].
struct FoldParams {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* m;
  float* l;
  float* o;
  int64_t q_sb, q_sh, q_sr;
  int64_t k_sb, k_sh, k_sr;
  int64_t v_sb, v_sh, v_sr;
  int64_t out_sb, out_sh, out_sr;
  int64_t st_bh;  // rows per (batch, head) in the state arrays
  int64_t k_off[kMaxResident];
  int64_t v_off[kMaxResident];
  int32_t q_len[kMaxResident];
  int32_t kv_len[kMaxResident];
  int64_t q_row0[kMaxResident];
  int32_t B, H, n_res;
  int32_t q_rows;
  int32_t flags;
  float scale_log2;  // softmax scale times log2(e): scores are exponentiated in base 2
  float* lse;        // with kWriteOut, if not null: m + ln l of each row (the state row layout)
  // Causal masking (mask != kMaskNone): query row r of resident r_ and key row c
  // of its visiting block sit at sequence positions pos(q_blk[r_], r) and
  // pos(kv_blk[r_], c) of a P-device ring over N = P blk + rem tokens (device
  // j's block holds blk rows, one more when j < rem); keys after the query are
  // masked.
  int32_t mask;
  int32_t P, blk, rem;
  int32_t q_blk[kMaxResident];
  int32_t kv_blk[kMaxResident];
  // The ring hand-off fused into the fold (bf16 kernel, no mask, resident
  // blocks all of one length), if send_k is not null: resident r's visiting
  // block is also written, K to send_k and V to send_v, at element offset
  // b * send_sb + h * send_sh + send_off[r] + row * d -- the slot the next
  // ring step reads.  Each tile is written by one workgroup of the resident.
  void* send_k;
  void* send_v;
  int64_t send_sb, send_sh;
  int64_t send_off[kMaxResident];
};

// Masking modes (the token layout of the ring when causal).
enum MaskMode : int {
  kMaskNone = 0,
  kMaskContiguous = 1,  // device j holds the next run of tokens after device j - 1
  kMaskStriped = 2,     // device j holds tokens j, j + P, j + 2P, ...
  kMaskZigzag = 3,      // device j holds chunks j and 2P - 1 - j of b / 2 tokens (rem = 0)
};

// Rows of device j's block and, for the contiguous split, its first position.
__host__ __device__ inline int32_t block_len(int32_t b, int32_t rem, int32_t j) { return b + (j < rem ? 1 : 0); }
__host__ __device__ inline int32_t block_start(int32_t b, int32_t rem, int32_t j) { return j * b + (j < rem ? j : rem); }

// Sequence position of row r of device j's block.
__host__ __device__ inline int32_t token_pos(int mode, int32_t P, int32_t b, int32_t rem, int32_t j, int32_t r) {
  if (mode == kMaskStriped) return r * P + j;
  if (mode == kMaskZigzag) {
    const int32_t h = b >> 1;
    return r < h ? j * h + r : (2 * P - 1 - j) * h + (r - h);
  }
  return block_start(b, rem, j) + r;
}

// Every layout numbers the rows of a block in increasing position (zig-zag:
// chunk j < P comes before its mirror 2P - 1 - j), so the keys of device j's
// block at or before a position x are a prefix of the block.  Largest such key
// row (-1 if none).
__host__ __device__ inline int32_t last_key_at_or_before(int mode, int32_t P, int32_t b, int32_t rem, int32_t j,
                                                        int32_t x) {
  int32_t c;
  if (mode == kMaskStriped) {
    c = x < j ? -1 : (x - j) / P;
  } else if (mode == kMaskZigzag) {
    const int32_t h = b >> 1;
    const int32_t hi0 = (2 * P - 1 - j) * h;  // position of the mirror chunk's first row
    if (x >= hi0)
      c = h + (x - hi0);
    else
      c = x - j * h < h ? x - j * h : h - 1;
  } else {
    c = x - block_start(b, rem, j);
  }
  if (c < -1) c = -1;
  const int32_t n = block_len(b, rem, j);
  return c < n - 1 ? c : n - 1;
}

// One backward launch over n_res (resident query block, visiting block) pairs
// of one ring step.  The dQ pass (one workgroup per tile of query rows) folds
// the visiting block into dQ; the dK/dV pass (one workgroup per tile of keys) adds the
// resident block's share to the visiting block's dK, dV accumulators.  Row
// arrays (nl2, dd, dq_acc) follow the resident rows like the forward state;
// dk_acc, dv_acc are [B, H, N, d] over the whole sequence.
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  void* dq;
  int64_t q_sb, q_sh, q_sr;
  int64_t k_sb, k_sh, k_sr;
  int64_t v_sb, v_sh, v_sr;
  int64_t do_sb, do_sh, do_sr;
  int64_t dq_sb, dq_sh, dq_sr;
  const float* nl2;  // -(m + ln l) log2(e) of each query row; -inf for a row that saw no key
  const float* dd;   // rowsum(dO * O) of each query row
  float* dq_acc;     // dQ / scale so far, fp32
  float* dk_acc;     // dK / scale so far, fp32
  float* dv_acc;     // dV so far, fp32
  int64_t st_bh;     // rows per (batch, head) of nl2, dd, dq_acc
  int64_t acc_bh;    // rows per (batch, head) of dk_acc, dv_acc
  int64_t k_off[kMaxResident];
  int64_t v_off[kMaxResident];
  int64_t acc_row0[kMaxResident];  // first row of the visiting block in dk_acc / dv_acc
  int64_t q_row0[kMaxResident];    // first row of the resident block in q, dout, dq and the row arrays
  int32_t q_len[kMaxResident];
  int32_t kv_len[kMaxResident];
  int32_t q_blk[kMaxResident];
  int32_t kv_blk[kMaxResident];
  int32_t B, H, n_res;
  int32_t q_rows, kv_rows;  // largest q_len and kv_len: they size the grids
  int32_t flags;            // dQ pass: kLoadState / kStoreState / kWriteOut on dq_acc and dq
  float scale;
  float scale_log2;
  int32_t mask, P, blk, rem;
};

// Each launcher returns the launch status (hipGetLastError after the launch).
hipError_t launch_fold_bf16(const FoldParams& p, int d, hipStream_t s);
hipError_t launch_fold_f32(const FoldParams& p, int d, hipStream_t s);
hipError_t launch_state_init(float* m, float* l, float* o, int64_t rows_total, int d, hipStream_t s);
hipError_t launch_bwd_dq_bf16(const BwdParams& p, int d, hipStream_t s);
hipError_t launch_bwd_dkdv_bf16(const BwdParams& p, int d, hipStream_t s);
hipError_t launch_bwd_dq_f32(const BwdParams& p, int d, hipStream_t s);
hipError_t launch_bwd_dkdv_f32(const BwdParams& p, int d, hipStream_t s);
// Backward set-up per resident row: nl2 = -lse log2(e) (-inf where lse = -inf)
// and dd = rowsum(dO * O), for B*H*rows rows (row = (bi * H + hi) * rows + r).
hipError_t launch_bwd_prep(const float* lse, const void* dout, int64_t do_sb, int64_t do_sh, int64_t do_sr,
                           const void* out, int64_t o_sb, int64_t o_sh, int64_t o_sr, bool bf16, int B, int H,
                           int64_t rows, int d, float* nl2, float* dd, hipStream_t s);
// dst = alpha * acc ([B, H, rows, d] fp32, contiguous) in the output dtype with strides.
hipError_t launch_scale_cast(const float* acc, float alpha, void* dst, int64_t sb, int64_t sh, int64_t sr, bool bf16,
                             int B, int H, int64_t rows, int d, hipStream_t s);
// Fill `bytes` bytes (a multiple of 16, 16-byte aligned) with a repeated 32-bit word.
hipError_t launch_fill_u32(void* x, size_t bytes, unsigned value, hipStream_t s);
// Fill n floats with zero.
hipError_t launch_zero(float* x, int64_t n, hipStream_t s);
// out element (bi, hi, row, c) = o / l, 0 where l == 0; out_bf16 selects the output type.
hipError_t launch_finalize(const float* l, const float* o, void* out, bool out_bf16, int64_t out_sb,
                           int64_t out_sh, int64_t out_sr, int B, int H, int64_t rows, int d, hipStream_t s);

}  // namespace ra
