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
};

// One fold launch: n_res resident query blocks, each of q_rows rows, each
// folding its own visiting block of kv_rows rows.  Offsets and strides are in
// elements.  Resident r's query rows start at row r * q_rows of q and of out;
// its state row `row` is (bi * H + hi) * st_bh + r * q_rows + row of m and l
// (times d for o); its visiting block starts at k + k_off[r] / v + v_off[r].
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
  int32_t B, H, n_res;
  int32_t q_rows, kv_rows;
  int32_t flags;
  float scale_log2;  // softmax scale times log2(e): scores are exponentiated in base 2
};

// Each launcher returns the launch status (hipGetLastError after the launch).
hipError_t launch_fold_bf16(const FoldParams& p, int d, hipStream_t s);
hipError_t launch_fold_f32(const FoldParams& p, int d, hipStream_t s);
hipError_t launch_state_init(float* m, float* l, float* o, int64_t rows_total, int d, hipStream_t s);
// out element (bi, hi, row, c) = o / l, 0 where l == 0; out_bf16 selects the output type.
hipError_t launch_finalize(const float* l, const float* o, void* out, bool out_bf16, int64_t out_sb,
                           int64_t out_sh, int64_t out_sr, int B, int H, int64_t rows, int d, hipStream_t s);

}  // namespace ra
