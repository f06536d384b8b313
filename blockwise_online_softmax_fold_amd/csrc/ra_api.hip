// Host side of libra.so: argument checks, workspace layout, the ring driver
// (P virtual ring steps with a double-buffered K/V hand-off on a side stream)
// and the C entry points declared in include/ra.h.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <time.h>

#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"
#include "ra.h"

#define RA_API extern "C" __attribute__((visibility("default")))

namespace {

using ra::FoldParams;

thread_local std::string g_err;

ra_status_t fail(ra_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

ra_status_t hip_fail(hipError_t e, const char* what) {
  g_err = std::string(what) + ": " + hipGetErrorString(e);
  return e == hipErrorOutOfMemory ? RA_E_OOM : RA_E_HIP;
}

#define RA_HIP(call, what)                \
  do {                                    \
    hipError_t e_ = (call);               \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

bool valid_d(int64_t d) { return d == 64 || d == 128 || d == 256; }
bool valid_dt(ra_dtype_t dt) { return dt == RA_DTYPE_F32 || dt == RA_DTYPE_BF16; }
size_t esize(ra_dtype_t dt) { return dt == RA_DTYPE_BF16 ? 2 : 4; }

ra_status_t check_tensor(const char* name, const void* ptr, const int64_t* strides, ra_dtype_t dt) {
  if (ptr == nullptr) return fail(RA_E_INVALID_ARG, "%s is NULL", name);
  if (strides == nullptr) return fail(RA_E_INVALID_ARG, "%s strides are NULL", name);
  if (((uintptr_t)ptr & 15) != 0) return fail(RA_E_INVALID_ARG, "%s is not 16-byte aligned", name);
  const int64_t q = dt == RA_DTYPE_BF16 ? 8 : 4;
  for (int i = 0; i < 3; ++i) {
    if (strides[i] < 0) return fail(RA_E_INVALID_ARG, "%s stride %d is negative", name, i);
    if (strides[i] % q != 0)
      return fail(RA_E_INVALID_ARG, "%s stride %d (%lld) is not a multiple of %lld elements", name, i,
                  (long long)strides[i], (long long)q);
  }
  return RA_OK;
}

// The kernels address the rows of one LDS tile (at most 64 rows) with 32-bit
// byte offsets from the tile's first row: streamed operands (K, V in the
// forward and the dQ kernel, Q, dO and V in the dK/dV kernel) need row strides
// below 2^24 elements.
constexpr int64_t kMaxTileRowStride = (int64_t)1 << 24;
ra_status_t check_tile_row_stride(const char* name, const int64_t* strides) {
  if (strides[2] >= kMaxTileRowStride)
    return fail(RA_E_UNSUPPORTED, "%s row stride %lld is not below 2^24 elements", name, (long long)strides[2]);
  return RA_OK;
}

ra_status_t check_state(const float* m, const float* l, const float* o) {
  if (!m || !l || !o) return fail(RA_E_INVALID_ARG, "state pointer m, l or o is NULL");
  if (((uintptr_t)o & 15) != 0) return fail(RA_E_INVALID_ARG, "state o is not 16-byte aligned");
  if (((uintptr_t)m & 3) != 0 || ((uintptr_t)l & 3) != 0)
    return fail(RA_E_INVALID_ARG, "state m or l is not 4-byte aligned");
  return RA_OK;
}

ra_status_t check_common(ra_dtype_t dt, int64_t B, int64_t H, int64_t d) {
  if (!valid_dt(dt)) return fail(RA_E_INVALID_ARG, "unknown dtype %d", (int)dt);
  if (B < 1 || H < 1) return fail(RA_E_INVALID_ARG, "B=%lld and H=%lld must be >= 1", (long long)B, (long long)H);
  if (B > 65535 || H > 65535) return fail(RA_E_UNSUPPORTED, "B and H must be <= 65535");
  if (!valid_d(d)) return fail(RA_E_UNSUPPORTED, "head dim d=%lld is not 64, 128 or 256", (long long)d);
  return RA_OK;
}

ra_status_t resolve_scale(float scale, int64_t d, float* out) {
  if (scale == 0.0f) {
    *out = (float)(1.0 / sqrt((double)d));
    return RA_OK;
  }
  if (!(scale > 0.0f) || !isfinite(scale))
    return fail(RA_E_INVALID_ARG, "scale must be 0 (meaning 1/sqrt(d)) or finite and > 0");
  *out = scale;
  return RA_OK;
}

float to_log2_scale(float scale) { return (float)((double)scale * 1.4426950408889634); }

// Device scratch of ra_ring_forward_noalloc: the ring workspace for callers
// that cannot allocate.  Each GPU holds its own copy from the time the library
// is first used on it until the process ends.  In host code the name below is
// not a device address; the address comes from hipGetSymbolAddress, once per
// device (DevRes::scratch).
constexpr size_t kScratchBytes = RA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Per-device resources owned by the library: the side stream of the hand-off
// and the events ordering it against the caller's stream.
struct DevRes {
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  hipEvent_t ready[2] = {nullptr, nullptr};
  hipEvent_t freed[2] = {nullptr, nullptr};
  void* scratch = nullptr;  // this device's address of `scratch`, once resolved
  std::mutex mu;  // one ring driver at a time per device uses these
};

std::mutex g_dev_mu;
std::map<int, DevRes*> g_dev;

ra_status_t get_dev(DevRes** out) {
  int dev = 0;
  RA_HIP(hipGetDevice(&dev), "hipGetDevice");
  std::lock_guard<std::mutex> g(g_dev_mu);
  auto it = g_dev.find(dev);
  if (it != g_dev.end()) {
    *out = it->second;
    return RA_OK;
  }
  DevRes* r = new DevRes;
  hipEvent_t* evs[6] = {&r->fork, &r->join, &r->ready[0], &r->ready[1], &r->freed[0], &r->freed[1]};
  // On a failure part-way, release what was created and leave no entry, so a
  // later call tries again.
  auto undo = [&](hipError_t e, const char* what) {
    for (hipEvent_t* ev : evs)
      if (*ev != nullptr) (void)hipEventDestroy(*ev);
    if (r->side != nullptr) (void)hipStreamDestroy(r->side);
    delete r;
    return hip_fail(e, what);
  };
  hipError_t e = hipStreamCreateWithFlags(&r->side, hipStreamNonBlocking);
  if (e != hipSuccess) return undo(e, "hipStreamCreateWithFlags");
  for (hipEvent_t* ev : evs) {
    e = hipEventCreateWithFlags(ev, hipEventDisableTiming);
    if (e != hipSuccess) return undo(e, "hipEventCreateWithFlags");
  }
  g_dev[dev] = r;
  *out = r;
  return RA_OK;
}

// Undoes a ring driver's set-up when it returns early on an error: the side
// stream is joined back into the caller's stream (so no hand-off copy still
// reads K or V after the call has returned) and a workspace the library
// allocated is freed.  The success path does both itself, checking each
// call, after clearing the fields.  Errors here are not reported: the call
// already returns the first one.
struct RingCleanup {
  hipStream_t stream = nullptr;
  hipStream_t side = nullptr;  // set while the side stream is forked
  hipEvent_t join = nullptr;
  void* ws = nullptr;  // set while an internally allocated workspace is live
  ~RingCleanup() {
    if (side != nullptr && hipEventRecord(join, side) == hipSuccess) (void)hipStreamWaitEvent(stream, join, 0);
    if (ws != nullptr) (void)hipFreeAsync(ws, stream);
  }
};

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Blocks of the ring: N = P b + rem tokens; device j's block holds
// block_len(b, rem, j) rows (b, one more for j < rem) starting at row
// block_start(b, rem, j) of the sequence.
struct Blocks {
  int64_t b = 0, rem = 0, b_max = 0;
  int64_t len(int64_t j) const { return ra::block_len((int32_t)b, (int32_t)rem, (int32_t)j); }
  int64_t start(int64_t j) const { return ra::block_start((int32_t)b, (int32_t)rem, (int32_t)j); }
};

Blocks ring_blocks(int64_t N, int32_t P) {
  Blocks k;
  k.b = N / P;
  k.rem = N % P;
  k.b_max = k.b + (k.rem ? 1 : 0);
  return k;
}

// Workspace of the ring driver: state of the n_q resident blocks
// (m, l: [B, H, rows]; o: [B, H, rows, d], rows = the residents' rows, at most
// n_q * b_max) followed by the K and V halves of the double buffer, each
// [slot][B][H][n_q * b_max][d]: in each head, resident r's visiting block
// starts at row r * b_max.  With every block resident in ring order and equal
// blocks, a slot's head is then the whole sequence rotated by whole blocks,
// which the hand-off fills with two contiguous copies.
struct RingLayout {
  Blocks blk;
  int nslots = 0;
  size_t off_m = 0, off_l = 0, off_o = 0, off_k = 0, off_v = 0, total = 0;
  int64_t head_rows = 0;   // rows of one (batch, head) in a slot: n_q * b_max
  int64_t slot_elems = 0;  // elements of one slot over all residents
};

RingLayout ring_layout(ra_dtype_t dt, int64_t B, int64_t H, int64_t N, int64_t d, int32_t P, int32_t n_q) {
  RingLayout L;
  L.blk = ring_blocks(N, P);
  const int64_t rows = (int64_t)n_q * L.blk.b_max;
  L.nslots = P - 1 < 2 ? P - 1 : 2;  // two visiting blocks, not P
  const size_t st_rows = (size_t)B * H * rows;
  L.off_m = 0;
  L.off_l = round_up(L.off_m + st_rows * 4);
  L.off_o = round_up(L.off_l + st_rows * 4);
  L.off_k = round_up(L.off_o + st_rows * (size_t)d * 4);
  L.head_rows = (int64_t)n_q * L.blk.b_max;
  L.slot_elems = B * H * L.head_rows * d;
  const size_t buf = (size_t)L.nslots * L.slot_elems * esize(dt);
  L.off_v = round_up(L.off_k + buf);
  L.total = round_up(L.off_v + buf);
  return L;
}

ra_status_t check_ring(const void* q, const int64_t* q_strides, const void* k, const int64_t* k_strides,
                       const void* v, const int64_t* v_strides, const void* out, const int64_t* out_strides,
                       ra_dtype_t dt, int64_t B, int64_t H, int64_t N, int64_t d, int32_t P,
                       const int32_t* query_blocks, int32_t n_q) {
  ra_status_t st = check_common(dt, B, H, d);
  if (st != RA_OK) return st;
  if (P < 1) return fail(RA_E_INVALID_ARG, "P=%d must be >= 1", (int)P);
  if (N < P) return fail(RA_E_INVALID_ARG, "N=%lld must be >= P=%d", (long long)N, (int)P);
  if (N / P + 1 > 0x7fffffffLL / 4) return fail(RA_E_UNSUPPORTED, "block size N/P is too large");
  if (n_q < 1) return fail(RA_E_INVALID_ARG, "n_q=%d must be >= 1", (int)n_q);
  if (query_blocks == nullptr && n_q != P)
    return fail(RA_E_INVALID_ARG, "query_blocks is NULL (all blocks) but n_q=%d != P=%d", (int)n_q, (int)P);
  if (query_blocks != nullptr)
    for (int32_t i = 0; i < n_q; ++i)
      if (query_blocks[i] < 0 || query_blocks[i] >= P)
        return fail(RA_E_INVALID_ARG, "query_blocks[%d]=%d is outside [0, P=%d)", (int)i, (int)query_blocks[i],
                    (int)P);
  if ((st = check_tensor("q", q, q_strides, dt)) != RA_OK) return st;
  if ((st = check_tensor("k", k, k_strides, dt)) != RA_OK) return st;
  if ((st = check_tensor("v", v, v_strides, dt)) != RA_OK) return st;
  if ((st = check_tensor("out", out, out_strides, dt)) != RA_OK) return st;
  if ((st = check_tile_row_stride("k", k_strides)) != RA_OK) return st;
  if ((st = check_tile_row_stride("v", v_strides)) != RA_OK) return st;
  return RA_OK;
}

void set_strides(int64_t* dst_b, int64_t* dst_h, int64_t* dst_r, const int64_t* s) {
  *dst_b = s[0];
  *dst_h = s[1];
  *dst_r = s[2];
}

// Copy rows [start, start + n) of src ([B, H, N, d] with strides s) into dst,
// whose heads are dst_head_rows rows of d elements apart and whose batches are
// H heads apart (the hand-off of one or more consecutive visiting blocks).
ra_status_t copy_block(void* dst, const void* src, const int64_t* s, int64_t B, int64_t H, int64_t start, int64_t n,
                       int64_t dst_head_rows, int64_t d, size_t es, hipStream_t stream) {
  const char* sp = (const char*)src;
  char* dp = (char*)dst;
  const size_t row_bytes = (size_t)d * es;
  const size_t blk_bytes = (size_t)n * row_bytes;
  const size_t dst_head = (size_t)dst_head_rows * row_bytes;
  if (s[2] == d && (H == 1 || s[1] * (int64_t)es >= (int64_t)blk_bytes)) {
    // rows of a block are contiguous: one 2-D copy over heads per batch
    const size_t spitch = H == 1 ? blk_bytes : (size_t)s[1] * es;
    for (int64_t bi = 0; bi < B; ++bi) {
      const char* from = sp + (size_t)(bi * s[0] + start * d) * es;
      char* to = dp + (size_t)bi * H * dst_head;
      RA_HIP(hipMemcpy2DAsync(to, dst_head, from, spitch, blk_bytes, (size_t)H, hipMemcpyDeviceToDevice, stream),
             "hipMemcpy2DAsync (hand-off)");
    }
    return RA_OK;
  }
  for (int64_t bi = 0; bi < B; ++bi)
    for (int64_t hi = 0; hi < H; ++hi) {
      const char* from = sp + (size_t)(bi * s[0] + hi * s[1] + start * s[2]) * es;
      char* to = dp + (size_t)(bi * H + hi) * dst_head;
      RA_HIP(hipMemcpy2DAsync(to, row_bytes, from, (size_t)s[2] * es, row_bytes, (size_t)n, hipMemcpyDeviceToDevice,
                              stream),
             "hipMemcpy2DAsync (hand-off)");
    }
  return RA_OK;
}

hipError_t launch_fold(const FoldParams& p, ra_dtype_t dt, int d, hipStream_t s) {
  return dt == RA_DTYPE_BF16 ? ra::launch_fold_bf16(p, d, s) : ra::launch_fold_f32(p, d, s);
}

// Optional per-launch timing of the fold kernels (ra_profile_folds).
struct FoldProfile {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> ev;  // pairs: start, stop
  size_t used = 0;             // pairs recorded
};
FoldProfile g_prof;
constexpr size_t kMaxProfiled = 4096;

// Record the start event of a timed launch; returns the pair index or -1.
long prof_begin(hipStream_t s) {
  std::lock_guard<std::mutex> g(g_prof.mu);
  if (!g_prof.on || g_prof.used >= kMaxProfiled) return -1;
  const size_t i = g_prof.used;
  while (g_prof.ev.size() < 2 * (i + 1)) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return -1;
    g_prof.ev.push_back(e);
  }
  if (hipEventRecord(g_prof.ev[2 * i], s) != hipSuccess) return -1;
  g_prof.used = i + 1;
  return (long)i;
}

void prof_end(long i, hipStream_t s) {
  if (i < 0) return;
  std::lock_guard<std::mutex> g(g_prof.mu);
  (void)hipEventRecord(g_prof.ev[2 * i + 1], s);
}

bool env_flag(const char* name) {
  const char* v = getenv(name);
  return v != nullptr && v[0] != '\0' && v[0] != '0';
}

long env_long(const char* name) {
  const char* v = getenv(name);
  return v == nullptr ? 0 : strtol(v, nullptr, 10);
}

// Host callback of the delayed hand-off (RA_DEBUG_DELAY_US): holds the side
// stream for the given number of microseconds.
void sleep_cb(void* us) {
  const long n = (long)(intptr_t)us;
  struct timespec ts;
  ts.tv_sec = n / 1000000;
  ts.tv_nsec = (n % 1000000) * 1000;
  nanosleep(&ts, nullptr);
}

// Quiet NaN patterns of a poisoned hand-off slot, as 32-bit words.
constexpr unsigned kNanBf16x2 = 0x7fc07fc0u;
constexpr unsigned kNanF32 = 0x7fc00000u;

}  // namespace

RA_API const char* ra_last_error(void) { return g_err.c_str(); }

RA_API const char* ra_version(void) { return "0.2.0"; }

RA_API ra_status_t ra_state_init(float* m, float* l, float* o, int64_t B, int64_t H, int64_t rows, int64_t d,
                                 void* stream) {
  g_err.clear();
  ra_status_t st = check_common(RA_DTYPE_F32, B, H, d);
  if (st != RA_OK) return st;
  if (rows < 0) return fail(RA_E_INVALID_ARG, "rows=%lld must be >= 0", (long long)rows);
  if (rows == 0) return RA_OK;
  if ((st = check_state(m, l, o)) != RA_OK) return st;
  RA_HIP(ra::launch_state_init(m, l, o, B * H * rows, (int)d, (hipStream_t)stream), "state init launch");
  return RA_OK;
}

namespace {

// Shared body of ra_fold_block and ra_fold_block_causal.
ra_status_t fold_block_impl(const void* q, const int64_t q_strides[3], const void* k, const int64_t k_strides[3],
                            const void* v, const int64_t v_strides[3], ra_dtype_t dt, int64_t B, int64_t H,
                            int64_t q_rows, int64_t kv_rows, int64_t d, float scale, float* m, float* l, float* o,
                            int mask, int32_t P, int32_t blk, int32_t rem, int32_t q_block, int32_t kv_block,
                            void* stream) {
  ra_status_t st = check_common(dt, B, H, d);
  if (st != RA_OK) return st;
  if (q_rows < 0 || kv_rows < 0) return fail(RA_E_INVALID_ARG, "q_rows and kv_rows must be >= 0");
  if (q_rows > 0x7fffffffLL / 4 || kv_rows > 0x7fffffffLL / 4)
    return fail(RA_E_UNSUPPORTED, "q_rows or kv_rows is too large for one launch");
  float sc;
  if ((st = resolve_scale(scale, d, &sc)) != RA_OK) return st;
  if (q_rows == 0) return RA_OK;  // no query rows: nothing is read or written
  if ((st = check_tensor("q", q, q_strides, dt)) != RA_OK) return st;
  if ((st = check_state(m, l, o)) != RA_OK) return st;
  if (kv_rows == 0) return RA_OK;  // an empty block leaves the state as it is
  if ((st = check_tensor("k", k, k_strides, dt)) != RA_OK) return st;
  if ((st = check_tensor("v", v, v_strides, dt)) != RA_OK) return st;
  if ((st = check_tile_row_stride("k", k_strides)) != RA_OK) return st;
  if ((st = check_tile_row_stride("v", v_strides)) != RA_OK) return st;

  FoldParams p = {};
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = nullptr;
  p.m = m;
  p.l = l;
  p.o = o;
  set_strides(&p.q_sb, &p.q_sh, &p.q_sr, q_strides);
  set_strides(&p.k_sb, &p.k_sh, &p.k_sr, k_strides);
  set_strides(&p.v_sb, &p.v_sh, &p.v_sr, v_strides);
  p.st_bh = q_rows;
  p.k_off[0] = 0;
  p.v_off[0] = 0;
  p.B = (int32_t)B;
  p.H = (int32_t)H;
  p.n_res = 1;
  p.q_rows = (int32_t)q_rows;
  p.q_len[0] = (int32_t)q_rows;
  p.kv_len[0] = (int32_t)kv_rows;
  p.q_row0[0] = 0;
  p.flags = ra::kLoadState | ra::kStoreState;
  p.scale_log2 = to_log2_scale(sc);
  p.mask = mask;
  p.P = P;
  p.blk = blk;
  p.rem = rem;
  p.q_blk[0] = q_block;
  p.kv_blk[0] = kv_block;
  RA_HIP(launch_fold(p, dt, (int)d, (hipStream_t)stream), "fold launch");
  return RA_OK;
}

bool valid_layout(int layout) {
  return layout == RA_CAUSAL_NONE || layout == RA_CAUSAL_CONTIGUOUS || layout == RA_CAUSAL_STRIPED ||
         layout == RA_CAUSAL_ZIGZAG;
}

// Positions of a causal ring over N tokens must fit the kernels' int32; the
// zig-zag split cuts the sequence into 2P equal chunks.
ra_status_t check_causal(int layout, int64_t P, int64_t N) {
  if (!valid_layout(layout)) return fail(RA_E_INVALID_ARG, "unknown causal layout %d", layout);
  if (layout == RA_CAUSAL_NONE) return RA_OK;
  if (N > 0x7fffffffLL) return fail(RA_E_UNSUPPORTED, "N=%lld positions do not fit 32 bits", (long long)N);
  if (layout == RA_CAUSAL_ZIGZAG && N % (2 * P) != 0)
    return fail(RA_E_INVALID_ARG, "zig-zag layout needs N a multiple of 2P, got N=%lld, P=%lld", (long long)N,
                (long long)P);
  return RA_OK;
}

}  // namespace

RA_API ra_status_t ra_fold_block(const void* q, const int64_t q_strides[3], const void* k, const int64_t k_strides[3],
                                 const void* v, const int64_t v_strides[3], ra_dtype_t dt, int64_t B, int64_t H,
                                 int64_t q_rows, int64_t kv_rows, int64_t d, float scale, float* m, float* l,
                                 float* o, void* stream) {
  g_err.clear();
  return fold_block_impl(q, q_strides, k, k_strides, v, v_strides, dt, B, H, q_rows, kv_rows, d, scale, m, l, o,
                         ra::kMaskNone, 1, (int32_t)kv_rows, 0, 0, 0, stream);
}

RA_API ra_status_t ra_fold_block_causal(const void* q, const int64_t q_strides[3], const void* k,
                                        const int64_t k_strides[3], const void* v, const int64_t v_strides[3],
                                        ra_dtype_t dt, int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                                        ra_causal_t layout, int32_t P, int32_t q_block, int32_t kv_block, float* m,
                                        float* l, float* o, void* stream) {
  g_err.clear();
  ra_status_t st;
  if (!valid_layout((int)layout)) return fail(RA_E_INVALID_ARG, "unknown causal layout %d", (int)layout);
  if (P < 1) return fail(RA_E_INVALID_ARG, "P=%d must be >= 1", (int)P);
  if (N < P) return fail(RA_E_INVALID_ARG, "N=%lld must be >= P=%d", (long long)N, (int)P);
  if (q_block < 0 || q_block >= P || kv_block < 0 || kv_block >= P)
    return fail(RA_E_INVALID_ARG, "q_block=%d and kv_block=%d must lie in [0, P=%d)", (int)q_block, (int)kv_block,
                (int)P);
  if (N / P + 1 > 0x7fffffffLL / 4) return fail(RA_E_UNSUPPORTED, "block size N/P is too large");
  if ((st = check_causal((int)layout, P, N)) != RA_OK) return st;
  const Blocks bk = ring_blocks(N, P);
  return fold_block_impl(q, q_strides, k, k_strides, v, v_strides, dt, B, H, bk.len(q_block), bk.len(kv_block), d,
                         scale, m, l, o, (int)layout, P, (int32_t)bk.b, (int32_t)bk.rem, q_block, kv_block, stream);
}

RA_API ra_status_t ra_finalize(const float* l, const float* o, void* out, const int64_t out_strides[3],
                               ra_dtype_t out_dt, int64_t B, int64_t H, int64_t rows, int64_t d, void* stream) {
  g_err.clear();
  ra_status_t st = check_common(out_dt, B, H, d);
  if (st != RA_OK) return st;
  if (rows < 0) return fail(RA_E_INVALID_ARG, "rows=%lld must be >= 0", (long long)rows);
  if (rows == 0) return RA_OK;
  if (l == nullptr || o == nullptr) return fail(RA_E_INVALID_ARG, "state pointer l or o is NULL");
  if (((uintptr_t)o & 15) != 0) return fail(RA_E_INVALID_ARG, "state o is not 16-byte aligned");
  if ((st = check_tensor("out", out, out_strides, out_dt)) != RA_OK) return st;
  RA_HIP(ra::launch_finalize(l, o, out, out_dt == RA_DTYPE_BF16, out_strides[0], out_strides[1], out_strides[2],
                             (int)B, (int)H, rows, (int)d, (hipStream_t)stream),
         "finalize launch");
  return RA_OK;
}

RA_API size_t ra_ring_workspace_bytes(ra_dtype_t dt, int64_t B, int64_t H, int64_t N, int64_t d, int32_t P,
                                      int32_t n_q) {
  const std::string saved = g_err;
  const bool ok = check_common(dt, B, H, d) == RA_OK && P >= 1 && N >= P && n_q >= 1 &&
                  N / P + 1 <= 0x7fffffffLL / 4;
  g_err = saved;
  if (!ok) return 0;
  return ring_layout(dt, B, H, N, d, P, n_q).total;
}

namespace {

// use_scratch: run in the device's static scratch (ra_ring_forward_noalloc)
// instead of `workspace`, which must then be NULL.
ra_status_t ring_forward_impl(const void* q, const int64_t q_strides[3], const void* k, const int64_t k_strides[3],
                              const void* v, const int64_t v_strides[3], void* out, const int64_t out_strides[3],
                              ra_dtype_t dt, int64_t B, int64_t H, int64_t N, int64_t d, int32_t P,
                              const int32_t* query_blocks, int32_t n_q, float scale, int mask, float* lse,
                              void* workspace, size_t workspace_bytes, void* stream_, bool use_scratch = false) {
  ra_status_t st = check_ring(q, q_strides, k, k_strides, v, v_strides, out, out_strides, dt, B, H, N, d, P,
                              query_blocks, n_q);
  if (st != RA_OK) return st;
  if ((st = check_causal(mask, P, N)) != RA_OK) return st;
  if (lse != nullptr && ((uintptr_t)lse & 3) != 0) return fail(RA_E_INVALID_ARG, "lse is not 4-byte aligned");
  float sc;
  if ((st = resolve_scale(scale, d, &sc)) != RA_OK) return st;
  const RingLayout L = ring_layout(dt, B, H, N, d, P, n_q);
  if (use_scratch && L.total > kScratchBytes)
    return fail(RA_E_INVALID_ARG,
                "this ring needs %zu bytes of workspace, more than the %zu-byte static scratch of "
                "ra_ring_forward_noalloc",
                L.total, kScratchBytes);
  if (workspace != nullptr) {
    if (workspace_bytes < L.total)
      return fail(RA_E_INVALID_ARG, "workspace of %zu bytes is smaller than the %zu bytes needed", workspace_bytes,
                  L.total);
    if (((uintptr_t)workspace & (kAlign - 1)) != 0)
      return fail(RA_E_INVALID_ARG, "workspace is not %zu-byte aligned", kAlign);
  }
  auto qb = [&](int32_t r) { return query_blocks ? query_blocks[r] : r; };
  const Blocks& bk = L.blk;
  // Resident r's rows start at row_of[r] of q, out and the state.
  std::vector<int64_t> row_of(n_q + 1, 0);
  for (int32_t r = 0; r < n_q; ++r) row_of[r + 1] = row_of[r] + bk.len(qb(r));
  const int64_t rows = row_of[n_q];

  hipStream_t stream = (hipStream_t)stream_;
  DevRes* dr = nullptr;
  if ((st = get_dev(&dr)) != RA_OK) return st;
  std::lock_guard<std::mutex> guard(dr->mu);
  RingCleanup cleanup;  // after the lock: runs while the device's resources are still held
  cleanup.stream = stream;

  void* ws = workspace;
  if (use_scratch) {
    // Resolved once per device, with that device current (get_dev found the
    // current device's resources); the array's name is never used as an address.
    if (dr->scratch == nullptr) {
      void* ptr = nullptr;
      RA_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress (scratch)");
      dr->scratch = ptr;
    }
    ws = dr->scratch;
  }
  const bool own_ws = ws == nullptr;
  if (own_ws) {
    RA_HIP(hipMallocAsync(&ws, L.total, stream), "hipMallocAsync (ring workspace)");
    cleanup.ws = ws;
  }
  char* base = (char*)ws;
  float* m = (float*)(base + L.off_m);
  float* l = (float*)(base + L.off_l);
  float* o = (float*)(base + L.off_o);
  char* kbuf = base + L.off_k;
  char* vbuf = base + L.off_v;
  const size_t es = esize(dt);
  const int64_t bm = bk.b_max;

  const bool serial = env_flag("RA_SYNC_EACH_STEP");
  // Hand-off hazard checks (debug modes for eager calls; not for graph capture):
  // RA_DEBUG_POISON fills each slot with NaN on the caller's stream right after
  // the fold that reads it, so a refill ordered too early (a missing "freed"
  // edge) or a fold that does not wait for its copy (a missing "ready" edge)
  // shows up as NaN in the output; RA_DEBUG_DELAY_US holds the side stream
  // that long before each hand-off, so a missing "ready" edge reads stale data.
  const bool poison = env_flag("RA_DEBUG_POISON");
  const long delay_us = env_long("RA_DEBUG_DELAY_US");
  hipStream_t side = serial ? stream : dr->side;
  if (!serial) {
    RA_HIP(hipEventRecord(dr->fork, stream), "hipEventRecord");
    RA_HIP(hipStreamWaitEvent(side, dr->fork, 0), "hipStreamWaitEvent");
    cleanup.side = side;
    cleanup.join = dr->join;
  }
  // Data for step t >= 1 lives in slot (t - 1) % 2.
  auto slot_of = [](int t) { return (t - 1) & 1; };
  // Every block resident in ring order, all of one length: each slot head is
  // the sequence rotated by whole blocks (two copies per batch and tensor).
  bool rotated = n_q == P && bk.rem == 0;
  for (int32_t r = 0; rotated && r < n_q; ++r) rotated = qb(r) == r;
  // Then, for bf16 without a mask (every workgroup loads every tile of its
  // visiting block), the fold itself writes the block it visits into the
  // other slot, at the position of the next resident, which visits that block
  // at the next step: the ring's send/receive without a separate copy (the
  // tiles are already in LDS).  Fold t reads slot (t - 1) % 2 (step 0: the
  // input) and writes slot t % 2, which fold t - 1 read; the stream orders
  // them.  RA_HANDOFF_COPY=1 keeps the side-stream copies instead.
  const bool fused = rotated && dt == RA_DTYPE_BF16 && mask == ra::kMaskNone && !env_flag("RA_HANDOFF_COPY");

  for (int t = 0; t < P; ++t) {
    if (t + 1 < P && !fused) {
      // Hand-off for step t + 1 (the "send to i+1 / receive from i-1" of
      // step t), issued before step t's fold so the two overlap.
      const int s = slot_of(t + 1);
      if (!serial && t + 1 >= 3) RA_HIP(hipStreamWaitEvent(side, dr->freed[s], 0), "hipStreamWaitEvent");
      char* ks = kbuf + (size_t)s * L.slot_elems * es;
      char* vs = vbuf + (size_t)s * L.slot_elems * es;
      if (delay_us > 0)
        RA_HIP(hipLaunchHostFunc(side, sleep_cb, (void*)(intptr_t)delay_us), "hipLaunchHostFunc (delayed hand-off)");
      if (rotated) {
        // Resident r visits block r - (t + 1): per head, slot rows [0, u b) are
        // sequence rows [N - u b, N) and slot rows [u b, N) are rows [0, N - u b),
        // u = t + 1.
        const int64_t u = (int64_t)(t + 1) * bk.b;
        const size_t off = (size_t)u * d * es;
        if ((st = copy_block(ks, k, k_strides, B, H, N - u, u, L.head_rows, d, es, side)) != RA_OK) return st;
        if ((st = copy_block(ks + off, k, k_strides, B, H, 0, N - u, L.head_rows, d, es, side)) != RA_OK) return st;
        if ((st = copy_block(vs, v, v_strides, B, H, N - u, u, L.head_rows, d, es, side)) != RA_OK) return st;
        if ((st = copy_block(vs + off, v, v_strides, B, H, 0, N - u, L.head_rows, d, es, side)) != RA_OK) return st;
      } else {
        for (int32_t r = 0; r < n_q; ++r) {
          const int64_t j = ((int64_t)qb(r) - (t + 1)) % P;
          const int64_t jj = j < 0 ? j + P : j;
          const size_t off = (size_t)r * bm * d * es;
          if ((st = copy_block(ks + off, k, k_strides, B, H, bk.start(jj), bk.len(jj), L.head_rows, d, es, side)) !=
              RA_OK)
            return st;
          if ((st = copy_block(vs + off, v, v_strides, B, H, bk.start(jj), bk.len(jj), L.head_rows, d, es, side)) !=
              RA_OK)
            return st;
        }
      }
      if (!serial) RA_HIP(hipEventRecord(dr->ready[s], side), "hipEventRecord");
    }
    if (t >= 1 && !serial && !fused) RA_HIP(hipStreamWaitEvent(stream, dr->ready[slot_of(t)], 0), "hipStreamWaitEvent");

    for (int32_t r0 = 0; r0 < n_q; r0 += ra::kMaxResident) {
      const int32_t nr = n_q - r0 < ra::kMaxResident ? n_q - r0 : ra::kMaxResident;
      FoldParams p = {};
      p.q = (const char*)q + (size_t)row_of[r0] * q_strides[2] * es;
      p.out = (char*)out + (size_t)row_of[r0] * out_strides[2] * es;
      p.m = m + row_of[r0];
      p.l = l + row_of[r0];
      p.o = o + (size_t)row_of[r0] * d;
      set_strides(&p.q_sb, &p.q_sh, &p.q_sr, q_strides);
      set_strides(&p.out_sb, &p.out_sh, &p.out_sr, out_strides);
      p.st_bh = rows;
      if (t == 0) {  // the own block, read in place
        p.k = k;
        p.v = v;
        set_strides(&p.k_sb, &p.k_sh, &p.k_sr, k_strides);
        set_strides(&p.v_sb, &p.v_sh, &p.v_sr, v_strides);
        for (int32_t r = 0; r < nr; ++r) {
          p.k_off[r] = bk.start(qb(r0 + r)) * k_strides[2];
          p.v_off[r] = bk.start(qb(r0 + r)) * v_strides[2];
        }
      } else {
        const int s = slot_of(t);
        p.k = kbuf + (size_t)s * L.slot_elems * es;
        p.v = vbuf + (size_t)s * L.slot_elems * es;
        p.k_sb = p.v_sb = H * L.head_rows * d;
        p.k_sh = p.v_sh = L.head_rows * d;
        p.k_sr = p.v_sr = d;
        for (int32_t r = 0; r < nr; ++r) p.k_off[r] = p.v_off[r] = (int64_t)(r0 + r) * bm * d;
      }
      p.B = (int32_t)B;
      p.H = (int32_t)H;
      p.n_res = nr;
      // The spilled state never leaves the ring, so it may stay relative to
      // the kernels' reference maximum (kRefState).
      p.flags = (t == 0 ? 0 : ra::kLoadState) | (t == P - 1 ? ra::kWriteOut : ra::kStoreState) | ra::kRefState;
      p.scale_log2 = to_log2_scale(sc);
      p.mask = mask;
      p.P = P;
      p.blk = (int32_t)bk.b;
      p.rem = (int32_t)bk.rem;
      p.lse = lse == nullptr ? nullptr : lse + row_of[r0];
      if (fused && t + 1 < P) {
        const size_t slot_bytes = (size_t)L.slot_elems * es;
        p.send_k = kbuf + (size_t)(t & 1) * slot_bytes;
        p.send_v = vbuf + (size_t)(t & 1) * slot_bytes;
        p.send_sb = H * L.head_rows * d;
        p.send_sh = L.head_rows * d;
        for (int32_t r = 0; r < nr; ++r) p.send_off[r] = (int64_t)((r0 + r + 1) % n_q) * bm * d;
      }
      p.q_rows = 0;
      for (int32_t r = 0; r < nr; ++r) {
        const int32_t i = qb(r0 + r);
        const int32_t j = (int32_t)(((int64_t)i - t) % P + P) % P;
        p.q_blk[r] = i;
        p.kv_blk[r] = j;
        p.q_len[r] = (int32_t)bk.len(i);
        p.kv_len[r] = (int32_t)bk.len(j);
        p.q_row0[r] = row_of[r0 + r] - row_of[r0];
        if (p.q_len[r] > p.q_rows) p.q_rows = p.q_len[r];
      }
      const long pi = prof_begin(stream);
      RA_HIP(launch_fold(p, dt, (int)d, stream), "fold launch");
      prof_end(pi, stream);
    }
    if (poison && t >= 1) {
      const size_t slot_bytes = (size_t)L.slot_elems * es;
      const unsigned nan = dt == RA_DTYPE_BF16 ? kNanBf16x2 : kNanF32;
      RA_HIP(ra::launch_fill_u32(kbuf + (size_t)slot_of(t) * slot_bytes, slot_bytes, nan, stream), "poison launch");
      RA_HIP(ra::launch_fill_u32(vbuf + (size_t)slot_of(t) * slot_bytes, slot_bytes, nan, stream), "poison launch");
    }
    // The slot read by this step is refilled two steps later.
    if (t >= 1 && t + 2 <= P - 1 && !serial && !fused)
      RA_HIP(hipEventRecord(dr->freed[slot_of(t)], stream), "hipEventRecord");
  }
  if (!serial) {
    RA_HIP(hipEventRecord(dr->join, side), "hipEventRecord");
    RA_HIP(hipStreamWaitEvent(stream, dr->join, 0), "hipStreamWaitEvent");
    cleanup.side = nullptr;
  }
  if (own_ws) {
    cleanup.ws = nullptr;
    RA_HIP(hipFreeAsync(ws, stream), "hipFreeAsync (ring workspace)");
  }
  return RA_OK;
}

}  // namespace

RA_API ra_status_t ra_ring_forward(const void* q, const int64_t q_strides[3], const void* k,
                                   const int64_t k_strides[3], const void* v, const int64_t v_strides[3], void* out,
                                   const int64_t out_strides[3], ra_dtype_t dt, int64_t B, int64_t H, int64_t N,
                                   int64_t d, int32_t P, const int32_t* query_blocks, int32_t n_q, float scale,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  return ring_forward_impl(q, q_strides, k, k_strides, v, v_strides, out, out_strides, dt, B, H, N, d, P,
                           query_blocks, n_q, scale, ra::kMaskNone, nullptr, workspace, workspace_bytes, stream);
}

RA_API ra_status_t ra_ring_forward_noalloc(const void* q, const int64_t q_strides[3], const void* k,
                                           const int64_t k_strides[3], const void* v, const int64_t v_strides[3],
                                           void* out, const int64_t out_strides[3], ra_dtype_t dt, int64_t B,
                                           int64_t H, int64_t N, int64_t d, int32_t P, const int32_t* query_blocks,
                                           int32_t n_q, float scale, void* stream) {
  g_err.clear();
  return ring_forward_impl(q, q_strides, k, k_strides, v, v_strides, out, out_strides, dt, B, H, N, d, P,
                           query_blocks, n_q, scale, ra::kMaskNone, nullptr, nullptr, 0, stream, true);
}

RA_API ra_status_t ra_ring_forward_causal(const void* q, const int64_t q_strides[3], const void* k,
                                          const int64_t k_strides[3], const void* v, const int64_t v_strides[3],
                                          void* out, const int64_t out_strides[3], ra_dtype_t dt, int64_t B,
                                          int64_t H, int64_t N, int64_t d, int32_t P, const int32_t* query_blocks,
                                          int32_t n_q, float scale, ra_causal_t layout, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (!valid_layout((int)layout)) return fail(RA_E_INVALID_ARG, "unknown causal layout %d", (int)layout);
  return ring_forward_impl(q, q_strides, k, k_strides, v, v_strides, out, out_strides, dt, B, H, N, d, P,
                           query_blocks, n_q, scale, (int)layout, nullptr, workspace, workspace_bytes, stream);
}

RA_API ra_status_t ra_ring_forward_ex(const void* q, const int64_t q_strides[3], const void* k,
                                      const int64_t k_strides[3], const void* v, const int64_t v_strides[3], void* out,
                                      const int64_t out_strides[3], float* lse, ra_dtype_t dt, int64_t B, int64_t H,
                                      int64_t N, int64_t d, int32_t P, const int32_t* query_blocks, int32_t n_q,
                                      float scale, ra_causal_t layout, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  g_err.clear();
  if (!valid_layout((int)layout)) return fail(RA_E_INVALID_ARG, "unknown causal layout %d", (int)layout);
  return ring_forward_impl(q, q_strides, k, k_strides, v, v_strides, out, out_strides, dt, B, H, N, d, P,
                           query_blocks, n_q, scale, (int)layout, lse, workspace, workspace_bytes, stream);
}

namespace {

// Workspace of the ring backward: per resident row nl2 and dd, the fp32 dQ
// accumulator, then fp32 dK and dV accumulators over the whole sequence.
struct BwdLayout {
  Blocks blk;
  size_t off_nl2 = 0, off_dd = 0, off_dq = 0, off_dk = 0, off_dv = 0, total = 0;
};

BwdLayout bwd_layout(int64_t B, int64_t H, int64_t N, int64_t d, int32_t P, int32_t n_q) {
  BwdLayout L;
  L.blk = ring_blocks(N, P);
  const size_t rows = (size_t)B * H * n_q * L.blk.b_max;
  const size_t seq = (size_t)B * H * N;
  L.off_nl2 = 0;
  L.off_dd = round_up(L.off_nl2 + rows * 4);
  L.off_dq = round_up(L.off_dd + rows * 4);
  L.off_dk = round_up(L.off_dq + rows * (size_t)d * 4);
  L.off_dv = round_up(L.off_dk + seq * (size_t)d * 4);
  L.total = round_up(L.off_dv + seq * (size_t)d * 4);
  return L;
}

hipError_t launch_bwd(const ra::BwdParams& p, ra_dtype_t dt, int d, hipStream_t s) {
  hipError_t e = dt == RA_DTYPE_BF16 ? ra::launch_bwd_dq_bf16(p, d, s) : ra::launch_bwd_dq_f32(p, d, s);
  if (e != hipSuccess) return e;
  return dt == RA_DTYPE_BF16 ? ra::launch_bwd_dkdv_bf16(p, d, s) : ra::launch_bwd_dkdv_f32(p, d, s);
}

}  // namespace

RA_API size_t ra_ring_backward_workspace_bytes(ra_dtype_t dt, int64_t B, int64_t H, int64_t N, int64_t d, int32_t P,
                                               int32_t n_q) {
  const std::string saved = g_err;
  const bool ok = check_common(dt, B, H, d) == RA_OK && P >= 1 && N >= P && n_q >= 1 &&
                  N / P + 1 <= 0x7fffffffLL / 4;
  g_err = saved;
  if (!ok) return 0;
  return bwd_layout(B, H, N, d, P, n_q).total;
}

RA_API ra_status_t ra_ring_backward(const void* q, const int64_t q_strides[3], const void* k,
                                    const int64_t k_strides[3], const void* v, const int64_t v_strides[3],
                                    const void* out, const int64_t out_strides[3], const void* dout,
                                    const int64_t dout_strides[3], const float* lse, void* dq,
                                    const int64_t dq_strides[3], void* dk, const int64_t dk_strides[3], void* dv,
                                    const int64_t dv_strides[3], ra_dtype_t dt, int64_t B, int64_t H, int64_t N,
                                    int64_t d, int32_t P, const int32_t* query_blocks, int32_t n_q, float scale,
                                    ra_causal_t layout, void* workspace, size_t workspace_bytes, void* stream_) {
  g_err.clear();
  ra_status_t st = check_ring(q, q_strides, k, k_strides, v, v_strides, out, out_strides, dt, B, H, N, d, P,
                              query_blocks, n_q);
  if (st != RA_OK) return st;
  if (!valid_layout((int)layout)) return fail(RA_E_INVALID_ARG, "unknown causal layout %d", (int)layout);
  if ((st = check_causal((int)layout, P, N)) != RA_OK) return st;
  if ((st = check_tensor("dout", dout, dout_strides, dt)) != RA_OK) return st;
  if ((st = check_tile_row_stride("q", q_strides)) != RA_OK) return st;
  if ((st = check_tile_row_stride("dout", dout_strides)) != RA_OK) return st;
  if ((st = check_tensor("dq", dq, dq_strides, dt)) != RA_OK) return st;
  if ((st = check_tensor("dk", dk, dk_strides, dt)) != RA_OK) return st;
  if ((st = check_tensor("dv", dv, dv_strides, dt)) != RA_OK) return st;
  if (lse == nullptr) return fail(RA_E_INVALID_ARG, "lse is NULL");
  if (((uintptr_t)lse & 3) != 0) return fail(RA_E_INVALID_ARG, "lse is not 4-byte aligned");
  // Two residents of one block would visit the same key block in the same
  // step, and the dK/dV kernel gives each tile of keys to one workgroup per
  // resident with no atomics: their read-modify-writes of dk_acc / dv_acc
  // would race.  A ring holds each block once, so duplicates are refused.
  if (query_blocks != nullptr) {
    std::vector<char> seen(P, 0);
    for (int32_t r = 0; r < n_q; ++r) {
      if (seen[query_blocks[r]])
        return fail(RA_E_INVALID_ARG, "query_blocks[%d]=%d repeats a block; the backward needs distinct blocks",
                    (int)r, (int)query_blocks[r]);
      seen[query_blocks[r]] = 1;
    }
  }
  float sc;
  if ((st = resolve_scale(scale, d, &sc)) != RA_OK) return st;
  const BwdLayout L = bwd_layout(B, H, N, d, P, n_q);
  if (workspace != nullptr) {
    if (workspace_bytes < L.total)
      return fail(RA_E_INVALID_ARG, "workspace of %zu bytes is smaller than the %zu bytes needed", workspace_bytes,
                  L.total);
    if (((uintptr_t)workspace & (kAlign - 1)) != 0)
      return fail(RA_E_INVALID_ARG, "workspace is not %zu-byte aligned", kAlign);
  }
  auto qb = [&](int32_t r) { return query_blocks ? query_blocks[r] : r; };
  const Blocks& bk = L.blk;
  std::vector<int64_t> row_of(n_q + 1, 0);
  for (int32_t r = 0; r < n_q; ++r) row_of[r + 1] = row_of[r] + bk.len(qb(r));
  const int64_t rows = row_of[n_q];
  hipStream_t stream = (hipStream_t)stream_;
  const size_t es = esize(dt);
  const bool bf16 = dt == RA_DTYPE_BF16;

  RingCleanup cleanup;
  cleanup.stream = stream;
  void* ws = workspace;
  const bool own_ws = ws == nullptr;
  if (own_ws) {
    RA_HIP(hipMallocAsync(&ws, L.total, stream), "hipMallocAsync (backward workspace)");
    cleanup.ws = ws;
  }
  char* base = (char*)ws;
  float* nl2 = (float*)(base + L.off_nl2);
  float* dd = (float*)(base + L.off_dd);
  float* dq_acc = (float*)(base + L.off_dq);
  float* dk_acc = (float*)(base + L.off_dk);
  float* dv_acc = (float*)(base + L.off_dv);

  RA_HIP(ra::launch_bwd_prep(lse, dout, dout_strides[0], dout_strides[1], dout_strides[2], out, out_strides[0],
                             out_strides[1], out_strides[2], bf16, (int)B, (int)H, rows, (int)d, nl2, dd, stream),
         "backward set-up launch");
  RA_HIP(ra::launch_zero(dk_acc, B * H * N * d, stream), "zero launch");
  RA_HIP(ra::launch_zero(dv_acc, B * H * N * d, stream), "zero launch");

  for (int t = 0; t < P; ++t) {
    for (int32_t r0 = 0; r0 < n_q; r0 += ra::kMaxResident) {
      const int32_t nr = n_q - r0 < ra::kMaxResident ? n_q - r0 : ra::kMaxResident;
      ra::BwdParams p = {};
      p.q = (const char*)q + (size_t)row_of[r0] * q_strides[2] * es;
      p.dout = (const char*)dout + (size_t)row_of[r0] * dout_strides[2] * es;
      p.dq = (char*)dq + (size_t)row_of[r0] * dq_strides[2] * es;
      p.k = k;
      p.v = v;
      set_strides(&p.q_sb, &p.q_sh, &p.q_sr, q_strides);
      set_strides(&p.k_sb, &p.k_sh, &p.k_sr, k_strides);
      set_strides(&p.v_sb, &p.v_sh, &p.v_sr, v_strides);
      set_strides(&p.do_sb, &p.do_sh, &p.do_sr, dout_strides);
      set_strides(&p.dq_sb, &p.dq_sh, &p.dq_sr, dq_strides);
      p.nl2 = nl2 + row_of[r0];
      p.dd = dd + row_of[r0];
      p.dq_acc = dq_acc + (size_t)row_of[r0] * d;
      p.dk_acc = dk_acc;
      p.dv_acc = dv_acc;
      p.st_bh = rows;
      p.acc_bh = N;
      p.B = (int32_t)B;
      p.H = (int32_t)H;
      p.n_res = nr;
      p.flags = (t == 0 ? 0 : ra::kLoadState) | (t == P - 1 ? ra::kWriteOut : ra::kStoreState);
      p.scale = sc;
      p.scale_log2 = to_log2_scale(sc);
      p.mask = (int)layout;
      p.P = P;
      p.blk = (int32_t)bk.b;
      p.rem = (int32_t)bk.rem;
      p.q_rows = 0;
      p.kv_rows = 0;
      for (int32_t r = 0; r < nr; ++r) {
        const int32_t i = qb(r0 + r);
        const int32_t j = (int32_t)(((int64_t)i - t) % P + P) % P;
        p.q_blk[r] = i;
        p.kv_blk[r] = j;
        p.q_len[r] = (int32_t)bk.len(i);
        p.kv_len[r] = (int32_t)bk.len(j);
        p.q_row0[r] = row_of[r0 + r] - row_of[r0];
        p.k_off[r] = bk.start(j) * k_strides[2];
        p.v_off[r] = bk.start(j) * v_strides[2];
        p.acc_row0[r] = bk.start(j);
        if (p.q_len[r] > p.q_rows) p.q_rows = p.q_len[r];
        if (p.kv_len[r] > p.kv_rows) p.kv_rows = p.kv_len[r];
      }
      const long pi = prof_begin(stream);
      RA_HIP(launch_bwd(p, dt, (int)d, stream), "backward launch");
      prof_end(pi, stream);
    }
  }
  RA_HIP(ra::launch_scale_cast(dk_acc, sc, dk, dk_strides[0], dk_strides[1], dk_strides[2], bf16, (int)B, (int)H, N,
                               (int)d, stream),
         "dK cast launch");
  RA_HIP(ra::launch_scale_cast(dv_acc, 1.0f, dv, dv_strides[0], dv_strides[1], dv_strides[2], bf16, (int)B, (int)H, N,
                               (int)d, stream),
         "dV cast launch");
  if (own_ws) {
    cleanup.ws = nullptr;
    RA_HIP(hipFreeAsync(ws, stream), "hipFreeAsync (backward workspace)");
  }
  return RA_OK;
}

RA_API ra_status_t ra_profile_folds(int enable) {
  g_err.clear();
  std::lock_guard<std::mutex> g(g_prof.mu);
  g_prof.on = enable != 0;
  g_prof.used = 0;
  return RA_OK;
}

RA_API ra_status_t ra_profile_read(int64_t* launches, double* total_ms, double* max_ms) {
  g_err.clear();
  if (!launches || !total_ms || !max_ms) return fail(RA_E_INVALID_ARG, "output pointer is NULL");
  std::lock_guard<std::mutex> g(g_prof.mu);
  double tot = 0.0, mx = 0.0;
  for (size_t i = 0; i < g_prof.used; ++i) {
    RA_HIP(hipEventSynchronize(g_prof.ev[2 * i + 1]), "hipEventSynchronize");
    float ms = 0.0f;
    RA_HIP(hipEventElapsedTime(&ms, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]), "hipEventElapsedTime");
    tot += ms;
    if (ms > mx) mx = ms;
  }
  *launches = (int64_t)g_prof.used;
  *total_ms = tot;
  *max_ms = mx;
  g_prof.used = 0;
  return RA_OK;
}
