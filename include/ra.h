/*
 * ra.h -- C ABI of the ring-attention fold library (libra.so) for AMD MI355X (gfx950).
 *
 * The operation is one device's share of Ring Attention:
 *
 *   * the fold (aicassindra.com "Ring Attention, math", the per-query
 *     pseudo-code under "The online-softmax identity that makes streaming
 *     legal"; bembew.net "Ring Attention", "Conceptual Algorithm"):
 *     for every query row, with the visiting block's scores s = q.k / sqrt(d),
 *        m' = max(m, max_j s_j),  alpha = exp(m - m'),
 *        l' = alpha*l + sum_j exp(s_j - m'),
 *        o' = alpha*o + sum_j exp(s_j - m') * v_j;
 *   * the ring loop (same page, "The ring schedule" and "Accumulation math,
 *     step by step"): device i folds block (i - t) mod P on step t = 0..P-1,
 *     starting from (m, l, o) = (-inf, 0, 0) with its own block, then O_i = o / l.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *   * Tensors q, k, v, out have logical shape [B, H, rows, d] with the d axis
 *     contiguous; their strides are given in ELEMENTS as {batch, head, row}.
 *     Every such pointer must be 16-byte aligned and every stride a multiple of
 *     8 elements (bf16) or 4 elements (fp32); the row strides of k and v (and,
 *     for ra_ring_backward, of q and dout) must be below 2^24 elements
 *     (RA_E_UNSUPPORTED otherwise): those rows stream through LDS tiles
 *     addressed with 32-bit offsets.
 *   * The running state is float32 and contiguous: m, l are [B, H, rows]; o is
 *     [B, H, rows, d].  m is in natural-log units of the scaled scores, exactly
 *     as the pages define it, so it can be compared with any reference.
 *   * All data pointers are DEVICE pointers owned by the caller.  The library
 *     never frees caller memory; it owns only its optional internal workspace
 *     and a cached side stream plus events per device.
 *   * `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every call only enqueues work and returns; all of it, including work on
 *     the library's side stream, is ordered before later work on `stream`.
 *   * scale: 0 selects 1/sqrt(d); otherwise it must be finite and > 0.
 *   * d must be 64, 128 or 256.
 *   * Arguments are checked on the host before any GPU work; a bad argument
 *     returns RA_E_INVALID_ARG / RA_E_UNSUPPORTED, launches nothing and sets
 *     the text returned by ra_last_error().  HIP failures return RA_E_HIP or
 *     RA_E_OOM.  No C++ exception crosses this boundary.
 *   * No atomics are used: results are bitwise reproducible run to run on the
 *     same GPU and build.
 */
#ifndef RA_H
#define RA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RA_OK = 0,
  RA_E_INVALID_ARG = 1, /* null pointer, bad size, bad stride, bad scale, workspace too small */
  RA_E_UNSUPPORTED = 2, /* valid request this build does not implement (d, N % P != 0, ...) */
  RA_E_HIP = 3,         /* a HIP runtime call or kernel launch failed */
  RA_E_OOM = 4          /* the internal workspace could not be allocated */
} ra_status_t;

typedef enum { RA_DTYPE_F32 = 0, RA_DTYPE_BF16 = 1 } ra_dtype_t;

/*
 * Causal masking and the token layout it assumes.  A query sees only keys at
 * or before its own position (math page, "Causal masking, load balance, and
 * other wrinkles"; bembew.net "Implementation Considerations", causal
 * masking).  The ring's N = P*b tokens are dealt to the P devices in one of
 * three ways (vibeengines.com, "The causal-mask catch"); row r of device j's
 * block (b = N/P rows when P divides N; see "Blocks of the ring") holds
 * sequence position
 *   RA_CAUSAL_CONTIGUOUS: start_j + r, start_j = j*b + min(j, N mod P)
 *   RA_CAUSAL_STRIPED:    r*P + j                     (tokens handed out in turn)
 *   RA_CAUSAL_ZIGZAG:     j*h + r          for r < h  (h = b/2: chunk j and its
 *                         (2P-1-j)*h + r-h for r >= h  mirror chunk 2P-1-j)
 * RA_CAUSAL_NONE is full (non-causal) attention.  In every layout positions
 * rise with r, so the keys a query row sees form a prefix of each block; the
 * kernels skip whole key tiles past the last visible key (a block entirely in
 * a row's future costs no arithmetic) and mask keys only inside the tiles
 * that straddle the boundary.  A row that sees no key of a block keeps its
 * state exactly as it was (m' = -inf is guarded: alpha = 1, weights 0).
 */
typedef enum {
  RA_CAUSAL_NONE = 0,
  RA_CAUSAL_CONTIGUOUS = 1,
  RA_CAUSAL_STRIPED = 2,
  RA_CAUSAL_ZIGZAG = 3
} ra_causal_t;

/*
 * ra_state_init -- set (m, l, o) = (-inf, 0, 0) for B*H*rows query rows.
 * Math page, "Accumulation math, step by step" (loop set-up).
 * m, l: [B, H, rows] float32; o: [B, H, rows, d] float32; all contiguous.
 * rows == 0 is a no-op (the pointers may then be NULL).
 */
ra_status_t ra_state_init(float* m, float* l, float* o, int64_t B, int64_t H, int64_t rows, int64_t d,
                          void* stream);

/*
 * ra_fold_block -- fold ONE visiting K/V block into the running state.
 * Math page, the per-query pseudo-code under the online-softmax identity;
 * bembew.net "Conceptual Algorithm", the loop body.
 *
 * q: [B, H, q_rows, d], k and v: [B, H, kv_rows, d], all of dtype `dt`, strides
 * in elements {batch, head, row}.  m, l, o: the state of the q_rows query rows
 * (layout above), read and updated in place.  Scores are computed with fp32
 * accumulation; for bf16 the weights exp(s - m') are rounded to bf16 before
 * the value product and l sums the same rounded weights.  Blocks may be folded
 * in any order (the math page's worked example: the result does not depend on
 * the order).  kv_rows == 0 leaves the state unchanged (k and v may then be
 * NULL); q_rows == 0 is a no-op (every pointer may then be NULL).  Any
 * q_rows, kv_rows >= 0 are accepted (ragged tails are masked).
 */
ra_status_t ra_fold_block(const void* q, const int64_t q_strides[3], const void* k, const int64_t k_strides[3],
                          const void* v, const int64_t v_strides[3], ra_dtype_t dt, int64_t B, int64_t H,
                          int64_t q_rows, int64_t kv_rows, int64_t d, float scale, float* m, float* l, float* o,
                          void* stream);

/*
 * ra_fold_block_causal -- ra_fold_block under a causal mask: the query block
 * is device q_block's and the visiting block device kv_block's of a P-device
 * ring over N tokens in the given layout, 0 <= q_block, kv_block < P.  The
 * blocks' row counts follow from N and P (see "Blocks of the ring" below): q
 * and the state hold block q_block's rows, k and v block kv_block's.
 * Arguments and state otherwise as for ra_fold_block.  RA_CAUSAL_ZIGZAG needs
 * N a multiple of 2P; N must stay below 2^31.  layout RA_CAUSAL_NONE folds the
 * same two blocks without a mask.  A pair with no visible key (for instance
 * kv_block > q_block in the contiguous layout) leaves the state bit for bit as
 * it was.
 */
ra_status_t ra_fold_block_causal(const void* q, const int64_t q_strides[3], const void* k,
                                 const int64_t k_strides[3], const void* v, const int64_t v_strides[3],
                                 ra_dtype_t dt, int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                                 ra_causal_t layout, int32_t P, int32_t q_block, int32_t kv_block, float* m,
                                 float* l, float* o, void* stream);

/*
 * ra_finalize -- O = o / l after the last block (math page, end of the loop).
 * l: [B, H, rows], o: [B, H, rows, d] (float32, contiguous); out: [B, H, rows, d]
 * of dtype out_dt with strides out_strides (elements).  Rows with l == 0 (never
 * folded) are written as 0.  The cast to bf16 rounds to nearest even.
 * rows == 0 is a no-op (the pointers may then be NULL).
 */
ra_status_t ra_finalize(const float* l, const float* o, void* out, const int64_t out_strides[3], ra_dtype_t out_dt,
                        int64_t B, int64_t H, int64_t rows, int64_t d, void* stream);

/*
 * Blocks of the ring.  N tokens are split over P devices, 1 <= P <= N.  When P
 * divides N every block holds b = N/P rows; otherwise (bembew.net
 * "Implementation Considerations": padding or dynamic partitioning) the first
 * N mod P devices hold N/P + 1 rows and the others N/P, so block j starts at
 * row j*(N/P) + min(j, N mod P).  Handing tokens out in turn (the striped
 * layout) gives exactly these sizes.
 */

/*
 * ra_ring_workspace_bytes -- device workspace ra_ring_forward needs: the fp32
 * state of the n_q resident query blocks plus, per resident block, the
 * visiting K/V double buffer (two blocks, not P: math page, "Memory: O(1)
 * extra per device").  Returns 0 for arguments ra_ring_forward would reject.
 */
size_t ra_ring_workspace_bytes(ra_dtype_t dt, int64_t B, int64_t H, int64_t N, int64_t d, int32_t P,
                               int32_t n_q);

/*
 * ra_ring_forward -- the whole per-device loop for n_q resident query blocks
 * of a P-device ring, run as P virtual ring steps on one GPU.
 * Math page, "Sharding the sequence", "The ring schedule", "Accumulation math,
 * step by step"; bembew.net "Conceptual Algorithm".
 *
 * q:   [B, H, rows, d] -- the resident query blocks stacked along rows in
 *      query_blocks order (rows = the sum of their block sizes, n_q*N/P when P
 *      divides N); strides q_strides.
 * k,v: [B, H, N, d] -- the whole sequence; block j is its rows as given under
 *      "Blocks of the ring" (rows [j*b, (j+1)*b) when P divides N).
 * out: [B, H, rows, d] -- like q; receives O_i = o / l.
 * query_blocks: HOST array of n_q block ids in [0, P); NULL means 0..P-1
 *      (then n_q must equal P).
 * On step t resident block i folds block (i - t) mod P.  Step 0 reads the own
 * block in place; the next block is moved into the other half of a per-block
 * double buffer while the current step's fold runs (the stand-in for the
 * ring's send to i+1 / receive from i-1):
 *   * every block resident in ring order (query_blocks NULL or 0..P-1), P
 *     dividing N, bf16: the fold kernel itself writes the block it visits,
 *     from LDS, to the next resident's place in the other half (stream order
 *     separates the writer and the readers; environment variable
 *     RA_HANDOFF_COPY=1 selects the copies below instead);
 *   * otherwise hipMemcpy2DAsync on a side stream, ordered by events: with
 *     every block resident in ring order and P dividing N (fp32), the blocks
 *     of one step are the sequence rotated by whole blocks, copied as two
 *     contiguous pieces per batch and tensor; else block by block.
 * The (m, l, o) spilled between the ring's steps stays inside the workspace;
 * for bf16 (d = 64, 128, 256) it is kept relative to a reference maximum at
 * most the running maximum (raised lazily) instead of the running maximum
 * itself.  O equals that of the same folds through ra_fold_block followed by
 * ra_finalize up to rounding, not bit for bit.
 * workspace: device buffer of at least ra_ring_workspace_bytes(...) bytes,
 *      256-byte aligned, or NULL to let the library allocate and free one in
 *      stream order.  Two calls that share a workspace must be ordered on
 *      their streams.
 */
ra_status_t ra_ring_forward(const void* q, const int64_t q_strides[3], const void* k, const int64_t k_strides[3],
                            const void* v, const int64_t v_strides[3], void* out, const int64_t out_strides[3],
                            ra_dtype_t dt, int64_t B, int64_t H, int64_t N, int64_t d, int32_t P,
                            const int32_t* query_blocks, int32_t n_q, float scale, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * ra_ring_forward_noalloc -- ra_ring_forward for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, checks, schedule and kernels as
 * ra_ring_forward with a NULL workspace, but the workspace is a static device
 * array of RA_NOALLOC_SCRATCH_BYTES bytes inside the library instead of an
 * allocation: the call allocates and frees nothing.
 *   * A ring whose ra_ring_workspace_bytes(...) exceeds RA_NOALLOC_SCRATCH_BYTES
 *     is rejected with RA_E_INVALID_ARG before any GPU work.
 *   * Each GPU the library runs on holds its own copy of the array until the
 *     process ends; its address is resolved on the first call on that device,
 *     which also creates the device's side stream and events (as the first
 *     ring call of any kind does): make that first call outside graph capture.
 *   * Every call on one GPU shares that GPU's array and leaves the last call's
 *     contents in it; nothing in it needs to start at zero (each call writes
 *     every byte it reads).  Calls that may run at the same time on one GPU
 *     (on different streams, or captured in graphs launched concurrently) race
 *     on it: order them.
 */
#define RA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
ra_status_t ra_ring_forward_noalloc(const void* q, const int64_t q_strides[3], const void* k,
                                    const int64_t k_strides[3], const void* v, const int64_t v_strides[3], void* out,
                                    const int64_t out_strides[3], ra_dtype_t dt, int64_t B, int64_t H, int64_t N,
                                    int64_t d, int32_t P, const int32_t* query_blocks, int32_t n_q, float scale,
                                    void* stream);

/*
 * ra_ring_forward_causal -- ra_ring_forward under a causal mask.  q, k, v and
 * out are in the layout's device order: block j is device j's share, holding
 * the positions given above for `layout` (contiguous: block j's first
 * position is its first row's index in the sequence).  Every other argument,
 * the workspace and the schedule are those of ra_ring_forward;
 * RA_CAUSAL_ZIGZAG needs N a multiple of 2P and N must stay below 2^31.
 * Steps whose visiting block lies entirely in the resident block's future
 * fold nothing (the hand-off still moves the block, as the ring would).
 * Every row sees at least its own position, so no output row has l = 0.
 */
ra_status_t ra_ring_forward_causal(const void* q, const int64_t q_strides[3], const void* k,
                                   const int64_t k_strides[3], const void* v, const int64_t v_strides[3], void* out,
                                   const int64_t out_strides[3], ra_dtype_t dt, int64_t B, int64_t H, int64_t N,
                                   int64_t d, int32_t P, const int32_t* query_blocks, int32_t n_q, float scale,
                                   ra_causal_t layout, void* workspace, size_t workspace_bytes, void* stream);

/*
 * ra_ring_forward_ex -- ra_ring_forward_causal (RA_CAUSAL_NONE: ra_ring_forward)
 * that also writes, when lse is not NULL, each resident row's log-sum-exp
 * L = m + ln l (natural log, the scaled scores' units) into lse: float32
 * [B, H, rows] contiguous, rows stacked like q; -inf for a row that saw no
 * key.  The backward pass needs L to rebuild the attention weights.
 */
ra_status_t ra_ring_forward_ex(const void* q, const int64_t q_strides[3], const void* k, const int64_t k_strides[3],
                               const void* v, const int64_t v_strides[3], void* out, const int64_t out_strides[3],
                               float* lse, ra_dtype_t dt, int64_t B, int64_t H, int64_t N, int64_t d, int32_t P,
                               const int32_t* query_blocks, int32_t n_q, float scale, ra_causal_t layout,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * ra_ring_backward_workspace_bytes -- device workspace ra_ring_backward needs:
 * per resident row two floats and a float32 dQ row, plus float32 dK and dV
 * accumulators over the whole sequence ([B, H, N, d] each).  Returns 0 for
 * arguments ra_ring_backward would reject.
 */
size_t ra_ring_backward_workspace_bytes(ra_dtype_t dt, int64_t B, int64_t H, int64_t N, int64_t d, int32_t P,
                                        int32_t n_q);

/*
 * ra_ring_backward -- the backward pass on the same ring (vibeengines.com "Ring
 * attention, explained", method step 6): on step t resident block i folds
 * block j = (i - t) mod P, adding to its own dQ_i and to the visiting block's
 * dK_j, dV_j accumulators (which, on a real ring, travel with the block).
 * With P = softmax weights rebuilt from lse: dV = P^T dO, dP = dO V^T,
 * D = rowsum(dO * O), dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q.
 *
 * q, k, v, layout, query_blocks, n_q, scale: exactly as given to the forward;
 *      the block ids in query_blocks must be distinct (RA_E_INVALID_ARG
 *      otherwise: two residents of one block would add to the same dK, dV rows
 *      at once).
 * out, lse: the forward's output and log-sum-exp (ra_ring_forward_ex).
 * dout: dL/dO, like out.  dq: like q, receives dL/dQ of the resident rows.
 * dk, dv: [B, H, N, d] like k and v, overwritten with the resident blocks'
 *      shares of dL/dK and dL/dV (the full gradients when every block is
 *      resident).  All of dtype dt; strides in elements.
 * Accumulation is in float32; bf16 inputs use bf16 MFMA products with the
 * weights and dS rounded to bf16.  K and V are read in place (one GPU: the
 * blocks do not move).  workspace: at least ra_ring_backward_workspace_bytes
 * bytes, 256-byte aligned, or NULL for a stream-ordered internal one.
 */
ra_status_t ra_ring_backward(const void* q, const int64_t q_strides[3], const void* k, const int64_t k_strides[3],
                             const void* v, const int64_t v_strides[3], const void* out,
                             const int64_t out_strides[3], const void* dout, const int64_t dout_strides[3],
                             const float* lse, void* dq, const int64_t dq_strides[3], void* dk,
                             const int64_t dk_strides[3], void* dv, const int64_t dv_strides[3], ra_dtype_t dt,
                             int64_t B, int64_t H, int64_t N, int64_t d, int32_t P, const int32_t* query_blocks,
                             int32_t n_q, float scale, ra_causal_t layout, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * Measurement support (not part of the method).  While enabled on the calling
 * process, the ring drivers record a HIP event pair around every fold launch
 * (forward) and every step's dQ + dK/dV launch pair (backward), on the
 * caller's stream that the launches use.  ra_profile_read waits for the
 * recorded events, returns the number of fold launches, their summed and
 * largest durations in milliseconds, and clears the record.  Enabling or
 * disabling also clears it.  At most 4096 launches are recorded; later ones
 * are not timed (the count says how many were).
 */
ra_status_t ra_profile_folds(int enable);
ra_status_t ra_profile_read(int64_t* launches, double* total_ms, double* max_ms);

/* Text of the last error on the calling thread ("" after success).  Valid
 * until the next ra_* call on the same thread. */
const char* ra_last_error(void);

/* Library version, "major.minor.patch". */
const char* ra_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RA_H */
