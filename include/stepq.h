/*
 * stepq.h -- C ABI of libstepq.so, the MI355X (gfx950) STEPQuant packed-state decode step.
 *
 * The method (page: "STEPQuant" paper digest, vibe-research silicon-writer readme):
 *   Background -- a Gated-DeltaNet / Kimi-Delta-Attention head keeps a d_k x d_v recurrent
 *   state S that each decode step updates from key k, value v and retention gate and reads out
 *   with query q; A_t holds both the gate and the delta update.  Here
 *       S_t = A_t S_{t-1} + beta_t k_t v_t^T,   A_t = Diag(a)(I - beta_t k_t k_t^T),
 *       o_t = S_t^T q_t,
 *   with a_i = alpha (one scalar) for GDN and a per-key-row vector alpha_i for KDA.
 *   Method 3 -- the state is stored as X_hat[i,j] = r_i c_j z[i,j]: a row factor, a column factor
 *   and a low-bit integer code per entry (widths 2/4/6/8, Method 1), with a few FP16 pivot units
 *   stored raw.
 *   Method 4 -- per step: reconstruct the tile, run retention + delta update + readout on the
 *   float tile, hand the output on without waiting for requantization, refit r and c, and pack
 *   codes and factors back in place, with no resident FP32 copy of the state.
 *
 * Conventions for every call:
 *   - Device pointers are HIP device memory on the plan's device, owned by the caller, fp32
 *     unless stated, C-contiguous.  The pool must be 256-byte aligned.
 *   - stream is a hipStream_t cast to void* (NULL = the default stream).  Calls only enqueue
 *     work; faults inside kernels surface at the caller's next synchronisation.
 *   - Every int-returning call returns STEPQ_OK (0) or a negative STEPQ_ERR_* code and sets the
 *     calling thread's message (stepq_last_error).  No C++ exception crosses this boundary.
 *   - The pool is updated in place: calls on the same plan and pool must be ordered by the
 *     caller (same stream, or events).
 */
#ifndef STEPQ_H
#define STEPQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct stepq_plan* stepq_plan_t;

enum {
  STEPQ_OK = 0,
  STEPQ_ERR_INVALID_ARG = -1, /* bad pointer, size, width, omega, batch (B < 0, B above
                                 max_batch in split mode, B * n_heads above INT_MAX) ...   */
  STEPQ_ERR_UNSUPPORTED = -2, /* valid but not built (e.g. d_k != d_v)                   */
  STEPQ_ERR_HIP = -3,         /* a HIP runtime call failed; message has the HIP error    */
  STEPQ_ERR_OOM = -4,         /* device or host allocation failed                        */
  STEPQ_ERR_NOT_READY = -5    /* reserved                                                */
};

enum { STEPQ_KIND_GDN = 0, STEPQ_KIND_KDA = 1 };
enum { STEPQ_MODE_FUSED = 0, STEPQ_MODE_SPLIT = 1 };
/* gate order of A_t (see stepq_plan_desc.order) */
enum { STEPQ_ORDER_DELTA_FIRST = 0, STEPQ_ORDER_DECAY_FIRST = 1 };

/* status word bits (stepq_get_status) */
#define STEPQ_FLAG_NONFINITE 1u /* a row of an updated state was not finite               */
#define STEPQ_FLAG_SCALE_OVF 2u /* a row or column factor overflowed binary16             */
#define STEPQ_FLAG_PIVOT_OVF 4u /* an FP16 pivot entry overflowed binary16                */
#define STEPQ_FLAG_BAD_SLOT 8u  /* a slot index outside [0, n_slots) other than -1          */

/*
 * Plan description (Method 1: the offline precision map, pivots and impact scores).
 *   kind      STEPQ_KIND_GDN: the allocation unit is a head -- every row of a head has the same
 *             width and either all or none of a head's rows are pivots.  STEPQ_KIND_KDA: the
 *             unit is a key row -- widths and pivot flags may vary row by row.
 *   n_heads   heads per request (one layer), 1 .. 65535.
 *   d_k, d_v  state shape; the library supports d_k == d_v in {64, 128}.
 *   bits      [n_heads * d_k] int8, widths in {2, 4, 6, 8} (ignored on pivot rows).
 *   pivot     [n_heads * d_k] uint8, 1 = FP16 pivot row (stored raw, not quantized).
 *   omega     [n_heads * d_k] float, row impact omega_i = E[(A_t^T q_t)_i^2] (Method 2),
 *             finite and >= 0.
 *   mode      STEPQ_MODE_FUSED: one kernel per step.  STEPQ_MODE_SPLIT: the readout kernel runs
 *             on the caller's stream and the refit + pack kernel on a library-owned side stream
 *             (Method 4: scale fitting and packed writeback overlap later layers).
 *   max_batch largest B any call will pass (sizes the split-mode hand-over buffer).
 *   device    HIP device ordinal the plan lives on.
 *   order     how A_t composes the gate and the delta update (Background: A_t holds both).
 *             STEPQ_ORDER_DELTA_FIRST: A_t = Diag(a)(I - beta k k^T), the reading this library
 *             takes by default.  STEPQ_ORDER_DECAY_FIRST: A_t = (I - beta k k^T) Diag(a), the rows
 *             decay before the delta update (the key projection sees the decayed state).  For
 *             GDN's scalar gate the two are one map and differ only in rounding.
 * All host arrays are copied; the caller may free them after the call.
 */
typedef struct {
  int kind;
  int n_heads;
  int d_k, d_v;
  const int8_t* bits;
  const uint8_t* pivot;
  const float* omega;
  int mode;
  int max_batch;
  int device;
  int order;
} stepq_plan_desc;

/* Validate desc, build the packed layout and upload the plan tables to the device. */
int stepq_plan_create(const stepq_plan_desc* desc, stepq_plan_t* out);

/* Wait for the plan's side-stream work, then release everything the plan owns.  NULL is a
   no-op. */
int stepq_plan_destroy(stepq_plan_t plan);

/* Bytes of one request's packed state (all heads; 256-byte multiple) and the actual stored
   bits per state value (codes + binary16 factors + binary16 pivots + padding).  Either output
   may be NULL.  Pool size = B * bytes_per_request. */
int stepq_pool_bytes(stepq_plan_t plan, size_t* bytes_per_request, double* bits_per_value);

/* Byte offset and size of head h's segment inside one request's packed state. */
int stepq_head_segment(stepq_plan_t plan, int head, size_t* offset, size_t* bytes);

/* Encode fp32 states S [B, n_heads, d_k, d_v] into pool [B * bytes_per_request] (the refit and
   pack half of a step: row factors, first quantization, weighted least-squares column refit,
   final requantization; pivots rounded to binary16).  Used to enter a state produced outside
   the decode path (e.g. after prefill). */
int stepq_encode_state(stepq_plan_t plan, const float* S, void* pool, int B, void* stream);

/*
 * One decode step for B requests (Method 4).  In:
 *   pool   [B * bytes_per_request] packed states, updated in place;
 *   q, k, v [B, n_heads, d] (q and k as the model produced them; no scaling is applied);
 *   alpha  GDN: [B, n_heads];  KDA: [B, n_heads, d_k];
 *   beta   [B, n_heads].
 * Out: out [B, n_heads, d_v] = S_t^T q_t computed on the updated float tile before
 * requantization.  In split mode out is complete when the work on `stream` is; the pool is
 * complete when the side stream's work is, and the next call on this plan (any pool) makes
 * `stream` wait for it.  In split mode the inputs are consumed by the stream-side kernel; the
 * caller may reuse them once the work on `stream` has completed.
 * Graph capture: a fused plan's decode, encode and unpack calls only enqueue kernels on
 * `stream`, so they may be captured into a HIP graph and replayed (each replay is one more step
 * on the same buffers).  A split-mode plan returns STEPQ_ERR_UNSUPPORTED on a capturing stream:
 * its side stream is joined back lazily, by the plan's next call.
 */
int stepq_decode_step(stepq_plan_t plan, void* pool, int B, const float* q, const float* k,
                      const float* v, const float* alpha, const float* beta, float* out,
                      void* stream);

/*
 * Slot-indexed pools.  The digest runs the packed kernel inside a serving framework whose
 * request state lives in a shared pool addressed by per-request slot indices (Method 4 and its
 * deployment notes: the state pool grows with concurrency); these two calls take such a pool.
 *   pool     [n_slots * bytes_per_request], 256-byte aligned: slot s is the packed state of one
 *            request, laid out exactly as one row of the plain calls' pool.
 *   slots    device int32 [B]: batch row b (its q, k, v, alpha, beta, out and S rows) uses
 *            slot slots[b].  slots[b] = -1 marks a padding row: its slot, stash and out row are
 *            not touched.  Any other value outside [0, n_slots) is skipped the same way and
 *            raises STEPQ_FLAG_BAD_SLOT.  Two rows must not name the same slot (they would race).
 * Everything else -- argument meaning, layout, ordering, split-mode streams -- is as for
 * stepq_decode_step and stepq_encode_state; with slots[b] = b and n_slots = B the results are
 * identical to theirs.  In split mode the readout kernel copies the resolved slots into a
 * plan-owned buffer, so the caller may reuse `slots` once the work on `stream` has completed.
 */
int stepq_decode_step_slots(stepq_plan_t plan, void* pool, int n_slots, const int32_t* slots,
                            int B, const float* q, const float* k, const float* v,
                            const float* alpha, const float* beta, float* out, void* stream);
int stepq_encode_state_slots(stepq_plan_t plan, const float* S, void* pool, int n_slots,
                             const int32_t* slots, int B, void* stream);

/*
 * stepq_decode_step without any device allocation, for callers that cannot allocate: code that
 * must not call hipMalloc (tight serving loops, harnesses that forbid allocation).  Arguments,
 * layout, results and stream ordering are those of stepq_decode_step; the results are
 * bit-identical to it.
 *   Fused plan: the same kernel as stepq_decode_step (it uses no scratch memory).
 *   Split plan: the readout kernel hands its per-tile update factors to the side-stream
 *   writeback through a library-static device array of 32 MiB per GPU (held from the plan's
 *   creation until the process ends) instead of the plan's own buffer; B may exceed the plan's
 *   max_batch up to that array's size: B * n_heads * d_k * 16 bytes <= 32 MiB (16384 tiles at
 *   d_k = 128, 32768 at 64).  Larger B: STEPQ_ERR_INVALID_ARG, nothing enqueued.
 * Every split plan on one GPU shares that GPU's array, which keeps the last call's contents.  A
 * call waits (on `stream`) for the previous call's writeback on the same GPU before its readout
 * overwrites the array, so calls issued one after another from one host thread are ordered;
 * calls issued concurrently from several host threads on one GPU race.  The call allocates
 * nothing: no hipMalloc, hipFree or allocating library routine (the array's device address is
 * resolved once per GPU when a split plan is created there).
 */
int stepq_decode_step_noalloc(stepq_plan_t plan, void* pool, int B, const float* q,
                              const float* k, const float* v, const float* alpha,
                              const float* beta, float* out, void* stream);

/* Debug decode of a pool: S_hat [B, n_heads, d_k, d_v] = r_i c_j z_ij (pivots as stored),
   r [B, n_heads, d_k] and c [B, n_heads, d_v] binary16 bit patterns, z [B, n_heads, d_k, d_v]
   codes (0 on pivot rows).  Any output may be NULL. */
int stepq_unpack_debug(stepq_plan_t plan, const void* pool, int B, float* S_hat, uint16_t* r,
                       uint16_t* c, int8_t* z, void* stream);

/* Wait for all work the plan enqueued (both streams), then read (and optionally clear) the
   status word accumulated by its kernels. */
int stepq_get_status(stepq_plan_t plan, uint32_t* flags, int reset);

/* Wait for the plan's side stream (split mode) to drain. */
int stepq_sync(stepq_plan_t plan);

/* Test hook for the split-mode ordering: before each side-stream writeback, spin for `cycles`
   GPU clocks (bounded, 0 = off, at most 2e9).  A missing wait between a writeback and the next
   step's readout would then make that readout consume stale codes. */
int stepq_debug_side_delay(stepq_plan_t plan, long long cycles);

/* Thread-local message describing the last failed call on this thread ("" if none). */
const char* stepq_last_error(void);

/* ---------------------------------------------------------------------------------------- */
/* Offline planning on the host (Method 1, Method 2).  binary64, host pointers.            */
/* ---------------------------------------------------------------------------------------- */

/* L_u = sum_{j=0}^{H-1} exp(2 j l_u) for n units (Method 1, lifetime weight over the next H
   steps; l_u = mean log retention gate of unit u, <= 0). */
int stepq_lifetime_weights(const double* l_u, int n, int H, double* L_out);

/* Accumulate row impact (Method 2): for n samples of one head, g = A^T q with A as selected by
   order (STEPQ_ORDER_DELTA_FIRST: Diag(a)(I - beta k k^T), g = a*q - beta k (k . (a*q));
   STEPQ_ORDER_DECAY_FIRST: (I - beta k k^T) Diag(a), g = a*(q - beta k (k . q)));
   acc[i] += sum over samples of g_i^2.  q, k, a: [n, d] float, beta: [n] float.
   omega = acc / (number of samples) once all samples are in. */
int stepq_row_impact_accumulate(int n, int d, const float* q, const float* k, const float* a,
                                const float* beta, int order, double* acc);

/* Row impact on the device (Method 2), for calibration before any plan exists.  For every head
   h of one layer and each of the B requests of one step: g = A^T q with A as selected by order
   (as for stepq_row_impact_accumulate); acc[h*d + i] += sum over the requests of g_i^2, in
   binary64 (requests in index order, so the result is deterministic).
     kind   STEPQ_KIND_GDN (alpha [B, n_heads]) or STEPQ_KIND_KDA (alpha [B, n_heads, d]);
     order  STEPQ_ORDER_DELTA_FIRST or STEPQ_ORDER_DECAY_FIRST;
     q, k   [B, n_heads, d] fp32 device;  beta [B, n_heads] fp32 device;
     acc    [n_heads * d] binary64 device, added to (zero it before the first step).
   d in {64, 128}.  omega = acc / (requests x steps accumulated).  Enqueued on `stream` on the
   current device. */
int stepq_row_impact_gpu(int kind, int order, int n_heads, int d, int B, const float* q,
                         const float* k, const float* alpha, const float* beta, double* acc,
                         void* stream);

/* The n_pivots units of largest risk (e.g. L_u d_u(b_max)); ties to the lower index.
   out_idx [n_pivots] ascending. */
int stepq_select_pivots(const double* risk, int n, int n_pivots, int32_t* out_idx);

/* Multiple-choice DP over equal-size units (GDN, unit = head): minimise sum_u cost[u][c]
   subject to sum_u choices[c_u] <= capacity_bits.  cost [n_units, n_choices] row-major,
   choices ascending even widths.  bits_out [n_units]; objective may be NULL. */
int stepq_alloc_mcdp(const double* cost, int n_units, const int* choices, int n_choices,
                     long capacity_bits, int* bits_out, double* objective);

/* Lagrangian allocation with discrete budget repair (KDA, unit = key row): minimise
   sum_u L_u d_u(b_u) subject to sum_u n_u b_u <= budget_bits.  d [n_units, n_choices]
   row-major, n [n_units] unit sizes, choices ascending.  bits_out [n_units]. */
int stepq_alloc_lagrangian(const double* L, const double* d, const double* n, int n_units,
                           const int* choices, int n_choices, double budget_bits, int iters,
                           int* bits_out, double* objective);

#ifdef __cplusplus
}
#endif
#endif /* STEPQ_H */
