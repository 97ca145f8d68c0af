// stepq_api.cpp -- host side of libstepq.so: argument checks, packed layout, plan tables,
// launches and stream ordering.  The ABI is declared (and each call documented) in stepq.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "stepq.h"
#include "stepq_internal.h"

using namespace stepq;

namespace stepq {

namespace {
thread_local std::string g_err;
}  // namespace

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

void clear_error() { g_err.clear(); }

const char* last_error() { return g_err.c_str(); }

}  // namespace stepq

namespace {

int ok() {
  clear_error();
  return STEPQ_OK;
}

#define HIP_TRY(expr)                                                                    \
  do {                                                                                   \
    hipError_t e_ = (expr);                                                              \
    if (e_ != hipSuccess)                                                                \
      return fail(STEPQ_ERR_HIP, "%s failed: %s", #expr, hipGetErrorString(e_));         \
  } while (0)

// Pairwise tree sum in binary32, the same evaluation order as the kernels' reductions.
float tree_sum(const float* x, int n) {
  if (n == 1) return x[0];
  return tree_sum(x, n / 2) + tree_sum(x + n / 2, n - n / 2);
}

// Makes the plan's device current and restores the caller's on scope exit; when it is already
// current (the usual case) no device switch is made either way.
struct DeviceGuard {
  int prev = -1;
  bool ok_ = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) {
      prev = -1;
      return;
    }
    if (prev == dev) {
      prev = -1;
      ok_ = true;
      return;
    }
    if (hipSetDevice(dev) == hipSuccess) ok_ = true;
  }
  ~DeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

}  // namespace

struct stepq_plan {
  int kind = 0, H = 0, D = 0, mode = 0, max_batch = 0, device = 0;
  long long bpr = 0;
  double bpv = 0.0;
  std::vector<long long> head_off, head_bytes;
  void* dtab = nullptr;     // all device tables in one allocation
  unsigned* status = nullptr;
  float* stash = nullptr;   // split-mode hand-over
  int* slot_stash = nullptr; // split mode: each row's resolved pool slot, for the writeback
  DevPlan dp{};
  hipStream_t side = nullptr;
  hipEvent_t ev_read = nullptr, ev_write = nullptr;
  bool write_pending = false;
  long long spin_cycles = 0;
  void* scratch = nullptr;   // split mode: this device's scratch array (no-allocation entry)
};

namespace {
// Per device, the split plan whose side-stream writeback last read the device scratch through
// stepq_decode_step_noalloc: the next such call waits for that writeback before its readout
// kernel overwrites the hand-over.
std::mutex g_scratch_mu;
stepq_plan* g_scratch_owner[64] = {};
}  // namespace

namespace {

int check_plan(stepq_plan_t p) {
  if (!p) return fail(STEPQ_ERR_INVALID_ARG, "plan is NULL");
  return STEPQ_OK;
}

void destroy_plan(stepq_plan* p) {
  if (!p) return;
  if (p->side) (void)hipStreamSynchronize(p->side);
  {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (p->device >= 0 && p->device < 64 && g_scratch_owner[p->device] == p)
      g_scratch_owner[p->device] = nullptr;
  }
  if (p->ev_read) (void)hipEventDestroy(p->ev_read);
  if (p->ev_write) (void)hipEventDestroy(p->ev_write);
  if (p->side) (void)hipStreamDestroy(p->side);
  if (p->stash) (void)hipFree(p->stash);
  if (p->slot_stash) (void)hipFree(p->slot_stash);
  if (p->dtab) (void)hipFree(p->dtab);
  delete p;
}

// Orders `stream` after the plan's pending side-stream writeback (split mode).
hipError_t wait_writeback(stepq_plan* p, hipStream_t stream) {
  if (p->mode == STEPQ_MODE_SPLIT && p->write_pending) return hipStreamWaitEvent(stream, p->ev_write, 0);
  return hipSuccess;
}

// One workgroup per (request, head) on a (B, n_heads) grid; the tile count B * n_heads is kept
// below INT_MAX (tile indices and the split-mode hand-over size are computed from it).
int check_grid(const stepq_plan* p, int B) {
  if ((long long)B * p->H > INT_MAX)
    return fail(STEPQ_ERR_INVALID_ARG, "B * n_heads = %lld exceeds the launch grid",
                (long long)B * p->H);
  return STEPQ_OK;
}

// A split-mode plan joins its side stream back lazily (the next call waits for the pending
// writeback), which a stream capture cannot express: such plans refuse to run on a capturing
// stream.  Fused plans enqueue kernels only and can be captured.
int refuse_capture(stepq_plan* p, hipStream_t stream, const char* what) {
  if (p->mode != STEPQ_MODE_SPLIT) return STEPQ_OK;
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &st) == hipSuccess && st != hipStreamCaptureStatusNone)
    return fail(STEPQ_ERR_UNSUPPORTED, "%s: a split-mode plan cannot run on a capturing stream "
                "(use a fused plan inside graphs)", what);
  return STEPQ_OK;
}

}  // namespace

extern "C" {

const char* stepq_last_error(void) { return stepq::last_error(); }

int stepq_plan_create(const stepq_plan_desc* d, stepq_plan_t* out) {
  if (!d || !out) return fail(STEPQ_ERR_INVALID_ARG, "desc and out must be non-NULL");
  *out = nullptr;
  if (d->kind != STEPQ_KIND_GDN && d->kind != STEPQ_KIND_KDA)
    return fail(STEPQ_ERR_INVALID_ARG, "kind must be STEPQ_KIND_GDN or STEPQ_KIND_KDA");
  if (d->n_heads < 1) return fail(STEPQ_ERR_INVALID_ARG, "n_heads must be >= 1");
  // the step kernels' launch grid is (requests, heads): heads are its second dimension
  if (d->n_heads > 65535) return fail(STEPQ_ERR_INVALID_ARG, "n_heads must be <= 65535");
  if (d->d_k != d->d_v) return fail(STEPQ_ERR_UNSUPPORTED, "the library supports d_k == d_v only");
  if (d->d_k != 64 && d->d_k != 128)
    return fail(STEPQ_ERR_UNSUPPORTED, "d_k must be 64 or 128 (got %d)", d->d_k);
  if (!d->bits || !d->pivot || !d->omega)
    return fail(STEPQ_ERR_INVALID_ARG, "bits, pivot and omega must be non-NULL");
  if (d->mode != STEPQ_MODE_FUSED && d->mode != STEPQ_MODE_SPLIT)
    return fail(STEPQ_ERR_INVALID_ARG, "mode must be STEPQ_MODE_FUSED or STEPQ_MODE_SPLIT");
  if (d->order != STEPQ_ORDER_DELTA_FIRST && d->order != STEPQ_ORDER_DECAY_FIRST)
    return fail(STEPQ_ERR_INVALID_ARG, "order must be STEPQ_ORDER_DELTA_FIRST or STEPQ_ORDER_DECAY_FIRST");
  if (d->mode == STEPQ_MODE_SPLIT && d->max_batch < 1)
    return fail(STEPQ_ERR_INVALID_ARG, "split mode needs max_batch >= 1");
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || d->device < 0 || d->device >= ndev)
    return fail(STEPQ_ERR_INVALID_ARG, "device %d not available (%d devices)", d->device, ndev);

  const int H = d->n_heads, D = d->d_k, G = D / 64;
  const long long nrow = (long long)H * D;
  for (long long i = 0; i < nrow; i++) {
    if (d->pivot[i] > 1) return fail(STEPQ_ERR_INVALID_ARG, "pivot[%lld] must be 0 or 1", i);
    const int b = d->bits[i];
    if (!d->pivot[i] && b != 2 && b != 4 && b != 6 && b != 8)
      return fail(STEPQ_ERR_INVALID_ARG, "bits[%lld] = %d not in {2,4,6,8}", i, b);
    if (!std::isfinite(d->omega[i]) || d->omega[i] < 0.0f)
      return fail(STEPQ_ERR_INVALID_ARG, "omega[%lld] must be finite and >= 0", i);
  }

  // per-head layout (segment: code block, pivot rows, row factors, column factors)
  std::vector<int> head_type(H), off_piv(H), off_r(H), off_c(H), words(H);
  std::vector<long long> head_off(H), head_bytes(H);
  std::vector<float> den(nrow), iq(nrow), omega(d->omega, d->omega + nrow);  // den: 1/den_i
  std::vector<int> bits(nrow), rowpos(nrow), pividx(nrow), rowmeta(nrow);
  long long off = 0;
  for (int h = 0; h < H; h++) {
    const int8_t* hb = d->bits + (long long)h * D;
    const uint8_t* hp = d->pivot + (long long)h * D;
    int npiv = 0, b0 = -1;
    bool uniform = true;
    long long lane_bits = 0;
    for (int i = 0; i < D; i++) {
      const long long r = (long long)h * D + i;
      if (hp[i]) {
        rowmeta[r] = (int)(0x80000000u | (unsigned)npiv);
        pividx[r] = npiv++;
        rowpos[r] = -1;
        bits[r] = 0;
        iq[r] = 0.0f;
      } else {
        pividx[r] = -1;
        rowpos[r] = (int)lane_bits;
        // bit offset in its first word | that word's index << 8 | width | the row's G codes
        // cross a word boundary | qmax
        rowmeta[r] = (int)(lane_bits & 31) | (int)((lane_bits >> 5) << 8) | (hb[i] << 16) |
                     ((int)((lane_bits & 31) + G * hb[i] > 32) << 20) |
                     (((1 << (hb[i] - 1)) - 1) << 24);
        bits[r] = hb[i];
        lane_bits += (long long)G * hb[i];
        iq[r] = 1.0f / (float)((1 << (hb[i] - 1)) - 1);
        if (b0 < 0) b0 = hb[i];
        else if (hb[i] != b0) uniform = false;
      }
    }
    const bool allpiv = npiv == D;
    if (d->kind == STEPQ_KIND_GDN) {
      if (npiv != 0 && !allpiv)
        return fail(STEPQ_ERR_INVALID_ARG, "GDN head %d: pivot must cover all or none of its rows", h);
      if (!uniform)
        return fail(STEPQ_ERR_INVALID_ARG, "GDN head %d: all rows must share one width", h);
      head_type[h] = allpiv ? kHeadPivot : b0;
    } else {
      head_type[h] = kHeadMixed;
    }
    words[h] = (int)((lane_bits + 31) / 32);
    off_piv[h] = 256 * words[h];
    off_r[h] = off_piv[h] + 2 * D * npiv;
    off_c[h] = off_r[h] + (allpiv ? 0 : 2 * D);
    const long long end = off_c[h] + (allpiv ? 0 : 2 * D);
    head_bytes[h] = (end + 255) / 256 * 256;
    head_off[h] = off;
    off += head_bytes[h];
    // den_i = 1 + omega_i / mean(omega): mean as a pairwise tree times 1/d
    const float* ho = d->omega + (long long)h * D;
    const float mean = tree_sum(ho, D) * (1.0f / (float)D);
    // the kernels scale by the reciprocal 1/den_i, rounded once here
    for (int i = 0; i < D; i++)
      den[(long long)h * D + i] = 1.0f / (mean > 0.0f ? 1.0f + ho[i] / mean : 1.0f);
  }

  // Dispatch order of the heads: the tiles with the most vector work first, the cheapest last
  // (4- and 2-bit, then 6-bit, then 8-bit heads, FP16 pivot heads at the end), so that the
  // launch ends on short tiles.  Ties keep the head index order.
  std::vector<int> head_order(H);
  for (int h = 0; h < H; h++) head_order[h] = h;
  auto rank = [&](int h) {
    const int t = head_type[h];
    return t == kHeadPivot ? 0 : t == 8 ? 1 : t == 6 ? 2 : 3;
  };
  std::stable_sort(head_order.begin(), head_order.end(),
                   [&](int x, int y) { return rank(x) > rank(y); });
  std::vector<HeadDisp> disp(H);
  for (int j = 0; j < H; j++) {
    const int h = head_order[j];
    disp[j] = HeadDisp{head_off[h], h, head_type[h], off_r[h], off_c[h], {0, 0}};
  }

  auto* p = new (std::nothrow) stepq_plan();
  if (!p) return fail(STEPQ_ERR_OOM, "host allocation failed");
  p->kind = d->kind;
  p->H = H;
  p->D = D;
  p->mode = d->mode;
  p->max_batch = d->max_batch;
  p->device = d->device;
  p->bpr = off;
  p->bpv = 8.0 * (double)off / ((double)H * D * D);
  p->head_off = head_off;
  p->head_bytes = head_bytes;

  DeviceGuard dg(d->device);
  if (!dg.ok_) {
    destroy_plan(p);
    return fail(STEPQ_ERR_HIP, "hipSetDevice(%d) failed", d->device);
  }
  // one device allocation for every table, each 256-byte aligned
  struct Piece { const void* src; size_t bytes; size_t off; };
  std::vector<Piece> pieces;
  size_t total = 0;
  auto add = [&](const void* src, size_t bytes) {
    pieces.push_back({src, bytes, total});
    total += (bytes + 255) / 256 * 256;
    return pieces.size() - 1;
  };
  const size_t i_hoff = add(head_off.data(), H * sizeof(long long));
  const size_t i_disp = add(disp.data(), H * sizeof(HeadDisp));
  const size_t i_opiv = add(off_piv.data(), H * sizeof(int));
  const size_t i_or = add(off_r.data(), H * sizeof(int));
  const size_t i_oc = add(off_c.data(), H * sizeof(int));
  const size_t i_w = add(words.data(), H * sizeof(int));
  const size_t i_den = add(den.data(), nrow * sizeof(float));
  const size_t i_om = add(omega.data(), nrow * sizeof(float));
  const size_t i_iq = add(iq.data(), nrow * sizeof(float));
  const size_t i_bits = add(bits.data(), nrow * sizeof(int));
  const size_t i_pos = add(rowpos.data(), nrow * sizeof(int));
  const size_t i_pid = add(pividx.data(), nrow * sizeof(int));
  const size_t i_meta = add(rowmeta.data(), nrow * sizeof(int));
  const unsigned zero = 0;
  const size_t i_st = add(&zero, sizeof(unsigned));
  hipError_t e = hipMalloc(&p->dtab, total);
  if (e != hipSuccess) {
    destroy_plan(p);
    return fail(STEPQ_ERR_OOM, "hipMalloc(%zu) for plan tables: %s", total, hipGetErrorString(e));
  }
  for (const Piece& pc : pieces) {
    e = hipMemcpy((char*)p->dtab + pc.off, pc.src, pc.bytes, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      destroy_plan(p);
      return fail(STEPQ_ERR_HIP, "plan table upload: %s", hipGetErrorString(e));
    }
  }
  auto at = [&](size_t i) { return (void*)((char*)p->dtab + pieces[i].off); };
  DevPlan& dp = p->dp;
  dp.H = H;
  dp.D = D;
  dp.order = d->order;
  dp.bpr = p->bpr;
  dp.head_off = (const long long*)at(i_hoff);
  dp.disp = (const HeadDisp*)at(i_disp);
  dp.off_piv = (const int*)at(i_opiv);
  dp.off_r = (const int*)at(i_or);
  dp.off_c = (const int*)at(i_oc);
  dp.words = (const int*)at(i_w);
  dp.iden = (const float*)at(i_den);
  dp.omega = (const float*)at(i_om);
  dp.iq = (const float*)at(i_iq);
  dp.bits = (const int*)at(i_bits);
  dp.rowpos = (const int*)at(i_pos);
  dp.pividx = (const int*)at(i_pid);
  dp.rowmeta = (const int*)at(i_meta);
  dp.status = (unsigned*)at(i_st);
  p->status = dp.status;

  if (d->mode == STEPQ_MODE_SPLIT) {
    const size_t n = (size_t)d->max_batch * H * 4 * D * sizeof(float);
    e = hipMalloc((void**)&p->stash, n);
    if (e == hipSuccess) e = hipMalloc((void**)&p->slot_stash, (size_t)d->max_batch * sizeof(int));
    if (e != hipSuccess) {
      destroy_plan(p);
      return fail(STEPQ_ERR_OOM, "hipMalloc(%zu) for the split-mode hand-over: %s", n,
                  hipGetErrorString(e));
    }
    if (int rc = scratch_resolve(d->device, &p->scratch)) {
      destroy_plan(p);
      return rc;
    }
    if ((e = hipStreamCreateWithFlags(&p->side, hipStreamNonBlocking)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&p->ev_read, hipEventDisableTiming)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&p->ev_write, hipEventDisableTiming)) != hipSuccess) {
      destroy_plan(p);
      return fail(STEPQ_ERR_HIP, "side stream / events: %s", hipGetErrorString(e));
    }
  }
  *out = p;
  return ok();
}

int stepq_plan_destroy(stepq_plan_t p) {
  if (!p) return ok();
  DeviceGuard dg(p->device);
  destroy_plan(p);
  return ok();
}

int stepq_pool_bytes(stepq_plan_t p, size_t* bytes_per_request, double* bits_per_value) {
  if (int rc = check_plan(p)) return rc;
  if (bytes_per_request) *bytes_per_request = (size_t)p->bpr;
  if (bits_per_value) *bits_per_value = p->bpv;
  return ok();
}

int stepq_head_segment(stepq_plan_t p, int head, size_t* offset, size_t* bytes) {
  if (int rc = check_plan(p)) return rc;
  if (head < 0 || head >= p->H) return fail(STEPQ_ERR_INVALID_ARG, "head %d out of range", head);
  if (offset) *offset = (size_t)p->head_off[head];
  if (bytes) *bytes = (size_t)p->head_bytes[head];
  return ok();
}

static int check_pool(const void* pool, int B) {
  if (B < 0) return fail(STEPQ_ERR_INVALID_ARG, "B must be >= 0");
  if (B > 0 && !pool) return fail(STEPQ_ERR_INVALID_ARG, "pool is NULL");
  if (((uintptr_t)pool & 255u) != 0) return fail(STEPQ_ERR_INVALID_ARG, "pool must be 256-byte aligned");
  return STEPQ_OK;
}

static int check_slots(const void* pool, int n_slots, const int32_t* slots, int B) {
  if (B < 0) return fail(STEPQ_ERR_INVALID_ARG, "B must be >= 0");
  if (B == 0) return STEPQ_OK;
  if (n_slots < 1) return fail(STEPQ_ERR_INVALID_ARG, "n_slots must be >= 1");
  if (!slots) return fail(STEPQ_ERR_INVALID_ARG, "slots is NULL");
  return check_pool(pool, n_slots);
}

namespace {

int encode_impl(stepq_plan_t p, const float* S, void* pool, int n_slots, const int32_t* slots,
                int B, void* stream) {
  if (B > 0 && !S) return fail(STEPQ_ERR_INVALID_ARG, "S is NULL");
  if (int rc = check_grid(p, B)) return rc;
  if (p->mode == STEPQ_MODE_SPLIT && B > p->max_batch)
    return fail(STEPQ_ERR_INVALID_ARG, "B = %d exceeds max_batch %d", B, p->max_batch);
  DeviceGuard dg(p->device);
  hipStream_t s = (hipStream_t)stream;
  if (int rc = refuse_capture(p, s, "encode")) return rc;
  HIP_TRY(wait_writeback(p, s));
  StepArgs a{};
  a.P = p->dp;
  a.pool = (uint8_t*)pool;
  a.B = B;
  a.S_in = S;
  a.stash = p->stash;
  a.slots = slots;
  a.n_slots = n_slots;
  if (B > 0) HIP_TRY(launch_step(p->kind, ENCODE, a, s));
  return ok();
}

int decode_impl(stepq_plan_t p, void* pool, int n_slots, const int32_t* slots, int B,
                const float* q, const float* k, const float* v, const float* alpha,
                const float* beta, float* out, void* stream, float* stash = nullptr) {
  if (B > 0 && (!q || !k || !v || !alpha || !beta || !out))
    return fail(STEPQ_ERR_INVALID_ARG, "q, k, v, alpha, beta and out must be non-NULL");
  if (int rc = check_grid(p, B)) return rc;
  if (p->mode == STEPQ_MODE_SPLIT && !stash && B > p->max_batch)
    return fail(STEPQ_ERR_INVALID_ARG, "B = %d exceeds max_batch %d", B, p->max_batch);
  if (B == 0) return ok();
  DeviceGuard dg(p->device);
  hipStream_t s = (hipStream_t)stream;
  if (int rc = refuse_capture(p, s, "decode_step")) return rc;
  StepArgs a{};
  a.P = p->dp;
  a.pool = (uint8_t*)pool;
  a.B = B;
  a.q = q;
  a.k = k;
  a.v = v;
  a.alpha = alpha;
  a.beta = beta;
  a.out = out;
  a.stash = stash ? stash : p->stash;
  a.slots = slots;
  a.n_slots = n_slots;
  if (p->mode == STEPQ_MODE_FUSED) {
    HIP_TRY(launch_step(p->kind, FUSED, a, s));
    return ok();
  }
  // split: readout on the caller's stream; refit + pack on the side stream once it is done.
  // The readout kernel records each row's resolved slot, so the writeback never reads the
  // caller's slot array (which the caller may reuse once `stream` has run).
  HIP_TRY(wait_writeback(p, s));
  if (slots) a.slot_out = p->slot_stash;
  HIP_TRY(launch_step(p->kind, READ, a, s));
  HIP_TRY(hipEventRecord(p->ev_read, s));
  HIP_TRY(hipStreamWaitEvent(p->side, p->ev_read, 0));
  if (p->spin_cycles > 0) HIP_TRY(launch_spin(p->spin_cycles, p->side));
  if (slots) a.slots = p->slot_stash;
  HIP_TRY(launch_step(p->kind, WRITE, a, p->side));
  HIP_TRY(hipEventRecord(p->ev_write, p->side));
  p->write_pending = true;
  return ok();
}

}  // namespace

int stepq_encode_state(stepq_plan_t p, const float* S, void* pool, int B, void* stream) {
  if (int rc = check_plan(p)) return rc;
  if (int rc = check_pool(pool, B)) return rc;
  return encode_impl(p, S, pool, B, nullptr, B, stream);
}

int stepq_encode_state_slots(stepq_plan_t p, const float* S, void* pool, int n_slots,
                             const int32_t* slots, int B, void* stream) {
  if (int rc = check_plan(p)) return rc;
  if (int rc = check_slots(pool, n_slots, slots, B)) return rc;
  return encode_impl(p, S, pool, n_slots, slots, B, stream);
}

int stepq_decode_step(stepq_plan_t p, void* pool, int B, const float* q, const float* k,
                      const float* v, const float* alpha, const float* beta, float* out,
                      void* stream) {
  if (int rc = check_plan(p)) return rc;
  if (int rc = check_pool(pool, B)) return rc;
  return decode_impl(p, pool, B, nullptr, B, q, k, v, alpha, beta, out, stream);
}

int stepq_decode_step_slots(stepq_plan_t p, void* pool, int n_slots, const int32_t* slots,
                            int B, const float* q, const float* k, const float* v,
                            const float* alpha, const float* beta, float* out, void* stream) {
  if (int rc = check_plan(p)) return rc;
  if (int rc = check_slots(pool, n_slots, slots, B)) return rc;
  return decode_impl(p, pool, n_slots, slots, B, q, k, v, alpha, beta, out, stream);
}

int stepq_decode_step_noalloc(stepq_plan_t p, void* pool, int B, const float* q,
                              const float* k, const float* v, const float* alpha,
                              const float* beta, float* out, void* stream) {
  if (int rc = check_plan(p)) return rc;
  if (int rc = check_pool(pool, B)) return rc;
  if (p->mode == STEPQ_MODE_FUSED)  // the fused kernel uses no scratch: the plain call
    return decode_impl(p, pool, B, nullptr, B, q, k, v, alpha, beta, out, stream);
  const size_t need = (size_t)B * p->H * 4 * p->D * sizeof(float);
  if (need > kScratchBytes)
    return fail(STEPQ_ERR_INVALID_ARG, "decode_step_noalloc: B * n_heads = %lld tiles need %zu "
                "bytes of scratch, above its %zu (at most %zu tiles at d = %d)",
                (long long)B * p->H, need, kScratchBytes, kScratchBytes / (16 * (size_t)p->D),
                p->D);
  if (B == 0) return ok();
  if (!p->scratch) return fail(STEPQ_ERR_HIP, "decode_step_noalloc: scratch not resolved");
  // the previous no-allocation writeback on this device (another plan's) must have read the
  // hand-over before this readout kernel overwrites it; this plan's own is waited for below
  {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    stepq_plan* prev = g_scratch_owner[p->device];
    if (prev && prev != p && prev->write_pending) {
      DeviceGuard dg(p->device);
      HIP_TRY(hipStreamWaitEvent((hipStream_t)stream, prev->ev_write, 0));
    }
    g_scratch_owner[p->device] = p;
  }
  return decode_impl(p, pool, B, nullptr, B, q, k, v, alpha, beta, out, stream,
                     (float*)p->scratch);
}

int stepq_unpack_debug(stepq_plan_t p, const void* pool, int B, float* S_hat, uint16_t* r,
                       uint16_t* c, int8_t* z, void* stream) {
  if (int rc = check_plan(p)) return rc;
  if (int rc = check_pool(pool, B)) return rc;
  DeviceGuard dg(p->device);
  hipStream_t s = (hipStream_t)stream;
  if (int rc = check_grid(p, B)) return rc;
  if (int rc = refuse_capture(p, s, "unpack_debug")) return rc;
  HIP_TRY(wait_writeback(p, s));
  HIP_TRY(launch_unpack(p->dp, (const uint8_t*)pool, B, S_hat, r, c, z, s));
  return ok();
}

int stepq_sync(stepq_plan_t p) {
  if (int rc = check_plan(p)) return rc;
  DeviceGuard dg(p->device);
  if (p->side) HIP_TRY(hipStreamSynchronize(p->side));
  return ok();
}

int stepq_get_status(stepq_plan_t p, uint32_t* flags, int reset) {
  if (int rc = check_plan(p)) return rc;
  if (!flags) return fail(STEPQ_ERR_INVALID_ARG, "flags is NULL");
  DeviceGuard dg(p->device);
  HIP_TRY(hipDeviceSynchronize());
  unsigned v = 0;
  HIP_TRY(hipMemcpy(&v, p->status, sizeof v, hipMemcpyDeviceToHost));
  *flags = v;
  if (reset) {
    const unsigned zero = 0;
    HIP_TRY(hipMemcpy(p->status, &zero, sizeof zero, hipMemcpyHostToDevice));
  }
  return ok();
}

int stepq_row_impact_gpu(int kind, int order, int n_heads, int d, int B, const float* q,
                         const float* k, const float* alpha, const float* beta, double* acc,
                         void* stream) {
  if (kind != STEPQ_KIND_GDN && kind != STEPQ_KIND_KDA)
    return fail(STEPQ_ERR_INVALID_ARG, "kind must be STEPQ_KIND_GDN or STEPQ_KIND_KDA");
  if (order != STEPQ_ORDER_DELTA_FIRST && order != STEPQ_ORDER_DECAY_FIRST)
    return fail(STEPQ_ERR_INVALID_ARG, "order must be STEPQ_ORDER_DELTA_FIRST or STEPQ_ORDER_DECAY_FIRST");
  if (n_heads < 1 || B < 0) return fail(STEPQ_ERR_INVALID_ARG, "n_heads >= 1 and B >= 0 required");
  if (d != 64 && d != 128) return fail(STEPQ_ERR_UNSUPPORTED, "d must be 64 or 128 (got %d)", d);
  if (!acc || (B > 0 && (!q || !k || !alpha || !beta)))
    return fail(STEPQ_ERR_INVALID_ARG, "q, k, alpha, beta and acc must be non-NULL");
  HIP_TRY(launch_row_impact(kind, order, n_heads, d, B, q, k, alpha, beta, acc,
                            (hipStream_t)stream));
  return ok();
}

// Test hook: a bounded spin of `cycles` clocks on the side stream before each split-mode
// writeback, to show that the next step's readout waits for it.
int stepq_debug_side_delay(stepq_plan_t p, long long cycles) {
  if (int rc = check_plan(p)) return rc;
  if (cycles < 0 || cycles > 2000000000LL)
    return fail(STEPQ_ERR_INVALID_ARG, "cycles must be in [0, 2e9]");
  p->spin_cycles = cycles;
  return ok();
}

}  // extern "C"
