// stepq_internal.h -- shared between the host API (stepq_api.cpp, stepq_offline.cpp) and the
// kernels (stepq_device.h, instantiated by stepq_k128_gdn.hip, stepq_k128_kda.hip and
// stepq_k64.hip).  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace stepq {

// Head types of the per-head dispatch: 2/4/6/8 = head quantized at that width (GDN),
// 0 = FP16 pivot head (GDN), -1 = rows of mixed widths and pivots (KDA).
constexpr int kHeadPivot = 0;
constexpr int kHeadMixed = -1;

// Kernel modes.  FUSED: the whole step.  READ: decode, update, readout, hand-over of the
// per-row/per-column update factors.  WRITE: decode, update from the hand-over, refit, pack.
// ENCODE: refit and pack an fp32 state given in memory.
enum Mode { FUSED = 0, READ = 1, WRITE = 2, ENCODE = 3 };

// One dispatch position j of the GDN kernels (grid index y): the j-th head of the plan's
// dispatch order, its type and its segment layout, so a workgroup finds everything it needs to
// start loading with one 32-byte scalar load.
struct alignas(32) HeadDisp {
  long long off;  // segment byte offset inside one request
  int h;          // the head
  int type;       // its head_type
  int off_r;      // row-factor block offset inside the segment
  int off_c;      // column-factor block offset
  int pad[2];
};
static_assert(sizeof(HeadDisp) == 32, "one 32-byte scalar load per dispatch position");

// Device-resident plan tables (all arrays in device memory; per-row arrays are [H * d]).
struct DevPlan {
  int H, D;                  // heads, d_k = d_v
  int order;                 // 0: A = Diag(a)(I - beta k k^T); 1: A = (I - beta k k^T) Diag(a)
  long long bpr;             // bytes per request
  const long long* head_off; // [H] segment byte offset inside one request
  const HeadDisp* disp;      // [H] GDN kernels, per dispatch position: the head and its layout
  const int* off_piv;        // [H] pivot block offset inside the segment
  const int* off_r;          // [H] row-factor block offset
  const int* off_c;          // [H] column-factor block offset
  const int* words;          // [H] words per lane of the code block
  const float* iden;         // [H*d] 1 / den_i, den_i = 1 + omega_i / mean(omega)
  const float* omega;        // [H*d]
  const float* iq;           // [H*d] 1/qmax, 0 on pivot rows
  const int* bits;           // [H*d] width (0 on pivot rows)
  const int* rowpos;         // [H*d] stream bit offset of the row's first code (-1 on pivots)
  const int* pividx;         // [H*d] row index inside the pivot block (-1 otherwise)
  const int* rowmeta;        // [H*d] packed: pivot 0x80000000 | pividx, else rowpos & 31 |
                             //   (rowpos >> 5) << 8 | bits << 16 | (codes cross a word
                             //   boundary) << 20 | qmax << 24
  unsigned* status;          // accumulated STEPQ_FLAG_* bits
};

struct StepArgs {
  DevPlan P;
  uint8_t* pool;
  int B;
  const float* q;
  const float* k;
  const float* v;
  const float* alpha;
  const float* beta;
  float* out;
  float* stash;      // split-mode hand-over, [B*H][4*D]
  const float* S_in; // ENCODE input [B*H][D][D]
  // Slot-indexed pools: batch row b uses pool slot slots[b] (nullptr: slot b).  A value outside
  // [0, n_slots) skips the row (-1 silently, anything else also raises the bad-slot flag).
  // READ writes each row's resolved slot (-1 = skipped) to slot_out[b] for the WRITE kernel.
  const int* slots;
  int n_slots;
  int* slot_out;
};

// Launchers (stepq_k64.hip; stepq_calib.hip for the row impact).  kind: 0 = GDN, 1 = KDA.
hipError_t launch_step(int kind, Mode mode, const StepArgs& a, hipStream_t s);
hipError_t launch_unpack(const DevPlan& P, const uint8_t* pool, int B, float* S, uint16_t* r,
                         uint16_t* c, int8_t* z, hipStream_t s);
hipError_t launch_row_impact(int kind, int order, int H, int D, int B, const float* q,
                             const float* k, const float* alpha, const float* beta, double* acc,
                             hipStream_t s);
hipError_t launch_spin(long long cycles, hipStream_t s);

// The no-allocation entry point's device scratch (stepq_noalloc.hip): kScratchBytes per GPU,
// resolved once per device; the current device must be `device`.
constexpr size_t kScratchBytes = size_t(32) << 20;
int scratch_resolve(int device, void** out);

// The calling thread's message of the last call (stepq_last_error): fail() records a printf-style
// message and returns code; clear_error() empties it.  Shared by every host entry point.
int fail(int code, const char* fmt, ...);
void clear_error();

}  // namespace stepq
