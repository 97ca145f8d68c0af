// stepq_device.h -- gfx950 kernels of the STEPQuant packed-state decode step (device templates;
// stepq_k*.hip instantiate them per tile size and kind).
//
// Method (page: "STEPQuant" paper digest, vibe-research silicon-writer readme):
//   Method 4 "the execution path of each decode step": reconstruct the tile from integer codes,
//   row/column factors and FP16 pivots; retention + delta update + readout on the float tile;
//   the output leaves before requantization; refit the row/column factors; pack codes and
//   factors, pivots stay FP16; no resident FP32 copy of the state.
//   Method 3 "Key-Row-Aware Dual-Axis Fitting": X_hat[i,j] = r_i c_j z[i,j]; r_i from the row's
//   mean magnitude and omega_i, c_j an omega-weighted least-squares fit with r fixed.
//   Background: S_t = A_t S_{t-1} + beta k v^T with A_t = Diag(a)(I - beta k k^T).
//
// Work mapping (one workgroup per (request, head) tile, d = d_k = d_v in {64, 128}):
//   d/32 waves; wave w owns rows 32w .. 32w+31, lane L owns the G = d/64 columns
//   G*L .. G*L+G-1.  The tile lives in VGPRs (32*G floats per lane).  Every reduction over rows
//   (k^T S, q^T S, the column maximum, the least-squares sums) runs inside a lane, the waves
//   adding their partials through LDS as a pairwise tree.  The one reduction over columns (the
//   row's mean magnitude) goes through an LDS transpose inside the wave, after which lanes L and
//   L+32 own row 32w + L (one half of the columns each).  Per-row scalars are read from LDS at
//   wave-uniform addresses (broadcast reads, no VALU work).
//
// Arithmetic matches a fixed binary32 evaluation order bit for bit:
//   dequant  X_ij = c_j z_ij (exact); f_i = r_i (pivot rows: X = the binary16 values, f = 1)
//   update   u = dot_i(kc_i, X) with kc_i = k_i f_i (or k_i M_i when the rows decay first);
//            e = fma(-a_i, u_j, v_j) (or v_j - u_j);  T = fma(K_i, e, X);  the updated state is
//            S_ij = M_i T_ij with M_i = a_i f_i, K_i = (beta k_i) / M_i (rows whose gate is
//            below 2^-72 drop X, and they and dead rows take M_i = beta k_i, K_i = 1)
//   scales   readout coefficient q_i M_i, row magnitude |M_i| tree_j |T_ij|, y = T (M_i / r_i)
//   sums     one fma chain over each wave's 32 rows (first term a rounded product), the waves'
//            partials added as a pairwise tree; the row magnitude sum is a pairwise tree over
//            columns
//   codes    round-half-even of the exact product y * (1/c): fma(y, 1/c, 1.5*2^23) rounds the
//            exact product once onto the integer grid of [2^23, 2^24); the low b bits of that
//            float are the two's-complement code, and the clamp to +-qmax is applied in the same
//            offset domain.
// The build passes -ffp-contract=off: no multiply-add is fused unless written as fmaf.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "stepq_internal.h"

namespace stepq {
namespace dev {

constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
constexpr float kGateErase = 0x1p-72f; // a gate below this erases the row's previous state
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr unsigned kFlagNonfinite = 1u, kFlagScaleOvf = 2u, kFlagPivotOvf = 4u,
                   kFlagBadSlot = 8u;

template <int N, typename F>
__device__ __forceinline__ void sfor(F&& f) {
  [&]<int... I>(std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
  }(std::make_integer_sequence<int, N>{});
}

#define CI(x) decltype(x)::value

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

__device__ __forceinline__ float h2f(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// binary32 -> binary16, nearest even (v_cvt_f16_f32).  The empty asm pins x as a rounded binary32
// value: without it the compiler may fold a producing fma into v_fma_mix{lo,hi}_f16, which
// rounds the exact fma result straight to binary16 and differs on binary16 ties.
__device__ __forceinline__ uint16_t f2h(float x) {
  asm volatile("" : "+v"(x));
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

__device__ __forceinline__ float rcp0(float x) { return x == 0.0f ? 0.0f : 1.0f / x; }

// rcp0 of a value widened from binary16 (a stored row or column factor): v_rcp_f32 followed by
// one Newton step with fma, y0 + y0 (1 - x y0).  The residual 1 - x y0 is exact, and for every
// finite nonzero binary16 x the result equals the correctly rounded binary32 1/x (checked
// exhaustively on gfx950 over all 63,486 such inputs; the raw v_rcp_f32 alone is off by one ulp
// on 5,492 of them).  Zero and infinity map to 0, as 1/x does for infinity.
__device__ __forceinline__ float rcp16(float x) {
  const float y0 = __builtin_amdgcn_rcpf(x);
  const float r = __builtin_fmaf(y0, __builtin_fmaf(-x, y0, 1.0f), y0);
  return __builtin_amdgcn_classf(x, 0x264) ? 0.0f : r;  // class bits: -inf, -0, +0, +inf
}

__device__ __forceinline__ bool is_inf16(uint16_t h) { return (h & 0x7FFFu) == 0x7C00u; }

// fma(a, b, kMagic) as one v_fmaak_f32 (the constant rides in the instruction).  In the KDA
// packing loop the compiler otherwise materializes kMagic with a v_mov before every fma.
__device__ __forceinline__ float fma_magic(float a, float b) {
  float d;
  asm("v_fmaak_f32 %0, %1, %2, 0x4b400000" : "=v"(d) : "v"(a), "v"(b));
  return d;
}

// code offset by kMagic: fma rounds the exact product y*ic once; then clamp to +-qm
__device__ __forceinline__ float quant_off(float y, float ic, float qm) {
  return __builtin_amdgcn_fmed3f(__builtin_fmaf(y, ic, kMagic), kMagic - qm, kMagic + qm);
}

// Visibility of this wave's own LDS writes to its other lanes (no s_barrier needed).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Pairwise tree over leaves pushed in index order: leaf M joins the partial sums on the levels
// where M has trailing one bits (a binary counter), so lv[L] holds a finished subtree of 2^L.
template <int M, int L = 0>
__device__ __forceinline__ void tree_push(float* lv, float x) {
  if constexpr (((M >> L) & 1) == 0) {
    lv[L] = x;
  } else {
    tree_push<M, L + 1>(lv, lv[L] + x);
  }
}

// Tile geometry: d/32 waves of 32 rows; lane L owns the G = d/64 columns G*L .. G*L+G-1.
template <int D>
struct Geo {
  static constexpr int G = D / 64;    // columns per lane
  static constexpr int R = 32;        // rows per wave
  static constexpr int NW = D / R;    // waves per tile
  static constexpr int NT = 64 * NW;  // threads per tile
};

// Per-row record, read at wave-uniform addresses (broadcast reads).  One interleaved record per
// row keeps every field of a wave's 32 rows within ds_read's immediate offset range of a single
// base register.  GDN rows share one gate (alpha) and one width, so they carry no a or 1/qmax.
//   kr   key-projection coefficient k f (or k M when the rows decay first)
//   K    (beta k) / M: the update T = fma(K, e, X)
//   M    row scale of the updated state S = M T
//   rho  M / r_hat (after the row factor; 0 on pivot and dead rows): y = T rho
//   W    omega r_hat^2 (before the row factor: omega, or -1 on a KDA pivot row)
//   qm   readout coefficient q M
template <bool KDA>
struct Row;
template <>
struct Row<false> {
  float kr, K, qm, M, rho, W;
};
template <>
struct Row<true> {
  float kr, K, qm, M, rho, W, a;  // a: the row's gate
};

// Read-only data in the constant address space: loads at wave-uniform addresses become scalar
// loads through the scalar cache.
template <typename T>
using KConst = const __attribute__((address_space(4))) T;

// A wave-uniform element of a read-only table (plan tables, slot indices): one scalar load.
template <typename T>
__device__ __forceinline__ T kread(const T* p, long long i) {
  return ((KConst<T>*)p)[i];
}

// Dispatch position j's record (one scalar load of its fields).
__device__ __forceinline__ HeadDisp kread_disp(KConst<HeadDisp>* p, int j) {
  KConst<int>* const q = (KConst<int>*)(p + j);
  HeadDisp r;
  r.off = *(KConst<long long>*)q;
  r.h = q[2];
  r.type = q[3];
  r.off_r = q[4];
  r.off_c = q[5];
  return r;
}

// The same uniform pointer, made opaque to the optimizer: loads through it are not merged with
// loads of the same data elsewhere (which would keep them live, in scalar registers, across
// phases).
template <typename T>
__device__ __forceinline__ KConst<T>* opaque_s(KConst<T>* p) {
  asm volatile("" : "+s"(p));
  return p;
}

// Per-row layout metadata of mixed-width tiles, packed by the plan into one int: a pivot row is
// 0x80000000 | (its index in the pivot block); a quantized row is the bit offset of its first
// code in its first stream word (bits 0..4) | that word's index << 8 | width << 16 | (its G
// codes cross a word boundary) << 20 | qmax << 24.  Read once per row and phase as a
// wave-uniform scalar; the word index arrives ready as a byte offset into the [word][lane]
// staging (word * 256), and shifts use the low five bits as they are.
__device__ __forceinline__ bool meta_pivot(int m) { return m < 0; }
__device__ __forceinline__ int meta_pividx(int m) { return m & 0xFF; }
__device__ __forceinline__ int meta_shift(int m) { return m & 31; }
__device__ __forceinline__ int meta_lds(int m) { return m & 0x3F00; }  // word * 256 (0: pivot)
__device__ __forceinline__ int meta_bits(int m) { return (m >> 16) & 15; }
__device__ __forceinline__ bool meta_straddles(int m) { return (m >> 20) & 1; }
__device__ __forceinline__ int meta_qmax(int m) { return (m >> 24) & 0x7F; }
template <int D, bool KDA>
struct CodeKda {  // code block staging of mixed-width tiles
  uint32_t code[(2 * D * 8 / 32 + 1) * 64];
};
template <int D>
struct CodeKda<D, false> {};

// Both tile kinds fit in 40 KB, so four workgroups fit in a CU's 160 KB.  Only two cross-wave
// slots: GDN column maxima pass through each wave's own (by then dead) transpose section; KDA
// keeps them in the transpose area just past its code staging block (they come after the
// transposes).  RO (the split mode's readout kernels) keeps only what a readout uses -- no
// transpose area, and for KDA the code staging block -- so five workgroups fit per CU.
template <int D, bool KDA, bool RO = false>
struct Smem {
  static constexpr int NW = Geo<D>::NW;
  static constexpr bool kKDA = KDA;
  static constexpr int NSLOT = 2;
  static constexpr int kSec = 32 * 65;  // one wave's transpose section [row][lane], +1 pad
  // KDA: column-maximum slots [NW][D] after the code staging block, then the column statistics
  static constexpr int kKdaMax = KDA ? (int)(sizeof(CodeKda<D, KDA>) / sizeof(float)) : 0;
  static constexpr int kKdaCol = kKdaMax + NW * D;
  static constexpr int kTr = !RO ? NW * kSec : KDA ? kKdaMax : 1;
  Row<KDA> row[D];
  float red[NSLOT][NW][D];
  union {
    float tr[kTr];           // the waves' transpose sections (conflict-free), q, KDA maxima
    CodeKda<D, KDA> kc;      // used only before and after the transpose
  };
  static_assert(!KDA || kKdaMax <= kTr, "KDA staging overflows the transpose area");
  static_assert(!KDA || RO || kKdaCol + 3 * D <= kTr, "KDA column statistics overflow");
  static_assert(KDA || RO || D + 3 * D <= kSec, "GDN column statistics overflow wave 0's section");
};
static_assert(sizeof(Smem<128, false>) <= 40960 && sizeof(Smem<128, true>) <= 40960,
              "four workgroups per CU need at most 40 KB of LDS each");
static_assert(sizeof(Smem<128, false, true>) <= 32768 && sizeof(Smem<128, true, true>) <= 32768,
              "five readout workgroups per CU need at most 32 KB of LDS each");

// An integer the optimizer cannot see through: each array's row base below gets its own copy,
// so the array's address stays in its own VGPR and each access uses the instruction's small
// immediate offset (instead of one shared base plus a large constant re-added per access).
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// The same LDS address, held in one VGPR: accesses at constant distances from it then use the
// instruction's immediate offset instead of re-adding the member's offset each time.
template <typename T, typename SM>
__device__ __forceinline__ T* lds_pin(SM& sm, T* p) {
  char* const b = reinterpret_cast<char*>(&sm);
  return reinterpret_cast<T*>(b + opaque((int)(reinterpret_cast<char*>(p) - b)));
}

// Wave-local view of the per-row records (this wave's 32 rows; broadcast reads).
template <typename SM>
struct Rows {
  const Row<SM::kKDA>* r;
  __device__ __forceinline__ Rows(const SM& sm) {
    const int base = (threadIdx.x >> 6) * 32;
    r = &sm.row[opaque(base)];
  }
};

// ---------------------------------------------------------------------------------------------
// fixed-width code extraction and packing (compile-time positions)
// ---------------------------------------------------------------------------------------------

template <int BITS, int K>
__device__ __forceinline__ int get_code(const uint32_t* wd) {
  constexpr int p = K * BITS, wi = p / 32, o = p % 32;
  if constexpr (o + BITS <= 32) {
    return __builtin_amdgcn_sbfe((int)wd[wi], o, BITS);
  } else {
    uint32_t x = __builtin_amdgcn_alignbit(wd[wi + 1], wd[wi], o);
    return __builtin_amdgcn_sbfe((int)x, 0, BITS);
  }
}

// Decode of 2- and 4-bit codes through byte conversions: each variant m_v of a word holds one
// code of every byte in that byte's top BITS bits with zeros below (a shift and a mask per
// variant), so converting a sign-extended byte (the compiler's sub-dword conversion) gives
// z * 2^(8 - BITS) in one instruction; times c * 2^(BITS - 8) that is c z exactly (c is a
// widened binary16, so the power-of-two scaling is exact).  Against extract + convert per code
// this saves about 0.6 instructions per code.  The byte is taken by a cast to int8_t, not by
// __builtin_amdgcn_sbfe: on a masked word this LLVM turned the signed conversion of the sbfe
// result into an unsigned one (uitofp of a value that can be negative), which decodes every
// negative code wrong.
template <int BITS, int G, int WPW>
__device__ __forceinline__ void decode_narrow(const uint32_t* wd, const float* cc,
                                              float (&S)[32][G]) {
  constexpr int NV = 8 / BITS;  // codes per byte
  constexpr uint32_t kTop = BITS == 4 ? 0xF0F0F0F0u : 0xC0C0C0C0u;
  constexpr float kScale = BITS == 4 ? 0x1p-4f : 0x1p-6f;
  float cs[G];
  sfor<G>([&](auto gg) { cs[CI(gg)] = cc[CI(gg)] * kScale; });
  sfor<WPW>([&](auto xx) {
    constexpr int x = CI(xx);
    uint32_t m[NV];
    sfor<NV>([&](auto vv) {
      constexpr int sh = 8 - BITS - CI(vv) * BITS;
      m[CI(vv)] = (sh ? wd[x] << sh : wd[x]) & kTop;
    });
    sfor<32 / BITS>([&](auto kk) {
      constexpr int K = x * (32 / BITS) + CI(kk);
      constexpr int r = K / G, g = K % G;
      constexpr int o = (K * BITS) % 32, byte = o / 8, v = (o % 8) / BITS;
      S[r][g] = cs[g] * (float)(int)(int8_t)(m[v] >> (8 * byte));
    });
  });
}

// Appends code K (low BITS bits of f) to the lane's stream kept in acc, newest bits on top, and
// stores each 32-bit word as it completes.  A code that straddles two words is inserted twice:
// first its low part (finishing the word), then whole (its low part lands in bits that later
// insertions shift out).
template <int BITS, int K, typename Store>
__device__ __forceinline__ void put_code(uint32_t& acc, uint32_t f, Store&& store) {
  constexpr int p = K * BITS, wi = p / 32, o = p % 32;
  if constexpr (o + BITS > 32) {
    constexpr int nlow = 32 - o;
    acc = __builtin_amdgcn_alignbit(f, acc, nlow);
    store(std::integral_constant<int, wi>{}, acc);
    acc = __builtin_amdgcn_alignbit(f, acc, BITS);
  } else {
    acc = __builtin_amdgcn_alignbit(f, acc, BITS);
    if constexpr (o + BITS == 32) store(std::integral_constant<int, wi>{}, acc);
  }
}

template <typename Args>
__device__ __forceinline__ void raise_flags(const Args& A, unsigned fl) {
  if (fl) atomicOr(A.P.status, fl);
}

// ---------------------------------------------------------------------------------------------
// phases shared by the tile variants (S: this lane's 32 rows x G columns)
// ---------------------------------------------------------------------------------------------

// Per-row loop over the wave's 32 rows in groups of NG rows, software-pipelined: the
// group's per-row coefficients (LDS broadcast reads, xr(r)) are fetched one group ahead, and a
// scheduling fence closes each group.  Left to itself the compiler fetches all 32 coefficients
// up front (32 registers, which spills the tile); with a fence but no look-ahead every group
// waits for its LDS reads.  body(r, x) does the row's work with its coefficient x.
template <int NG = 4, typename XF, typename Body>
__device__ __forceinline__ void rows_pipelined(XF&& xr, Body&& body) {
  constexpr int NGR = 32 / NG;  // groups
  float x[2][NG];
  sfor<NG>([&](auto tt) { x[0][CI(tt)] = xr(CI(tt)); });
  sfor<NGR>([&](auto jj) {
    constexpr int j = CI(jj);
    if constexpr (j + 1 < NGR)
      sfor<NG>([&](auto tt) { x[(j + 1) & 1][CI(tt)] = xr(NG * (j + 1) + CI(tt)); });
    sfor<NG>([&](auto tt) {
      body(std::integral_constant<int, NG * j + CI(tt)>{}, x[j & 1][CI(tt)]);
    });
    __builtin_amdgcn_sched_barrier(0);
  });
}

// dot over the wave's 32 rows of a per-row scalar x_r with S[r][g]: one fma chain per column,
// first row to last.
template <int G, typename XF>
__device__ __forceinline__ void row_dot(const float (&S)[32][G], XF&& xr, float* res) {
  rows_pipelined(xr, [&](auto rr, float x) {
    constexpr int r = CI(rr);
    sfor<G>([&](auto gg) {
      constexpr int g = CI(gg);
      if constexpr (r == 0) res[g] = x * S[0][g];
      else res[g] = __builtin_fmaf(x, S[r][g], res[g]);
    });
  });
}

// Per-column error of the delta update with one gate for all rows: e = v - alpha u (the delta
// update sees the undecayed state), or e = v - u when the rows decayed first (the key
// projection already carries the gate).
template <int G>
__device__ __forceinline__ void col_error(int order, float alpha, const float* u, const float* vv,
                                          float* e) {
  sfor<G>([&](auto gg) {
    constexpr int g = CI(gg);
    e[g] = order ? vv[g] - u[g] : __builtin_fmaf(-alpha, u[g], vv[g]);
  });
}

// Cross-wave combination of this lane's per-wave partials (red[slot][w][col]).
template <int D, typename SM>
__device__ __forceinline__ void xwave_put(SM& sm, int slot, int w, int lane, const float* x) {
  constexpr int G = Geo<D>::G;
  float* const p = lds_pin(sm, &sm.red[slot][0][G * lane]);
  sfor<G>([&](auto gg) { p[w * D + CI(gg)] = x[CI(gg)]; });
}
// pairwise tree over the waves' partials (rows 0-31, 32-63, ...)
template <int D, typename SM>
__device__ __forceinline__ void xwave_sum(SM& sm, int slot, int lane, float* x) {
  constexpr int G = Geo<D>::G, NW = Geo<D>::NW;
  const float* const p = lds_pin(sm, &sm.red[slot][0][G * lane]);
  sfor<G>([&](auto gg) {
    constexpr int g = CI(gg);
    if constexpr (NW == 2) {
      x[g] = p[g] + p[D + g];
    } else {
      x[g] = (p[g] + p[D + g]) + (p[2 * D + g] + p[3 * D + g]);
    }
  });
}
// Column maxima across waves: GDN tiles stage them in each wave's own transpose section (dead
// once that wave's row factors are done), KDA tiles in the transpose area just past the code
// staging block (in wave 2's section: stored after the barrier that ends every transpose).
template <int D, typename SM>
__device__ __forceinline__ float* max_slot(SM& sm, int w) {
  if constexpr (SM::kKDA) return sm.tr + SM::kKdaMax + w * D;
  else return sm.tr + w * SM::kSec;
}
template <int D, typename SM>
__device__ __forceinline__ void xwave_max_put(SM& sm, int w, int lane, const float* x) {
  constexpr int G = Geo<D>::G;
  float* const dst = lds_pin(sm, max_slot<D>(sm, w) + G * lane);
  sfor<G>([&](auto gg) { dst[CI(gg)] = x[CI(gg)]; });
}

// Per-column statistics once per tile: wave g < G finishes column G*lane + g of every lane (one
// column per lane, instead of all G columns in every wave) and shares the result through LDS:
// GDN in wave 0's section past its maximum slot (that section's transpose is done by then), KDA
// past the maximum slots (also in wave 2's section).  [0, D): 1/c0; [D, 2D): 1/c_hat; then the
// binary16 c_hat of the D columns.
template <int D, typename SM>
__device__ __forceinline__ float* col_share(SM& sm) {
  return lds_pin(sm, sm.tr + (SM::kKDA ? SM::kKdaCol : D));
}
// maximum of the waves' partial maxima of column G*lane + g
template <int D, typename SM>
__device__ __forceinline__ float xwave_max_col(SM& sm, int lane, int g) {
  constexpr int G = Geo<D>::G, NW = Geo<D>::NW;
  constexpr int kStride = SM::kKDA ? D : SM::kSec;  // between the waves' partials
  const float* const p0 = lds_pin(sm, max_slot<D>(sm, 0) + G * lane) + g;
  float m = p0[0];
  sfor<NW - 1>([&](auto ww) { m = __builtin_fmaxf(m, p0[(CI(ww) + 1) * kStride]); });
  return m;
}
// pairwise tree over the waves' partials of column G*lane + g (the order xwave_sum uses)
template <int D, typename SM>
__device__ __forceinline__ float xwave_sum_col(SM& sm, int slot, int lane, int g) {
  constexpr int G = Geo<D>::G, NW = Geo<D>::NW;
  const float* const p = lds_pin(sm, &sm.red[slot][0][G * lane]) + g;
  if constexpr (NW == 2) return p[0] + p[D];
  else return (p[0] + p[D]) + (p[2 * D] + p[3 * D]);
}
// Column factor of one column from its least-squares sums (c0 when sq is not positive): its
// binary16 value in ch; returns 1/c_hat (0 if dead).
__device__ __forceinline__ float col_factor1(float num, float sq, float c0, uint16_t& ch,
                                             unsigned& fl) {
  const float c1 = sq > 0.0f ? num / sq : c0;
  ch = f2h(c1);
  if (is_inf16(ch)) fl |= kFlagScaleOvf;
  return rcp16(h2f(ch));
}
// The refit once the least-squares partial sums are staged: waves g < G finish column
// G*lane + g, every wave then reads 1/c_hat of its G columns, and wave 0 stores the lane's G
// binary16 factors with one store (cblk may be null), so each segment's factor block is written
// by whole words.
//
//
// kTest: waves w < G also pass their column's maximum ymax (the largest |y| of column
// G*lane + w over every row) and the head's qmax, and every wave gets back whether no code of
// the tile reaches the clamp: every column's fma(ymax, 1/c_hat, kMagic) lies at most qmax above
// kMagic, and its least-squares sums are not NaN.  The rounding of fma(y, ic, kMagic) is
// monotone in y and symmetric about kMagic (an even integer, unit spacing around it), so then
// every |y| <= ymax of the column rounds inside +-qmax and the clamp is the identity for the
// whole tile.  An infinite maximum fails the test; a NaN entry (which the maximum skips) makes
// the column's sum of squares NaN and fails it there.
template <int D, bool kTest = false, typename SM>
__device__ __forceinline__ bool col_refit(SM& sm, float* csh, int w, int lane, float c0w,
                                          uint16_t* cblk, float* ic, unsigned& fl,
                                          float ymax = 0.0f, float qm = 0.0f) {
  constexpr int G = Geo<D>::G;
  uint16_t* const chs = reinterpret_cast<uint16_t*>(csh + 2 * D);
  int* const clamp_free = reinterpret_cast<int*>(csh + 2 * D + D / 2);  // [G] wave verdicts
  if (w < G) {
    const float n = xwave_sum_col<D>(sm, 0, lane, w), q = xwave_sum_col<D>(sm, 1, lane, w);
    uint16_t ch;
    const float icw = col_factor1(n, q, c0w, ch, fl);
    csh[D + G * lane + w] = icw;
    chs[G * lane + w] = ch;
    if constexpr (kTest) {
      const bool inside = __builtin_fmaf(ymax, icw, kMagic) <= kMagic + qm && q == q;
      const bool all = __builtin_amdgcn_ballot_w64(inside) == ~0ull;
      if (lane == 0) clamp_free[w] = all;
    }
  }
  __syncthreads();
  sfor<G>([&](auto gg) { ic[CI(gg)] = csh[D + G * lane + CI(gg)]; });
  bool free_all = kTest;
  if constexpr (kTest) sfor<G>([&](auto gg) { free_all = free_all && clamp_free[CI(gg)] != 0; });
  if (w == 0 && cblk) {
    if constexpr (G == 2) {
      reinterpret_cast<uint32_t*>(cblk)[lane] = reinterpret_cast<const uint32_t*>(chs)[lane];
    } else {
      cblk[lane] = chs[lane];
    }
  }
  return free_all;
}

// |S| partial sums of each row over this lane's columns, transposed through LDS.
template <int D, typename SM>
__device__ __forceinline__ void put_rowabs(SM& sm, const float (&S)[32][Geo<D>::G], int lane) {
  constexpr int G = Geo<D>::G;
  float* const dst = lds_pin(sm, sm.tr + (threadIdx.x >> 6) * SM::kSec + lane);
  sfor<32>([&](auto rr) {
    constexpr int r = CI(rr);
    float a;
    if constexpr (G == 2) a = __builtin_fabsf(S[r][0]) + __builtin_fabsf(S[r][1]);
    else a = __builtin_fabsf(S[r][0]);
    dst[r * 65] = a;
  });
}

// Row factor of row 32w + (lane & 31): lanes L and L+32 each sum half of the row's |T| over its
// columns, the halves are added and scaled by |M|, and lane L < 32 writes r_hat to the pool
// (unless rblk is null) and rho = M (1/r_hat) (0 if dead or pivot) and W = (omega r_hat) r_hat
// (0 likewise) into the row record, whose rho and W slots hold the plan's 1/den and omega of
// the row until then.
template <int D, typename SM>
__device__ __forceinline__ void row_factor(SM& sm, int lane, int row, bool piv, uint16_t* rblk,
                                           unsigned& fl) {
  float lv[6];
  // the lane index is re-read here rather than kept live from the tile's start
  const int lt = opaque((int)threadIdx.x);
  const float* const src = lds_pin(
      sm, sm.tr + (lt >> 6) * SM::kSec + (lt & 31) * 65 + (lt & 32));
  sfor<32>([&](auto jj) { tree_push<CI(jj)>(lv, src[CI(jj)]); });
  const float other = __shfl_xor(lv[5], 32);
  const float Mr = sm.row[row].M;
  const float m =
      ((lane < 32 ? lv[5] + other : other + lv[5]) * __builtin_fabsf(Mr)) * (1.0f / (float)D);
  if (!__builtin_isfinite(m)) fl |= kFlagNonfinite;
  if (lane >= 32) return;
  if (piv) {
    sm.row[row].rho = 0.0f;
    sm.row[row].W = 0.0f;
    if (rblk) rblk[row] = 0;
    return;
  }
  const float iden = sm.row[row].rho, om = sm.row[row].W;  // parked there by load_inputs
  const float r = (m + 1e-8f) * iden;
  const uint16_t rh = f2h(r);
  if (is_inf16(rh)) fl |= kFlagScaleOvf;
  if (rblk) rblk[row] = rh;
  const float rf = h2f(rh);
  sm.row[row].rho = Mr * rcp16(rf);
  sm.row[row].W = (om * rf) * rf;
}

// y = T * rho (in place) and the column maximum max_i |y| of a one-width (GDN) tile: the 1/qmax
// factor is applied after the maximum (rounding is monotone).
template <int G, typename RW>
__device__ __forceinline__ void scale_rows(float (&S)[32][G], const RW& rows, float* mx) {
  sfor<G>([&](auto gg) { mx[CI(gg)] = 0.0f; });
  rows_pipelined([&](int r) { return rows.r[r].rho; }, [&](auto rr, float rho) {
    constexpr int r = CI(rr);
    sfor<G>([&](auto gg) {
      constexpr int g = CI(gg);
      S[r][g] = S[r][g] * rho;
      mx[g] = __builtin_fmaxf(mx[g], __builtin_fabsf(S[r][g]));
    });
  });
}

// First quantization z0 = rne(y / c0) and the sums of the omega-weighted least-squares fit:
// num = sum_i (W_i z0) y, sq = sum_i (W_i z0) z0, each one fma chain over the wave's rows.
template <int G, typename RW>
__device__ __forceinline__ void ls_sums(const float (&S)[32][G], const RW& rows, const float* ic0,
                                        float* num, float* sq) {
  rows_pipelined([&](int r) { return rows.r[r].W; }, [&](auto rr, float W) {
    constexpr int r = CI(rr);
    sfor<G>([&](auto gg) {
      constexpr int g = CI(gg);
      const float z0 = __builtin_fmaf(S[r][g], ic0[g], kMagic) - kMagic;  // |z0| <= qmax
      const float a = W * z0;
      if constexpr (r == 0) {
        num[g] = a * S[r][g];
        sq[g] = a * z0;
      } else {
        num[g] = __builtin_fmaf(a, S[r][g], num[g]);
        sq[g] = __builtin_fmaf(a, z0, sq[g]);
      }
    });
  });
}


// The readout of the lane's G columns, stored by one wave (`mine`).
template <int D>
__device__ __forceinline__ void store_out(const StepArgs& A, long long tile, bool mine, int lane,
                                          const float* o) {
  constexpr int G = Geo<D>::G;
  if (mine) sfor<G>([&](auto gg) { A.out[tile * D + G * lane + CI(gg)] = o[CI(gg)]; });
}

// Split-mode hand-over of the update factors, [4 D] floats per tile: the gate at [0, D) (KDA:
// a_i per row; GDN: the tile's one alpha at [0]), beta k_i per row at [D, 2 D) (lane L < 32 of
// each wave, written as soon as they are loaded); per column (wave 0, after the readout) either
// e_j at [2 D, 3 D) (UV false: GDN, or any gate decaying the rows first) or u_j and v_j at
// [2 D, 4 D) (UV true: per-row gate applied after the delta update, e_ij = v_j - a_i u_j).
template <int D, bool KDA>
__device__ __forceinline__ void put_stash_rows(const StepArgs& A, long long tile, int lane,
                                               int row, float a_row, float bk_row) {
  float* st = A.stash + tile * 4 * D;
  if (lane < 32) {
    if (KDA || row == 0) st[KDA ? row : 0] = a_row;
    st[D + row] = bk_row;
  }
}

template <int D, bool UV>
__device__ __forceinline__ void put_stash_cols(const StepArgs& A, long long tile, int w,
                                               int lane, const float* e, const float* u,
                                               const float* vv) {
  constexpr int G = Geo<D>::G;
  float* st = A.stash + tile * 4 * D;
  if (w == 0) {
    sfor<G>([&](auto gg) {
      constexpr int g = CI(gg);
      if constexpr (UV) {
        st[2 * D + G * lane + g] = u[g];
        st[3 * D + G * lane + g] = vv[g];
      } else {
        st[2 * D + G * lane + g] = e[g];
      }
    });
  }
}

template <int D>
__device__ __forceinline__ void load_state(const StepArgs& A, long long tile, int row0, int lane,
                                           float (&S)[32][Geo<D>::G]) {
  constexpr int G = Geo<D>::G;
  const float* src = A.S_in + tile * D * D;
  sfor<32>([&](auto rr) {
    sfor<G>([&](auto gg) { S[CI(rr)][CI(gg)] = src[(row0 + CI(rr)) * D + G * lane + CI(gg)]; });
  });
}

// Per-tile inputs of a step: row records (lanes 0..31 of each wave fill their wave's rows),
// per-column v or the hand-over.  Returns alpha (GDN) and fills vv / e / u, and each lane's row
// gate a_row and beta k (bk_row) for the split-mode hand-over.  UV: the hand-over carries u and v
// (per-row e) instead of e.  The row records get M = a f (f = r_hat, or 1 on pivot rows and
// FP16 pivot heads), K = (beta k) / M -- or M = beta k, K = 1 for a row whose gate is below
// 2^-72 (its state is erased) or whose factor is 0 -- the key-projection coefficient k f, or
// k M when the gate decays the rows before the delta update (plan order 1), and the readout
// coefficient q M.  Encoding: M = 1.
template <int D, int MODE, bool KDA, bool UV = KDA, typename SM, typename Mid>
__device__ __forceinline__ void load_inputs(const StepArgs& A, SM& sm, long long tile, int h,
                                            int lane, int row, const uint16_t* rblk,
                                            float& alpha, float* vv, float* e, float* u,
                                            float& a_row, float& bk_row, Mid&& mid) {
  constexpr bool kWrite = MODE != READ;
  constexpr int G = Geo<D>::G;
  constexpr bool kRead = MODE == FUSED || MODE == READ;
  if constexpr (kRead) {
    sfor<G>([&](auto gg) { vv[CI(gg)] = A.v[tile * D + G * lane + CI(gg)]; });
    if constexpr (!KDA) alpha = A.alpha[tile];
  }
  if constexpr (MODE == WRITE) {
    const float* st = A.stash + tile * 4 * D;
    if constexpr (UV) {
      sfor<G>([&](auto gg) {
        u[CI(gg)] = st[2 * D + G * lane + CI(gg)];
        vv[CI(gg)] = st[3 * D + G * lane + CI(gg)];
      });
    } else {
      if constexpr (!KDA) alpha = st[0];
      sfor<G>([&](auto gg) { e[CI(gg)] = st[2 * D + G * lane + CI(gg)]; });
    }
  }
  // Every load first, in all lanes (lanes 32..63 read the same rows as lanes 0..31), then the
  // arithmetic and the record writes of lanes 0..31: the tile waits for memory once.  Without
  // stored row factors (FP16 pivot heads, encoding) a 16-bit word of the head's 1/den row is
  // read in their place and not used.
  const uint16_t* const rsrc = rblk ? rblk : reinterpret_cast<const uint16_t*>(A.P.iden + h * D);
  const uint16_t rh = rsrc[row];
  int meta = 0;
  if constexpr (KDA) meta = A.P.rowmeta[h * D + row];
  // the row factor's plan values ride in the record's rho and W slots until row_factor()
  float iden = 1.0f, om = 0.0f;
  if constexpr (kWrite) {
    iden = A.P.iden[h * D + row];
    om = A.P.omega[h * D + row];
  }
  float a = alpha, beta = 0.0f, kk = 0.0f, qv = 0.0f, bk = 0.0f;
  if constexpr (kRead) {
    beta = A.beta[tile];
    kk = A.k[tile * D + row];
    qv = A.q[tile * D + row];
    if constexpr (KDA) a = A.alpha[tile * D + row];
  }
  if constexpr (MODE == WRITE) {
    const float* st = A.stash + tile * 4 * D;
    if constexpr (KDA) a = st[row];  // GDN: alpha, read from st[0] above
    bk = st[D + row];
  }
  // the caller's own loads go out behind these (the fences keep the scheduler from hoisting
  // them): the arithmetic below then waits for the small inputs only, while the caller's
  // (larger) loads are still in flight
  __builtin_amdgcn_sched_barrier(0);
  mid();
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (kRead) bk = beta * kk;
  a_row = a;
  bk_row = bk;
  if (lane < 32) {
    auto& rec = sm.row[row];
    // row factor: r_hat of a quantized row; 1 on pivot rows and FP16 pivot heads
    const float rf = rblk && !(KDA && meta_pivot(meta)) ? h2f(rh) : 1.0f;
    if constexpr (KDA) rec.a = a;
    rec.rho = iden;
    rec.W = KDA && meta_pivot(meta) ? -1.0f : om;  // omega >= 0 (or -0) on every other row
    if constexpr (MODE == ENCODE) {
      rec.M = 1.0f;
    } else {
      const float m = a * rf;
      const bool flat = __builtin_fabsf(a) < kGateErase || rf == 0.0f;
      const float Mv = flat ? bk : m;
      rec.M = Mv;
      rec.K = flat ? 1.0f : bk / m;
      if constexpr (kRead) {
        rec.kr = A.P.order ? kk * m : kk * rf;
        rec.qm = qv * Mv;
      }
    }
  }
}

// A gate below 2^-72 erases its row's previous state: the decoded row is dropped after the key
// projection has used it (rows in the bits of `mask`, wave-uniform).  The zeros are written by
// volatile moves so that they stay inside the rarely taken branch (as plain stores of 0 the
// compiler materializes them on the common path).
template <int G>
__device__ __forceinline__ void erase_rows(float (&S)[32][G], uint64_t mask) {
  if (mask) {
#pragma unroll
    for (int r = 0; r < 32; r++) {
      if ((mask >> r) & 1) {
#pragma unroll
        for (int g = 0; g < G; g++) asm volatile("v_mov_b32 %0, 0" : "=v"(S[r][g]));
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// GDN: a whole head at one width
// ---------------------------------------------------------------------------------------------

template <int D, int MODE, int BITS, typename SM>
__device__ __forceinline__ void gdn_tile(const StepArgs& A, int b, long long slot,
                                         const HeadDisp& hd, SM& sm) {
  using Gm = Geo<D>;
  constexpr int G = Gm::G, R = Gm::R;
  constexpr int WPW = R * G * BITS / 32;  // code words per lane for one wave's rows
  constexpr float QM = (float)((1 << (BITS - 1)) - 1);
  constexpr float IQ = 1.0f / QM;
  constexpr bool kRead = MODE == FUSED || MODE == READ;   // computes u and the readout
  constexpr bool kWrite = MODE != READ;                   // refits and packs
  const int lane = threadIdx.x & 63, w = wave_id(), row0 = w * R, row = row0 + (lane & 31);
  const int h = hd.h;
  const long long tile = (long long)b * A.P.H + h;
  uint8_t* seg = A.pool + slot * A.P.bpr + hd.off;
  // this lane's code words: word x of the wave's rows at wl[64 x] (one base, immediate offsets)
  uint32_t* const wl = reinterpret_cast<uint32_t*>(seg) + (w * WPW * 64 + lane);
  uint16_t* rblk = reinterpret_cast<uint16_t*>(seg + hd.off_r);
  uint16_t* cblk = reinterpret_cast<uint16_t*>(seg + hd.off_c);
  const Rows<SM> rows(sm);
  unsigned fl = 0;

  float S[R][G];
  float e[G], u[G], vv[G], cc[G];
  uint32_t wd[WPW];
  float alpha = 0.0f;

  // ---- phase 0: the small per-tile inputs, then the code words (issued before the inputs'
  // arithmetic, so the decode below waits for each word only as it reaches it)
  float a_row, bk_row;
  load_inputs<D, MODE, false>(A, sm, tile, h, lane, row, MODE != ENCODE ? rblk : nullptr, alpha,
                              vv, e, u, a_row, bk_row, [&] {
    if constexpr (MODE != ENCODE) {
      sfor<G>([&](auto gg) { cc[CI(gg)] = h2f(cblk[G * lane + CI(gg)]); });
      __builtin_amdgcn_sched_barrier(0);  // the column factors ahead of the first code word
      sfor<WPW>([&](auto xx) {
        wd[CI(xx)] = __builtin_nontemporal_load(&wl[CI(xx) * 64]);
      });
    }
  });
  if constexpr (MODE == READ) put_stash_rows<D, false>(A, tile, lane, row, a_row, bk_row);
  wave_lds_sync();

  if constexpr (MODE == ENCODE) {
    load_state<D>(A, tile, row0, lane, S);
  } else {
    // ---- phase 1: dequantize, and u = S_hat^T k
    if constexpr (BITS <= 4) {
      decode_narrow<BITS, G, WPW>(wd, cc, S);
    } else {
      sfor<R>([&](auto rr) {
        constexpr int r = CI(rr);
        sfor<G>([&](auto gg) {
          constexpr int g = CI(gg);
          S[r][g] = cc[g] * (float)get_code<BITS, r * G + g>(wd);
        });
      });
    }
    if constexpr (kRead) {
      row_dot<G>(S, [&](int r) { return rows.r[r].kr; }, u);
      xwave_put<D>(sm, 0, w, lane, u);
      __syncthreads();
      xwave_sum<D>(sm, 0, lane, u);
      col_error<G>(A.P.order, alpha, u, vv, e);
    }
    erase_rows<G>(S, __builtin_fabsf(alpha) < kGateErase ? ~0ull : 0ull);

    // ---- phase 2: gated delta update T = fma(K, e, X) (the state is M T) and readout
    rows_pipelined([&](int r) { return rows.r[r].K; }, [&](auto rr, float K) {
      sfor<G>([&](auto gg) { S[CI(rr)][CI(gg)] = __builtin_fmaf(K, e[CI(gg)], S[CI(rr)][CI(gg)]); });
    });
    if constexpr (kRead) {
      float o[G];
      row_dot<G>(S, [&](int r) { return rows.r[r].qm; }, o);
      xwave_put<D>(sm, 1, w, lane, o);
      if constexpr (MODE == READ) {
        __syncthreads();
        xwave_sum<D>(sm, 1, lane, o);
        store_out<D>(A, tile, w == 0, lane, o);
        put_stash_cols<D, false>(A, tile, w, lane, e, u, vv);
        return;
      }
      // the fused step adds the waves' readout partials after the column-maximum barrier below
      // (slot 1 is next written after the barrier that follows that one)
    }
  }
  if constexpr (kWrite) {
    // ---- row factor from the row magnitudes
    put_rowabs<D>(sm, S, lane);
    wave_lds_sync();
    row_factor<D>(sm, lane, row, false, rblk, fl);
    wave_lds_sync();

    // ---- phase 3: y = S / r_hat = T M / r_hat, first column factor c0 = max_i |y_ij| / qmax
    float mx[G];
    scale_rows<G>(S, rows, mx);
    xwave_max_put<D>(sm, w, lane, mx);
    __syncthreads();
    float* const csh = col_share<D>(sm);
    float c0w = 0.0f, ymaxw = 0.0f;  // c0 and max |y| of column G*lane + w (waves w < G)
    if (w < G) {
      ymaxw = xwave_max_col<D>(sm, lane, w);
      c0w = ymaxw * IQ;
      csh[G * lane + w] = rcp0(c0w);
    }
    if constexpr (kRead) {
      // the fused step's readout, by the last wave (one that finishes no column statistics)
      static_assert(Gm::NW - 1 >= G, "the readout wave must not be a column-statistics wave");
      if (w == Gm::NW - 1) {
        float o[G];
        xwave_sum<D>(sm, 1, lane, o);
        store_out<D>(A, tile, true, lane, o);
      }
    }
    __syncthreads();
    float ic0[G];
    sfor<G>([&](auto gg) { ic0[CI(gg)] = csh[G * lane + CI(gg)]; });

    // ---- phase 4: first quantization and the least-squares column refit
    float num[G], sq[G], ic[G];
    ls_sums<G>(S, rows, ic0, num, sq);
    xwave_put<D>(sm, 0, w, lane, num);  // slot 0 (u) and slot 1 (readout) were last read
    xwave_put<D>(sm, 1, w, lane, sq);   // before the barriers above
    __syncthreads();
    const bool clamp_free = col_refit<D, true>(sm, csh, w, lane, c0w, cblk, ic, fl, ymaxw, QM);

    // ---- phase 5: final requantization and packing.  When no code of the tile can reach
    // +-qmax (the usual case after the refit) the clamp is the identity and is left out: the
    // same bits, one instruction per entry fewer.
    uint32_t acc = 0;
    auto store = [&](auto wi, uint32_t x) {
      __builtin_nontemporal_store(x, &wl[CI(wi) * 64]);
    };
    if (clamp_free) {
      sfor<R * G>([&](auto kk) {
        constexpr int K = CI(kk), r = K / G, g = K % G;
        put_code<BITS, K>(acc, __builtin_bit_cast(uint32_t, fma_magic(S[r][g], ic[g])), store);
      });
    } else {
      sfor<R * G>([&](auto kk) {
        constexpr int K = CI(kk), r = K / G, g = K % G;
        put_code<BITS, K>(acc, __builtin_bit_cast(uint32_t, quant_off(S[r][g], ic[g], QM)),
                          store);
      });
    }
  }
  raise_flags(A, fl);
}

// ---------------------------------------------------------------------------------------------
// GDN FP16 pivot head: the tile is stored raw in binary16, row-major
// ---------------------------------------------------------------------------------------------

template <int D, int MODE, typename SM>
__device__ __forceinline__ void pivot_tile(const StepArgs& A, int b, long long slot,
                                           const HeadDisp& hd, SM& sm) {
  using Gm = Geo<D>;
  constexpr int G = Gm::G, R = Gm::R;
  constexpr bool kRead = MODE == FUSED || MODE == READ;
  constexpr bool kWrite = MODE != READ;
  const int lane = threadIdx.x & 63, w = wave_id(), row0 = w * R, row = row0 + (lane & 31);
  const int h = hd.h;
  const long long tile = (long long)b * A.P.H + h;
  uint8_t* seg = A.pool + slot * A.P.bpr + hd.off;
  uint16_t* hblk = reinterpret_cast<uint16_t*>(seg);
  const Rows<SM> rows(sm);
  unsigned fl = 0;
  float S[R][G];
  float e[G], u[G], vv[G];
  float alpha = 0.0f;

  if constexpr (MODE == ENCODE) {
    load_state<D>(A, tile, row0, lane, S);
  } else {
    sfor<R>([&](auto rr) {
      sfor<G>([&](auto gg) {
        S[CI(rr)][CI(gg)] = h2f(hblk[(row0 + CI(rr)) * D + G * lane + CI(gg)]);
      });
    });
  }
  float a_row, bk_row;
  load_inputs<D, MODE, false>(A, sm, tile, h, lane, row, nullptr, alpha, vv, e, u, a_row, bk_row,
                              [] {});
  if constexpr (MODE == READ) put_stash_rows<D, false>(A, tile, lane, row, a_row, bk_row);
  wave_lds_sync();
  if constexpr (MODE != ENCODE) {
    if constexpr (kRead) {
      row_dot<G>(S, [&](int r) { return rows.r[r].kr; }, u);
      xwave_put<D>(sm, 0, w, lane, u);
      __syncthreads();
      xwave_sum<D>(sm, 0, lane, u);
      col_error<G>(A.P.order, alpha, u, vv, e);
    }
    erase_rows<G>(S, __builtin_fabsf(alpha) < kGateErase ? ~0ull : 0ull);
    sfor<R>([&](auto rr) {
      constexpr int r = CI(rr);
      const float K = rows.r[r].K;
      sfor<G>([&](auto gg) { S[r][CI(gg)] = __builtin_fmaf(K, e[CI(gg)], S[r][CI(gg)]); });
    });
    if constexpr (kRead) {
      float o[G];
      row_dot<G>(S, [&](int r) { return rows.r[r].qm; }, o);
      xwave_put<D>(sm, 1, w, lane, o);
      __syncthreads();
      xwave_sum<D>(sm, 1, lane, o);
      store_out<D>(A, tile, w == 0, lane, o);
      if constexpr (MODE == READ) {
        put_stash_cols<D, false>(A, tile, w, lane, e, u, vv);
        return;
      }
    }
  }
  if constexpr (kWrite) {
    put_rowabs<D>(sm, S, lane);
    sfor<R>([&](auto rr) {
      const float M = rows.r[CI(rr)].M;
      sfor<G>([&](auto gg) {
        const uint16_t hv = f2h(S[CI(rr)][CI(gg)] * M);
        if (is_inf16(hv)) fl |= kFlagPivotOvf;
        hblk[(row0 + CI(rr)) * D + G * lane + CI(gg)] = hv;
      });
    });
    wave_lds_sync();
    row_factor<D>(sm, lane, row, true, nullptr, fl);
  }
  raise_flags(A, fl);
}

// ---------------------------------------------------------------------------------------------
// KDA: per-row widths and pivot rows (wave-uniform per row).  The code block is staged in LDS;
// a row's codes sit at a uniform stream bit offset, read as a 64-bit window of the lane stream.
// ---------------------------------------------------------------------------------------------

// ORDER 0: A = Diag(a)(I - beta k k^T), a per-row error e_ij = v_j - a_i u_j.  ORDER 1:
// A = (I - beta k k^T) Diag(a): the key projection carries the gate, one error e_j = v_j - u_j
// per column.
template <int D, int MODE, int ORDER, typename SM>
__device__ __forceinline__ void kda_tile(const StepArgs& A, int b, long long slot, int h, SM& sm) {
  using Gm = Geo<D>;
  constexpr int G = Gm::G, R = Gm::R, NT = Gm::NT;
  constexpr bool kRead = MODE == FUSED || MODE == READ;
  constexpr bool kWrite = MODE != READ;
  constexpr bool kUV = ORDER == 0;  // split-mode hand-over carries u and v (per-row error)
  // passes of the workgroup over the largest code block (8-bit rows), in 16-byte units
  constexpr int kStageIt = (G * D * 8 / 32 * 16 + NT - 1) / NT;
  const int lane = threadIdx.x & 63, w = wave_id(), row0 = w * R, row = row0 + (lane & 31);
  const int tid = threadIdx.x;
  const long long tile = (long long)b * A.P.H + h;
  uint8_t* seg = A.pool + slot * A.P.bpr + kread(A.P.head_off, h);
  uint32_t* words = reinterpret_cast<uint32_t*>(seg);
  uint16_t* pblk = reinterpret_cast<uint16_t*>(seg + kread(A.P.off_piv, h));
  const int nwords = kread(A.P.words, h);
  // a head whose rows are all FP16 pivots stores no row or column factors
  uint16_t* rblk = nwords > 0 ? reinterpret_cast<uint16_t*>(seg + kread(A.P.off_r, h)) : nullptr;
  uint16_t* cblk = nwords > 0 ? reinterpret_cast<uint16_t*>(seg + kread(A.P.off_c, h)) : nullptr;
  const Rows<SM> rows(sm);
  // the wave's row metadata and 1/qmax, read in groups of eight through the scalar cache
  KConst<int>* const gmeta = (KConst<int>*)(A.P.rowmeta + (h * D + row0));
  KConst<float>* const giq = (KConst<float>*)(A.P.iq + (h * D + row0));
  unsigned fl = 0;
  float S[R][G];
  float e[G], u[G], vv[G], cc[G];
  float alpha = 0.0f;

  // ---- phase 0: stage the code block in LDS (coalesced 16-byte copies), per-row inputs.  Every
  // global load of the phase is issued before the first LDS write, so the tile waits for memory
  // once.  The column factors are read unconditionally: a head without them (all rows pivots)
  // reads its pivot block instead and never uses the values.
  const int n4 = nwords * 16;  // 16-byte units: nwords * 64 lanes * 4 bytes / 16
  u32x4* const l4 = reinterpret_cast<u32x4*>(sm.kc.code);
  u32x4 st[kStageIt];
  if constexpr (MODE != ENCODE) {
    const u32x4* g4 = reinterpret_cast<const u32x4*>(words);
    sfor<kStageIt>([&](auto ii) {
      const int x = tid + CI(ii) * NT;
      if (x < n4) st[CI(ii)] = __builtin_nontemporal_load(&g4[x]);
    });
    const uint16_t* const cread = nwords > 0 ? cblk : pblk;
    sfor<G>([&](auto gg) { cc[CI(gg)] = h2f(cread[G * lane + CI(gg)]); });
  }
  float a_row, bk_row;
  load_inputs<D, MODE, true, kUV>(A, sm, tile, h, lane, row, MODE != ENCODE ? rblk : nullptr,
                                  alpha, vv, e, u, a_row, bk_row, [] {});
  if constexpr (MODE == READ) put_stash_rows<D, true>(A, tile, lane, row, a_row, bk_row);
  if constexpr (MODE != ENCODE) {
    sfor<kStageIt>([&](auto ii) {
      const int x = tid + CI(ii) * NT;
      if (x < n4) l4[x] = st[CI(ii)];
    });
    if (tid < 16) l4[n4 + tid] = u32x4{0u, 0u, 0u, 0u};  // window over the last word
  }
  __syncthreads();

  // ---- phase 1: dequantize, u
  if constexpr (MODE == ENCODE) {
    load_state<D>(A, tile, row0, lane, S);
  } else {
    // rows in groups of eight: the group's metadata first (one scalar load of eight words), then
    // its decode; a group without a pivot row (the common case) takes a branch-free path
    sfor<R / 8>([&](auto qq) {
      constexpr int r0 = 8 * CI(qq);
      int ms[8];
      KConst<int>* const gm = opaque_s(gmeta);
      sfor<8>([&](auto tt) { ms[CI(tt)] = gm[r0 + CI(tt)]; });
      int any = 0;  // sign bit set: the group holds a pivot row
      sfor<8>([&](auto tt) { any |= ms[CI(tt)]; });
      // every row's two stream words are read before any row is decoded: one LDS wait per group
      // instead of one per row (a pivot row reads the block's first words and does not use them)
      uint32_t lo[8], hi[8];
      const char* const lane_words = reinterpret_cast<const char*>(&sm.kc.code[lane]);
      sfor<8>([&](auto tt) {
        const uint32_t* const src =
            reinterpret_cast<const uint32_t*>(lane_words + meta_lds(ms[CI(tt)]));
        lo[CI(tt)] = src[0];
        hi[CI(tt)] = src[64];
      });
      __builtin_amdgcn_sched_barrier(0);
      auto decode = [&](auto tt) {
        constexpr int t = CI(tt), r = r0 + t;
        const int bw = meta_bits(ms[t]);
        const uint32_t x = __builtin_amdgcn_alignbit(hi[t], lo[t], meta_shift(ms[t]));
        sfor<G>([&](auto gg) {
          constexpr int g = CI(gg);
          const int z = __builtin_amdgcn_sbfe((int)x, g * bw, bw);
          S[r][g] = cc[g] * (float)z;
        });
      };
      if (!meta_pivot(any)) {
        sfor<8>(decode);
      } else {
        sfor<8>([&](auto tt) {
          constexpr int t = CI(tt), r = r0 + t;
          if (meta_pivot(ms[t])) {
            const int pv = meta_pividx(ms[t]);
            sfor<G>([&](auto gg) { S[r][CI(gg)] = h2f(pblk[pv * D + G * lane + CI(gg)]); });
          } else {
            decode(tt);
          }
        });
      }
    });
    if constexpr (kRead) {
      row_dot<G>(S, [&](int r) { return rows.r[r].kr; }, u);
      xwave_put<D>(sm, 0, w, lane, u);
    }
  }
  __syncthreads();  // code block reads done (LDS reused below), cross-wave u staged
  if constexpr (kRead) {
    xwave_sum<D>(sm, 0, lane, u);
    if constexpr (!kUV) sfor<G>([&](auto gg) { e[CI(gg)] = vv[CI(gg)] - u[CI(gg)]; });
  }

  // ---- phase 2: update T = fma(K, e, X) (the state is M T), readout
  if constexpr (MODE != ENCODE) {
    erase_rows<G>(S, __builtin_amdgcn_ballot_w64(lane < 32 &&
                                                 __builtin_fabsf(a_row) < kGateErase));
    sfor<R>([&](auto rr) {
      constexpr int r = CI(rr);
      const float a = rows.r[r].a, K = rows.r[r].K;
      sfor<G>([&](auto gg) {
        constexpr int g = CI(gg);
        const float ev = kUV ? __builtin_fmaf(-a, u[g], vv[g]) : e[g];
        S[r][g] = __builtin_fmaf(K, ev, S[r][g]);
      });
    });
    if constexpr (kRead) {
      float o[G];
      row_dot<G>(S, [&](int r) { return rows.r[r].qm; }, o);
      xwave_put<D>(sm, 1, w, lane, o);
      if constexpr (MODE == READ) {
        __syncthreads();
        xwave_sum<D>(sm, 1, lane, o);
        store_out<D>(A, tile, w == 0, lane, o);
        put_stash_cols<D, kUV>(A, tile, w, lane, e, u, vv);
        return;
      }
      // the fused step adds the waves' readout partials after the next barrier (slot 1 is next
      // written after the column-maximum barrier)
    }
  }
  if constexpr (kWrite) {
    put_rowabs<D>(sm, S, lane);
    wave_lds_sync();
    const bool piv = sm.row[row].W < 0.0f;
    row_factor<D>(sm, lane, row, piv, rblk, fl);
    __syncthreads();  // every wave's transposes are done: zero the code staging for packing
    if constexpr (kRead) {
      // the fused step's readout, by the last wave
      if (w == Gm::NW - 1) {
        float o[G];
        xwave_sum<D>(sm, 1, lane, o);
        store_out<D>(A, tile, true, lane, o);
      }
    }
    {
      const int n4 = nwords * 16;
      u32x4* l4 = reinterpret_cast<u32x4*>(sm.kc.code);
      for (int x = tid; x < n4; x += NT) l4[x] = u32x4{0u, 0u, 0u, 0u};
    }

    // ---- phase 3: pivot rows stored as binary16; y and c0 = max_i |y_ij| / qmax_i (rows in
    // groups of eight: metadata and 1/qmax first, then the rows)
    float mx[G];
    sfor<G>([&](auto gg) { mx[CI(gg)] = 0.0f; });
    sfor<R / 8>([&](auto qq) {
      constexpr int r0 = 8 * CI(qq);
      int ms[8];
      float iqs[8];
      KConst<int>* const gm = opaque_s(gmeta);
      KConst<float>* const gq = opaque_s(giq);
      sfor<8>([&](auto tt) { ms[CI(tt)] = gm[r0 + CI(tt)]; });
      sfor<8>([&](auto tt) { iqs[CI(tt)] = gq[r0 + CI(tt)]; });
      int any = 0;  // sign bit set: the group holds a pivot row
      sfor<8>([&](auto tt) { any |= ms[CI(tt)]; });
      if (meta_pivot(any)) {
        sfor<8>([&](auto tt) {
          constexpr int r = r0 + CI(tt);
          if (meta_pivot(ms[CI(tt)])) {
            const int pv = meta_pividx(ms[CI(tt)]);
            const float M = rows.r[r].M;
            sfor<G>([&](auto gg) {
              const uint16_t hv = f2h(S[r][CI(gg)] * M);
              if (is_inf16(hv)) fl |= kFlagPivotOvf;
              pblk[pv * D + G * lane + CI(gg)] = hv;
            });
          }
        });
      }
      sfor<8>([&](auto tt) {
        constexpr int r = r0 + CI(tt);
        const float rho = rows.r[r].rho, iq = iqs[CI(tt)];
        sfor<G>([&](auto gg) {
          constexpr int g = CI(gg);
          S[r][g] = S[r][g] * rho;
          mx[g] = __builtin_fmaxf(mx[g], __builtin_fabsf(S[r][g]) * iq);
        });
      });
    });
    xwave_max_put<D>(sm, w, lane, mx);
    __syncthreads();  // also orders the zeroing above before the packing below
    float* const csh = col_share<D>(sm);
    float c0w = 0.0f;  // c0 of column G*lane + w (waves w < G)
    if (w < G) {
      c0w = xwave_max_col<D>(sm, lane, w);
      csh[G * lane + w] = rcp0(c0w);
    }
    __syncthreads();
    float ic0[G];
    sfor<G>([&](auto gg) { ic0[CI(gg)] = csh[G * lane + CI(gg)]; });

    // ---- phase 4: z0 and least-squares sums
    float num[G], sq[G], ic[G];
    ls_sums<G>(S, rows, ic0, num, sq);
    xwave_put<D>(sm, 0, w, lane, num);
    xwave_put<D>(sm, 1, w, lane, sq);
    __syncthreads();
    col_refit<D>(sm, csh, w, lane, c0w, cblk, ic, fl);

    // ---- phase 5: requantize and pack into the zeroed LDS stream, then copy out.  A row's G
    // codes (G * b bits) land at its uniform stream position: OR-ed into one word, or two when
    // they straddle a word boundary; words shared with a neighbouring wave's rows combine the
    // same way.  The clamp bounds +-qmax in the offset domain are the integers 0x4B400000 +-
    // qmax read as binary32 (the grid spacing there is 1).
    char* const lane_words = reinterpret_cast<char*>(&sm.kc.code[lane]);
    // a zero the optimizer cannot see: it stays in one register as the low half of every row's
    // 64-bit shift below (as a known 0 it is rematerialized by a move per row)
    const uint32_t zero = (uint32_t)opaque(0);
    sfor<R / 8>([&](auto qq) {
      constexpr int r0 = 8 * CI(qq);
      int ms[8];
      KConst<int>* const gm = opaque_s(gmeta);
      sfor<8>([&](auto tt) { ms[CI(tt)] = gm[r0 + CI(tt)]; });
      int any = 0;  // sign bit set: the group holds a pivot row
      sfor<8>([&](auto tt) { any |= ms[CI(tt)]; });
      auto pack = [&](auto tt) {
        constexpr int r = r0 + CI(tt);
        const int m = ms[CI(tt)];
        const int bw = meta_bits(m), qmi = meta_qmax(m);
        const float lo_b = __builtin_bit_cast(float, 0x4B400000 - qmi);
        const float hi_b = __builtin_bit_cast(float, 0x4B400000 | qmi);
        // each code's low bw bits enter at the top of acc (one funnel shift per code, no
        // mask): after the row's G codes they fill its top G * bw bits, code 0 lowest, zeros
        // below
        uint32_t acc = 0;
        sfor<G>([&](auto gg) {
          const float t = __builtin_amdgcn_fmed3f(fma_magic(S[r][CI(gg)], ic[CI(gg)]), lo_b, hi_b);
          acc = __builtin_amdgcn_alignbit(__builtin_bit_cast(uint32_t, t), acc, bw);
        });
        // one 64-bit shift moves them from the top of the pair (acc, 0) to bit `sh` of their
        // first stream word; the upper half is what runs into the next word
        const uint64_t y = (((uint64_t)acc << 32) | zero) >> (64 - G * bw - meta_shift(m));
        uint32_t* const dst = reinterpret_cast<uint32_t*>(lane_words + meta_lds(m));
        atomicOr(dst, (uint32_t)y);
        if (meta_straddles(m)) atomicOr(dst + 64, (uint32_t)(y >> 32));
      };
      if (!meta_pivot(any)) {
        sfor<8>(pack);
      } else {
        sfor<8>([&](auto tt) {
          if (!meta_pivot(ms[CI(tt)])) pack(tt);
        });
      }
    });
    __syncthreads();
    {
      const int n4 = nwords * 16;
      u32x4* g4 = reinterpret_cast<u32x4*>(words);
      const u32x4* l4 = reinterpret_cast<const u32x4*>(sm.kc.code);
      u32x4 st[kStageIt];
      sfor<kStageIt>([&](auto ii) {
        const int x = tid + CI(ii) * NT;
        if (x < n4) st[CI(ii)] = l4[x];
      });
      sfor<kStageIt>([&](auto ii) {
        const int x = tid + CI(ii) * NT;
        if (x < n4) __builtin_nontemporal_store(st[CI(ii)], &g4[x]);
      });
    }
  }
  raise_flags(A, fl);
}

// ---------------------------------------------------------------------------------------------
// kernels
// ---------------------------------------------------------------------------------------------

// Pool slot of batch row b (uniform over the workgroup): b itself, or slots[b] for a
// slot-indexed pool; -1 = skip the row.  Thread 0 of each request's head-0 tile records the
// resolved slot for the split-mode writeback and raises the bad-slot flag.
template <int MODE>
__device__ __forceinline__ long long pool_slot(const StepArgs& A, int b, int h) {
  if (!A.slots) return b;
  const int s = kread(A.slots, b);
  const bool valid = s >= 0 && s < A.n_slots;
  if (h == 0 && threadIdx.x == 0) {
    if (MODE == READ) A.slot_out[b] = valid ? s : -1;
    if (MODE != WRITE && !valid && s != -1) atomicOr(A.P.status, kFlagBadSlot);
  }
  return valid ? s : -1;
}

// Grid (B, H): workgroup (b, j) runs head head_order[j] of request b, the requests of one head
// dispatched together and the heads in the plan's order (longest tiles first, FP16 pivot heads
// last), which shortens the launch's ragged end.  The two grid indices need no division, and
// the dispatch position's record gives the head, its type and its segment layout at once.
template <int D, int MODE>
__global__ __launch_bounds__(Geo<D>::NT, MODE == READ ? 5 : 4) void k_gdn(StepArgs A) {
  __shared__ Smem<D, false, MODE == READ> sm;
  const int hs = blockIdx.y, b = blockIdx.x;
  const HeadDisp hd = kread_disp((KConst<HeadDisp>*)A.P.disp, hs);
  const long long slot = pool_slot<MODE>(A, b, hd.h);
  if (slot < 0) return;
  // Each tile path reads the arguments it uses itself, through an opaque pointer to the kernel
  // argument segment: argument values shared by several paths are then not loaded once before
  // the switch and held live across it (which spilled about 20 scalar registers per tile).
  // The dispatch record is re-read the same way (a scalar-cache hit by then).
  auto args = [&]() -> const StepArgs& {
    KConst<StepArgs>* const p = (KConst<StepArgs>*)__builtin_amdgcn_kernarg_segment_ptr();
    return *(const StepArgs*)opaque_s(p);
  };
  auto rec = [&]() { return kread_disp(opaque_s((KConst<HeadDisp>*)args().P.disp), hs); };
  switch (hd.type) {
    case 2: gdn_tile<D, MODE, 2>(args(), b, slot, rec(), sm); break;
    case 4: gdn_tile<D, MODE, 4>(args(), b, slot, rec(), sm); break;
    case 6: gdn_tile<D, MODE, 6>(args(), b, slot, rec(), sm); break;
    case 8: gdn_tile<D, MODE, 8>(args(), b, slot, rec(), sm); break;
    default: pivot_tile<D, MODE>(args(), b, slot, rec(), sm); break;
  }
}

template <int D, int MODE>
__global__ __launch_bounds__(Geo<D>::NT, MODE == READ ? 5 : 4) void k_kda(StepArgs A) {
  __shared__ Smem<D, true, MODE == READ> sm;
  const int b = blockIdx.x, h = blockIdx.y;  // grid (B, H)
  const long long slot = pool_slot<MODE>(A, b, h);
  if (slot < 0) return;
  if (A.P.order) kda_tile<D, MODE, 1>(A, b, slot, h, sm);
  else kda_tile<D, MODE, 0>(A, b, slot, h, sm);
}

// Debug decode: one workgroup per tile, same lane/row mapping, any head type.
template <int D>
__global__ __launch_bounds__(D) void k_unpack(DevPlan P, const uint8_t* pool, float* S,
                                              uint16_t* rout, uint16_t* cout, int8_t* zout) {
  constexpr int G = D / 64;
  const int tile = blockIdx.x;
  const int b = tile / P.H, h = tile - b * P.H;
  const int lane = threadIdx.x & 63, w = wave_id(), trow = threadIdx.x;
  const uint8_t* seg = pool + (long long)b * P.bpr + P.head_off[h];
  const uint32_t* words = reinterpret_cast<const uint32_t*>(seg);
  const uint16_t* pblk = reinterpret_cast<const uint16_t*>(seg + P.off_piv[h]);
  const bool allpiv = P.words[h] == 0;  // every row an FP16 pivot: no factor blocks
  const uint16_t* rblk = reinterpret_cast<const uint16_t*>(seg + P.off_r[h]);
  const uint16_t* cblk = reinterpret_cast<const uint16_t*>(seg + P.off_c[h]);
  if (rout) rout[(long long)tile * D + trow] = allpiv ? 0 : rblk[trow];
  if (cout) cout[(long long)tile * D + trow] = allpiv ? 0 : cblk[trow];
  for (int r = 0; r < 64; r++) {
    const int row = w * 64 + r;
    const int pr = h * D + row;
    const int pv = P.pividx[pr];
    for (int g = 0; g < G; g++) {
      const int col = G * lane + g;
      float s;
      int z = 0;
      if (pv >= 0) {
        s = h2f(pblk[pv * D + col]);
      } else {
        const int bw = P.bits[pr];
        const long long p = (long long)P.rowpos[pr] + g * bw;
        const uint32_t lo = words[(p >> 5) * 64 + lane];
        const uint32_t hi = words[((p >> 5) + 1) * 64 + lane];
        const uint32_t x = __builtin_amdgcn_alignbit(hi, lo, (uint32_t)(p & 31));
        z = __builtin_amdgcn_sbfe((int)x, 0, bw);
        s = h2f(rblk[row]) * (h2f(cblk[col]) * (float)z);
      }
      const long long e = ((long long)tile * D + row) * D + col;
      if (S) S[e] = s;
      if (zout) zout[e] = (int8_t)z;
    }
  }
}

template <int D, int KIND>
hipError_t launch_kind(Mode mode, const StepArgs& a, hipStream_t s) {
  const dim3 grid(a.B, a.P.H), block(Geo<D>::NT);
  switch (mode) {
    case FUSED:
      if constexpr (KIND == 0) hipLaunchKernelGGL((k_gdn<D, FUSED>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((k_kda<D, FUSED>), grid, block, 0, s, a);
      break;
    case READ:
      if constexpr (KIND == 0) hipLaunchKernelGGL((k_gdn<D, READ>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((k_kda<D, READ>), grid, block, 0, s, a);
      break;
    case WRITE:
      if constexpr (KIND == 0) hipLaunchKernelGGL((k_gdn<D, WRITE>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((k_kda<D, WRITE>), grid, block, 0, s, a);
      break;
    case ENCODE:
      if constexpr (KIND == 0) hipLaunchKernelGGL((k_gdn<D, ENCODE>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((k_kda<D, ENCODE>), grid, block, 0, s, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace dev
}  // namespace stepq
