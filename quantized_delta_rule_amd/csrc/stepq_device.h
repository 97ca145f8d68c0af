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
//   wave w owns rows 64w .. 64w+63, lane L owns the G = d/64 columns G*L .. G*L+G-1.  The tile
//   lives in VGPRs (64*G floats per lane).  Every reduction over rows (k^T S, q^T S, the column
//   maximum, the least-squares sums) runs inside a lane, the two waves of a d = 128 tile adding
//   their halves through LDS.  The one reduction over columns (the row's mean magnitude) goes
//   through an LDS transpose inside the wave, after which lane L owns row 64w + L.  Per-row
//   scalars are read from LDS at wave-uniform addresses (broadcast reads, no VALU work).
//
// Arithmetic matches a fixed binary32 evaluation order bit for bit:
//   dequant  S_hat = r_i c_j z_ij rounded once (c_j z_ij is exact)
//   update   e = fma(-a_i, u_j, v_j);  S = fma(a_i, S_hat, (beta k_i) e)
//   sums     aligned groups of 4 rows accumulated with fma first to last, the group sums then
//            added as a pairwise tree; the row magnitude sum is a pairwise tree over columns
//   rounding round-half-even; x + 1.5*2^23 leaves rne(x) in the low mantissa bits, whose low b
//            bits are then the two's-complement code.
// The build passes -ffp-contract=off: no multiply-add is fused unless written as fmaf.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "stepq_internal.h"

namespace stepq {
namespace dev {

constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr unsigned kFlagNonfinite = 1u, kFlagScaleOvf = 2u, kFlagPivotOvf = 4u;

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

__device__ __forceinline__ uint16_t f2h(float x) {  // v_cvt_f16_f32: nearest even, IEEE mode
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

__device__ __forceinline__ float rcp0(float x) { return x == 0.0f ? 0.0f : 1.0f / x; }

__device__ __forceinline__ bool is_inf16(uint16_t h) { return (h & 0x7FFFu) == 0x7C00u; }

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

template <int D>
struct Smem {
  static constexpr int NW = D / 64;
  float r[D], k[D], bk[D], q[D], a[D], ir[D], W[D], iq[D], qm[D];
  float red[2][NW][D];
  union {
    float absT[NW][64][65];                    // [wave][row][lane], +1 pad: conflict-free
    uint32_t code[(2 * D * 8 / 32 + 1) * 64];  // mixed-width tiles: code block staging
  };
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

__device__ __forceinline__ void raise_flags(const StepArgs& A, unsigned fl) {
  if (fl) atomicOr(A.P.status, fl);
}

// ---------------------------------------------------------------------------------------------
// shared phases
// ---------------------------------------------------------------------------------------------

// Row factor of row trow (one lane per row) from this wave's transposed |S| partials.  Writes
// r_hat to the pool (unless rblk is null) and ir = 1/r_hat (0 if dead or pivot) and
// W = (omega r_hat) r_hat (0 likewise) to LDS.
template <int D>
__device__ __forceinline__ void row_factor(Smem<D>& sm, int w, int lane, int trow, float den,
                                           float om, bool piv, uint16_t* rblk, unsigned& fl) {
  float lv[7];
  const float* src = &sm.absT[w][lane][0];
  sfor<64>([&](auto jj) { tree_push<CI(jj)>(lv, src[CI(jj)]); });
  const float m = lv[6] * (1.0f / (float)D);
  if (!__builtin_isfinite(m)) fl |= kFlagNonfinite;
  if (piv) {
    sm.ir[trow] = 0.0f;
    sm.W[trow] = 0.0f;
    if (rblk) rblk[trow] = 0;
    return;
  }
  const float r = (m + 1e-8f) / den;
  const uint16_t rh = f2h(r);
  if (is_inf16(rh)) fl |= kFlagScaleOvf;
  if (rblk) rblk[trow] = rh;
  const float rf = h2f(rh);
  sm.ir[trow] = rcp0(rf);
  sm.W[trow] = (om * rf) * rf;
}

// Adds the per-wave partials of this lane's columns across waves: red[slot][w][col].
template <int D, int G>
__device__ __forceinline__ void xwave_sum(Smem<D>& sm, int slot, int lane, float* x) {
  if constexpr (D / 64 > 1) {
    sfor<G>([&](auto gg) {
      x[CI(gg)] = sm.red[slot][0][G * lane + CI(gg)] + sm.red[slot][1][G * lane + CI(gg)];
    });
  }
}

// Stages per-wave partials for xwave_sum (caller then __syncthreads()).
template <int D, int G>
__device__ __forceinline__ void xwave_put(Smem<D>& sm, int slot, int w, int lane,
                                          const float* x) {
  if constexpr (D / 64 > 1) {
    sfor<G>([&](auto gg) { sm.red[slot][w][G * lane + CI(gg)] = x[CI(gg)]; });
  }
}

// Readout out = S^T q for this lane's columns (wave 0 stores).
template <int D, int G>
__device__ __forceinline__ void store_out(const StepArgs& A, long long tile, int w, int lane,
                                          const float* o) {
  if (w == 0) sfor<G>([&](auto gg) { A.out[tile * D + G * lane + CI(gg)] = o[CI(gg)]; });
}

// Split-mode hand-over of the update factors: a (GDN: a[0] = alpha), beta k, and e (GDN) or
// u and v (KDA) per column.
template <int D, int G, bool KDA>
__device__ __forceinline__ void put_stash(const StepArgs& A, long long tile, int w, int lane,
                                          int trow, float a_row, float bk_row, const float* e,
                                          const float* u, const float* vv) {
  float* st = A.stash + tile * 4 * D;
  st[trow] = a_row;
  st[D + trow] = bk_row;
  if (w == 0) {
    sfor<G>([&](auto gg) {
      constexpr int g = CI(gg);
      if constexpr (KDA) {
        st[2 * D + G * lane + g] = u[g];
        st[3 * D + G * lane + g] = vv[g];
      } else {
        st[2 * D + G * lane + g] = e[g];
      }
    });
  }
}

// ---------------------------------------------------------------------------------------------
// GDN: a whole head at one width
// ---------------------------------------------------------------------------------------------

template <int D, int MODE, int BITS>
__device__ __forceinline__ void gdn_tile(const StepArgs& A, int b, int h, Smem<D>& sm) {
  constexpr int G = D / 64, R = 64, NQ = R / 4;
  constexpr int WPW = R * G * BITS / 32;  // code words per lane for one wave's rows
  constexpr float QM = (float)((1 << (BITS - 1)) - 1);
  constexpr float IQ = 1.0f / QM;
  constexpr bool kRead = MODE == FUSED || MODE == READ;   // computes u and the readout
  constexpr bool kWrite = MODE != READ;                   // refits and packs
  const int lane = threadIdx.x & 63, w = wave_id(), trow = threadIdx.x, row0 = w * R;
  const long long tile = (long long)b * A.P.H + h;
  uint8_t* seg = A.pool + (long long)b * A.P.bpr + A.P.head_off[h];
  uint32_t* words = reinterpret_cast<uint32_t*>(seg);
  uint16_t* rblk = reinterpret_cast<uint16_t*>(seg + A.P.off_r[h]);
  uint16_t* cblk = reinterpret_cast<uint16_t*>(seg + A.P.off_c[h]);
  const int prow = h * D + trow;
  unsigned fl = 0;

  float S[R][G];
  float e[G], u[G], vv[G], cc[G];
  uint32_t wd[WPW > 0 ? WPW : 1];
  float alpha = 0.0f, beta = 0.0f, den = 1.0f, om = 0.0f, kk = 0.0f;

  // ---- phase 0: code loads first (they stream from HBM), then the small per-tile inputs
  if constexpr (MODE != ENCODE) {
    sfor<WPW>([&](auto xx) {
      wd[CI(xx)] = __builtin_nontemporal_load(&words[(w * WPW + CI(xx)) * 64 + lane]);
    });
    sfor<G>([&](auto gg) { cc[CI(gg)] = h2f(cblk[G * lane + CI(gg)]); });
    sm.r[trow] = h2f(rblk[trow]);
  }
  if constexpr (kRead) {
    alpha = A.alpha[tile];
    beta = A.beta[tile];
    kk = A.k[tile * D + trow];
    sm.k[trow] = kk;
    sm.bk[trow] = beta * kk;
    sm.q[trow] = A.q[tile * D + trow];
    sfor<G>([&](auto gg) { vv[CI(gg)] = A.v[tile * D + G * lane + CI(gg)]; });
  }
  if constexpr (MODE == WRITE) {
    const float* st = A.stash + tile * 4 * D;
    alpha = st[0];
    sm.bk[trow] = st[D + trow];
    sfor<G>([&](auto gg) { e[CI(gg)] = st[2 * D + G * lane + CI(gg)]; });
  }
  if constexpr (kWrite) {
    den = A.P.den[prow];
    om = A.P.omega[prow];
  }
  wave_lds_sync();

  // ---- phase 1: dequantize, and u = S_hat^T k
  if constexpr (MODE == ENCODE) {
    const float* src = A.S_in + tile * D * D;
    sfor<R>([&](auto rr) {
      sfor<G>([&](auto gg) { S[CI(rr)][CI(gg)] = src[(row0 + CI(rr)) * D + G * lane + CI(gg)]; });
    });
  } else {
    float lv[G][5];
    sfor<NQ>([&](auto mm) {
      constexpr int m = CI(mm);
      sfor<4>([&](auto tt) {
        constexpr int r = 4 * m + CI(tt);
        const float rh = sm.r[row0 + r];
        sfor<G>([&](auto gg) {
          constexpr int g = CI(gg);
          S[r][g] = rh * (cc[g] * (float)get_code<BITS, r * G + g>(wd));
        });
      });
      if constexpr (kRead) {
        const float k0 = sm.k[row0 + 4 * m], k1 = sm.k[row0 + 4 * m + 1];
        const float k2 = sm.k[row0 + 4 * m + 2], k3 = sm.k[row0 + 4 * m + 3];
        sfor<G>([&](auto gg) {
          constexpr int g = CI(gg);
          float s = k0 * S[4 * m][g];
          s = __builtin_fmaf(k1, S[4 * m + 1][g], s);
          s = __builtin_fmaf(k2, S[4 * m + 2][g], s);
          s = __builtin_fmaf(k3, S[4 * m + 3][g], s);
          tree_push<m>(lv[g], s);
        });
      }
    });
    if constexpr (kRead) {
      sfor<G>([&](auto gg) { u[CI(gg)] = lv[CI(gg)][4]; });
      xwave_put<D, G>(sm, 0, w, lane, u);
      __syncthreads();
      xwave_sum<D, G>(sm, 0, lane, u);
      sfor<G>([&](auto gg) { e[CI(gg)] = __builtin_fmaf(-alpha, u[CI(gg)], vv[CI(gg)]); });
    }
  }

  // ---- phase 2: gated delta update, readout, row magnitudes
  if constexpr (MODE != ENCODE) {
    float lv[G][5];
    sfor<NQ>([&](auto mm) {
      constexpr int m = CI(mm);
      sfor<4>([&](auto tt) {
        constexpr int r = 4 * m + CI(tt);
        const float bk = sm.bk[row0 + r];
        sfor<G>([&](auto gg) {
          constexpr int g = CI(gg);
          S[r][g] = __builtin_fmaf(alpha, S[r][g], bk * e[g]);
        });
      });
      if constexpr (kRead) {
        const float q0 = sm.q[row0 + 4 * m], q1 = sm.q[row0 + 4 * m + 1];
        const float q2 = sm.q[row0 + 4 * m + 2], q3 = sm.q[row0 + 4 * m + 3];
        sfor<G>([&](auto gg) {
          constexpr int g = CI(gg);
          float s = q0 * S[4 * m][g];
          s = __builtin_fmaf(q1, S[4 * m + 1][g], s);
          s = __builtin_fmaf(q2, S[4 * m + 2][g], s);
          s = __builtin_fmaf(q3, S[4 * m + 3][g], s);
          tree_push<m>(lv[g], s);
        });
      }
    });
    if constexpr (kRead) {
      float o[G];
      sfor<G>([&](auto gg) { o[CI(gg)] = lv[CI(gg)][4]; });
      xwave_put<D, G>(sm, 1, w, lane, o);
      __syncthreads();
      xwave_sum<D, G>(sm, 1, lane, o);
      store_out<D, G>(A, tile, w, lane, o);
      if constexpr (MODE == READ) {
        put_stash<D, G, false>(A, tile, w, lane, trow, alpha, sm.bk[trow], e, u, vv);
        return;
      }
    }
  }
  if constexpr (kWrite) {
    sfor<R>([&](auto rr) {
      constexpr int r = CI(rr);
      float a;
      if constexpr (G == 2) a = __builtin_fabsf(S[r][0]) + __builtin_fabsf(S[r][1]);
      else a = __builtin_fabsf(S[r][0]);
      sm.absT[w][r][lane] = a;
    });
    wave_lds_sync();
    row_factor<D>(sm, w, lane, trow, den, om, false, rblk, fl);
    wave_lds_sync();

    // ---- phase 3: y = S / r_hat, first column factor c0 = max_i |y_ij| / qmax
    float mx[G];
    sfor<G>([&](auto gg) { mx[CI(gg)] = 0.0f; });
    sfor<R>([&](auto rr) {
      constexpr int r = CI(rr);
      const float ir = sm.ir[row0 + r];
      sfor<G>([&](auto gg) {
        constexpr int g = CI(gg);
        S[r][g] = S[r][g] * ir;
        mx[g] = __builtin_fmaxf(mx[g], __builtin_fabsf(S[r][g]));
      });
    });
    if constexpr (D / 64 > 1) {
      sfor<G>([&](auto gg) { sm.red[0][w][G * lane + CI(gg)] = mx[CI(gg)]; });
      __syncthreads();
      sfor<G>([&](auto gg) {
        mx[CI(gg)] = __builtin_fmaxf(sm.red[0][0][G * lane + CI(gg)],
                                     sm.red[0][1][G * lane + CI(gg)]);
      });
    }
    float c0[G], ic0[G];
    sfor<G>([&](auto gg) {
      c0[CI(gg)] = mx[CI(gg)] * IQ;  // = max_i(|y| * 1/qmax): rounding is monotone
      ic0[CI(gg)] = rcp0(c0[CI(gg)]);
    });

    // ---- phase 4: first quantization z0 and the omega-weighted least-squares sums
    float ln[G][5], ls[G][5];
    sfor<NQ>([&](auto mm) {
      constexpr int m = CI(mm);
      float W4[4];
      sfor<4>([&](auto tt) { W4[CI(tt)] = sm.W[row0 + 4 * m + CI(tt)]; });
      sfor<G>([&](auto gg) {
        constexpr int g = CI(gg);
        float sn = 0.0f, sq = 0.0f;
        sfor<4>([&](auto tt) {
          constexpr int r = 4 * m + CI(tt);
          const float z0 = __builtin_rintf(S[r][g] * ic0[g]);  // |z0| <= qmax: no clamp
          const float a = W4[CI(tt)] * z0;
          if constexpr (CI(tt) == 0) {
            sn = a * S[r][g];
            sq = a * z0;
          } else {
            sn = __builtin_fmaf(a, S[r][g], sn);
            sq = __builtin_fmaf(a, z0, sq);
          }
        });
        tree_push<m>(ln[g], sn);
        tree_push<m>(ls[g], sq);
      });
    });
    float num[G], sq[G];
    sfor<G>([&](auto gg) {
      num[CI(gg)] = ln[CI(gg)][4];
      sq[CI(gg)] = ls[CI(gg)][4];
    });
    if constexpr (D / 64 > 1) {
      xwave_put<D, G>(sm, 0, w, lane, num);
      xwave_put<D, G>(sm, 1, w, lane, sq);
      __syncthreads();
      xwave_sum<D, G>(sm, 0, lane, num);
      xwave_sum<D, G>(sm, 1, lane, sq);
    }
    float ic[G];
    sfor<G>([&](auto gg) {
      constexpr int g = CI(gg);
      const float c1 = sq[g] > 0.0f ? num[g] / sq[g] : c0[g];
      const uint16_t ch = f2h(c1);
      if (is_inf16(ch)) fl |= kFlagScaleOvf;
      if (w == 0) cblk[G * lane + g] = ch;
      ic[g] = rcp0(h2f(ch));
    });

    // ---- phase 5: final round-half-even requantization and packing
    uint32_t acc = 0;
    auto store = [&](auto wi, uint32_t x) {
      __builtin_nontemporal_store(x, &words[(w * WPW + CI(wi)) * 64 + lane]);
    };
    sfor<R * G>([&](auto kk2) {
      constexpr int K = CI(kk2), r = K / G, g = K % G;
      float t = __builtin_amdgcn_fmed3f(S[r][g] * ic[g], -QM, QM);
      uint32_t f = __builtin_bit_cast(uint32_t, t + kMagic);
      put_code<BITS, K>(acc, f, store);
    });
  }
  raise_flags(A, fl);
}

// ---------------------------------------------------------------------------------------------
// GDN FP16 pivot head: the tile is stored raw in binary16, row-major
// ---------------------------------------------------------------------------------------------

template <int D, int MODE>
__device__ __forceinline__ void pivot_tile(const StepArgs& A, int b, int h, Smem<D>& sm) {
  constexpr int G = D / 64, R = 64, NQ = R / 4;
  constexpr bool kRead = MODE == FUSED || MODE == READ;
  constexpr bool kWrite = MODE != READ;
  const int lane = threadIdx.x & 63, w = wave_id(), trow = threadIdx.x, row0 = w * R;
  const long long tile = (long long)b * A.P.H + h;
  uint8_t* seg = A.pool + (long long)b * A.P.bpr + A.P.head_off[h];
  uint16_t* hblk = reinterpret_cast<uint16_t*>(seg);
  unsigned fl = 0;
  float S[R][G];
  float e[G], u[G], vv[G];
  float alpha = 0.0f, beta = 0.0f;

  if constexpr (MODE == ENCODE) {
    const float* src = A.S_in + tile * D * D;
    sfor<R>([&](auto rr) {
      sfor<G>([&](auto gg) { S[CI(rr)][CI(gg)] = src[(row0 + CI(rr)) * D + G * lane + CI(gg)]; });
    });
  } else {
    sfor<R>([&](auto rr) {
      sfor<G>([&](auto gg) {
        S[CI(rr)][CI(gg)] = h2f(hblk[(row0 + CI(rr)) * D + G * lane + CI(gg)]);
      });
    });
  }
  if constexpr (kRead) {
    alpha = A.alpha[tile];
    beta = A.beta[tile];
    const float kk = A.k[tile * D + trow];
    sm.k[trow] = kk;
    sm.bk[trow] = beta * kk;
    sm.q[trow] = A.q[tile * D + trow];
    sfor<G>([&](auto gg) { vv[CI(gg)] = A.v[tile * D + G * lane + CI(gg)]; });
  }
  if constexpr (MODE == WRITE) {
    const float* st = A.stash + tile * 4 * D;
    alpha = st[0];
    sm.bk[trow] = st[D + trow];
    sfor<G>([&](auto gg) { e[CI(gg)] = st[2 * D + G * lane + CI(gg)]; });
  }
  wave_lds_sync();
  if constexpr (kRead) {
    float lv[G][5];
    sfor<NQ>([&](auto mm) {
      constexpr int m = CI(mm);
      const float k0 = sm.k[row0 + 4 * m], k1 = sm.k[row0 + 4 * m + 1];
      const float k2 = sm.k[row0 + 4 * m + 2], k3 = sm.k[row0 + 4 * m + 3];
      sfor<G>([&](auto gg) {
        constexpr int g = CI(gg);
        float s = k0 * S[4 * m][g];
        s = __builtin_fmaf(k1, S[4 * m + 1][g], s);
        s = __builtin_fmaf(k2, S[4 * m + 2][g], s);
        s = __builtin_fmaf(k3, S[4 * m + 3][g], s);
        tree_push<m>(lv[g], s);
      });
    });
    sfor<G>([&](auto gg) { u[CI(gg)] = lv[CI(gg)][4]; });
    xwave_put<D, G>(sm, 0, w, lane, u);
    __syncthreads();
    xwave_sum<D, G>(sm, 0, lane, u);
    sfor<G>([&](auto gg) { e[CI(gg)] = __builtin_fmaf(-alpha, u[CI(gg)], vv[CI(gg)]); });
  }
  if constexpr (MODE != ENCODE) {
    float lv[G][5];
    sfor<NQ>([&](auto mm) {
      constexpr int m = CI(mm);
      sfor<4>([&](auto tt) {
        constexpr int r = 4 * m + CI(tt);
        const float bk = sm.bk[row0 + r];
        sfor<G>([&](auto gg) {
          S[r][CI(gg)] = __builtin_fmaf(alpha, S[r][CI(gg)], bk * e[CI(gg)]);
        });
      });
      if constexpr (kRead) {
        const float q0 = sm.q[row0 + 4 * m], q1 = sm.q[row0 + 4 * m + 1];
        const float q2 = sm.q[row0 + 4 * m + 2], q3 = sm.q[row0 + 4 * m + 3];
        sfor<G>([&](auto gg) {
          constexpr int g = CI(gg);
          float s = q0 * S[4 * m][g];
          s = __builtin_fmaf(q1, S[4 * m + 1][g], s);
          s = __builtin_fmaf(q2, S[4 * m + 2][g], s);
          s = __builtin_fmaf(q3, S[4 * m + 3][g], s);
          tree_push<m>(lv[g], s);
        });
      }
    });
    if constexpr (kRead) {
      float o[G];
      sfor<G>([&](auto gg) { o[CI(gg)] = lv[CI(gg)][4]; });
      xwave_put<D, G>(sm, 1, w, lane, o);
      __syncthreads();
      xwave_sum<D, G>(sm, 1, lane, o);
      store_out<D, G>(A, tile, w, lane, o);
      if constexpr (MODE == READ) {
        put_stash<D, G, false>(A, tile, w, lane, trow, alpha, sm.bk[trow], e, u, vv);
        return;
      }
    }
  }
  if constexpr (kWrite) {
    sfor<R>([&](auto rr) {
      constexpr int r = CI(rr);
      float a;
      if constexpr (G == 2) a = __builtin_fabsf(S[r][0]) + __builtin_fabsf(S[r][1]);
      else a = __builtin_fabsf(S[r][0]);
      sm.absT[w][r][lane] = a;
      sfor<G>([&](auto gg) {
        const uint16_t hv = f2h(S[r][CI(gg)]);
        if (is_inf16(hv)) fl |= kFlagPivotOvf;
        hblk[(row0 + r) * D + G * lane + CI(gg)] = hv;
      });
    });
    wave_lds_sync();
    row_factor<D>(sm, w, lane, trow, 1.0f, 0.0f, true, nullptr, fl);
  }
  raise_flags(A, fl);
}

// ---------------------------------------------------------------------------------------------
// KDA: per-row widths and pivot rows (wave-uniform per row).  The code block is staged in LDS;
// a row's codes sit at a uniform stream bit offset, read as a 64-bit window of the lane stream.
// ---------------------------------------------------------------------------------------------

template <int D, int MODE>
__device__ __forceinline__ void kda_tile(const StepArgs& A, int b, int h, Smem<D>& sm) {
  constexpr int G = D / 64, R = 64, NQ = R / 4, NT = D;
  constexpr bool kRead = MODE == FUSED || MODE == READ;
  constexpr bool kWrite = MODE != READ;
  const int lane = threadIdx.x & 63, w = wave_id(), trow = threadIdx.x, row0 = w * R;
  const long long tile = (long long)b * A.P.H + h;
  uint8_t* seg = A.pool + (long long)b * A.P.bpr + A.P.head_off[h];
  uint32_t* words = reinterpret_cast<uint32_t*>(seg);
  uint16_t* pblk = reinterpret_cast<uint16_t*>(seg + A.P.off_piv[h]);
  uint16_t* rblk = reinterpret_cast<uint16_t*>(seg + A.P.off_r[h]);
  uint16_t* cblk = reinterpret_cast<uint16_t*>(seg + A.P.off_c[h]);
  const int nwords = A.P.words[h];
  const int* bitsv = A.P.bits + h * D;
  const int* posv = A.P.rowpos + h * D;
  const int* pidv = A.P.pividx + h * D;
  const int prow = h * D + trow;
  unsigned fl = 0;
  float S[R][G];
  float u[G], vv[G], cc[G];
  float beta = 0.0f, den = 1.0f, om = 0.0f;

  // ---- phase 0: stage the code block in LDS (coalesced 16-byte copies), per-row inputs
  if constexpr (MODE != ENCODE) {
    const int n4 = nwords * 16;  // uint4 count: nwords * 64 lanes / 4
    const u32x4* g4 = reinterpret_cast<const u32x4*>(words);
    u32x4* l4 = reinterpret_cast<u32x4*>(sm.code);
    for (int x = trow; x < n4; x += NT) l4[x] = __builtin_nontemporal_load(&g4[x]);
    if (trow < 16) l4[n4 + trow] = u32x4{0u, 0u, 0u, 0u};  // window over the last word
    sfor<G>([&](auto gg) { cc[CI(gg)] = h2f(cblk[G * lane + CI(gg)]); });
    sm.r[trow] = h2f(rblk[trow]);
  }
  if constexpr (kRead) {
    beta = A.beta[tile];
    const float kk = A.k[tile * D + trow];
    const float ar = A.alpha[tile * D + trow];
    sm.k[trow] = kk;
    sm.bk[trow] = beta * kk;
    sm.a[trow] = ar;
    sm.q[trow] = A.q[tile * D + trow];
    sfor<G>([&](auto gg) { vv[CI(gg)] = A.v[tile * D + G * lane + CI(gg)]; });
  }
  if constexpr (MODE == WRITE) {
    const float* st = A.stash + tile * 4 * D;
    sm.a[trow] = st[trow];
    sm.bk[trow] = st[D + trow];
    sfor<G>([&](auto gg) {
      u[CI(gg)] = st[2 * D + G * lane + CI(gg)];
      vv[CI(gg)] = st[3 * D + G * lane + CI(gg)];
    });
  }
  if constexpr (kWrite) {
    den = A.P.den[prow];
    om = A.P.omega[prow];
    sm.iq[trow] = A.P.iq[prow];
    sm.qm[trow] = A.P.qmax[prow];
  }
  __syncthreads();

  // ---- phase 1: dequantize, u
  if constexpr (MODE == ENCODE) {
    const float* src = A.S_in + tile * D * D;
    sfor<R>([&](auto rr) {
      sfor<G>([&](auto gg) { S[CI(rr)][CI(gg)] = src[(row0 + CI(rr)) * D + G * lane + CI(gg)]; });
    });
  } else {
    sfor<R>([&](auto rr) {
      constexpr int r = CI(rr);
      const int row = row0 + r;
      const int pv = __builtin_amdgcn_readfirstlane(pidv[row]);
      if (pv >= 0) {
        sfor<G>([&](auto gg) { S[r][CI(gg)] = h2f(pblk[pv * D + G * lane + CI(gg)]); });
      } else {
        const int bw = __builtin_amdgcn_readfirstlane(bitsv[row]);
        const int p = __builtin_amdgcn_readfirstlane(posv[row]);
        const uint32_t lo = sm.code[(p >> 5) * 64 + lane];
        const uint32_t hi = sm.code[((p >> 5) + 1) * 64 + lane];
        const uint32_t x = __builtin_amdgcn_alignbit(hi, lo, p & 31);
        const float rh = sm.r[row];
        sfor<G>([&](auto gg) {
          constexpr int g = CI(gg);
          const int z = __builtin_amdgcn_sbfe((int)x, g * bw, bw);
          S[r][g] = rh * (cc[g] * (float)z);
        });
      }
    });
    if constexpr (kRead) {
      float lv[G][5];
      sfor<NQ>([&](auto mm) {
        constexpr int m = CI(mm);
        const float k0 = sm.k[row0 + 4 * m], k1 = sm.k[row0 + 4 * m + 1];
        const float k2 = sm.k[row0 + 4 * m + 2], k3 = sm.k[row0 + 4 * m + 3];
        sfor<G>([&](auto gg) {
          constexpr int g = CI(gg);
          float s = k0 * S[4 * m][g];
          s = __builtin_fmaf(k1, S[4 * m + 1][g], s);
          s = __builtin_fmaf(k2, S[4 * m + 2][g], s);
          s = __builtin_fmaf(k3, S[4 * m + 3][g], s);
          tree_push<m>(lv[g], s);
        });
      });
      sfor<G>([&](auto gg) { u[CI(gg)] = lv[CI(gg)][4]; });
      xwave_put<D, G>(sm, 0, w, lane, u);
    }
  }
  __syncthreads();  // code block reads done (LDS reused below), cross-wave u staged
  if constexpr (kRead) xwave_sum<D, G>(sm, 0, lane, u);

  // ---- phase 2: update, readout, row magnitudes
  if constexpr (MODE != ENCODE) {
    float lv[G][5];
    sfor<NQ>([&](auto mm) {
      constexpr int m = CI(mm);
      sfor<4>([&](auto tt) {
        constexpr int r = 4 * m + CI(tt);
        const float ar = sm.a[row0 + r], bk = sm.bk[row0 + r];
        sfor<G>([&](auto gg) {
          constexpr int g = CI(gg);
          const float ev = __builtin_fmaf(-ar, u[g], vv[g]);
          S[r][g] = __builtin_fmaf(ar, S[r][g], bk * ev);
        });
      });
      if constexpr (kRead) {
        const float q0 = sm.q[row0 + 4 * m], q1 = sm.q[row0 + 4 * m + 1];
        const float q2 = sm.q[row0 + 4 * m + 2], q3 = sm.q[row0 + 4 * m + 3];
        sfor<G>([&](auto gg) {
          constexpr int g = CI(gg);
          float s = q0 * S[4 * m][g];
          s = __builtin_fmaf(q1, S[4 * m + 1][g], s);
          s = __builtin_fmaf(q2, S[4 * m + 2][g], s);
          s = __builtin_fmaf(q3, S[4 * m + 3][g], s);
          tree_push<m>(lv[g], s);
        });
      }
    });
    if constexpr (kRead) {
      float o[G];
      sfor<G>([&](auto gg) { o[CI(gg)] = lv[CI(gg)][4]; });
      xwave_put<D, G>(sm, 1, w, lane, o);
      __syncthreads();
      xwave_sum<D, G>(sm, 1, lane, o);
      store_out<D, G>(A, tile, w, lane, o);
      if constexpr (MODE == READ) {
        put_stash<D, G, true>(A, tile, w, lane, trow, sm.a[trow], sm.bk[trow], nullptr, u, vv);
        return;
      }
    }
  }
  if constexpr (kWrite) {
    sfor<R>([&](auto rr) {
      constexpr int r = CI(rr);
      float a;
      if constexpr (G == 2) a = __builtin_fabsf(S[r][0]) + __builtin_fabsf(S[r][1]);
      else a = __builtin_fabsf(S[r][0]);
      sm.absT[w][r][lane] = a;
    });
    wave_lds_sync();
    const bool piv = A.P.pividx[prow] >= 0;
    row_factor<D>(sm, w, lane, trow, den, om, piv, rblk, fl);
    __syncthreads();  // absT dead for every wave: the code staging area is zeroed for packing
    {
      const int n4 = nwords * 16;
      u32x4* l4 = reinterpret_cast<u32x4*>(sm.code);
      for (int x = trow; x < n4; x += NT) l4[x] = u32x4{0u, 0u, 0u, 0u};
    }

    // ---- phase 3: y, c0 = max_i |y_ij| / qmax_i ; pivot rows: store binary16
    float mx[G];
    sfor<G>([&](auto gg) { mx[CI(gg)] = 0.0f; });
    sfor<R>([&](auto rr) {
      constexpr int r = CI(rr);
      const int row = row0 + r;
      const int pv = __builtin_amdgcn_readfirstlane(pidv[row]);
      if (pv >= 0) {
        sfor<G>([&](auto gg) {
          const uint16_t hv = f2h(S[r][CI(gg)]);
          if (is_inf16(hv)) fl |= kFlagPivotOvf;
          pblk[pv * D + G * lane + CI(gg)] = hv;
        });
      }
      const float ir = sm.ir[row], iq = sm.iq[row];
      sfor<G>([&](auto gg) {
        constexpr int g = CI(gg);
        S[r][g] = S[r][g] * ir;
        mx[g] = __builtin_fmaxf(mx[g], __builtin_fabsf(S[r][g]) * iq);
      });
    });
    if constexpr (D / 64 > 1) {
      sfor<G>([&](auto gg) { sm.red[0][w][G * lane + CI(gg)] = mx[CI(gg)]; });
    }
    __syncthreads();  // also orders the zeroing above before the packing below
    if constexpr (D / 64 > 1) {
      sfor<G>([&](auto gg) {
        mx[CI(gg)] = __builtin_fmaxf(sm.red[0][0][G * lane + CI(gg)],
                                     sm.red[0][1][G * lane + CI(gg)]);
      });
    }
    float c0[G], ic0[G];
    sfor<G>([&](auto gg) {
      c0[CI(gg)] = mx[CI(gg)];
      ic0[CI(gg)] = rcp0(mx[CI(gg)]);
    });

    // ---- phase 4: z0 and least-squares sums
    float ln[G][5], ls[G][5];
    sfor<NQ>([&](auto mm) {
      constexpr int m = CI(mm);
      float W4[4];
      sfor<4>([&](auto tt) { W4[CI(tt)] = sm.W[row0 + 4 * m + CI(tt)]; });
      sfor<G>([&](auto gg) {
        constexpr int g = CI(gg);
        float sn = 0.0f, sq = 0.0f;
        sfor<4>([&](auto tt) {
          constexpr int r = 4 * m + CI(tt);
          const float z0 = __builtin_rintf(S[r][g] * ic0[g]);
          const float a = W4[CI(tt)] * z0;
          if constexpr (CI(tt) == 0) {
            sn = a * S[r][g];
            sq = a * z0;
          } else {
            sn = __builtin_fmaf(a, S[r][g], sn);
            sq = __builtin_fmaf(a, z0, sq);
          }
        });
        tree_push<m>(ln[g], sn);
        tree_push<m>(ls[g], sq);
      });
    });
    float num[G], sq[G];
    sfor<G>([&](auto gg) {
      num[CI(gg)] = ln[CI(gg)][4];
      sq[CI(gg)] = ls[CI(gg)][4];
    });
    if constexpr (D / 64 > 1) {
      xwave_put<D, G>(sm, 0, w, lane, num);
      xwave_put<D, G>(sm, 1, w, lane, sq);
      __syncthreads();
      xwave_sum<D, G>(sm, 0, lane, num);
      xwave_sum<D, G>(sm, 1, lane, sq);
    }
    float ic[G];
    sfor<G>([&](auto gg) {
      constexpr int g = CI(gg);
      const float c1 = sq[g] > 0.0f ? num[g] / sq[g] : c0[g];
      const uint16_t ch = f2h(c1);
      if (is_inf16(ch)) fl |= kFlagScaleOvf;
      if (w == 0) cblk[G * lane + g] = ch;
      ic[g] = rcp0(h2f(ch));
    });

    // ---- phase 5: requantize and pack into the LDS stream (uniform positions), then copy out
    {
      unsigned long long acc = 0;
      int cw = -1;         // word index held in the low half of acc
      bool first = true;   // the wave's first word may be shared with the previous wave
      auto flush = [&](bool shared) {
        const uint32_t lo = (uint32_t)acc;
        if (shared) atomicOr(&sm.code[cw * 64 + lane], lo);
        else sm.code[cw * 64 + lane] = lo;
      };
      sfor<R>([&](auto rr) {
        constexpr int r = CI(rr);
        const int row = row0 + r;
        const int bw = __builtin_amdgcn_readfirstlane(bitsv[row]);
        if (__builtin_amdgcn_readfirstlane(pidv[row]) < 0) {
          const int p = __builtin_amdgcn_readfirstlane(posv[row]);
          const float qm = sm.qm[row];
          const uint32_t mask = (1u << bw) - 1u;
          uint32_t wv = 0;
          sfor<G>([&](auto gg) {
            constexpr int g = CI(gg);
            const float t = __builtin_amdgcn_fmed3f(S[r][g] * ic[g], -qm, qm);
            const uint32_t f = __builtin_bit_cast(uint32_t, t + kMagic) & mask;
            wv |= f << (g * bw);
          });
          if (cw < 0) cw = p >> 5;
          while ((p >> 5) > cw) {  // uniform: move to the word holding this row's first bit
            flush(first);
            first = false;
            acc >>= 32;
            cw++;
          }
          acc |= (unsigned long long)wv << (p & 31);
        }
      });
      if (cw >= 0) {
        flush(true);  // the last word may be shared with the next wave
        // bits of a row that straddles past this word belong to word cw + 1
        const uint32_t hi = (uint32_t)(acc >> 32);
        if (hi) atomicOr(&sm.code[(cw + 1) * 64 + lane], hi);
      }
    }
    __syncthreads();
    {
      const int n4 = nwords * 16;
      u32x4* g4 = reinterpret_cast<u32x4*>(words);
      const u32x4* l4 = reinterpret_cast<const u32x4*>(sm.code);
      for (int x = trow; x < n4; x += NT) __builtin_nontemporal_store(l4[x], &g4[x]);
    }
  }
  raise_flags(A, fl);
}

// ---------------------------------------------------------------------------------------------
// kernels
// ---------------------------------------------------------------------------------------------

template <int D, int MODE>
__global__ __launch_bounds__(D) void k_gdn(StepArgs A) {
  __shared__ Smem<D> sm;
  const int tile = blockIdx.x;
  const int b = tile / A.P.H, h = tile - b * A.P.H;
  switch (A.P.head_type[h]) {
    case 2: gdn_tile<D, MODE, 2>(A, b, h, sm); break;
    case 4: gdn_tile<D, MODE, 4>(A, b, h, sm); break;
    case 6: gdn_tile<D, MODE, 6>(A, b, h, sm); break;
    case 8: gdn_tile<D, MODE, 8>(A, b, h, sm); break;
    default: pivot_tile<D, MODE>(A, b, h, sm); break;
  }
}

template <int D, int MODE>
__global__ __launch_bounds__(D) void k_kda(StepArgs A) {
  __shared__ Smem<D> sm;
  const int tile = blockIdx.x;
  const int b = tile / A.P.H, h = tile - b * A.P.H;
  kda_tile<D, MODE>(A, b, h, sm);
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
  const bool allpiv = P.head_type[h] == kHeadPivot;
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
  const dim3 grid(a.B * a.P.H), block(D);
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
