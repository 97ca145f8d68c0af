// stepq_offline.cpp -- offline planning on the host (binary64): lifetime weight, row impact,
// pivot choice and the two bit allocators.
//
// Page: "STEPQuant" paper digest (vibe-research silicon-writer readme).
//   Method 1 "Lifetime-aware Bit Allocation": per unit u, a distortion table d_u(b) and the mean
//   log retention gate l_u; over a window of H future steps the error lifetime weight is
//   L_u = sum_{j<H} exp(2 j l_u); minimise sum_u L_u d_u(b_u) under an average-bit budget, by a
//   multiple-choice dynamic program when the unit is a head (GDN) and by a Lagrangian solve with
//   discrete budget repair when the unit is a key row (KDA); a few FP16 pivot units protect the
//   hardest units.
//   Method 2 "Row-impact": g_t = A_t^T q_t, omega_i = E[g_{t,i}^2].
#include <algorithm>
#include <cmath>
#include <limits>
#include <numeric>
#include <string>
#include <vector>

#include "stepq.h"
#include "stepq_internal.h"

namespace {
// a refused call: its message goes to the library's error slot (stepq_last_error)
int bad(const char* m) { return stepq::fail(STEPQ_ERR_INVALID_ARG, "%s", m); }
}  // namespace

extern "C" {

int stepq_lifetime_weights(const double* l_u, int n, int H, double* L_out) {
  if (!l_u || !L_out || n < 0 || H < 1) return bad("lifetime_weights: bad arguments");
  for (int u = 0; u < n; u++) {
    const double l = l_u[u];
    if (!(l <= 0.0) || !std::isfinite(l)) return bad("lifetime_weights: l_u must be finite and <= 0");
    // geometric series sum_{j<H} x^j with x = exp(2l), written with expm1 so l -> 0 stays exact
    L_out[u] = l == 0.0 ? (double)H : std::expm1(2.0 * H * l) / std::expm1(2.0 * l);
  }
  stepq::clear_error();
  return STEPQ_OK;
}

int stepq_row_impact_accumulate(int n, int d, const float* q, const float* k, const float* a,
                                const float* beta, int order, double* acc) {
  if (n < 0 || d < 1 || (n > 0 && (!q || !k || !a || !beta)) || !acc ||
      (order != STEPQ_ORDER_DELTA_FIRST && order != STEPQ_ORDER_DECAY_FIRST))
    return bad("row_impact_accumulate: bad arguments");
  std::vector<double> aq(d);
  for (int t = 0; t < n; t++) {
    const float* qt = q + (long long)t * d;
    const float* kt = k + (long long)t * d;
    const float* at = a + (long long)t * d;
    double kx = 0.0;  // k . (a*q), or k . q when the rows decay first
    for (int i = 0; i < d; i++) {
      aq[i] = (double)at[i] * (double)qt[i];
      kx += (double)kt[i] * (order == STEPQ_ORDER_DECAY_FIRST ? (double)qt[i] : aq[i]);
    }
    const double s = (double)beta[t] * kx;
    for (int i = 0; i < d; i++) {
      // g = A^T q:  Diag(a)(I - b k k^T) -> a*q - s k;  (I - b k k^T) Diag(a) -> a (q - s k)
      const double g = order == STEPQ_ORDER_DECAY_FIRST
                           ? (double)at[i] * ((double)qt[i] - s * (double)kt[i])
                           : aq[i] - s * (double)kt[i];
      acc[i] += g * g;
    }
  }
  stepq::clear_error();
  return STEPQ_OK;
}

int stepq_select_pivots(const double* risk, int n, int n_pivots, int32_t* out_idx) {
  if (!risk || n < 0 || n_pivots < 0 || n_pivots > n || (n_pivots > 0 && !out_idx))
    return bad("select_pivots: bad arguments");
  std::vector<int> idx(n);
  std::iota(idx.begin(), idx.end(), 0);
  std::stable_sort(idx.begin(), idx.end(), [&](int x, int y) { return risk[x] > risk[y]; });
  std::vector<int> pick(idx.begin(), idx.begin() + n_pivots);
  std::sort(pick.begin(), pick.end());
  for (int i = 0; i < n_pivots; i++) out_idx[i] = pick[i];
  stepq::clear_error();
  return STEPQ_OK;
}

int stepq_alloc_mcdp(const double* cost, int n_units, const int* choices, int n_choices,
                     long capacity_bits, int* bits_out, double* objective) {
  if (!cost || !choices || !bits_out || n_units < 0 || n_choices < 1 || capacity_bits < 0)
    return bad("alloc_mcdp: bad arguments");
  for (int c = 0; c < n_choices; c++)
    if (choices[c] < 2 || choices[c] % 2 || (c && choices[c] <= choices[c - 1]))
      return bad("alloc_mcdp: choices must be ascending even widths");
  // States count bits in steps of two: dp[c] = cheapest cost of the units so far using exactly
  // 2c bits.  Choices are tried in ascending width and replace the incumbent only when strictly
  // cheaper, so equal costs keep the narrower width.
  const long cap = capacity_bits / 2;
  const double INF = std::numeric_limits<double>::infinity();
  std::vector<double> dp(cap + 1, INF), nd(cap + 1);
  std::vector<signed char> pick((size_t)n_units * (cap + 1), -1);
  dp[0] = 0.0;
  for (int u = 0; u < n_units; u++) {
    std::fill(nd.begin(), nd.end(), INF);
    for (long c = 0; c <= cap; c++) {
      for (int ci = 0; ci < n_choices; ci++) {
        const long wc = choices[ci] / 2;
        if (c - wc < 0 || dp[c - wc] == INF) continue;
        const double val = dp[c - wc] + cost[(size_t)u * n_choices + ci];
        if (val < nd[c]) {
          nd[c] = val;
          pick[(size_t)u * (cap + 1) + c] = (signed char)ci;
        }
      }
    }
    dp.swap(nd);
  }
  long best_c = -1;
  double best = INF;
  for (long c = 0; c <= cap; c++)
    if (dp[c] < best) {
      best = dp[c];
      best_c = c;
    }
  if (best_c < 0) return bad("alloc_mcdp: budget below the narrowest width");
  long c = best_c;
  for (int u = n_units - 1; u >= 0; u--) {
    const int ci = pick[(size_t)u * (cap + 1) + c];
    bits_out[u] = choices[ci];
    c -= choices[ci] / 2;
  }
  if (objective) *objective = best;
  stepq::clear_error();
  return STEPQ_OK;
}

int stepq_alloc_lagrangian(const double* L, const double* d, const double* n, int n_units,
                           const int* choices, int n_choices, double budget_bits, int iters,
                           int* bits_out, double* objective) {
  if (!L || !d || !n || !choices || !bits_out || n_units < 0 || n_choices < 1 || iters < 0)
    return bad("alloc_lagrangian: bad arguments");
  const int N = n_units;
  std::vector<int> bi(N);
  auto assign = [&](double lam) {
    for (int u = 0; u < N; u++) {
      double best = 0.0;
      int arg = 0;
      for (int ci = 0; ci < n_choices; ci++) {
        const double val = L[u] * d[(size_t)u * n_choices + ci] + lam * n[u] * choices[ci];
        if (ci == 0 || val < best) {
          best = val;
          arg = ci;
        }
      }
      bi[u] = arg;
    }
  };
  auto total = [&]() {
    double t = 0.0;
    for (int u = 0; u < N; u++) t += n[u] * choices[bi[u]];
    return t;
  };
  // the multiplier: double until feasible, then bisect keeping the feasible end
  double hi = 1.0;
  assign(hi);
  while (total() > budget_bits) {
    hi *= 2.0;
    if (hi > 1e300) return bad("alloc_lagrangian: budget below the narrowest width");
    assign(hi);
  }
  double lo = 0.0;
  for (int it = 0; it < iters; it++) {
    const double mid = 0.5 * (lo + hi);
    assign(mid);
    if (total() <= budget_bits) hi = mid;
    else lo = mid;
  }
  assign(hi);
  double used = total();
  // repair: spend what is left on the best single-step upgrades (ties to the lower unit)
  for (;;) {
    double best = 0.0;
    int bu = -1;
    for (int u = 0; u < N; u++) {
      const int ci = bi[u];
      if (ci + 1 >= n_choices) continue;
      const double extra = n[u] * (choices[ci + 1] - choices[ci]);
      if (used + extra > budget_bits) continue;
      const double gain =
          (L[u] * (d[(size_t)u * n_choices + ci] - d[(size_t)u * n_choices + ci + 1])) / extra;
      if (bu < 0 || gain > best) {
        best = gain;
        bu = u;
      }
    }
    if (bu < 0 || best <= 0.0) break;
    used += n[bu] * (choices[bi[bu] + 1] - choices[bi[bu]]);
    bi[bu] += 1;
  }
  double obj = 0.0;
  for (int u = 0; u < N; u++) {
    bits_out[u] = choices[bi[u]];
    obj += L[u] * d[(size_t)u * n_choices + bi[u]];
  }
  if (objective) *objective = obj;
  stepq::clear_error();
  return STEPQ_OK;
}

}  // extern "C"
