// Budgeted per-matrix bitrates: one candidate rate per matrix under a total bit budget.
//
// [ABS]: compression at arbitrary target rates with sampled storage estimates; [README]
// 性能 / [NEWS] 官方基準: whole-model packs at a fixed average rate (e.g. 2.3 / 3.0 bpp for
// the 276 layers of a diffusion transformer).  Spending those bits unevenly — more where
// a matrix's error falls fastest — is the data-free part of mixed-precision allocation:
// every matrix i comes with measured (bits, cost) points, one per candidate target
// (bits = stored bits, cost = the caller's weight x squared reconstruction error), and
//
//   1. for a multiplier lambda >= 0 every matrix takes the candidate minimising
//      cost + lambda bits (ties: fewer bits, then the lower index); the total bits of
//      that pick never grow with lambda;
//   2. lambda = 0 if its pick fits the budget; otherwise the smallest lambda among the
//      points where some matrix's pick changes, (cost_j - cost_k) / (bits_k - bits_j),
//      whose pick fits; if rounding at the last such point leaves a matrix above its
//      fewest bits, every matrix takes its fewest bits (ties: lower cost, then the lower
//      index) — the limit of large lambda (EP_E_RANGE if even that does not fit);
//   3. the leftover budget is spent greedily: repeatedly the upgrade (a candidate with
//      more bits and lower cost, fitting the leftover) with the largest cost saved per
//      extra bit (ties: lower matrix, then lower candidate index).
#include <algorithm>
#include <cmath>
#include <vector>

#include "ep_internal.h"

namespace ep {
namespace {

struct Planner {
  int n, m;
  const double* bits;
  const double* cost;
  double b(int i, int j) const { return bits[(size_t)i * m + j]; }
  double c(int i, int j) const { return cost[(size_t)i * m + j]; }
  int pick(int i, double lam) const {
    int best = 0;
    double bv = c(i, 0) + lam * b(i, 0);
    for (int j = 1; j < m; ++j) {
      const double v = c(i, j) + lam * b(i, j);
      if (v < bv || (v == bv && b(i, j) < b(i, best))) {
        best = j;
        bv = v;
      }
    }
    return best;
  }
  int fewest(int i) const {
    int best = 0;
    for (int j = 1; j < m; ++j)
      if (b(i, j) < b(i, best) || (b(i, j) == b(i, best) && c(i, j) < c(i, best))) best = j;
    return best;
  }
  double total(double lam, int* ch) const {
    double t = 0.0;
    for (int i = 0; i < n; ++i) {
      ch[i] = pick(i, lam);
      t += b(i, ch[i]);
    }
    return t;
  }
};

}  // namespace
}  // namespace ep

using namespace ep;

extern "C" {

int ep_plan_bitrates(int n, int n_cand, const double* bits, const double* cost, double budget_bits, int* choice) {
  set_error("");
  if (n < 1 || n_cand < 1 || !bits || !cost || !choice) return fail(EP_E_ARG, "null pointer or empty plan");
  for (size_t q = 0; q < (size_t)n * n_cand; ++q)
    if (!std::isfinite(bits[q]) || !std::isfinite(cost[q]) || bits[q] < 0.0 || cost[q] < 0.0)
      return fail(EP_E_ARG, "bits and costs must be finite and non-negative");
  if (!std::isfinite(budget_bits)) return fail(EP_E_RANGE, "budget must be finite");
  const Planner P{n, n_cand, bits, cost};
  std::vector<int> ch((size_t)n);
  // the fewest bits any pick can reach
  double least = 0.0;
  for (int i = 0; i < n; ++i) {
    double mb = P.b(i, 0);
    for (int j = 1; j < n_cand; ++j) mb = std::min(mb, P.b(i, j));
    least += mb;
  }
  if (least > budget_bits) return fail(EP_E_RANGE, "budget below the smallest candidates");
  if (P.total(0.0, ch.data()) > budget_bits) {
    std::vector<double> lams;
    for (int i = 0; i < n; ++i)
      for (int j = 0; j < n_cand; ++j)
        for (int k = 0; k < n_cand; ++k)
          if (P.b(i, k) > P.b(i, j) && P.c(i, j) > P.c(i, k)) lams.push_back((P.c(i, j) - P.c(i, k)) / (P.b(i, k) - P.b(i, j)));
    std::sort(lams.begin(), lams.end());
    lams.erase(std::unique(lams.begin(), lams.end()), lams.end());
    // smallest lambda whose pick fits (the total never grows with lambda, also with the
    // rounding of cost + lambda bits at a breakpoint: there it can only keep the pick of
    // the lambdas below)
    size_t lo = 0, hi = lams.size();
    while (lo < hi) {
      const size_t mid = (lo + hi) / 2;
      if (P.total(lams[mid], ch.data()) <= budget_bits) hi = mid;
      else lo = mid + 1;
    }
    if (lo < lams.size()) P.total(lams[lo], ch.data());
    else
      for (int i = 0; i < n; ++i) ch[i] = P.fewest(i);
  }
  // greedy use of the leftover budget
  double used = 0.0;
  for (int i = 0; i < n; ++i) used += P.b(i, ch[i]);
  for (;;) {
    double best_r = 0.0;
    int bi = -1, bk = -1;
    for (int i = 0; i < n; ++i) {
      const double b0 = P.b(i, ch[i]), c0 = P.c(i, ch[i]);
      for (int k = 0; k < n_cand; ++k) {
        const double db = P.b(i, k) - b0, dc = c0 - P.c(i, k);
        if (db <= 0.0 || dc <= 0.0 || used + db > budget_bits) continue;
        const double r = dc / db;
        if (bi < 0 || r > best_r) {
          best_r = r;
          bi = i;
          bk = k;
        }
      }
    }
    if (bi < 0) break;
    used += P.b(bi, bk) - P.b(bi, ch[bi]);
    ch[bi] = bk;
  }
  for (int i = 0; i < n; ++i) choice[i] = ch[i];
  return EP_OK;
}

int ep_blob_distortion(const ep_blob* blob, double* sq_err, double* sq_ref) {
  set_error("");
  if (!blob || !sq_err || !sq_ref) return fail(EP_E_ARG, "null pointer");
  if (blob->b.kind != kKindLossy) return fail(EP_E_ARG, "a lossless blob has no reconstruction error");
  if (blob->b.dist.sq_err < 0.0) return fail(EP_E_STATE, "distortion is known only for blobs compressed in this process");
  *sq_err = blob->b.dist.sq_err;
  *sq_ref = blob->b.dist.sq_ref;
  return EP_OK;
}

}  // extern "C"
