// plan.cpp -- Lagrangian allocation of a byte budget over cells (host code): one multiplier chooses every
// cell's option (a rank, a residual width) under a shared byte budget ("JoLT: Near-Lossless KV Cache
// Compression" thesis page, "How JoLT works"; "A JoLT for the KV cache", abstract).
//
// For a multiplier lam >= 0 a cell takes the option minimizing D + lam B (ties: fewer bytes).  As lam falls
// from infinity the choice walks up the cell's lower convex hull of (bytes, distortion) points, switching at
// breakpoints.  Each cell's hull is built once (gift wrapping from its cheapest option: the next vertex is the
// option of more bytes and less distortion with the largest crossing multiplier, the farthest of equal ones),
// and the choice at a multiplier is read off by comparing it with the breakpoints, never by evaluating
// D + lam B: rounding then cannot make the bytes increase with lam, so bisection over the sorted breakpoints
// finds the smallest one whose choices fit.  At it, cells on a breakpoint equal to lam (ties between two hull
// vertices) move on, in cell order, while the bytes fit.  Every cell minimizes D + lam B, so no allocation of at
// most the same bytes has less total distortion (Everett's theorem).
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

#include "../../include/kvc.h"

namespace kvc {

namespace {

struct Hull {
  std::vector<int32_t> vert;  // option index of each vertex, bytes strictly increasing
  std::vector<double> lam;    // lam[k]: the multiplier below which vertex k + 1 replaces vertex k (non-increasing)
};

Hull build_hull(const double* D, const double* B, int n) {
  Hull h;
  int v = 0;
  for (int o = 1; o < n; ++o)
    if (B[o] < B[v] || (B[o] == B[v] && D[o] < D[v])) v = o;  // equal bytes and distortion: the lower index
  h.vert.push_back(v);
  for (;;) {
    int best = -1;
    double bl = 0.0;
    for (int p = 0; p < n; ++p) {
      if (!(B[p] > B[v] && D[p] < D[v])) continue;
      const double l = (D[v] - D[p]) / (B[p] - B[v]);
      if (best < 0 || l > bl || (l == bl && B[p] > B[best])) {  // equal (lam, bytes): the lower index stays
        best = p;
        bl = l;
      }
    }
    if (best < 0) return h;
    if (!h.lam.empty() && bl > h.lam.back()) bl = h.lam.back();
    h.vert.push_back(best);
    h.lam.push_back(bl);
    v = best;
  }
}

// vertex chosen at multiplier lam: every breakpoint strictly above lam is passed
int walk(const Hull& h, double lam) {
  int k = 0;
  while (k < (int)h.lam.size() && h.lam[k] > lam) ++k;
  return k;
}

double used_at(const std::vector<Hull>& hs, const double* bytes, int n, double lam, std::vector<int>* ks) {
  double used = 0.0;
  for (size_t c = 0; c < hs.size(); ++c) {
    const int k = walk(hs[c], lam);
    if (ks) (*ks)[c] = k;
    used += bytes[c * (size_t)n + hs[c].vert[k]];
  }
  return used;
}

}  // namespace

kvc_status plan_impl(const kvc_plan_in& in, int32_t* choice, double* lambda) {
  if (in.n_cells < 1 || in.n_options < 1 || in.n_options > 1024 || !in.distortion || !in.bytes || !choice)
    return KVC_ERR_INVALID_ARG;
  if ((int64_t)in.n_cells * in.n_options > ((int64_t)1 << 22)) return KVC_ERR_INVALID_ARG;
  const int n = in.n_options;
  for (int64_t i = 0; i < (int64_t)in.n_cells * n; ++i)
    if (!std::isfinite(in.distortion[i]) || !std::isfinite(in.bytes[i]) || in.bytes[i] < 0.0) return KVC_ERR_INVALID_ARG;
  if (!std::isfinite(in.budget)) return KVC_ERR_INVALID_ARG;
  std::vector<Hull> hs;
  hs.reserve(in.n_cells);
  std::vector<double> lams{0.0};
  for (int c = 0; c < in.n_cells; ++c) {
    hs.push_back(build_hull(in.distortion + (size_t)c * n, in.bytes + (size_t)c * n, n));
    lams.insert(lams.end(), hs.back().lam.begin(), hs.back().lam.end());
  }
  std::sort(lams.begin(), lams.end());
  lams.erase(std::unique(lams.begin(), lams.end()), lams.end());
  // at the largest multiplier every cell sits on its cheapest option
  if (used_at(hs, in.bytes, n, lams.back(), nullptr) > in.budget) return KVC_ERR_INVALID_ARG;
  size_t lo = 0, hi = lams.size() - 1;  // the bytes never increase along the sorted multipliers
  while (lo < hi) {
    const size_t mid = lo + (hi - lo) / 2;
    if (used_at(hs, in.bytes, n, lams[mid], nullptr) <= in.budget)
      hi = mid;
    else
      lo = mid + 1;
  }
  const double lam = lams[lo];
  std::vector<int> ks(in.n_cells);
  double used = used_at(hs, in.bytes, n, lam, &ks);
  for (int c = 0; c < in.n_cells; ++c) {  // tie fill
    const Hull& h = hs[c];
    const double* B = in.bytes + (size_t)c * n;
    while (ks[c] < (int)h.lam.size() && h.lam[ks[c]] == lam) {
      const double extra = B[h.vert[ks[c] + 1]] - B[h.vert[ks[c]]];
      if (used + extra > in.budget) break;
      used += extra;
      ++ks[c];
    }
    choice[c] = h.vert[ks[c]];
  }
  if (lambda) *lambda = lam;
  return KVC_OK;
}

}  // namespace kvc
