// Hardware-aware prefix scheduler (host code).
//
// DSpark tutorial, confidence-scheduled verification, "hardware-aware prefix
// scheduler": each request's drafted positions carry conditional survival
// probabilities c_k; the scheduler picks every request's verify length l_r to
// maximise Theta = tau * SPS(B), B the verify batch in tokens and SPS(B) a
// measured steps-per-second curve.  Candidate tokens are taken in order of
// cumulative survival prod_{i <= k} c_i, highest first, one at a time, and
// the walk stops at the first token that does not raise Theta.
//
// Readings: a request verifying l_r drafts adds l_r + 1 tokens to B; tau is
// the expected number of emitted tokens, sum_r (1 + sum_{k <= l_r} prod c);
// SPS is interpolated linearly in the table and clamped at its ends; equal
// cumulative survivals go to the lower request, then the lower position.
#include "bd_launch.hpp"

#include <algorithm>
#include <vector>

namespace bd {

namespace {

struct Cand {
  double s;  // cumulative survival
  int r, k;  // request, position (1-based)
};

// the table sorted by batch; linear in between, the end values outside
double sps_at(const std::vector<std::pair<double, double>>& tab, double B) {
  if (B <= tab.front().first) return tab.front().second;
  if (B >= tab.back().first) return tab.back().second;
  const auto it = std::upper_bound(tab.begin(), tab.end(), B,
                                   [](double x, const std::pair<double, double>& e) { return x < e.first; });
  const auto& hi = *it;
  const auto& lo = *(it - 1);
  if (hi.first == lo.first) return hi.second;
  const double slope = (hi.second - lo.second) / (hi.first - lo.first);
  return slope * (B - lo.first) + lo.second;
}

}  // namespace

int prefix_schedule(const float* surv, const int32_t* surv_cu, int R, const float* sps_b, const float* sps_v,
                    int n_sps, int32_t* ell, double* theta) {
  std::vector<std::pair<double, double>> tab(n_sps);
  for (int j = 0; j < n_sps; ++j) tab[j] = {double(sps_b[j]), double(sps_v[j])};
  std::stable_sort(tab.begin(), tab.end(),
                   [](const std::pair<double, double>& x, const std::pair<double, double>& y) {
                     return x.first < y.first;
                   });
  std::vector<Cand> cands;
  for (int r = 0; r < R; ++r) {
    double cum = 1.0;
    for (int k = 1; k <= surv_cu[r + 1] - surv_cu[r]; ++k) {
      cum *= double(surv[surv_cu[r] + k - 1]);
      cands.push_back({cum, r, k});
    }
  }
  std::sort(cands.begin(), cands.end(), [](const Cand& x, const Cand& y) {
    if (x.s != y.s) return x.s > y.s;
    if (x.r != y.r) return x.r < y.r;
    return x.k < y.k;
  });
  for (int r = 0; r < R; ++r) ell[r] = 0;
  long long B = R;
  double tau = double(R);
  double th = R > 0 ? tau * sps_at(tab, double(B)) : 0.0;
  for (const Cand& c : cands) {
    if (c.k != ell[c.r] + 1) continue;
    const double tau2 = tau + c.s;
    const double th2 = tau2 * sps_at(tab, double(B + 1));
    if (!(th2 > th)) break;
    ell[c.r] = c.k;
    ++B;
    tau = tau2;
    th = th2;
  }
  if (theta) *theta = th;
  return 0;
}

}  // namespace bd
