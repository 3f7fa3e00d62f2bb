// Host-side analysis of alpha and channel masks (LeanK page, section 6 and
// section 2.1).  Offline tools over small host arrays; no device work.

#include <math.h>

#include <algorithm>
#include <numeric>
#include <vector>

#include "common.h"

namespace {

// Ranks 1..n of x, equal values given the mean of the ranks they span.
std::vector<double> average_ranks(const float* x, int64_t n) {
  std::vector<int64_t> order(n);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int64_t a, int64_t b) { return x[a] < x[b]; });
  std::vector<double> ranks(n);
  for (int64_t i = 0; i < n;) {
    int64_t j = i;
    while (j + 1 < n && x[order[j + 1]] == x[order[i]]) ++j;
    const double r = 0.5 * static_cast<double>(i + j) + 1.0;
    for (int64_t k = i; k <= j; ++k) ranks[order[k]] = r;
    i = j + 1;
  }
  return ranks;
}

template <typename X, typename Y>
double pearson(const X& x, const Y& y, int64_t n) {
  double mx = 0.0, my = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    mx += static_cast<double>(x[i]);
    my += static_cast<double>(y[i]);
  }
  mx /= static_cast<double>(n);
  my /= static_cast<double>(n);
  double sxy = 0.0, sxx = 0.0, syy = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    const double dx = static_cast<double>(x[i]) - mx, dy = static_cast<double>(y[i]) - my;
    sxy += dx * dy;
    sxx += dx * dx;
    syy += dy * dy;
  }
  const double den = sqrt(sxx * syy);
  return den > 0.0 ? sxy / den : 0.0;
}

}  // namespace

extern "C" int leank_pair_retention(const uint8_t* mask, int32_t n_layers, int32_t n_kv_heads,
                                    int32_t head_dim, double* retention_out) {
  if (!mask || !retention_out || n_layers < 1 || n_kv_heads < 1) return LEANK_EINVAL;
  if (head_dim < 2 || head_dim % 2) return LEANK_EINVAL;
  const int half = head_dim / 2;
  const int64_t rows = static_cast<int64_t>(n_layers) * n_kv_heads;
  for (int i = 0; i < half; ++i) {
    double sum = 0.0;
    for (int64_t r = 0; r < rows; ++r) {
      const uint8_t* m = mask + r * head_dim;
      sum += 0.5 * ((m[i] ? 1.0 : 0.0) + (m[i + half] ? 1.0 : 0.0));
    }
    retention_out[i] = sum / static_cast<double>(rows);
  }
  return LEANK_OK;
}

extern "C" int leank_head_hf_ratio(const float* alpha, int32_t n_layers, int32_t n_kv_heads,
                                   int32_t head_dim, int32_t n_hf_pairs, double* w_hf_out) {
  if (!alpha || !w_hf_out || n_layers < 1 || n_kv_heads < 1) return LEANK_EINVAL;
  if (head_dim < 2 || head_dim % 2 || n_hf_pairs < 0 || n_hf_pairs > head_dim / 2) return LEANK_EINVAL;
  const int half = head_dim / 2;
  const int64_t rows = static_cast<int64_t>(n_layers) * n_kv_heads;
  for (int64_t r = 0; r < rows; ++r) {
    const float* a = alpha + r * head_dim;
    double hf = 0.0, total = 0.0;
    for (int c = 0; c < head_dim; ++c) {
      if (a[c] != a[c]) return LEANK_EINVAL;
      const double v = fabs(static_cast<double>(a[c]));
      total += v;
      if ((c < half ? c : c - half) < n_hf_pairs) hf += v;
    }
    w_hf_out[r] = total > 0.0 ? hf / total : 0.0;
  }
  return LEANK_OK;
}

extern "C" int leank_rank_correlation(const float* a, const float* b, int64_t n,
                                      double* pearson_out, double* rank_pearson_out) {
  if (!a || !b || !pearson_out || !rank_pearson_out || n < 2) return LEANK_EINVAL;
  for (int64_t i = 0; i < n; ++i)
    if (a[i] != a[i] || b[i] != b[i]) return LEANK_EINVAL;
  *pearson_out = pearson(a, b, n);
  const std::vector<double> ra = average_ranks(a, n), rb = average_ranks(b, n);
  *rank_pearson_out = pearson(ra, rb, n);
  return LEANK_OK;
}
