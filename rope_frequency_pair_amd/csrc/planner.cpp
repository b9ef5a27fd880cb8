// Host-side window planner (see planner.h).
#include "planner.h"

#include <algorithm>
#include <cmath>

// Every formula here is evaluated in IEEE double exactly as written (no fused
// multiply-add contraction), so the integer windows match other IEEE double
// evaluations of the same expressions bit for bit.
#pragma STDC FP_CONTRACT OFF

namespace atw {

void window_widths(int head_dim, double rope_base, double k_turns, bool window_on, int64_t* w) {
  const int h = head_dim / 2;
  if (!window_on || std::isinf(k_turns)) {
    for (int r = 0; r < h; ++r) w[r] = kUnbounded;
    return;
  }
  const double two_pi = 2.0 * 3.141592653589793;
  for (int r = 0; r < h; ++r) {
    // same operation order as the definition: theta, wavelength, k * wavelength
    const double theta = std::pow(rope_base, (-2.0 * r) / head_dim);
    const double lam = two_pi / theta;
    const double x = std::floor(k_turns * lam);
    w[r] = (x >= 4611686018427387904.0) ? kUnbounded : static_cast<int64_t>(x);
  }
}

void pair_turns_per_position(int head_dim, double rope_base, double* phi) {
  const int h = head_dim / 2;
  const double two_pi = 2.0 * 3.141592653589793;
  for (int r = 0; r < h; ++r) phi[r] = std::pow(rope_base, (-2.0 * r) / head_dim) / two_pi;
}

bool rope_theta(const RopeSpec& spec, int head_dim, double* theta, const char** why) {
  const int h = head_dim / 2;
  const double two_pi = 2.0 * 3.141592653589793;
  auto bad = [&](const char* m) {
    if (why) *why = m;
    return false;
  };
  if (spec.kind == kRopeTable) {
    if (spec.theta == nullptr) return bad("table frequencies are NULL");
    for (int r = 0; r < h; ++r) theta[r] = spec.theta[r];
  } else {
    if (!(spec.base > 1.0) || std::isinf(spec.base)) return bad("rope base must be a finite value > 1");
    for (int r = 0; r < h; ++r) theta[r] = std::pow(spec.base, (-2.0 * r) / head_dim);
    if (spec.kind == kRopeLinear) {
      if (!(spec.factor > 0.0) || std::isinf(spec.factor)) return bad("linear factor must be finite and > 0");
      for (int r = 0; r < h; ++r) theta[r] = theta[r] / spec.factor;
    } else if (spec.kind == kRopeLlama3) {
      const double f = spec.factor, lo = spec.low_freq_factor, hi = spec.high_freq_factor;
      const double L = spec.original_max_position;
      if (!(f > 0.0) || std::isinf(f) || !(lo > 0.0) || !(hi > lo) || std::isinf(hi) ||
          !(L > 0.0) || std::isinf(L))
        return bad("llama3 scaling needs factor > 0, 0 < low_freq_factor < high_freq_factor, "
                   "original_max_position > 0 (all finite)");
      const double lo_wavelen = L / lo, hi_wavelen = L / hi;
      for (int r = 0; r < h; ++r) {
        const double t = theta[r];
        const double wavelen = two_pi / t;
        if (wavelen < hi_wavelen) {
          theta[r] = t;
        } else if (wavelen > lo_wavelen) {
          theta[r] = t / f;
        } else {
          const double sm = (L / wavelen - lo) / (hi - lo);
          theta[r] = (1.0 - sm) * t / f + sm * t;
        }
      }
    } else if (spec.kind != kRopePlain) {
      return bad("unknown rope kind");
    }
  }
  for (int r = 0; r < h; ++r) {
    if (!(theta[r] > 0.0) || std::isinf(theta[r])) return bad("every theta_r must be finite and > 0");
    if (r > 0 && theta[r] > theta[r - 1]) return bad("theta_r must be non-increasing in r");
  }
  return true;
}

void window_widths_theta(int h, const double* theta, double k_turns, bool window_on, int64_t* w) {
  if (!window_on || std::isinf(k_turns)) {
    for (int r = 0; r < h; ++r) w[r] = kUnbounded;
    return;
  }
  const double two_pi = 2.0 * 3.141592653589793;
  for (int r = 0; r < h; ++r) {
    const double lam = two_pi / theta[r];
    const double x = std::floor(k_turns * lam);
    w[r] = (x >= 4611686018427387904.0) ? kUnbounded : static_cast<int64_t>(x);
  }
}

bool explicit_widths(int h, const int64_t* table, bool window_on, int64_t* w, const char** why) {
  for (int r = 0; r < h; ++r) {
    if (table[r] < 0) {
      *why = "every explicit window must be >= 0";
      return false;
    }
    if (r > 0 && table[r] < table[r - 1]) {
      *why = "explicit windows must be non-decreasing in the pair index";
      return false;
    }
  }
  for (int r = 0; r < h; ++r) w[r] = (!window_on || table[r] > kUnbounded) ? kUnbounded : table[r];
  return true;
}

int first_retained_pair(const int64_t* w, int h, int64_t delta) {
  // w is sorted; count of entries < delta
  return static_cast<int>(std::lower_bound(w, w + h, delta) - w);
}

namespace {

using i128 = __int128;

// sum_{x=a}^{b-1} x  (0 if b <= a)
i128 series(i128 a, i128 b) {
  if (b <= a) return 0;
  return (a + b - 1) * (b - a) / 2;
}

// sum over rows n in [A, B) of clamp(n - W, 0, n_kv): the number of causal
// cells of row n at distance > W (row n sees distances max(0,n-n_kv+1)..n).
i128 causal_pruned_rows(i128 A, i128 B, i128 W, i128 n_kv) {
  // n <= W: 0;  W < n < W + n_kv: n - W;  n >= W + n_kv: n_kv
  const i128 lo = std::max(A, W + 1), hi = std::min(B, W + n_kv);
  i128 s = series(lo - W, hi - W);
  const i128 full_lo = std::max(A, W + n_kv);
  if (B > full_lo) s += (B - full_lo) * n_kv;
  return s;
}

// sum over rows n in [A, B) of #{m in [0, n_kv): m - n > W} = clamp(K - n, 0, .)
// with K = n_kv - 1 - W (non-causal, keys after the query).
i128 noncausal_after_rows(i128 A, i128 B, i128 W, i128 n_kv) {
  const i128 K = n_kv - 1 - W;
  const i128 hi = std::min(B, K);
  if (hi <= A) return 0;
  // sum_{n=A}^{hi-1} (K - n) = sum_{x=K-hi+1}^{K-A} x
  return series(K - hi + 1, K - A + 1);
}

// sum_{x=lo}^{hi-1} clamp(x, 0, L)
i128 sum_clamp(i128 lo, i128 hi, i128 L) {
  if (hi <= lo || L <= 0) return 0;
  i128 s = series(std::max<i128>(lo, 1), std::min<i128>(hi, L + 1));
  const i128 full_lo = std::max<i128>(lo, L + 1);
  if (hi > full_lo) s += (hi - full_lo) * L;
  return s;
}

// Cells (n, m) of the rectangle rows [A, B) x keys [m0, m1) (positions) with
// n - m > W, and with m - n > W.
i128 rect_before(i128 A, i128 B, i128 m0, i128 m1, i128 W) {
  return sum_clamp(A - W - m0, B - W - m0, m1 - m0);   // #{m in [m0, m1): m < n - W}
}
i128 rect_after(i128 A, i128 B, i128 m0, i128 m1, i128 W) {
  return sum_clamp(m1 - W - B, m1 - W - A, m1 - m0);   // #{m in [m0, m1): m > n + W}
}

}  // namespace

void pruned_terms(int64_t n_q, int64_t n_kv, int64_t q_pos0, int head_dim, const int64_t* w,
                  bool causal, int64_t* pruned, int64_t* total) {
  const int h = head_dim / 2;
  if (n_q <= 0 || n_kv <= 0) {
    *pruned = 0;
    *total = 0;
    return;
  }
  const i128 A = q_pos0, B = (i128)q_pos0 + n_q, NKV = n_kv;
  i128 p = 0, visible;
  if (causal) {
    // row n sees min(n + 1, n_kv) keys
    const i128 split = std::min(B, std::max(A, NKV - 1));  // rows n < n_kv - 1 see n + 1
    visible = series(A + 1, split + 1) + (B - split) * NKV;
    for (int r = 0; r < h; ++r) p += causal_pruned_rows(A, B, w[r], NKV);
  } else {
    visible = (i128)n_q * NKV;
    for (int r = 0; r < h; ++r)
      p += causal_pruned_rows(A, B, w[r], NKV) + noncausal_after_rows(A, B, w[r], NKV);
  }
  *pruned = static_cast<int64_t>(p);
  *total = static_cast<int64_t>(visible * h);
}

bool tile_distance_range(int64_t n_lo, int64_t n_hi, int64_t m_lo, int64_t m_hi, bool causal,
                         int64_t* dmin, int64_t* dmax) {
  if (n_hi < n_lo || m_hi < m_lo) return false;
  if (causal) {
    if (m_lo > n_hi) return false;
    *dmin = std::max<int64_t>(0, n_lo - m_hi);
    *dmax = n_hi - m_lo;
  } else {
    if (m_hi < n_lo) *dmin = n_lo - m_hi;
    else if (m_lo > n_hi) *dmin = m_lo - n_hi;
    else *dmin = 0;
    *dmax = std::max(std::abs(n_hi - m_lo), std::abs(n_lo - m_hi));
  }
  return true;
}

void tile_plan(int head_dim, const int64_t* w, int64_t n_q, int64_t n_kv, int64_t q_pos0,
               bool causal, int tile_q, int tile_k, int32_t* plan) {
  const int h = head_dim / 2;
  const int64_t n_qt = (n_q + tile_q - 1) / tile_q, n_kt = (n_kv + tile_k - 1) / tile_k;
  for (int64_t a = 0; a < n_qt; ++a) {
    const int64_t n_lo = q_pos0 + a * tile_q;
    const int64_t n_hi = q_pos0 + std::min<int64_t>((a + 1) * tile_q, n_q) - 1;
    for (int64_t b = 0; b < n_kt; ++b) {
      const int64_t m_lo = b * tile_k, m_hi = std::min<int64_t>((b + 1) * tile_k, n_kv) - 1;
      int32_t* out = plan + (a * n_kt + b) * 2;
      int64_t dmin, dmax;
      if (!tile_distance_range(n_lo, n_hi, m_lo, m_hi, causal, &dmin, &dmax)) {
        out[0] = out[1] = -1;
        continue;
      }
      out[0] = first_retained_pair(w, h, dmin);
      out[1] = first_retained_pair(w, h, dmax);
    }
  }
}

void pruned_terms_blocks(int64_t n_q, int64_t n_kv, int64_t q_pos0, int head_dim, const int64_t* w,
                         bool causal, const uint32_t* mask, int64_t mask_words, int block,
                         int64_t* pruned, int64_t* total) {
  const int h = head_dim / 2;
  const int64_t n_qb = (n_q + block - 1) / block, n_kb = (n_kv + block - 1) / block;
  i128 p = 0, visible = 0;
  for (int64_t qb = 0; qb < n_qb; ++qb) {
    const i128 A = (i128)q_pos0 + qb * block, B = (i128)q_pos0 + std::min<int64_t>(n_q, (qb + 1) * block);
    const uint32_t* row = mask + qb * mask_words;
    for (int64_t kb = 0; kb < n_kb; ++kb) {
      if (!((row[kb >> 5] >> (kb & 31)) & 1u)) continue;
      const i128 m0 = kb * block, m1 = std::min<int64_t>(n_kv, (kb + 1) * block);
      if (causal) {
        const i128 vis = rect_before(A, B, m0, m1, -1);   // m <= n
        if (vis == 0) continue;
        visible += vis;
        for (int r = 0; r < h; ++r) p += rect_before(A, B, m0, m1, w[r]);
      } else {
        visible += (B - A) * (m1 - m0);
        for (int r = 0; r < h; ++r) p += rect_before(A, B, m0, m1, w[r]) + rect_after(A, B, m0, m1, w[r]);
      }
    }
  }
  *pruned = static_cast<int64_t>(p);
  *total = static_cast<int64_t>(visible * h);
}

}  // namespace atw
