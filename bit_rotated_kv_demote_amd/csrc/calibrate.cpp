// Offline calibration of one layer on the host (fp64), with the method's
// rotation or one of the baselines the pages compare it against.
//
// "OSCAR: Offline Spectral Covariance-Aware Rotation for 2-bit KV Cache
// Quantization" (gist.science), 2.1 and 2.2 A: the key target is the query
// covariance C_Q = (1/N) sum q^T q, the value target the score-weighted
// covariance C_S = (1/N) V^T S^T S V; their eigenbases U_Q, U_S are composed
// with a Hadamard transform and a bit-reversal permutation into
// R_K = U_Q H P_br and R_V = U_S H P_br; per-layer clip thresholds come from
// the rotated calibration activations.  "OSCAR：面向2-bit KV缓存量化的谱协方差感知
// 旋转方法" (zingnex.cn), 离线优化的优势: the rotation is computed once offline and
// applied unchanged at inference, and layers may share it (here: the mean of
// the layers' targets, tau over all of their activations).  Per KV head, each
// KV head is calibrated from its own query heads, keys and values.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

#include "calibrate.h"

namespace oscar {
namespace {

constexpr int D = 128;

// Sum of q^T q over tokens and query heads, added per KV head into
// c[hkv][D*D] (query head h belongs to KV head h / (hq / hkv)).
void add_query_moments(const float* q, int64_t n, int hq, int hkv, double* c) {
  const int g = hq / hkv;
  const int64_t rows = n * hq;
  const unsigned nt = std::max(1u, std::min(8u, std::thread::hardware_concurrency()));
  std::vector<std::vector<double>> part(nt, std::vector<double>((size_t)hkv * D * D, 0.0));
  std::vector<std::thread> th;
  for (unsigned t = 0; t < nt; ++t)
    th.emplace_back([&, t] {
      for (int64_t r = t; r < rows; r += nt) {
        const float* x = q + r * D;
        double* acc = part[t].data() + (size_t)((r % hq) / g) * D * D;
        for (int i = 0; i < D; ++i) {
          const double xi = x[i];
          double* row = acc + i * D;
          for (int j = 0; j < D; ++j) row[j] += xi * (double)x[j];
        }
      }
    });
  for (auto& t : th) t.join();
  for (unsigned t = 0; t < nt; ++t)
    for (size_t i = 0; i < (size_t)hkv * D * D; ++i) c[i] += part[t][i];
}

// Sum over query heads h and tokens n of o_{h,n}^T o_{h,n}, with
// o_{h,n} = sum_{m<=n} softmax_m(q_n . k_m / sqrt(d)) v_m, added per KV head
// into c[hkv][D*D] (the value target C_S before its 1/(N Hq)).  With the keys
// passed as v this is the attention-weighted key moment (S_h K)^T (S_h K).
void add_score_moments(const float* q, const float* k, const float* v, int64_t n, int hq, int hkv, double* c) {
  const int g = hq / hkv;
  const unsigned nt = std::max(1u, std::min(8u, std::thread::hardware_concurrency()));
  std::vector<std::vector<double>> part(nt, std::vector<double>((size_t)hkv * D * D, 0.0));
  std::vector<std::thread> th;
  const double inv_sqrt_d = 1.0 / std::sqrt((double)D);
  for (unsigned t = 0; t < nt; ++t)
    th.emplace_back([&, t] {
      std::vector<double> logit(n), o(D), qd(D);
      for (int64_t work = t; work < (int64_t)hq * n; work += nt) {
        const int h = (int)(work / n);
        const int64_t row = work % n;
        const int kv = h / g;
        double* acc = part[t].data() + (size_t)kv * D * D;
        const float* qr = q + (row * hq + h) * D;
        for (int i = 0; i < D; ++i) qd[i] = qr[i];
        double mx = -INFINITY;
        for (int64_t m = 0; m <= row; ++m) {
          const float* kr = k + (m * hkv + kv) * D;
          double s = 0.0;
          for (int i = 0; i < D; ++i) s += qd[i] * (double)kr[i];
          logit[m] = s * inv_sqrt_d;
          mx = std::max(mx, logit[m]);
        }
        double tot = 0.0;
        for (int64_t m = 0; m <= row; ++m) { logit[m] = std::exp(logit[m] - mx); tot += logit[m]; }
        std::fill(o.begin(), o.end(), 0.0);
        for (int64_t m = 0; m <= row; ++m) {
          const double w = logit[m] / tot;
          const float* vr = v + (m * hkv + kv) * D;
          for (int i = 0; i < D; ++i) o[i] += w * (double)vr[i];
        }
        for (int i = 0; i < D; ++i) {
          double* r = acc + i * D;
          for (int j = 0; j < D; ++j) r[j] += o[i] * o[j];
        }
      }
    });
  for (auto& t : th) t.join();
  for (unsigned t = 0; t < nt; ++t)
    for (size_t i = 0; i < (size_t)hkv * D * D; ++i) c[i] += part[t][i];
}

// Cyclic Jacobi eigen-decomposition of a symmetric matrix; eigenvectors as
// columns, sorted by descending eigenvalue, each column's largest-magnitude
// entry (first on ties) made positive.
void eigenbasis(const double* c, double* u) {
  std::vector<double> a(c, c + D * D), vv(D * D, 0.0);
  for (int i = 0; i < D; ++i) vv[i * D + i] = 1.0;
  double total = 0.0;
  for (int i = 0; i < D * D; ++i) total += a[i] * a[i];
  for (int sweep = 0; sweep < 100; ++sweep) {
    double off = 0.0;
    for (int p = 0; p < D; ++p)
      for (int q = p + 1; q < D; ++q) off += a[p * D + q] * a[p * D + q];
    if (off <= 1e-30 * total || off == 0.0) break;
    for (int p = 0; p < D; ++p)
      for (int q = p + 1; q < D; ++q) {
        const double apq = a[p * D + q];
        if (std::fabs(apq) < 1e-300) continue;
        const double theta = (a[q * D + q] - a[p * D + p]) / (2.0 * apq);
        const double t = (theta >= 0 ? 1.0 : -1.0) / (std::fabs(theta) + std::sqrt(theta * theta + 1.0));
        const double cs = 1.0 / std::sqrt(t * t + 1.0), sn = t * cs;
        for (int k = 0; k < D; ++k) {   // columns p, q
          const double akp = a[k * D + p], akq = a[k * D + q];
          a[k * D + p] = cs * akp - sn * akq;
          a[k * D + q] = sn * akp + cs * akq;
        }
        for (int k = 0; k < D; ++k) {   // rows p, q
          const double apk = a[p * D + k], aqk = a[q * D + k];
          a[p * D + k] = cs * apk - sn * aqk;
          a[q * D + k] = sn * apk + cs * aqk;
        }
        for (int k = 0; k < D; ++k) {
          const double vkp = vv[k * D + p], vkq = vv[k * D + q];
          vv[k * D + p] = cs * vkp - sn * vkq;
          vv[k * D + q] = sn * vkp + cs * vkq;
        }
      }
  }
  std::vector<int> order(D);
  for (int i = 0; i < D; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return a[x * D + x] > a[y * D + y]; });
  for (int col = 0; col < D; ++col) {
    const int src = order[col];
    int imax = 0;
    for (int i = 1; i < D; ++i)
      if (std::fabs(vv[i * D + src]) > std::fabs(vv[imax * D + src])) imax = i;
    const double sgn = vv[imax * D + src] < 0 ? -1.0 : 1.0;
    for (int i = 0; i < D; ++i) u[i * D + col] = sgn * vv[i * D + src];
  }
}

int bit_reverse7(int j) {
  int r = 0;
  for (int b = 0; b < 7; ++b) { r = (r << 1) | (j & 1); j >>= 1; }
  return r;
}

// R = U . H . P_br: H block-diagonal normalised Sylvester Hadamard
// ((-1)^popcount(i&j) / sqrt(b) inside each block), (x P)_j = x_{bitrev(j)}.
void compose_rotation(const double* u, int block, float* r) {
  std::vector<double> uh(D * D, 0.0);
  const double norm = 1.0 / std::sqrt((double)block);
  for (int i = 0; i < D; ++i)
    for (int j = 0; j < D; ++j) {
      const int b0 = (j / block) * block;
      double s = 0.0;
      for (int k = b0; k < b0 + block; ++k)
        s += u[i * D + k] * ((__builtin_popcount((unsigned)((k - b0) & (j - b0))) & 1) ? -norm : norm);
      uh[i * D + j] = s;
    }
  for (int i = 0; i < D; ++i)
    for (int j = 0; j < D; ++j) r[i * D + j] = (float)uh[i * D + bit_reverse7(j)];
}

// tau_j = linear-interpolated percentile of |x . R|_j over the rows
// x + (first + step * m) * D, m = 0 .. rows-1.
void clip_thresholds(const float* x, int64_t rows, int64_t first, int64_t step, const float* r, double pct,
                     float* tau) {
  std::vector<std::vector<double>> col(D, std::vector<double>(rows));
  std::vector<double> y(D);
  for (int64_t n = 0; n < rows; ++n) {
    const float* xr = x + (first + step * n) * D;
    std::fill(y.begin(), y.end(), 0.0);
    for (int i = 0; i < D; ++i) {
      const double xi = xr[i];
      for (int j = 0; j < D; ++j) y[j] += xi * (double)r[i * D + j];
    }
    for (int j = 0; j < D; ++j) col[j][n] = std::fabs(y[j]);
  }
  for (int j = 0; j < D; ++j) {
    auto& c = col[j];
    std::sort(c.begin(), c.end());
    const double pos = (double)(rows - 1) * pct / 100.0;
    const int64_t lo = (int64_t)std::floor(pos);
    const int64_t hi = std::min<int64_t>(lo + 1, rows - 1);
    const double f = pos - (double)lo;
    tau[j] = (float)(c[lo] + f * (c[hi] - c[lo]));
  }
}

}  // namespace

int calibrate_layers(int hq, int hkv, int n_layers, int hadamard_block, float percentile, int rotation,
                     bool per_kv_head, const float* q, const float* k, const float* v, int64_t n, float* rot_k,
                     float* rot_v, float* clip_k, float* clip_v) {
  if (rotation < kRotSpectral || rotation > kRotIdentity) return -2;
  for (const float* p : {q, k, v}) {
    const int64_t cnt = (int64_t)n_layers * n * (p == q ? hq : hkv) * D;
    for (int64_t i = 0; i < cnt; ++i)
      if (!std::isfinite(p[i])) return -1;
  }
  // Per-KV-head sums of the key and value moments over every layer; a set
  // (one KV head, or all of them) then averages its share: the targets of
  // each layer, averaged over the layers.
  const int n_sets = per_kv_head ? hkv : 1;
  const int heads_per_set = per_kv_head ? 1 : hkv;
  const double rows_per_set = (double)n_layers * (double)n * (double)(hq / hkv) * heads_per_set;
  std::vector<double> mk((size_t)hkv * D * D, 0.0), ms((size_t)hkv * D * D, 0.0);
  if (rotation == kRotSpectral || rotation == kRotKeyAttn) {
    for (int l = 0; l < n_layers; ++l) {
      const float* ql = q + (int64_t)l * n * hq * D;
      const float* kl = k + (int64_t)l * n * hkv * D;
      const float* vl = v + (int64_t)l * n * hkv * D;
      if (rotation == kRotSpectral)
        add_query_moments(ql, n, hq, hkv, mk.data());
      else
        add_score_moments(ql, kl, kl, n, hq, hkv, mk.data());
      add_score_moments(ql, kl, vl, n, hq, hkv, ms.data());
    }
  }
  std::vector<double> ck(D * D), cs(D * D), uk(D * D), us(D * D);
  for (int set = 0; set < n_sets; ++set) {
    float* rk = rot_k + (size_t)set * D * D;
    float* rv = rot_v + (size_t)set * D * D;
    switch (rotation) {
      case kRotSpectral:               // key target C_Q, value target C_S
      case kRotKeyAttn:                // key target C_SK, value target C_S
        std::fill(ck.begin(), ck.end(), 0.0);
        std::fill(cs.begin(), cs.end(), 0.0);
        for (int hd = set * heads_per_set; hd < (set + 1) * heads_per_set; ++hd)
          for (int i = 0; i < D * D; ++i) {
            ck[i] += mk[(size_t)hd * D * D + i];
            cs[i] += ms[(size_t)hd * D * D + i];
          }
        for (int i = 0; i < D * D; ++i) {
          ck[i] /= rows_per_set;
          cs[i] /= rows_per_set;
        }
        eigenbasis(ck.data(), uk.data());
        eigenbasis(cs.data(), us.data());
        compose_rotation(uk.data(), hadamard_block, rk);
        compose_rotation(us.data(), hadamard_block, rv);
        break;
      case kRotHadamard:               // U = I: R = H P_br
        std::fill(uk.begin(), uk.end(), 0.0);
        for (int i = 0; i < D; ++i) uk[i * D + i] = 1.0;
        compose_rotation(uk.data(), hadamard_block, rk);
        std::copy(rk, rk + D * D, rv);
        break;
      default:                         // kRotIdentity: R = I
        for (int i = 0; i < D * D; ++i) rk[i] = rv[i] = (i % (D + 1) == 0) ? 1.0f : 0.0f;
        break;
    }
    // the set's rows of every layer: all (layer, token, KV head) rows, or
    // those of KV head `set`
    const int64_t rows = per_kv_head ? (int64_t)n_layers * n : (int64_t)n_layers * n * hkv;
    const int64_t first = per_kv_head ? set : 0, step = per_kv_head ? hkv : 1;
    clip_thresholds(k, rows, first, step, rk, percentile, clip_k + (size_t)set * D);
    clip_thresholds(v, rows, first, step, rv, percentile, clip_v + (size_t)set * D);
  }
  for (int j = 0; j < n_sets * D; ++j)
    if (!std::isfinite(clip_k[j]) || !std::isfinite(clip_v[j]) || clip_k[j] > 65504.0f || clip_v[j] > 65504.0f ||
        !(clip_k[j] > 0.0f) || !(clip_v[j] > 0.0f))
      return -1;
  return 0;
}

}  // namespace oscar
