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
// applied unchanged at inference.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

#include "calibrate.h"

namespace oscar {
namespace {

constexpr int D = 128;

// C_Q: pooled over tokens and query heads.
void query_covariance(const float* q, int64_t n, int hq, double* c) {
  std::fill(c, c + D * D, 0.0);
  const int64_t rows = n * hq;
  const unsigned nt = std::max(1u, std::min(8u, std::thread::hardware_concurrency()));
  std::vector<std::vector<double>> part(nt, std::vector<double>(D * D, 0.0));
  std::vector<std::thread> th;
  for (unsigned t = 0; t < nt; ++t)
    th.emplace_back([&, t] {
      double* acc = part[t].data();
      for (int64_t r = t; r < rows; r += nt) {
        const float* x = q + r * D;
        for (int i = 0; i < D; ++i) {
          const double xi = x[i];
          double* row = acc + i * D;
          for (int j = 0; j < D; ++j) row[j] += xi * (double)x[j];
        }
      }
    });
  for (auto& t : th) t.join();
  for (unsigned t = 0; t < nt; ++t)
    for (int i = 0; i < D * D; ++i) c[i] += part[t][i];
  for (int i = 0; i < D * D; ++i) c[i] /= (double)rows;
}

// C_S = (1/(N Hq)) sum_h sum_n o_{h,n}^T o_{h,n}, o_{h,n} = sum_{m<=n} softmax_m(q_n . k_m / sqrt(d)) v_m.
// With the keys passed as v this is the attention-weighted key covariance
// C_SK = (1/(N Hq)) sum_h (S_h K)^T (S_h K).
void score_covariance(const float* q, const float* k, const float* v, int64_t n, int hq, int hkv, double* c) {
  std::fill(c, c + D * D, 0.0);
  const int g = hq / hkv;
  const unsigned nt = std::max(1u, std::min(8u, std::thread::hardware_concurrency()));
  std::vector<std::vector<double>> part(nt, std::vector<double>(D * D, 0.0));
  std::vector<std::thread> th;
  const double inv_sqrt_d = 1.0 / std::sqrt((double)D);
  for (unsigned t = 0; t < nt; ++t)
    th.emplace_back([&, t] {
      double* acc = part[t].data();
      std::vector<double> logit(n), o(D), qd(D);
      for (int64_t work = t; work < (int64_t)hq * n; work += nt) {
        const int h = (int)(work / n);
        const int64_t row = work % n;
        const int kv = h / g;
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
    for (int i = 0; i < D * D; ++i) c[i] += part[t][i];
  for (int i = 0; i < D * D; ++i) c[i] /= (double)(n * hq);
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

// tau_j = linear-interpolated percentile of |x . R|_j over all rows of x.
void clip_thresholds(const float* x, int64_t rows, const float* r, double pct, float* tau) {
  std::vector<std::vector<double>> col(D, std::vector<double>(rows));
  std::vector<double> y(D);
  for (int64_t n = 0; n < rows; ++n) {
    const float* xr = x + n * D;
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

int calibrate_layer(int hq, int hkv, int hadamard_block, float percentile, int rotation, const float* q,
                    const float* k, const float* v, int64_t n, float* rot_k, float* rot_v, float* clip_k,
                    float* clip_v) {
  for (const float* p : {q, k, v}) {
    const int64_t cnt = n * (p == q ? hq : hkv) * D;
    for (int64_t i = 0; i < cnt; ++i)
      if (!std::isfinite(p[i])) return -1;
  }
  std::vector<double> ck(D * D), cs(D * D), uk(D * D, 0.0), us(D * D, 0.0);
  switch (rotation) {
    case kRotSpectral:                 // key target C_Q, value target C_S
    case kRotKeyAttn:                  // key target C_SK, value target C_S
      if (rotation == kRotSpectral)
        query_covariance(q, n, hq, ck.data());
      else
        score_covariance(q, k, k, n, hq, hkv, ck.data());
      score_covariance(q, k, v, n, hq, hkv, cs.data());
      eigenbasis(ck.data(), uk.data());
      eigenbasis(cs.data(), us.data());
      compose_rotation(uk.data(), hadamard_block, rot_k);
      compose_rotation(us.data(), hadamard_block, rot_v);
      break;
    case kRotHadamard:                 // U = I: R = H P_br
      for (int i = 0; i < D; ++i) uk[i * D + i] = 1.0;
      compose_rotation(uk.data(), hadamard_block, rot_k);
      std::copy(rot_k, rot_k + D * D, rot_v);
      break;
    case kRotIdentity:                 // R = I
      for (int i = 0; i < D * D; ++i) rot_k[i] = rot_v[i] = (i % (D + 1) == 0) ? 1.0f : 0.0f;
      break;
    default:
      return -2;
  }
  clip_thresholds(k, n * hkv, rot_k, percentile, clip_k);
  clip_thresholds(v, n * hkv, rot_v, percentile, clip_v);
  for (int j = 0; j < D; ++j)
    if (!std::isfinite(clip_k[j]) || !std::isfinite(clip_v[j]) || clip_k[j] > 65504.0f || clip_v[j] > 65504.0f ||
        !(clip_k[j] > 0.0f) || !(clip_v[j] > 0.0f))
      return -1;
  return 0;
}

}  // namespace oscar
