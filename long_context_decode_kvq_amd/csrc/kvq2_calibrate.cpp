// kvq_calibrate: offline calibration of one layer on the host.
//
// OSCAR technical summary (gist.science 2605.17757), sec. 2.2-A:
//   item 1  C_Q = (1/N) sum q q^T (query-aware key target),
//           C_S = (1/N) V^T S^T S V (score-aware value target);
//   item 2  eigen-decomposition of both -> U_Q, U_S;
//   item 3  R_K = U_Q H_Had P_br, R_V = U_S H_Had P_br;
//   item 4  per-layer clip thresholds from the rotated calibration data.
// Readings: uncentered moments pooled over the query heads of each KV head
// (1/(N*G)); S is the causal softmax of the calibration tokens, so
// V^T S^T S V = O^T O with O = S V; eigen-columns in descending eigenvalue
// order, each made positive at its largest-magnitude entry; the clip is the
// nearest-rank quantile of |r| over all tokens, KV heads and channels.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <numeric>
#include <thread>
#include <vector>

#include "kvq2_internal.h"

namespace kvq {
namespace {

constexpr int D = kHeadDim;

double bf16_to_double(uint16_t b) {
  uint32_t u = uint32_t(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return double(f);
}

uint16_t float_to_bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

int bit_reverse7(int i) {
  int r = 0;
  for (int b = 0; b < 7; ++b) r |= ((i >> b) & 1) << (6 - b);
  return r;
}

// Cyclic Jacobi eigen-solver for a symmetric D x D matrix (row-major).
// On return A is (numerically) diagonal and V holds the eigenvectors as columns.
bool jacobi_eigh(std::vector<double>& A, std::vector<double>& V) {
  V.assign(D * D, 0.0);
  for (int i = 0; i < D; ++i) V[i * D + i] = 1.0;
  double norm2 = 0.0;
  for (double x : A) norm2 += x * x;
  if (norm2 == 0.0) return true;
  for (int sweep = 0; sweep < 64; ++sweep) {
    double off = 0.0;
    for (int p = 0; p < D; ++p)
      for (int q = p + 1; q < D; ++q) off += A[p * D + q] * A[p * D + q];
    if (off <= 1e-30 * norm2) return true;
    for (int p = 0; p < D - 1; ++p) {
      for (int q = p + 1; q < D; ++q) {
        const double apq = A[p * D + q];
        if (std::fabs(apq) <= 1e-300) continue;
        const double theta = (A[q * D + q] - A[p * D + p]) / (2.0 * apq);
        const double t = (theta >= 0 ? 1.0 : -1.0) / (std::fabs(theta) + std::sqrt(theta * theta + 1.0));
        const double c = 1.0 / std::sqrt(t * t + 1.0);
        const double s = t * c;
        for (int k = 0; k < D; ++k) {           // A <- A J
          const double akp = A[k * D + p], akq = A[k * D + q];
          A[k * D + p] = c * akp - s * akq;
          A[k * D + q] = s * akp + c * akq;
        }
        for (int k = 0; k < D; ++k) {           // A <- J^T A
          const double apk = A[p * D + k], aqk = A[q * D + k];
          A[p * D + k] = c * apk - s * aqk;
          A[q * D + k] = s * apk + c * aqk;
        }
        A[p * D + q] = A[q * D + p] = 0.0;
        for (int k = 0; k < D; ++k) {           // V <- V J
          const double vkp = V[k * D + p], vkq = V[k * D + q];
          V[k * D + p] = c * vkp - s * vkq;
          V[k * D + q] = s * vkp + c * vkq;
        }
      }
    }
  }
  return false;
}

// Eigenbasis with descending eigenvalues and the sign rule, then
// R = U . H . P (fp64) rounded to fp32.  H[i][j] = (-1)^popcount(i&j)/sqrt(D);
// (A P)[i][j] = A[i][bitrev(j)].
// R = U H P with H the Sylvester Hadamard of size `hb` on each diagonal
// block of hb channels (hb = 128: the full transform), scaled by 1/sqrt(hb).
bool rotation_from_covariance(std::vector<double> C, float* R_out, int hb) {
  std::vector<double> V;
  if (!jacobi_eigh(C, V)) return false;
  std::vector<int> order(D);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](int a, int b) { return C[a * D + a] > C[b * D + b]; });
  std::vector<double> U(D * D);
  for (int c = 0; c < D; ++c) {
    const int src = order[c];
    int arg = 0;
    double best = -1.0;
    for (int k = 0; k < D; ++k) {
      const double a = std::fabs(V[k * D + src]);
      if (a > best) { best = a; arg = k; }
    }
    const double sign = V[arg * D + src] < 0 ? -1.0 : 1.0;
    for (int k = 0; k < D; ++k) U[k * D + c] = sign * V[k * D + src];
  }
  const double inv_sqrt = 1.0 / std::sqrt(double(hb));
  for (int i = 0; i < D; ++i) {
    for (int j = 0; j < D; ++j) {
      const int jb = bit_reverse7(j);   // column j of H P is column jb of H
      const int blk = jb / hb;
      double acc = 0.0;
      for (int k = blk * hb; k < (blk + 1) * hb; ++k)
        acc += U[i * D + k] *
               ((__builtin_popcount((k % hb) & (jb % hb)) & 1) ? -inv_sqrt : inv_sqrt);
      R_out[i * D + j] = float(acc);
    }
  }
  return true;
}

// Pinned rotation r = bf16(fp32(R^T x)): fp64 accumulation in order j = 0..127.
void rotate_pinned(const double* x, const float* R, float* r_out) {
  for (int i = 0; i < D; ++i) {
    double acc = 0.0;
    for (int j = 0; j < D; ++j) acc = std::fma(x[j], double(R[j * D + i]), acc);
    const uint16_t b = float_to_bf16_rne(float(acc));
    r_out[i] = float(bf16_to_double(b));
  }
}

}  // namespace
}  // namespace kvq

using namespace kvq;

extern "C" int kvq_calibrate(const kvq_dims* dims, int32_t n_tokens, const uint16_t* q,
                             const uint16_t* k, const uint16_t* v, double clip_quantile,
                             float* R_K, float* R_V, float* clip_K, float* clip_V) {
  if (dims == nullptr || q == nullptr || k == nullptr || v == nullptr || R_K == nullptr ||
      R_V == nullptr || clip_K == nullptr || clip_V == nullptr)
    return KVQ_ERR_ARG;
  if (dims->head_dim != kHeadDim) return KVQ_ERR_UNSUPPORTED;
  const int Hq = dims->n_q_heads, Hkv = dims->n_kv_heads;
  const int hb = dims->hadamard_block > 0 ? dims->hadamard_block : D;
  if (hb != 32 && hb != 64 && hb != 128) return KVQ_ERR_UNSUPPORTED;
  if (Hkv < 1 || Hq < 1 || Hq % Hkv != 0 || n_tokens < 1) return KVQ_ERR_ARG;
  if (!(clip_quantile > 0.0) || !(clip_quantile <= 1.0)) return KVQ_ERR_ARG;
  const int G = Hq / Hkv;
  const int N = n_tokens;
  const double sm = dims->sm_scale > 0.0f ? double(dims->sm_scale) : 1.0 / std::sqrt(double(D));

  // Widen the bf16 inputs once; reject non-finite values.
  std::vector<double> Q(size_t(N) * Hq * D), K(size_t(N) * Hkv * D), Vv(size_t(N) * Hkv * D);
  for (size_t i = 0; i < Q.size(); ++i) Q[i] = bf16_to_double(q[i]);
  for (size_t i = 0; i < K.size(); ++i) K[i] = bf16_to_double(k[i]);
  for (size_t i = 0; i < Vv.size(); ++i) Vv[i] = bf16_to_double(v[i]);
  for (const auto* arr : {&Q, &K, &Vv})
    for (double x : *arr)
      if (!std::isfinite(x)) return KVQ_ERR_NUMERIC;

  std::vector<char> ok(Hkv, 0);
  auto work = [&](int h) {
    // C_Q, pooled over the G query heads of KV head h.
    std::vector<double> CQ(D * D, 0.0), CS(D * D, 0.0);
    for (int n = 0; n < N; ++n)
      for (int g = 0; g < G; ++g) {
        const double* x = &Q[(size_t(n) * Hq + h * G + g) * D];
        for (int i = 0; i < D; ++i)
          for (int j = 0; j < D; ++j) CQ[i * D + j] += x[i] * x[j];
      }
    // Contiguous copies of this head's keys and values.
    std::vector<double> Kh(size_t(N) * D), Vh(size_t(N) * D), logit(N), o(D);
    for (int n = 0; n < N; ++n)
      for (int i = 0; i < D; ++i) {
        Kh[size_t(n) * D + i] = K[(size_t(n) * Hkv + h) * D + i];
        Vh[size_t(n) * D + i] = Vv[(size_t(n) * Hkv + h) * D + i];
      }
    // C_S = (1/(N G)) sum O^T O with O the causal attention outputs.
    for (int g = 0; g < G; ++g) {
      for (int n = 0; n < N; ++n) {
        const double* x = &Q[(size_t(n) * Hq + h * G + g) * D];
        double mx = -INFINITY;
        for (int j = 0; j <= n; ++j) {
          const double* kj = &Kh[size_t(j) * D];
          double s = 0.0;
          for (int i = 0; i < D; ++i) s += x[i] * kj[i];
          logit[j] = sm * s;
          mx = std::max(mx, logit[j]);
        }
        double tot = 0.0;
        std::fill(o.begin(), o.end(), 0.0);
        for (int j = 0; j <= n; ++j) {
          const double p = std::exp(logit[j] - mx);
          tot += p;
          const double* vj = &Vh[size_t(j) * D];
          for (int i = 0; i < D; ++i) o[i] += p * vj[i];
        }
        for (int i = 0; i < D; ++i) o[i] /= tot;
        for (int i = 0; i < D; ++i)
          for (int j = 0; j < D; ++j) CS[i * D + j] += o[i] * o[j];
      }
    }
    const double inv = 1.0 / (double(N) * G);
    for (int i = 0; i < D * D; ++i) {
      CQ[i] *= inv;
      CS[i] *= inv;
    }
    ok[h] = rotation_from_covariance(CQ, R_K + size_t(h) * D * D, hb) &&
            rotation_from_covariance(CS, R_V + size_t(h) * D * D, hb);
  };
  {
    const int n_threads = std::max(1, std::min(Hkv, 16));
    for (int base = 0; base < Hkv; base += n_threads) {
      std::vector<std::thread> pool;
      for (int h = base; h < std::min(Hkv, base + n_threads); ++h) pool.emplace_back(work, h);
      for (auto& t : pool) t.join();
    }
  }
  for (int h = 0; h < Hkv; ++h)
    if (!ok[h]) return KVQ_ERR_NUMERIC;

  // Clip thresholds: nearest-rank quantile of |rotated bf16 value|.
  auto clip_of = [&](const std::vector<double>& X, const float* R, float* out) -> int {
    std::vector<float> mag(size_t(N) * Hkv * D);
    std::vector<float> r(D);
    for (int n = 0; n < N; ++n)
      for (int h = 0; h < Hkv; ++h) {
        rotate_pinned(&X[(size_t(n) * Hkv + h) * D], R + size_t(h) * D * D, r.data());
        for (int i = 0; i < D; ++i) mag[(size_t(n) * Hkv + h) * D + i] = std::fabs(r[i]);
      }
    const size_t cnt = mag.size();
    long long rank = static_cast<long long>(std::ceil(clip_quantile * double(cnt)));
    rank = std::min<long long>(std::max<long long>(rank, 1), static_cast<long long>(cnt));
    std::nth_element(mag.begin(), mag.begin() + (rank - 1), mag.end());
    const float c = mag[rank - 1];
    if (!(c > 0.0f) || !(c <= kMaxClip)) return KVQ_ERR_NUMERIC;
    *out = c;
    return KVQ_OK;
  };
  int rc = clip_of(K, R_K, clip_K);
  if (rc != KVQ_OK) return rc;
  return clip_of(Vv, R_V, clip_V);
}
