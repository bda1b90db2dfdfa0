// Host set-up computed once per process (Sec. 3, "Rotated low-bit residual" and Eq. (2)):
// the seeded Gaussian rotation (Q factor of a Householder QR, diag(R) > 0) and the eps^2(b)
// calibration on Gaussian rows.  Random numbers: SplitMix64 (Steele, Lea & Flood 2014) as a
// counter-based stream, Box-Muller for Gaussians; stream 1 = rotation, 3 = calibration.
#include <math.h>
#include <stdint.h>

#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "setup.hpp"

namespace jolt {

static const uint64_t kGamma = 0x9E3779B97F4A7C15ull;

static uint64_t mix64(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ull;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBull;
  z ^= z >> 31;
  return z;
}

uint64_t splitmix_word(uint64_t key, uint64_t n) { return mix64(key + (n + 1) * kGamma); }

uint64_t stream_key(uint64_t seed, uint64_t stream) { return splitmix_word(seed, stream); }

static inline double unif(uint64_t w) { return ((double)(w >> 11) + 0.5) * (1.0 / 9007199254740992.0); }

void gaussians(uint64_t seed, uint64_t stream, uint64_t start, uint64_t count, double *out) {
  const uint64_t key = stream_key(seed, stream);
  for (uint64_t i = 0; i < count; ++i) {
    const uint64_t e = start + i, k = e >> 1;
    const double u1 = unif(splitmix_word(key, 2 * k)), u2 = unif(splitmix_word(key, 2 * k + 1));
    const double r = sqrt(-2.0 * log(u1)), th = 2.0 * M_PI * u2;
    out[i] = (e & 1) ? r * sin(th) : r * cos(th);
  }
}

// Householder QR of the D x D Gaussian; returns Q (row-major) with columns signed so that
// diag(R) > 0.
static std::vector<double> rotation_compute(int D, uint64_t seed) {
  std::vector<double> A((size_t)D * D), Q((size_t)D * D, 0.0), vs((size_t)D * D, 0.0), betas(D, 0.0), rdiag(D);
  gaussians(seed, 1, 0, (uint64_t)D * D, A.data());
  for (int k = 0; k < D; ++k) {
    double norm2 = 0.0;
    for (int i = k; i < D; ++i) norm2 += A[(size_t)i * D + k] * A[(size_t)i * D + k];
    const double x0 = A[(size_t)k * D + k];
    const double nrm = sqrt(norm2);
    const double alpha = (x0 >= 0.0) ? -nrm : nrm;  // R[k][k] = alpha
    double *v = &vs[(size_t)k * D];
    for (int i = k; i < D; ++i) v[i] = A[(size_t)i * D + k];
    v[k] -= alpha;
    double vn = 0.0;
    for (int i = k; i < D; ++i) vn += v[i] * v[i];
    const double beta = (vn > 0.0) ? 2.0 / vn : 0.0;
    betas[k] = beta;
    for (int j = k; j < D; ++j) {
      double s = 0.0;
      for (int i = k; i < D; ++i) s += v[i] * A[(size_t)i * D + j];
      s *= beta;
      for (int i = k; i < D; ++i) A[(size_t)i * D + j] -= s * v[i];
    }
    rdiag[k] = A[(size_t)k * D + k];
  }
  // Q = H_0 H_1 ... H_{D-1} applied to the identity (backwards)
  for (int i = 0; i < D; ++i) Q[(size_t)i * D + i] = 1.0;
  for (int k = D - 1; k >= 0; --k) {
    const double *v = &vs[(size_t)k * D];
    for (int j = 0; j < D; ++j) {
      double s = 0.0;
      for (int i = k; i < D; ++i) s += v[i] * Q[(size_t)i * D + j];
      s *= betas[k];
      for (int i = k; i < D; ++i) Q[(size_t)i * D + j] -= s * v[i];
    }
  }
  for (int k = 0; k < D; ++k)
    if (rdiag[k] < 0.0)
      for (int i = 0; i < D; ++i) Q[(size_t)i * D + k] = -Q[(size_t)i * D + k];
  return Q;
}

const std::vector<double> &rotation(int D, uint64_t seed) {
  static std::mutex mu;
  static std::map<std::pair<int, uint64_t>, std::vector<double>> cache;
  std::lock_guard<std::mutex> g(mu);
  auto key = std::make_pair(D, seed);
  auto it = cache.find(key);
  if (it == cache.end()) it = cache.emplace(key, rotation_compute(D, seed)).first;
  return it->second;
}

// eps^2(b) on 2^18 Gaussian rows of length D (seed 0): the row quantiser with fp32 decisions
// (same rule as the device encoder), error measured against the fp64 rows.
const std::vector<double> &eps2_table(int D) {
  static std::mutex mu;
  static std::map<int, std::vector<double>> cache;
  std::lock_guard<std::mutex> g(mu);
  auto it = cache.find(D);
  if (it != cache.end()) return it->second;
  const int rows = 1 << 18;
  std::vector<double> num(9, 0.0);
  double den = 0.0;
  std::vector<double> xd(D);
  std::vector<float> xf(D);
  for (int r = 0; r < rows; ++r) {
    gaussians(0, 3, (uint64_t)r * D, D, xd.data());
    double rowden = 0.0;
    for (int i = 0; i < D; ++i) {
      xf[i] = (float)xd[i];
      rowden += xd[i] * xd[i];
    }
    den += rowden;
    for (int b = 1; b <= 8; ++b) {
      // error measured against the fp64 row
      float a = 0.f;
      for (int i = 0; i < D; ++i) a = fmaxf(a, fabsf(xf[i]));
      const int qm = (b >= 2) ? ((1 << (b - 1)) - 1) : 1;
      const float s = (b == 1) ? a : a / (float)qm;
      double e = 0.0;
      for (int i = 0; i < D; ++i) {
        float v;
        if (b == 1) v = (xf[i] >= 0.f) ? s : -s;
        else if (s > 0.f) {
          float q = rintf(xf[i] / s);
          q = fminf(fmaxf(q, (float)-qm), (float)qm);
          v = q * s;
        } else v = 0.f;
        e += (xd[i] - (double)v) * (xd[i] - (double)v);
      }
      num[b] += e;
    }
  }
  std::vector<double> t(9, 1.0);
  for (int b = 1; b <= 8; ++b) t[b] = num[b] / den;
  return cache.emplace(D, t).first->second;
}

}  // namespace jolt
