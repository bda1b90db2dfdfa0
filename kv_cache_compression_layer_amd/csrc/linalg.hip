// Small dense fp64 linear algebra on the GPU: symmetric eigenproblems (Householder
// tridiagonalisation, Sturm bisection, inverse iteration, back-transformation), Cholesky with
// triangular inverse for the thin QR, and an fp64 Gram of fp32 panels.
//
// These serve the mode spectra and factors of the method (token-mode and feature-mode
// singular values/vectors from Gram matrices; the FlashJoLT Rayleigh-Ritz step on B B^T), the
// matrices are at most a few thousand wide, and one workgroup owns one matrix for the
// sequential parts.  Algorithms: Golub & Van Loan, "Matrix Computations", Sec. 8.3
// (tridiagonalisation), Sec. 8.4 (Sturm-sequence bisection), Sec. 8.2/7.6 (inverse iteration);
// Cholesky QR as in Fukaya et al. (2014).
#include <math.h>

#include "common.hpp"
#include "linalg.hpp"

namespace jolt {

namespace {

constexpr int LT = 1024;  // threads of the one-workgroup-per-matrix kernels

__device__ double block_sum(double v, double *red) {
  v = warp_sum_d(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  double s = 0.0;
  for (int i = 0; i < nw; ++i) s += red[i];  // fixed order: deterministic
  return s;
}

// All eigenvalues of `batch` symmetric tridiagonals (d, e), descending, by multisection: a group
// of BL lanes brackets one eigenvalue and evaluates BL Sturm counts per iteration (BL - 1 interior
// shifts spaced evenly inside the bracket), narrowing the bracket (BL + 1)-fold per iteration.
// Sturm recurrence with a pivot guard, Gershgorin starting interval, stop at a relative width of
// about 2 ulp (Golub & Van Loan, Sec. 8.4).
// BL: 16 lanes for small problems (enough threads to fill the GPU), 4 where the problem is large
// enough to fill it anyway (fewer Sturm sweeps in total)

template <int BL>
__global__ void __launch_bounds__(256) bisect_kernel(const double *d_in, const double *e_in, long long t_bs, int n,
                                                     double *evals, long long ev_bs, int clamp, const unsigned *err,
                                                     long long err_bs) {
  extern __shared__ double smem[];
  __shared__ double red[3][4];
  const int b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (err && err[b * err_bs]) {  // the reduction reported a failed exchange: no eigenvalues
    const int j = (blockIdx.x * 256 + tid) / BL;
    if (j < n && (tid % BL) == 0) evals[b * ev_bs + j] = __longlong_as_double(0x7ff8000000000000LL);
    return;
  }
  const double *d = d_in + b * t_bs, *e = e_in + b * t_bs;
  double *sd = smem, *se2 = smem + n;
  double lo0 = 1e300, hi0 = -1e300;
  for (int i = tid; i < n; i += 256) {
    const double di = d[i], ei = (i + 1 < n) ? e[i] : 0.0, ep = (i > 0) ? e[i - 1] : 0.0;
    sd[i] = di;
    se2[i] = ei * ei;
    const double r = fabs(ep) + fabs(ei);
    lo0 = fmin(lo0, di - r);
    hi0 = fmax(hi0, di + r);
  }
  for (int o = 32; o > 0; o >>= 1) {
    lo0 = fmin(lo0, __shfl_xor(lo0, o, 64));
    hi0 = fmax(hi0, __shfl_xor(hi0, o, 64));
  }
  if (lane == 0) {
    red[0][wave] = lo0;
    red[1][wave] = hi0;
  }
  __syncthreads();
  lo0 = fmin(fmin(red[0][0], red[0][1]), fmin(red[0][2], red[0][3]));
  hi0 = fmax(fmax(red[1][0], red[1][1]), fmax(red[1][2], red[1][3]));
  const double tn = fmax(fabs(lo0), fabs(hi0));
  const double pivmin = fmax(1e-300, 1e-300 * tn * tn);
  lo0 -= 2.2e-16 * tn * 4 + pivmin;
  hi0 += 2.2e-16 * tn * 4 + pivmin;
  const int g = lane / BL, l = lane % BL;
  const int j = (blockIdx.x * 256 + tid) / BL;  // eigenvalue index (descending)
  if (j >= n) return;
  const int s = n - 1 - j;                     // j-th largest == s-th smallest
  double lo = lo0, hi = hi0;
  for (int it = 0; it < 200; ++it) {
    if (hi - lo <= 2.2e-16 * fmax(fabs(lo), fabs(hi)) * 2 + pivmin) break;
    const double x = lo + (hi - lo) * (double)(l + 1) / (double)(BL + 1);
    int cnt = 0;
    double q = sd[0] - x;
    if (fabs(q) < pivmin) q = -pivmin;
    cnt += (q < 0.0);
    for (int i = 1; i < n; ++i) {
      // e_{i-1}^2 / q by the hardware reciprocal and one Newton step (within an ulp or two of the
      // rounded quotient: the count keeps the backward stability of the recurrence)
      double y = __builtin_amdgcn_rcp(q);
      y = fma(y, fma(-q, y, 1.0), y);
      q = (sd[i] - x) - se2[i - 1] * y;
      if (fabs(q) < pivmin) q = -pivmin;
      cnt += (q < 0.0);
    }
    // first lane of the group whose count exceeds s: the eigenvalue lies in (x_{P-1}, x_P]
    const unsigned long long over = __ballot(cnt > s);
    const unsigned grp = (unsigned)((over >> (g * BL)) & ((1ull << BL) - 1ull));
    const int P = grp ? __builtin_ctz(grp) : BL;
    const double w = hi - lo;
    const double nlo = (P > 0) ? lo + w * (double)P / (double)(BL + 1) : lo;
    const double nhi = (P < BL) ? lo + w * (double)(P + 1) / (double)(BL + 1) : hi;
    if (!(nlo > lo || nhi < hi)) break;  // no progress at this precision
    lo = nlo;
    hi = nhi;
  }
  if (l == 0) {
    double v = 0.5 * (lo + hi);
    if (clamp && v < 0.0) v = 0.0;
    evals[b * ev_bs + j] = v;
  }
}

// ---------------------------------------------------------------------------------------------
// Householder tridiagonalisation + all eigenvalues by bisection.
// A: [batch][n][lda] fp64 symmetric (overwritten).  Output per batch: d[n], e[n] (e[n-1]=0),
// reflectors refl[n][n] (row k holds v_k for rows k+1.., v_k[0] = 1), beta[n],
// evals[n] descending (clamped at >= 0 when clamp != 0).  The working copy lives in LDS
// (n^2 + 2n doubles), so this kernel serves n <= 136.
// ---------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(LT) tridiag_values_kernel(double *A, long long a_bs, int lda, const int *n_of,
                                                            int n_fixed, double *d_out, double *e_out,
                                                            double *refl, double *beta, long long t_bs,
                                                            double *evals, long long ev_bs, int clamp,
                                                            int use_lds) {
  extern __shared__ double smem[];
  const int b = blockIdx.x;
  const int n = n_of ? n_of[b] : n_fixed;
  const int tid = threadIdx.x, nt = blockDim.x;
  double *Ag = A + b * a_bs;
  double *d = d_out + b * t_bs, *e = e_out + b * t_bs, *R = refl + b * t_bs * (long long)n_fixed,
         *be = beta + b * t_bs;
  // working copy in LDS (matrices that do not fit take tridiag_fused_kernel)
  (void)use_lds;
  double *W = smem;
  const int ldw = n;
  double *vbuf = smem + (long long)n * n, *pbuf = vbuf + n;
  for (int i = tid; i < n * n; i += nt) W[i] = Ag[(long long)(i / n) * lda + (i % n)];
  __syncthreads();

  const int lane = tid & 63, wv = tid >> 6, nwv = nt >> 6;
  // three barriers per step: the two reductions are formed by every wave on its own (same order
  // in every wave, so the values agree) and w = p - c v is formed inside the update
  for (int k = 0; k + 2 < n; ++k) {
    const int m = n - k - 1;  // trailing size
    const double *row = W + (long long)k * ldw + (k + 1);  // x = A[k][k+1..] (= column k by symmetry)
    double part = 0.0;
    for (int i = 1 + lane; i < m; i += 64) part += row[i] * row[i];
    const double sigma = warp_sum_d(part);
    const double alpha = row[0];
    double bet, v0, mu;
    if (sigma == 0.0) {
      bet = 0.0;
      v0 = 1.0;
      mu = alpha;
    } else {
      mu = sqrt(alpha * alpha + sigma);
      v0 = (alpha <= 0.0) ? (alpha - mu) : (-sigma / (alpha + mu));
      bet = 2.0 * v0 * v0 / (sigma + v0 * v0);
    }
    for (int i = tid; i < m; i += nt) {
      double vi = (i == 0) ? 1.0 : row[i] / v0;
      vbuf[i] = vi;
      R[(long long)k * n_fixed + k + 1 + i] = vi;
    }
    if (tid == 0) {
      d[k] = W[(long long)k * ldw + k];
      e[k] = (sigma == 0.0) ? alpha : mu;
      be[k] = bet;
    }
    __syncthreads();
    if (bet == 0.0) continue;
    // p = beta * A22 v: one wave per row, lanes along the (contiguous) row
    double *A22 = W + (long long)(k + 1) * ldw + (k + 1);
    for (int i = wv; i < m; i += nwv) {
      const double *ri = A22 + (long long)i * ldw;
      double s0 = 0.0, s1 = 0.0;
      int jj = lane;
      for (; jj + 64 < m; jj += 128) {
        s0 += ri[jj] * vbuf[jj];
        s1 += ri[jj + 64] * vbuf[jj + 64];
      }
      if (jj < m) s0 += ri[jj] * vbuf[jj];
      const double sr = warp_sum_d(s0 + s1);
      if (lane == 0) pbuf[i] = bet * sr;
    }
    __syncthreads();
    part = 0.0;
    for (int i = lane; i < m; i += 64) part += pbuf[i] * vbuf[i];
    const double c = 0.5 * bet * warp_sum_d(part);
    // A22 -= v w^T + w v^T with w = p - c v: one wave per row
    for (int i = wv; i < m; i += nwv) {
      double *ri = A22 + (long long)i * ldw;
      const double vi = vbuf[i], wi = pbuf[i] - c * vbuf[i];
      for (int jj = lane; jj < m; jj += 64) ri[jj] -= vi * (pbuf[jj] - c * vbuf[jj]) + wi * vbuf[jj];
    }
    __syncthreads();
  }
  if (tid == 0) {
    if (n >= 2) {
      d[n - 2] = W[(long long)(n - 2) * ldw + (n - 2)];
      d[n - 1] = W[(long long)(n - 1) * ldw + (n - 1)];
      e[n - 2] = W[(long long)(n - 1) * ldw + (n - 2)];
      be[n - 2] = 0.0;
    } else {
      d[0] = W[0];
    }
    e[n - 1] = 0.0;
    be[n - 1] = 0.0;
  }
  (void)evals;
  (void)ev_bs;
  (void)clamp;
}

// ---------------------------------------------------------------------------------------------
// The same reduction for matrices kept in global memory (too large for LDS), arranged so that the
// trailing matrix is swept once per step.  Step k (reflector v_k from row k, p_k = beta_k A v_k,
// w_k = p_k - (beta_k / 2)(p_k . v_k) v_k, A <- A - v_k w_k^T - w_k v_k^T on rows/cols > k):
//   1. wave 0 applies the update to row k+1 and forms reflector k+1 from it (one-step look-ahead);
//   2. every wave applies the update to its rows i > k+1 and, in the same pass over the row,
//      accumulates p_{k+1}[i] = beta_{k+1} sum_j A[i][j] v_{k+1}[j].
// Column k+1 of rows i > k+1 is never read again (its content is row k+1 by symmetry) and is not
// updated.  v and p live in LDS with absolute indices, two buffers each alternating by step, so a
// step needs two workgroup barriers.  Same formulas as tridiag_values_kernel; sums run in a fixed
// order, so results are deterministic.  LDS: 4n doubles.
// ---------------------------------------------------------------------------------------------
constexpr int TCH = 9;  // 64-wide row chunks a wave keeps in registers (one pass covers 576 columns)
constexpr int TRB = 2;  // rows a wave sweeps together (TRB * TCH loads in flight)

// Wave-level: Householder reflector from row r (x = W[r][r+1..n)), written to v (LDS, absolute
// columns), the reflector row R[r][..] and d/e/beta[r]; returns beta on every lane.  General
// width (re-reads the row); the fused kernel uses the register version below when it fits.
__device__ __forceinline__ double wave_reflector(double *W, int ldw, int n, int r, double *v, double *R, long long r_ld, double *d,
                                 double *e, double *be) {
  const int lane = threadIdx.x & 63;
  const double *x = W + (long long)r * ldw;
  double part = 0.0, alpha = 0.0;
  for (int j = r + 1 + lane; j < n; j += 64) {
    const double xj = x[j];
    if (j == r + 1) alpha = xj;
    else part += xj * xj;
  }
  const double sigma = warp_sum_d(part);
  alpha = __shfl(alpha, 0, 64);  // column r+1 is lane 0's first element
  double bet, v0, mu;
  if (sigma == 0.0) {
    bet = 0.0;
    v0 = 1.0;
    mu = alpha;
  } else {
    mu = sqrt(alpha * alpha + sigma);
    v0 = (alpha <= 0.0) ? (alpha - mu) : (-sigma / (alpha + mu));
    bet = 2.0 * v0 * v0 / (sigma + v0 * v0);
  }
  const double dr = x[r];
  for (int j = r + 1 + lane; j < n; j += 64) {
    const double vj = (j == r + 1) ? 1.0 : x[j] / v0;
    v[j] = vj;
    R[(long long)r * r_ld + j] = vj;  // may alias row r of W: each element is read before it is written
  }
  if (lane == 0) {
    d[r] = dr;
    e[r] = (sigma == 0.0) ? alpha : mu;
    be[r] = bet;
  }
  return bet;
}

// value of a double held by lane l (l a compile-time constant), by scalar lane reads
__device__ __forceinline__ double lane_bcast_d(double v, int l) {
  const int lo = __builtin_amdgcn_readlane(__double2loint(v), l);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(v), l);
  return __hiloint2double(hi, lo);
}

// Row r (columns r..n-1, n - r <= 64 * TCH) held in registers x[t] = row[r + lane + 64 t]:
// the same reflector, one read of the row.  A null R skips the reflector row, a null d the
// d/e/beta entries (v and the returned beta are always formed).
__device__ __forceinline__ double wave_reflector_regs(const double (&x)[TCH], int n, int r, double *v, double *R, long long r_ld,
                                      double *d, double *e, double *be) {
  const int lane = threadIdx.x & 63;
  double part = 0.0;
#pragma unroll
  for (int t = 0; t < TCH; ++t) {
    const int j = r + lane + 64 * t;
    if (j >= r + 2 && j < n) part += x[t] * x[t];
  }
  const double sigma = warp_sum_d(part);
  const double alpha = lane_bcast_d(x[0], 1), dr = lane_bcast_d(x[0], 0);
  double bet, v0, mu;
  if (sigma == 0.0) {
    bet = 0.0;
    v0 = 1.0;
    mu = alpha;
  } else {
    mu = sqrt(alpha * alpha + sigma);
    v0 = (alpha <= 0.0) ? (alpha - mu) : (-sigma / (alpha + mu));
    bet = 2.0 * v0 * v0 / (sigma + v0 * v0);
  }
#pragma unroll
  for (int t = 0; t < TCH; ++t) {
    const int j = r + lane + 64 * t;
    if (j >= r + 1 && j < n) {
      const double vj = (j == r + 1) ? 1.0 : x[t] / v0;
      v[j] = vj;
      if (R) R[(long long)r * r_ld + j] = vj;
    }
  }
  if (lane == 0 && d) {
    d[r] = dr;
    e[r] = (sigma == 0.0) ? alpha : mu;
    be[r] = bet;
  }
  return bet;
}

// UP (n <= 64 TCH): the sweep touches only the upper triangle of the trailing block (j >= i),
// read and written once; element (i, j), j > i, adds u v'_j to the row sum of i and u v'_i to the
// column sum of j, kept per lane for the lane's absolute columns lane + 64 t; the column sums of
// the waves are added to the row sums in LDS in wave order (deterministic), which takes a third
// barrier per step.  Half the traffic of the full sweep.  LDS: 5n + 64 TCH nwave doubles.
template <bool UP>
__global__ void __launch_bounds__(LT) tridiag_fused_kernel(double *A, long long a_bs, int lda, int n,
                                                           double *d_out, double *e_out, double *refl, double *beta,
                                                           long long t_bs, double *evals, long long ev_bs, int clamp) {
  extern __shared__ double smem[];
  __shared__ double sbeta[2];
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwave = blockDim.x >> 6;
  double *W = A + b * a_bs;
  const int ldw = lda;
  double *d = d_out + b * t_bs, *e = e_out + b * t_bs, *R = refl + b * t_bs * (long long)n, *be = beta + b * t_bs;
  // v_k at smem + (k % 2) n, p_k at smem + (2 + k % 2) n (pointers derived arithmetically from the
  // LDS array so that every access compiles to an LDS instruction)

  if (n >= 3) {
    // prologue: reflector 0 and p_0 = beta_0 A[1.., 1..] v_0
    if (wave == 0) {
      const double bt = wave_reflector(W, ldw, n, 0, smem, R, n, d, e, be);
      if (lane == 0) sbeta[0] = bt;
    }
    __syncthreads();
    {
      const double b0 = sbeta[0];
      for (int i = 1 + wave; i < n; i += nwave) {
        const double *ri = W + (long long)i * ldw;
        double s = 0.0;
        for (int j = 1 + lane; j < n; j += 64) s += ri[j] * smem[j];
        s = warp_sum_d(s);
        if (lane == 0) smem[2 * n + i] = b0 * s;
      }
    }
    __syncthreads();
    for (int k = 0; k + 2 < n; ++k) {
      const int cur = k & 1, nxt = cur ^ 1, r = k + 1;
      const double *vk = smem + cur * n, *pk = smem + (2 + cur) * n;
      double *vnx = smem + nxt * n;
      // c = (beta_k / 2) p_k . v_k, computed by every wave in the same order
      double part = 0.0;
      for (int j = r + lane; j < n; j += 64) part += pk[j] * vk[j];
      const double c = 0.5 * sbeta[cur] * warp_sum_d(part);
      const bool last = (r == n - 2);
      if (wave == 0) {
        // update row r (columns r..n-1), then the next reflector from it
        double *rr = W + (long long)r * ldw;
        const double wr = pk[r] - c * vk[r], vr = vk[r];
        if (n - r <= 64 * TCH) {
          double x[TCH];
#pragma unroll
          for (int t = 0; t < TCH; ++t) {
            const int j = r + lane + 64 * t;
            x[t] = (j < n) ? rr[j] : 0.0;
          }
#pragma unroll
          for (int t = 0; t < TCH; ++t) {
            const int j = r + lane + 64 * t;
            if (j < n) {
              x[t] -= vr * (pk[j] - c * vk[j]) + wr * vk[j];
              rr[j] = x[t];  // (columns > r are overwritten by the reflector when it aliases the row)
            }
          }
          if (!last) {
            const double bt = wave_reflector_regs(x, n, r, vnx, R, n, d, e, be);
            if (lane == 0) sbeta[nxt] = bt;
          } else {
            const double e2 = __shfl(x[0], 1, 64);  // column n-1 of row n-2
            if (lane == 0) {
              d[n - 2] = x[0];
              e[n - 2] = e2;
              be[n - 2] = 0.0;
            }
          }
        } else {
          for (int j = r + lane; j < n; j += 64) rr[j] -= vr * (pk[j] - c * vk[j]) + wr * vk[j];
          if (!last) {
            const double bt = wave_reflector(W, ldw, n, r, vnx, R, n, d, e, be);
            if (lane == 0) sbeta[nxt] = bt;
          } else if (lane == 0) {
            d[n - 2] = rr[n - 2];
            e[n - 2] = rr[n - 1];
            be[n - 2] = 0.0;
          }
        }
      }
      __syncthreads();
      // rows r+1..n-1: update columns r+1..n-1 and accumulate the next matvec in the same pass;
      // a wave sweeps TRB rows at once with every load of a chunk group issued before any use
      const double bn = last ? 0.0 : sbeta[nxt];
      const double *vn = vnx;
      double *pn = smem + (2 + nxt) * n;
      if constexpr (UP) {
        double *prow = smem + 4 * n, *pcol = smem + 5 * n;  // row sums [n]; column sums [nwave][64 TCH]
        double cacc[TCH];
#pragma unroll
        for (int t = 0; t < TCH; ++t) cacc[t] = 0.0;
        for (int i0 = r + 1 + wave * TRB; i0 < n; i0 += nwave * TRB) {
          double s[TRB], wi[TRB], vi[TRB], vni[TRB];
#pragma unroll
          for (int q = 0; q < TRB; ++q) {
            const int i = min(i0 + q, n - 1);
            s[q] = 0.0;
            wi[q] = pk[i] - c * vk[i];
            vi[q] = vk[i];
            vni[q] = last ? 0.0 : vn[i];
          }
          const int tstart = i0 >> 6;  // first 64-column chunk holding column i0 (uniform)
          double a[TRB][TCH];
#pragma unroll
          for (int t = 0; t < TCH; ++t)
            if (t >= tstart) {
              const int j = lane + 64 * t;
#pragma unroll
              for (int q = 0; q < TRB; ++q)
                a[q][t] = (i0 + q < n && j >= i0 + q && j < n) ? W[(long long)(i0 + q) * ldw + j] : 0.0;
            }
#pragma unroll
          for (int t = 0; t < TCH; ++t)
            if (t >= tstart) {
              const int j = lane + 64 * t;
              if (j >= i0 && j < n) {
                const double pj = pk[j] - c * vk[j], vj = vk[j], vnj = last ? 0.0 : vn[j];
#pragma unroll
                for (int q = 0; q < TRB; ++q) {
                  if (i0 + q < n && j >= i0 + q) {
                    const double u = a[q][t] - (vi[q] * pj + wi[q] * vj);
                    W[(long long)(i0 + q) * ldw + j] = u;
                    s[q] += u * vnj;
                    if (j > i0 + q) cacc[t] += u * vni[q];
                  }
                }
              }
            }
          if (!last) {
#pragma unroll
            for (int q = 0; q < TRB; ++q) {
              const double sq = warp_sum_d(s[q]);
              if (lane == 0 && i0 + q < n) prow[i0 + q] = sq;
            }
          }
        }
        if (!last) {
#pragma unroll
          for (int t = 0; t < TCH; ++t) pcol[wave * 64 * TCH + lane + 64 * t] = cacc[t];
        }
        __syncthreads();
        if (!last) {
          for (int j = r + 1 + tid; j < n; j += blockDim.x) {
            double sum = prow[j];
            for (int w = 0; w < nwave; ++w) sum += pcol[w * 64 * TCH + j];
            pn[j] = bn * sum;
          }
        }
        __syncthreads();
      } else {
        for (int i0 = r + 1 + wave * TRB; i0 < n; i0 += nwave * TRB) {
          double s[TRB], wi[TRB], vi[TRB];
#pragma unroll
          for (int q = 0; q < TRB; ++q) {
            const int i = min(i0 + q, n - 1);
            s[q] = 0.0;
            wi[q] = pk[i] - c * vk[i];
            vi[q] = vk[i];
          }
          for (int j0 = r + 1; j0 < n; j0 += 64 * TCH) {
            double a[TRB][TCH];
#pragma unroll
            for (int q = 0; q < TRB; ++q)
#pragma unroll
              for (int t = 0; t < TCH; ++t) {
                const int j = j0 + lane + 64 * t;
                a[q][t] = (i0 + q < n && j < n) ? W[(long long)(i0 + q) * ldw + j] : 0.0;
              }
#pragma unroll
            for (int t = 0; t < TCH; ++t) {
              const int j = j0 + lane + 64 * t;
              if (j < n) {
                const double pj = pk[j] - c * vk[j], vj = vk[j], vnj = last ? 0.0 : vn[j];
#pragma unroll
                for (int q = 0; q < TRB; ++q) {
                  if (i0 + q < n) {
                    const double u = a[q][t] - (vi[q] * pj + wi[q] * vj);
                    W[(long long)(i0 + q) * ldw + j] = u;
                    s[q] += u * vnj;
                  }
                }
              }
            }
          }
          if (!last) {
#pragma unroll
            for (int q = 0; q < TRB; ++q) {
              const double sq = warp_sum_d(s[q]);
              if (lane == 0 && i0 + q < n) pn[i0 + q] = bn * sq;
            }
          }
        }
        __syncthreads();
      }
    }
    if (tid == 0) {
      d[n - 1] = W[(long long)(n - 1) * ldw + (n - 1)];
      e[n - 1] = 0.0;
      be[n - 1] = 0.0;
    }
  } else if (tid == 0) {
    d[0] = W[0];
    if (n == 2) {
      d[1] = W[(long long)ldw + 1];
      e[0] = W[1];
    }
    e[n - 1] = 0.0;
    be[0] = 0.0;
    be[n - 1] = 0.0;
  }
  (void)evals;
  (void)ev_bs;
  (void)clamp;
}

// ---------------------------------------------------------------------------------------------
// The same reduction spread over P workgroups per matrix, for matrices whose rows fit in their
// combined LDS: workgroup w keeps the full rows i = w, w + P, w + 2P, ... (fp64) in LDS for the
// whole reduction, and only vectors cross workgroups.  Every workgroup forms each reflector itself
// from the published row, so a step takes one exchange.  Step j (reflector j from row j):
//   1. read p_{j-1} and row j (after update j-2) from the exchange slot of step j-1, form c_{j-1},
//      apply update j-1 to row j and form v_j, beta_j from it (wave 0 of every workgroup, the same
//      arithmetic everywhere; the owner of row j writes d, e, beta and the reflector row);
//   2. apply update j-1 to the own rows i > j (columns > j) and form p_j[i] = beta_j (A v_j)_i in
//      the same pass (a wave takes up to MR rows at once and reads the vectors once for them);
//   3. publish p_j of the own rows and, from the owner of row j+1, that row; wait for all P.
// Same formulas as tridiag_fused_kernel<false>; every sum runs in a fixed order (deterministic).
// Exchange: the published values are agent-coherent (write-through) stores and are read with
// agent-coherent loads; the publishing wave waits for its stores to complete before it bumps the
// per-matrix step counter, which each workgroup's first thread polls (then an acquire fence), so no
// L2 write-back is needed per step.  Every wait is bounded: one that runs out sets the matrix's
// error word (the bisection then reports NaN eigenvalues) and stops waiting.  The reflector row 0
// is written after the first exchange, when every workgroup has read row 0 of A (refl may alias A).
// Scratch per matrix: a 256-byte header (step counter, error word) and two slots of p and row
// (mwg_ldx(n) doubles each).  LDS: (ceil(n / P) + 3) n + ceil(n / P) doubles.
// ---------------------------------------------------------------------------------------------
constexpr int MWG_HDR = 32;  // header doubles per matrix
constexpr int MR = 3;        // rows a wave sweeps together
__host__ __device__ inline long long mwg_ldx(int n) { return ((long long)n + 63) / 64 * 64; }
__host__ __device__ inline long long mwg_doubles(int n) { return MWG_HDR + 4 * mwg_ldx(n); }

__global__ void mwg_reset_kernel(double *x, long long stride, int batch) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < batch) {
    unsigned *h = (unsigned *)(x + b * stride);
    h[0] = 0u;
    h[1] = 0u;
  }
}

__device__ __forceinline__ void xstore(double *p, double v) {
  __hip_atomic_store((unsigned long long *)p, (unsigned long long)__double_as_longlong(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double xload(const double *p) {
  return __longlong_as_double(
      (long long)__hip_atomic_load((unsigned long long *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

__global__ void __launch_bounds__(LT) tridiag_mwg_kernel(const double *A, long long a_bs, int lda, int n, int P,
                                                         double *d_out, double *e_out, double *refl, double *beta,
                                                         long long t_bs, double *xch, unsigned spin_limit,
                                                         unsigned target_extra) {
  extern __shared__ double smem[];
  __shared__ double sbeta[2];
  __shared__ int sfail;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwave = LT / 64;
  // block -> (matrix, member): with the usual round-robin placement of blocks on the 8 XCDs, the
  // members of a matrix share one XCD (and its L2) when the grid is a multiple of 8
  const int nblk = gridDim.x;
  const int L = (nblk & 7) == 0 ? (int)(blockIdx.x & 7) * (nblk >> 3) + (int)(blockIdx.x >> 3) : (int)blockIdx.x;
  const int b = L / P, w = L % P;
  const int nr = (n - w + P - 1) / P, nrmax = (n + P - 1) / P;
  double *rows = smem;                       // [nrmax][n]: local row li is row w + P li
  double *sv = rows + (long long)nrmax * n;  // v_j at sv + (j & 1) n (absolute columns)
  double *sp = sv + 2 * n;                   // p_{j-1}
  double *pout = sp + n;                     // p_j of the own rows, by local index
  const double *Ab = A + b * a_bs;
  double *d = d_out + b * t_bs, *e = e_out + b * t_bs, *R = refl + b * t_bs * (long long)n, *be = beta + b * t_bs;
  double *X = xch + b * mwg_doubles(n);
  unsigned *cnt = (unsigned *)X;  // [0] exchanges completed (P per step), [1] error word
  const long long ldx = mwg_ldx(n);
  double *XS = X + MWG_HDR;  // slot s: p at XS + 2 s ldx, row at XS + (2 s + 1) ldx
  auto own_first = [&](int i0) { return i0 <= w ? 0 : (i0 - w + P - 1) / P; };

  if (tid == 0) sfail = 0;
  for (long long q = tid; q < (long long)nr * n; q += LT) {
    const int li = (int)(q / n), c = (int)(q % n);
    rows[q] = Ab[(long long)(w + P * li) * lda + c];
  }
  // step 0: reflector 0 from row 0 of A (every workgroup; d/e/beta by the owner of row 0)
  if (wave == 0) {
    double x[TCH];
#pragma unroll
    for (int t = 0; t < TCH; ++t) {
      const int c = lane + 64 * t;
      x[t] = c < n ? Ab[c] : 0.0;
    }
    const double bt = wave_reflector_regs(x, n, 0, sv, nullptr, n, w == 0 ? d : nullptr, e, be);
    if (lane == 0) sbeta[0] = bt;
  }
  __syncthreads();

  // update j-1 on the own rows i > j (columns > j) and p_j of those rows
  auto sweep = [&](int j, double cprev) {
    const double *vp = sv + ((j + 1) & 1) * n;  // v_{j-1}
    const double *vj = sv + (j & 1) * n;
    const double bj = sbeta[j & 1];
    const int tstart = (j + 1) >> 6;
    for (int l0 = own_first(j + 1) + wave; l0 < nr; l0 += nwave * MR) {
      double vi[MR], wi[MR], s[MR];
#pragma unroll
      for (int q = 0; q < MR; ++q) {
        const int li = min(l0 + q * nwave, nr - 1), i = w + P * li;
        vi[q] = j >= 1 ? vp[i] : 0.0;
        wi[q] = j >= 1 ? sp[i] - cprev * vp[i] : 0.0;
        s[q] = 0.0;
      }
#pragma unroll
      for (int t = 0; t < TCH; ++t)
        if (t >= tstart) {
          const int c = lane + 64 * t;
          if (c > j && c < n) {
            const double vc = j >= 1 ? vp[c] : 0.0, wc = j >= 1 ? sp[c] - cprev * vc : 0.0, xc = vj[c];
            double a[MR];
#pragma unroll
            for (int q = 0; q < MR; ++q)
              if (l0 + q * nwave < nr) a[q] = rows[(long long)(l0 + q * nwave) * n + c];
#pragma unroll
            for (int q = 0; q < MR; ++q)
              if (l0 + q * nwave < nr) {
                double u = a[q];
                if (j >= 1) {
                  u = a[q] - (vi[q] * wc + wi[q] * vc);
                  rows[(long long)(l0 + q * nwave) * n + c] = u;
                }
                s[q] += u * xc;
              }
          }
        }
#pragma unroll
      for (int q = 0; q < MR; ++q)
        if (l0 + q * nwave < nr) {
          const double sq = warp_sum_d(s[q]);
          if (lane == 0) pout[l0 + q * nwave] = bj * sq;
        }
    }
  };
  // p_j of the own rows and (from its owner) row j+1 into slot j & 1; once those stores have
  // completed, count the step
  auto publish = [&](int j) {
    if (wave == 0) {
      double *xp = XS + 2 * (j & 1) * ldx, *xr = xp + ldx;
      for (int li = own_first(j + 1) + lane; li < nr; li += 64) xstore(xp + w + P * li, pout[li]);
      if ((j + 1) % P == w) {
        const double *rr = rows + (long long)((j + 1) / P) * n;
        for (int c = j + 1 + lane; c < n; c += 64) xstore(xr + c, rr[c]);
      }
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(0);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      if (lane == 0) __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  auto wait_all = [&](unsigned target) {
    target += target_extra;
    if (tid == 0 && !sfail) {
      unsigned it = 0;
      while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
        if (++it > spin_limit) {
          sfail = 1;
          __hip_atomic_fetch_or(cnt + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
  };

  sweep(0, 0.0);
  __syncthreads();
  publish(0);
  for (int j = 1; j <= n - 2; ++j) {
    wait_all((unsigned)P * (unsigned)j);
    const double *xp = XS + 2 * ((j - 1) & 1) * ldx, *xr = xp + ldx;
    double x[TCH];
    if (wave == 0) {  // row j, loaded beside p_{j-1}
#pragma unroll
      for (int t = 0; t < TCH; ++t) {
        const int c = j + lane + 64 * t;
        x[t] = c < n ? xload(xr + c) : 0.0;
      }
    }
    for (int c = j + tid; c < n; c += LT) sp[c] = xload(xp + c);
    if (j == 1 && w == 0)  // every workgroup has read row 0 of A
      for (int c = 1 + tid; c < n; c += LT) R[c] = sv[c];
    __syncthreads();
    // c_{j-1} = (beta_{j-1} / 2) p_{j-1} . v_{j-1}, the same in every wave
    const double *vp = sv + ((j - 1) & 1) * n;
    double part = 0.0;
#pragma unroll
    for (int t = 0; t < TCH; ++t) {
      const int c = j + lane + 64 * t;
      if (c < n) part += sp[c] * vp[c];
    }
    const double cprev = 0.5 * sbeta[(j - 1) & 1] * warp_sum_d(part);
    const bool last = (j == n - 2);
    if (wave == 0) {
      const double vr = vp[j], wr = sp[j] - cprev * vp[j];
#pragma unroll
      for (int t = 0; t < TCH; ++t) {
        const int c = j + lane + 64 * t;
        if (c < n) x[t] -= vr * (sp[c] - cprev * vp[c]) + wr * vp[c];
      }
      const bool own = (j % P) == w;
      if (!last) {
        const double bt = wave_reflector_regs(x, n, j, sv + (j & 1) * n, own ? R : nullptr, n, own ? d : nullptr, e, be);
        if (lane == 0) sbeta[j & 1] = bt;
      } else if (own) {
        const double e2 = lane_bcast_d(x[0], 1);  // column n-1 of row n-2
        if (lane == 0) {
          d[n - 2] = x[0];
          e[n - 2] = e2;
          be[n - 2] = 0.0;
        }
      }
    }
    __syncthreads();
    if (!last) {
      sweep(j, cprev);
      __syncthreads();
      publish(j);
    } else if (tid == 0 && (n - 1) % P == w) {
      // row n-1: update n-3 on its diagonal entry
      const int i = n - 1;
      const double vi = vp[i], wi = sp[i] - cprev * vp[i];
      d[i] = rows[(long long)(i / P) * n + i] - (vi * wi + wi * vi);
      e[i] = 0.0;
      be[i] = 0.0;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Inverse iteration for the k largest eigenvalues of the tridiagonal (d, e); one thread per
// eigenvector, rows of Z [k][n] (fp64).  Work arrays interleaved [i][j] for coalescing.
// Then clusters (gap <= 1e-9 ||T||) are re-orthogonalised by two passes of Gram-Schmidt: a computed
// vector is off its eigenvector by about eps ||T|| / gap (backward-stable solves from eigenvalues
// accurate to a few eps ||T||), so vectors farther apart than that are orthogonal to ~1e-7, well
// below the fp32 and 16-bit storage of the factors.
// ---------------------------------------------------------------------------------------------
constexpr int IT = 512;  // threads of the inverse-iteration kernel (one eigenvector each)

// grid (ceil(kmax / 64), batch) of one wave each: thread j of matrix b iterates eigenvector j.
__global__ void __launch_bounds__(64) invit_kernel(const double *d_in, const double *e_in, long long t_bs,
                                                   const double *evals_all, long long ev_bs, const int *k_of,
                                                   const int *n_of, int n_fixed, double *Z, long long z_bs,
                                                   double *work, long long w_bs, int kmax) {
  extern __shared__ double smem[];
  const int b = blockIdx.y;
  const int n = n_of ? n_of[b] : n_fixed;
  const int k = min(k_of[b], n);
  const int tid = threadIdx.x, nt = blockDim.x;
  const double *d = d_in + b * t_bs, *e = e_in + b * t_bs, *ev = evals_all + b * ev_bs;
  double *sd = smem, *se = smem + n;
  for (int i = tid; i < n; i += nt) {
    sd[i] = d[i];
    se[i] = (i + 1 < n) ? e[i] : 0.0;
  }
  __syncthreads();
  double tn = 0.0;
  for (int i = 0; i < n; ++i) tn = fmax(tn, fabs(sd[i]) + fabs(se[i]) + (i ? fabs(se[i - 1]) : 0.0));
  const double tiny = fmax(tn * 1e-15, 1e-300);
  double *Zb = Z + b * z_bs;
  double *wb = work + b * w_bs;
  // work layout: u0, u1, u2 (upper bands), multipliers, two iterate buffers, each [n][kmax];
  // then the pivot flags
  double *U0 = wb, *U1 = wb + (long long)n * kmax, *U2 = wb + 2LL * n * kmax, *Xv = wb + 3LL * n * kmax;
  double *Za = wb + 4LL * n * kmax, *Zb2 = wb + 5LL * n * kmax;
  unsigned char *piv = (unsigned char *)(wb + 6LL * n * kmax);
  for (int j = blockIdx.x * nt + tid; j < k; j += gridDim.x * nt) {
    const double lam = ev[j];
    // factor P (T - lam I) = L U with partial pivoting; L multipliers applied on the fly, so
    // they are stored in U2's slot of the row below only through piv/U arrays.
    // Elimination: rows i (current) and i+1.
    double a = sd[0] - lam, bb = se[0], cc = 0.0;  // row i: [a at col i, bb at i+1, cc at i+2]
    // storage for multipliers: reuse Xv temporarily is not possible (x needed), keep mult in U2 of next row
    for (int i = 0; i < n - 1; ++i) {
      const double sub = se[i];            // T[i+1][i]
      const double nd = sd[i + 1] - lam;   // T[i+1][i+1]
      const double ne = (i + 2 < n) ? se[i + 1] : 0.0;  // T[i+1][i+2]
      if (fabs(a) >= fabs(sub)) {
        // no swap
        double aa = (a == 0.0) ? tiny : a;
        double l = sub / aa;
        U0[(long long)i * kmax + j] = 1.0 / aa;  // reciprocal pivot (the solves multiply)
        U1[(long long)i * kmax + j] = bb;
        U2[(long long)i * kmax + j] = cc;
        piv[(long long)i * kmax + j] = 0;
        Xv[(long long)i * kmax + j] = l;  // multiplier (x is filled later)
        a = nd - l * bb;
        bb = ne - l * cc;
        cc = 0.0;
      } else {
        // swap rows i and i+1
        double l = a / sub;
        U0[(long long)i * kmax + j] = 1.0 / sub;
        U1[(long long)i * kmax + j] = nd;
        U2[(long long)i * kmax + j] = ne;
        piv[(long long)i * kmax + j] = 1;
        Xv[(long long)i * kmax + j] = l;
        double na = bb - l * nd;
        double nb = cc - l * ne;
        a = na;
        bb = nb;
        cc = 0.0;
      }
    }
    U0[(long long)(n - 1) * kmax + j] = 1.0 / ((a == 0.0) ? tiny : a);
    U1[(long long)(n - 1) * kmax + j] = 0.0;
    U2[(long long)(n - 1) * kmax + j] = 0.0;
    // iterate on vectors stored interleaved ([i][kmax], coalesced across threads), alternating
    // between two buffers so that loads never wait on this thread's own stores
    double *__restrict__ za = Za;
    double *__restrict__ zb = Zb2;
    // start vector: deterministic pseudo-random, entries in (0.5, 1.5)
    for (int i = 0; i < n; ++i) {
      uint64_t h = (uint64_t)(i + 1) * 0x9E3779B97F4A7C15ull ^ (uint64_t)(j + 7) * 0xBF58476D1CE4E5B9ull;
      h ^= h >> 31;
      h *= 0x94D049BB133111EBull;
      h ^= h >> 29;
      za[(long long)i * kmax + j] = 0.5 + (double)(h >> 11) * (1.0 / 9007199254740992.0);
    }
    // the iterate is rescaled by 1 / max|z| between iterations through the factor sc applied as
    // it is read (no extra pass over it); the unit 2-norm is taken once, on output
    double sc = 1.0;
    double scale = 0.0;
    for (int iter = 0; iter < 3; ++iter) {
      // apply L^{-1} P: za -> zb (the running entry stays in a register).  The operands of row
      // i + LP are requested as soon as row i has used its slot of a ring of LP (the whole chain is
      // one thread's, so the depth of that ring is what covers a memory round trip); the iterate is
      // scaled by sc where it is used, not where it is loaded, so no load is waited for early.
      double cur = za[j] * sc;
      {
        constexpr int LP = 16;
        double rl[LP], rx[LP];
        unsigned char rp[LP];
        // (rows past the last one are clamped to it: always a valid load, never consumed)
        auto load = [&](int t, int i) __attribute__((always_inline)) {
          const long long r = min(i, n - 2);
          rl[t] = Xv[r * kmax + j];
          rx[t] = za[(r + 1) * kmax + j];
          rp[t] = piv[r * kmax + j];
        };
        if (n >= 2) {
#pragma unroll
          for (int t = 0; t < LP; ++t) load(t, t);
        }
        for (int i0 = 0; i0 < n - 1; i0 += LP) {
#pragma unroll
          for (int t = 0; t < LP; ++t) {
            const int i = i0 + t;
            if (i < n - 1) {
              const double x = rx[t] * sc;
              if (rp[t]) {
                zb[(long long)i * kmax + j] = x;
                cur = cur - rl[t] * x;
              } else {
                zb[(long long)i * kmax + j] = cur;
                cur = x - rl[t] * cur;
              }
            }
            load(t, i + LP);
          }
        }
      }
      zb[(long long)(n - 1) * kmax + j] = cur;
      // back substitution with U (bands u0, u1, u2): zb -> za, the same ring of row operands
      double z1 = 0.0, z2 = 0.0;  // z[i + 1], z[i + 2]
      scale = 0.0;
      {
        constexpr int UP = 12;
        double r0[UP], r1[UP], r2[UP], rz[UP];
        // (rows before the first are clamped to it: always a valid load, never consumed)
        auto load = [&](int t, int i) __attribute__((always_inline)) {
          const long long r = max(i, 0);
          r0[t] = U0[r * kmax + j];
          r1[t] = U1[r * kmax + j];
          r2[t] = U2[r * kmax + j];
          rz[t] = zb[r * kmax + j];
        };
#pragma unroll
        for (int t = 0; t < UP; ++t) load(t, n - 1 - t);
        for (int i0 = n - 1; i0 >= 0; i0 -= UP) {
#pragma unroll
          for (int t = 0; t < UP; ++t) {
            const int i = i0 - t;
            if (i >= 0) {
              double sv = rz[t];
              if (i + 1 < n) sv -= r1[t] * z1;
              if (i + 2 < n) sv -= r2[t] * z2;
              const double zi = sv * r0[t];
              za[(long long)i * kmax + j] = zi;
              scale = fmax(scale, fabs(zi));
              z2 = z1;
              z1 = zi;
            }
            load(t, i - UP);
          }
        }
      }
      sc = (scale > 0.0) ? 1.0 / scale : 1.0;
    }
    // unit 2-norm of sc * z (entries read in groups of 8, all loads of a group in flight)
    constexpr int OG = 8;
    double nrm = 0.0;
    for (int i0 = 0; i0 < n; i0 += OG) {
      double x[OG];
#pragma unroll
      for (int t = 0; t < OG; ++t) x[t] = (i0 + t < n) ? za[(long long)(i0 + t) * kmax + j] * sc : 0.0;
#pragma unroll
      for (int t = 0; t < OG; ++t) nrm += x[t] * x[t];
    }
    const double f = sc / sqrt(nrm);
    double *z = Zb + (long long)j * n;  // output row j
    for (int i0 = 0; i0 < n; i0 += OG) {
      double x[OG];
#pragma unroll
      for (int t = 0; t < OG; ++t) x[t] = (i0 + t < n) ? za[(long long)(i0 + t) * kmax + j] : 0.0;
#pragma unroll
      for (int t = 0; t < OG; ++t)
        if (i0 + t < n) z[i0 + t] = x[t] * f;
    }
  }
}

// Cluster re-orthogonalisation of the inverse-iteration vectors (one workgroup per matrix,
// sequential over vectors, parallel over entries): eigenvalues closer than 1e-9 ||T|| form a
// cluster, whose vectors are orthogonalised in order by two passes of Gram-Schmidt.
__global__ void __launch_bounds__(IT) invit_cluster_kernel(const double *d_in, const double *e_in, long long t_bs,
                                                           const double *evals_all, long long ev_bs, const int *k_of,
                                                           const int *n_of, int n_fixed, double *Z, long long z_bs) {
  __shared__ double red[IT / 64];
  const int b = blockIdx.x;
  const int n = n_of ? n_of[b] : n_fixed;
  const int k = min(k_of[b], n);
  const int tid = threadIdx.x, nt = blockDim.x;
  const double *d = d_in + b * t_bs, *e = e_in + b * t_bs, *ev = evals_all + b * ev_bs;
  double *Zb = Z + b * z_bs;
  double tn = 0.0;
  for (int i = tid; i < n; i += nt) tn = fmax(tn, fabs(d[i]) + (i + 1 < n ? fabs(e[i]) : 0.0) + (i ? fabs(e[i - 1]) : 0.0));
  for (int o = 32; o > 0; o >>= 1) tn = fmax(tn, __shfl_xor(tn, o, 64));
  if ((tid & 63) == 0) red[tid >> 6] = tn;
  __syncthreads();
  tn = 0.0;
  for (int w = 0; w < nt / 64; ++w) tn = fmax(tn, red[w]);
  __syncthreads();
  const double ctol = 1e-9 * fmax(tn, 1e-300);
  // classical Gram-Schmidt, twice, of each clustered vector against the cluster's earlier vectors:
  // per pass all coefficients at once (thread per earlier vector, up to CB at a time), then the
  // update (thread per entry); the tail of a spectrum with a wide dynamic range can form one cluster
  // of hundreds of vectors, which one reduction per earlier vector would serialise
  constexpr int CB = 1024;
  __shared__ double cs[CB];
  for (int j = 1; j < k; ++j) {
    // start of j's cluster, found by every thread (uniform); vectors outside a cluster are final
    // already and need no barrier
    if (fabs(ev[j - 1] - ev[j]) > ctol) continue;
    int s = j;
    while (s > 0 && fabs(ev[s - 1] - ev[s]) <= ctol) --s;
    if (s < j) {
      double *zj = Zb + (long long)j * n;
      for (int pass = 0; pass < 2; ++pass) {
        for (int i0 = s; i0 < j; i0 += CB) {
          const int i1 = min(j, i0 + CB);
          for (int i = i0 + tid; i < i1; i += nt) {
            const double *zi = Zb + (long long)i * n;
            double c = 0.0;
            for (int q = 0; q < n; ++q) c += zi[q] * zj[q];
            cs[i - i0] = c;
          }
          __syncthreads();
          for (int q = tid; q < n; q += nt) {
            double v = zj[q];
            for (int i = i0; i < i1; ++i) v -= cs[i - i0] * Zb[(long long)i * n + q];
            zj[q] = v;
          }
          __syncthreads();
        }
        double part = 0.0;
        for (int q = tid; q < n; q += nt) part += zj[q] * zj[q];
        double nr = block_sum(part, red);
        nr = (nr > 0.0) ? 1.0 / sqrt(nr) : 0.0;
        for (int q = tid; q < n; q += nt) zj[q] *= nr;
        __syncthreads();
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------------
// Back-transformation z <- H_0 H_1 ... H_{n-3} z of eigenvector rows, then sign normalisation
// (largest-magnitude entry positive) and output as fp64 and/or fp32 rows.  Matrices above 576
// take the compact WY blocks of tridiag_blk.hip.
// ---------------------------------------------------------------------------------------------

// Register variant for n <= 64 NC: each wave owns VPW eigenvector rows, lane l holding entries
// l + 64 t, and walks all reflectors on its own (no workgroup barriers): per reflector one dot
// product per row (lane partials, wave sum) and the rank-one update, with the next reflector's
// entries loaded while the current one is applied.
template <int NC, int VPW>
__global__ void __launch_bounds__(256) backtransform_regs_kernel(const double *Zin, long long z_bs, const double *refl,
                                                                 const double *beta, long long t_bs, int n,
                                                                 const int *k_of, double *out64, float *out32,
                                                                 long long out_bs, int out_ld) {
  const int b = blockIdx.y, lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int k = min(k_of[b], n);
  const int q0 = (blockIdx.x * (blockDim.x >> 6) + wave) * VPW;
  if (q0 >= k) return;
  const double *Zb = Zin + b * z_bs;
  const double *Rb = refl + b * t_bs * (long long)n;
  const double *bb = beta + b * t_bs;
  double z[VPW][NC];
#pragma unroll
  for (int q = 0; q < VPW; ++q)
#pragma unroll
    for (int t = 0; t < NC; ++t) {
      const int p = lane + 64 * t;
      z[q][t] = (q0 + q < k && p < n) ? Zb[(long long)(q0 + q) * n + p] : 0.0;
    }
  // reflector kk holds v at absolute columns kk + 1 .. n - 1 of row kk
  auto load_v = [&](int kk, double (&v)[NC]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < NC; ++t) {
      const int p = lane + 64 * t;
      v[t] = (kk >= 0 && p > kk && p < n) ? Rb[(long long)kk * n + p] : 0.0;
    }
  };
  // reflectors and their beta go through a ring of RD slots: reflector kk is requested RD steps
  // before it is applied (one step's work is far shorter than a memory round trip)
  constexpr int RD = 6;
  double vr[RD][NC], br[RD];
  auto load_b = [&](int kk) __attribute__((always_inline)) { return kk >= 0 ? bb[kk] : 0.0; };
#pragma unroll
  for (int u = 0; u < RD; ++u) {
    load_v(n - 3 - u, vr[u]);
    br[u] = load_b(n - 3 - u);
  }
  for (int k0 = n - 3; k0 >= 0; k0 -= RD) {
#pragma unroll
    for (int u = 0; u < RD; ++u) {
      const int kk = k0 - u;
      const double bt = br[u];
      if (kk >= 0 && bt != 0.0) {
#pragma unroll
        for (int q = 0; q < VPW; ++q) {
          double s = 0.0;
#pragma unroll
          for (int t = 0; t < NC; ++t) s += vr[u][t] * z[q][t];
          const double c = bt * warp_sum_d(s);
#pragma unroll
          for (int t = 0; t < NC; ++t) z[q][t] -= c * vr[u][t];
        }
      }
      load_v(kk - RD, vr[u]);
      br[u] = load_b(kk - RD);
    }
  }
  // sign normalisation (largest-magnitude entry positive, first index on ties) and output
#pragma unroll
  for (int q = 0; q < VPW; ++q) {
    if (q0 + q >= k) break;
    double best = -1.0;
    int bi = 0;
#pragma unroll
    for (int t = 0; t < NC; ++t) {
      const int p = lane + 64 * t;
      const double a = fabs(z[q][t]);
      if (p < n && a > best) { best = a; bi = p; }
    }
    for (int o = 32; o > 0; o >>= 1) {
      const double ob = __shfl_xor(best, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
    }
    double val = 0.0;
#pragma unroll
    for (int t = 0; t < NC; ++t)
      if (lane + 64 * t == bi) val = z[q][t];
    val = __shfl(val, bi & 63, 64);
    const double sg = (val < 0.0) ? -1.0 : 1.0;
#pragma unroll
    for (int t = 0; t < NC; ++t) {
      const int p = lane + 64 * t;
      if (p < n) {
        const double x = sg * z[q][t];
        const long long o = b * out_bs + (long long)(q0 + q) * out_ld + p;
        if (out64) out64[o] = x;
        if (out32) out32[o] = (float)x;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Cholesky G = R^T R (R upper, fp64), right-looking in 32-column panels, one workgroup per
// matrix; the inverse R^{-1} follows in tri_inv_kernel (from the diagonal-block inverses that
// chol_diag_kernel leaves), which writes
// RinvT = (R^{-1})^T as fp32 [n][ld_out] and its max |entry| (for the fp16 split of the apply GEMM).  Non-positive pivots are replaced by a tiny
// multiple of the largest diagonal entry (documented regularisation).
// LDS: a 32 x 32 diagonal block and a 32 x (n - k0) panel (n <= 544 keeps the panel in LDS).
// ---------------------------------------------------------------------------------------------
constexpr int CNB = 32;
constexpr int CHOL_MAXN_LDS = 544;
// accumulator of v_mfma_f64_16x16x4 (lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16] and holds
// C rows 4 v + l / 16 of column l % 16)
typedef double td4 __attribute__((ext_vector_type(4)));
constexpr int CT = 1024;

// The Cholesky factorisation G = R^T R split into launches so that the trailing updates, which
// carry almost all of the n^3 / 3 flops, spread over the whole GPU.  Per matrix the scratch holds
// R (n^2, the result), the 32 x 32 diagonal-block inverses used by the triangular inverse, a
// working copy W of the trailing matrix (n^2), the inverse of the current diagonal block and the
// pivot floor.  chol_init copies the upper triangle of G into W and clears R; per 32-column
// panel, chol_diag (one wave per matrix) factors the diagonal block of W into R and inverts it,
// then chol_update (one workgroup per 32 x 32 upper tile of the trailing block of each matrix)
// solves the two panel tiles it needs with that inverse, writes the solved tile of R's row block
// (diagonal tiles only) and subtracts panel^T panel from its tile of W.
__device__ __forceinline__ long long chol_w_off(int n) { return (long long)n * n + (long long)((n + CNB - 1) / CNB) * CNB * CNB; }

__global__ void __launch_bounds__(256) chol_init_kernel(const double *G, long long g_bs, int ldg, int n, double *Rw,
                                                        long long r_bs, float *amax) {
  const int b = blockIdx.y;
  const double *Gb = G + b * g_bs;
  double *R = Rw + b * r_bs, *W = R + chol_w_off(n);
  for (long long idx = blockIdx.x * 256LL + threadIdx.x; idx < (long long)n * n; idx += (long long)gridDim.x * 256) {
    const int i = (int)(idx / n), j = (int)(idx % n);
    W[idx] = (j >= i) ? Gb[(long long)i * ldg + j] : 0.0;
    R[idx] = 0.0;
  }
  if (blockIdx.x == 0 && threadIdx.x < 64) {
    // pivot floor from the diagonal of G
    double dmax = 0.0;
    for (int i = threadIdx.x; i < n; i += 64) dmax = fmax(dmax, Gb[(long long)i * ldg + i]);
    for (int o = 32; o > 0; o >>= 1) dmax = fmax(dmax, __shfl_xor(dmax, o, 64));
    if (threadIdx.x == 0) {
      W[(long long)n * n + CNB * 33] = fmax(dmax * 1e-28, 1e-300);
      amax[b] = 0.f;  // max |R^{-1}| is accumulated by tri_inv_kernel
    }
  }
}

// inverse of the diagonal block of panel k0 for the trailing update, alternating between two
// slots by panel so that a launch can write the next panel's while its blocks read the current one
__device__ __forceinline__ double *chol_dvg(double *W, int n, int k0) {
  return W + (long long)n * n + (((k0 / CNB) & 1) ? CNB * 33 + 8 : 0);
}

// Factor the (updated) diagonal block of panel k0 of W into R and invert it; one wave (lane c
// of the calling wave), Dk [CNB * 33] and Dr [CNB] in the caller's LDS.
__device__ __forceinline__ void chol_diag_block(int n, double *R, double *W, int k0, double *Dk, double *Dr) {
  const int c = threadIdx.x & 63;
  const double floor_piv = W[(long long)n * n + CNB * 33];
  double *Dvg = chol_dvg(W, n, k0);
  const int kb = min(CNB, n - k0);
  // right-looking Cholesky of the diagonal block: lane c holds column c (a[r] = W[r][c], r <= c);
  // row j of the factor is published in LDS and read back by every lane (one wave: LDS order is
  // program order, no barrier).  The pivot chain uses 1/sqrt by the hardware estimate and two
  // Newton steps (each doubles the correct bits; the last leaves an error of an ulp or two), so a
  // column costs a multiply instead of a square root and a division.
  double a[CNB];
#pragma unroll
  for (int r = 0; r < CNB; ++r) a[r] = (c < kb && r <= c && r < kb) ? W[(long long)(k0 + r) * n + k0 + c] : 0.0;
#pragma unroll
  for (int jj = 0; jj < CNB; ++jj) {
    if (jj < kb) {
      const double dj = fmax(lane_bcast_d(a[jj], jj), floor_piv);
      double y = __builtin_amdgcn_rsq(dj);
      const double hd = 0.5 * dj;
      y = y * fma(-hd * y, y, 1.5);
      y = y * fma(-hd * y, y, 1.5);
      if (c == jj) a[jj] = dj * y;
      else if (c > jj) a[jj] *= y;  // R[jj][c]
      if (c == 0) Dr[jj] = y;
      if (c < CNB) Dk[jj * 33 + c] = (c >= jj) ? a[jj] : 0.0;
#pragma unroll
      for (int r = jj + 1; r < CNB; ++r) {
        const double rjr = Dk[jj * 33 + r];  // R[jj][r]
        if (r <= c) a[r] -= rjr * a[jj];
      }
    }
  }
  if (c < kb) {
#pragma unroll
    for (int r = 0; r < CNB; ++r)
      if (r < kb && r <= c) R[(long long)(k0 + r) * n + k0 + c] = a[r];
  }
  // inverse of the diagonal block: lane c solves R_kk x = e_c by back substitution; written for
  // the trailing update (stride 33) and as diagonal block k0 / 32 of the triangular inverse
  double x[CNB];
#pragma unroll
  for (int r = CNB - 1; r >= 0; --r) {
    double v = (r == c) ? 1.0 : 0.0;
#pragma unroll
    for (int q = r + 1; q < CNB; ++q)
      if (q <= c) v -= Dk[r * 33 + q] * x[q];
    x[r] = (r <= c && r < kb && c < kb) ? v * Dr[r] : 0.0;
  }
  if (c < CNB) {
    double *Dv = R + (long long)n * n + (long long)(k0 / CNB) * CNB * CNB;
#pragma unroll
    for (int r = 0; r < CNB; ++r) {
      Dvg[r * 33 + c] = x[r];  // (R_kk^{-1})[r][c]
      Dv[r * CNB + c] = x[r];
    }
  }
}

// the first panel's diagonal block (later ones are factored by the update of the panel before)
__global__ void __launch_bounds__(64) chol_diag_kernel(int n, double *Rw, long long r_bs, int k0) {
  __shared__ double Dk[CNB * 33];
  __shared__ double Dr[CNB];
  double *R = Rw + blockIdx.x * r_bs;
  chol_diag_block(n, R, R + chol_w_off(n), k0, Dk, Dr);
}

// grid (nt * nt, batch), nt = ceil(rem / 32): tile (ti, tj), tj >= ti, of the trailing upper block
__global__ void __launch_bounds__(256) chol_update_kernel(double *Rw, long long r_bs, int n, int k0) {
  __shared__ double Dv[CNB * 33];
  __shared__ double Pi[CNB][33], Pj[CNB][33], Ai[CNB][33], Aj[CNB][33];
  const int kb = min(CNB, n - k0), base = k0 + kb, rem = n - base;
  const int ntl = (rem + 31) / 32;
  const int ti = blockIdx.x / ntl, tj = blockIdx.x % ntl, b = blockIdx.y;
  if (tj < ti) return;
  double *R = Rw + b * r_bs, *W = R + chol_w_off(n);
  const double *Dvg = chol_dvg(W, n, k0);
  const int tid = threadIdx.x;
  for (int e = tid; e < CNB * 33; e += 256) Dv[e] = Dvg[e];
  for (int e = tid; e < CNB * 32; e += 256) {
    const int q = e / 32, x = e % 32;
    const int ci = ti * 32 + x, cj = tj * 32 + x;
    Ai[q][x] = (q < kb && ci < rem) ? W[(long long)(k0 + q) * n + base + ci] : 0.0;
    Aj[q][x] = (q < kb && cj < rem) ? W[(long long)(k0 + q) * n + base + cj] : 0.0;
  }
  __syncthreads();
  // On the fp64 matrix cores, wave w owning output tile (w / 2, w % 2) of 16 x 16:
  // solved panel tiles P[i][x] = sum_{q <= i} (R_kk^{-1})[q][i] A[q][x] (Dv is zero below its diagonal)
  const int wv = tid >> 6, ln = tid & 63, lr = ln & 15, lk = ln >> 4;
  const int ot = (wv >> 1) * 16, ox = (wv & 1) * 16;
  {
    td4 pi = {0.0, 0.0, 0.0, 0.0}, pj = pi;
#pragma unroll
    for (int ks = 0; ks < CNB; ks += 4) {
      const double a = Dv[(ks + lk) * 33 + ot + lr];
      pi = __builtin_amdgcn_mfma_f64_16x16x4f64(a, Ai[ks + lk][ox + lr], pi, 0, 0, 0);
      pj = __builtin_amdgcn_mfma_f64_16x16x4f64(a, Aj[ks + lk][ox + lr], pj, 0, 0, 0);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      Pi[ot + 4 * v + lk][ox + lr] = pi[v];
      Pj[ot + 4 * v + lk][ox + lr] = pj[v];
    }
  }
  __syncthreads();
  if (ti == tj) {  // the solved tile of R's row block
    for (int e = tid; e < CNB * 32; e += 256) {
      const int i = e / 32, x = e % 32, cj = tj * 32 + x;
      if (i < kb && cj < rem) R[(long long)(k0 + i) * n + base + cj] = Pj[i][x];
    }
  }
  // trailing tile -= Pi^T Pj (rows of Pi and Pj past kb are zero)
  {
    td4 u = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int ks = 0; ks < CNB; ks += 4)
      u = __builtin_amdgcn_mfma_f64_16x16x4f64(Pi[ks + lk][ot + lr], Pj[ks + lk][ox + lr], u, 0, 0, 0);
    const int jj = tj * 32 + ox + lr;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int ii = ti * 32 + ot + 4 * v + lk;
      if (ii < rem && jj < rem && jj >= ii) W[(long long)(base + ii) * n + base + jj] -= u[v];
    }
  }
  // the first trailing tile is the next panel's diagonal block, complete now: factor it here
  if (blockIdx.x == 0) {
    __syncthreads();
    if (tid < 64) chol_diag_block(n, R, W, base, &Ai[0][0], &Pi[0][0]);
  }
}

// X = R^{-1} by independent back substitutions over 16-column slabs: workgroup (cb, b) holds
// X[:, 16 cb .. 16 cb + 15] in LDS, starts from the diagonal-block inverse and walks the block
// rows upwards, X_i = -Dinv_i (R[i, >i] X[>i, slab]).  Writes (R^{-1})^T rows as fp32 and folds
// max |entry| into amax[b] (zeroed by the Cholesky kernel).
constexpr int SW = 16;   // slab width
constexpr int TKP = 4;   // k parts of a block row's dot products (8 waves: 2 row tiles x 4 parts)
constexpr int TKS = 32;  // 4-deep k steps whose R entries a lane requests together
__global__ void __launch_bounds__(512) tri_inv_kernel(const double *Rw, long long r_bs, int n, float *RinvT,
                                                      long long o_bs, int ld_out, float *amax) {
  extern __shared__ double sm[];
  __shared__ double Tp[TKP][CNB][SW];
  __shared__ double Ts[CNB][SW];
  __shared__ float fred[8];
  // the longest chains first: block L takes slab ncb - 1 - L / batch of matrix L % batch
  const int ncb = gridDim.x, batch = gridDim.y;
  const int L = blockIdx.x + ncb * blockIdx.y;
  const int cb = ncb - 1 - L / batch, b = L % batch, tid = threadIdx.x;
  const int c0 = cb * SW, cw = min(SW, n - c0);
  const int rd = c0 / CNB, rows = (rd + 1) * CNB;  // slab rows 0 .. rows-1 (zero past n)
  const double *R = Rw + b * r_bs;
  const double *Dinv = R + (long long)n * n;
  double *Xs = sm;  // [rows][SW]
  for (int idx = tid; idx < rows * SW; idx += 512) {
    const int r = idx / SW, c = idx % SW;
    double v = 0.0;
    if (r >= rd * CNB && c < cw) v = Dinv[(long long)rd * CNB * CNB + (r - rd * CNB) * CNB + (c0 - rd * CNB) + c];
    Xs[idx] = v;
  }
  __syncthreads();
  const int q = tid / SW, c = tid % SW;  // 32 x 16 threads: the diagonal-block products
  const int wv = tid >> 6, ln = tid & 63, tile = wv & 1, kp = wv >> 1, lr = ln & 15, lk = ln >> 4;
  for (int i = rd - 1; i >= 0; --i) {
    const int i0 = i * CNB, kbeg = i0 + CNB, kend = min(rows, n);
    // row q of Dinv_i (upper triangular), loaded now for use after the barriers
    const double *Di = Dinv + (long long)i * CNB * CNB + q * CNB;
    double dv[CNB];
#pragma unroll
    for (int p = 0; p < CNB; ++p) dv[p] = Di[p];
    // T = R[i0 .. i0 + 31][kbeg .. kend) X[kbeg .. kend)[slab] on the fp64 matrix cores: wave (tile,
    // kp) takes rows 16 tile .. 16 tile + 15 and the kp-th share of the 4-deep k steps; lane (lr, lk)
    // supplies A = R[row lr][k + lk] and B = X[k + lk][column lr], and holds T rows 4 v + lk of its
    // tile in column lr.  Its R entries for up to TKS steps are requested before the first product.
    const int nk4 = (kend - kbeg + 3) >> 2, per = (nk4 + TKP - 1) / TKP;
    const int sbeg = kp * per, send = min(nk4, sbeg + per);
    const double *Ra = R + (long long)(i0 + 16 * tile + lr) * n;
    td4 acc = {0.0, 0.0, 0.0, 0.0};
    for (int s0 = sbeg; s0 < send; s0 += TKS) {
      double a[TKS];
#pragma unroll
      for (int u = 0; u < TKS; ++u) {
        const int k = kbeg + 4 * (s0 + u) + lk;
        a[u] = (s0 + u < send && k < kend) ? Ra[k] : 0.0;
      }
#pragma unroll
      for (int u = 0; u < TKS; ++u) {
        if (s0 + u < send) {  // (wave-uniform)
          const int k = kbeg + 4 * (s0 + u) + lk;
          const double x = (k < kend) ? Xs[k * SW + lr] : 0.0;
          acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a[u], x, acc, 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) Tp[kp][16 * tile + 4 * v + lk][lr] = acc[v];
    __syncthreads();
    Ts[q][c] = ((Tp[0][q][c] + Tp[1][q][c]) + Tp[2][q][c]) + Tp[3][q][c];  // the parts in fixed order
    __syncthreads();
    double v = 0.0;
#pragma unroll
    for (int p = 0; p < CNB; ++p)
      if (p >= q) v -= dv[p] * Ts[p][c];
    Xs[(i0 + q) * SW + c] = v;
    __syncthreads();
  }
  // output rows c0 .. c0+cw-1 of (R^{-1})^T: RinvT[c0 + c][r] = X[r][c0 + c] (zero below row c0 + c)
  float lmax = 0.f;
  float *O = RinvT + b * o_bs;
  for (int idx = tid; idx < cw * n; idx += 512) {
    const int cc = idx / n, r = idx % n;
    const float v = (r <= c0 + cc) ? (float)Xs[r * SW + cc] : 0.f;
    O[(long long)(c0 + cc) * ld_out + r] = v;
    lmax = fmaxf(lmax, fabsf(v));
  }
  lmax = warp_max(lmax);
  if ((tid & 63) == 0) fred[tid >> 6] = lmax;
  __syncthreads();
  if (tid == 0) {
    float m = 0.f;
    for (int w = 0; w < 8; ++w) m = fmaxf(m, fred[w]);
    atomicMax((unsigned int *)(amax + b), __float_as_uint(m));
  }
}

// H[b] (fp64) = P[b] P[b]^T for fp32 rows P[b] [rows][ldp] (K columns): products of fp32 values
// are exact in fp64, accumulated by the fp64 matrix cores.  One block per 64 x 64 lower tile
// (mirrored into the upper one); each wave owns a 32 x 32 quadrant as 2 x 2 blocks of
// v_mfma_f64_16x16x4 (lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16] and receives
// C[4 v + l / 16][l % 16] in its v-th value).  32-deep slices of both row blocks are staged in LDS.
typedef double d4 __attribute__((ext_vector_type(4)));
__global__ void __launch_bounds__(256) gram64_kernel(const float *P, long long p_bs, int ldp, int rows, int K,
                                                     double *H, long long h_bs, int ldh) {
  constexpr int KT = 32;
  __shared__ float As[64][KT + 1], Bs[64][KT + 1];
  const int b = blockIdx.z;
  const int ti = blockIdx.y, tj = blockIdx.x;
  if (tj > ti) return;
  const int r0 = ti * 64, c0 = tj * 64;
  const float *Pb = P + b * p_bs;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1, rr = lane & 15, kq = lane >> 4;
  d4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = d4{0.0, 0.0, 0.0, 0.0};
  // the next 32-deep slice is loaded into registers (16-byte loads when rows are 16-byte
  // aligned) while the current one is multiplied
  const bool vec = (ldp % 4 == 0) && (K % 4 == 0) && (((uintptr_t)P & 15) == 0);
  float4 ra[2], rb[2];
  auto gload = [&](int k0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = tid + 256 * u, r = e >> 3, k = k0 + 4 * (e & 7);
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f), y = x;
      if (vec) {
        if (r0 + r < rows && k < K) x = *(const float4 *)(Pb + (long long)(r0 + r) * ldp + k);
        if (c0 + r < rows && k < K) y = *(const float4 *)(Pb + (long long)(c0 + r) * ldp + k);
      } else {
        float xa[4], ya[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          xa[j] = (r0 + r < rows && k + j < K) ? Pb[(long long)(r0 + r) * ldp + k + j] : 0.f;
          ya[j] = (c0 + r < rows && k + j < K) ? Pb[(long long)(c0 + r) * ldp + k + j] : 0.f;
        }
        x = make_float4(xa[0], xa[1], xa[2], xa[3]);
        y = make_float4(ya[0], ya[1], ya[2], ya[3]);
      }
      ra[u] = x;
      rb[u] = y;
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = tid + 256 * u, r = e >> 3, k = 4 * (e & 7);
      As[r][k] = ra[u].x; As[r][k + 1] = ra[u].y; As[r][k + 2] = ra[u].z; As[r][k + 3] = ra[u].w;
      Bs[r][k] = rb[u].x; Bs[r][k + 1] = rb[u].y; Bs[r][k + 2] = rb[u].z; Bs[r][k + 3] = rb[u].w;
    }
  };
  gload(0);
  for (int k0 = 0; k0 < K; k0 += KT) {
    lstore();
    __syncthreads();
    if (k0 + KT < K) gload(k0 + KT);
#pragma unroll
    for (int ks = 0; ks < KT; ks += 4) {
      double a[2], bb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = (double)As[wr * 32 + i * 16 + rr][ks + kq];
#pragma unroll
      for (int j = 0; j < 2; ++j) bb[j] = (double)Bs[wc * 32 + j * 16 + rr][ks + kq];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], bb[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
  double *Hb = H + b * h_bs;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = r0 + wr * 32 + i * 16 + 4 * v + kq, c = c0 + wc * 32 + j * 16 + rr;
        if (r < rows && c < rows && c <= r) {
          Hb[(long long)r * ldh + c] = acc[i][j][v];
          Hb[(long long)c * ldh + r] = acc[i][j][v];
        }
      }
}

}  // namespace

// allow the large dynamic LDS allocations of the one-workgroup kernels (gfx950: 160 KiB per CU)
void ensure_lds_attrs() {
  static bool done = false;
  if (done) return;
  int dev = 0, maxsh = 65536;
  HIP_TRY(hipGetDevice(&dev));
  if (hipDeviceGetAttribute(&maxsh, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) maxsh = 65536;
  const int want = maxsh - 2048;  // leave room for the kernels' static LDS
  // best effort: the runtime may already allow the full amount
  (void)hipFuncSetAttribute((const void *)tri_inv_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, want);
  (void)hipFuncSetAttribute((const void *)tridiag_values_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, want);
  (void)hipFuncSetAttribute((const void *)tridiag_fused_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize, want);
  (void)hipFuncSetAttribute((const void *)tridiag_fused_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize, want);
  (void)hipFuncSetAttribute((const void *)tridiag_mwg_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, want);
  (void)hipFuncSetAttribute((const void *)bisect_kernel<4>, hipFuncAttributeMaxDynamicSharedMemorySize, want);
  (void)hipFuncSetAttribute((const void *)bisect_kernel<16>, hipFuncAttributeMaxDynamicSharedMemorySize, want);
  (void)hipGetLastError();
  done = true;
}

size_t tridiag_lds_bytes(int n) { return ((size_t)n * n + 2 * (size_t)n) * sizeof(double); }

size_t tridiag_mwg_bytes(int n, int batch) {
  if (n > 64 * TCH && tridiag_blocked_fits(n)) return (size_t)batch * (size_t)tridiag_blocked_doubles(n) * sizeof(double);
  return (size_t)batch * (size_t)mwg_doubles(n) * sizeof(double);
}

namespace {

// Members per matrix for tridiag_mwg_kernel (the fewest whose rows fit in LDS) and the matrices
// per launch, so that every workgroup of a launch can be resident at once (its waits need that).
bool mwg_plan(int n, int batch, int &P, int &chunk, size_t &shm) {
  if (n > 64 * TCH) return false;
  int dev = 0, cus = 0, maxsh = 0;
  HIP_TRY(hipGetDevice(&dev));
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipDeviceGetAttribute(&maxsh, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  for (int p = 2; p <= 32; p *= 2) {
    const long long nrm = (n + p - 1) / p;
    const size_t bytes = (size_t)((nrm + 3) * n + nrm) * sizeof(double);
    if (bytes + 2048 > (size_t)maxsh) continue;
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, (const void *)tridiag_mwg_kernel, LT, bytes) != hipSuccess) {
      (void)hipGetLastError();
      return false;
    }
    const long long cap = (long long)cus * occ;
    if (occ < 1 || cap < p) return false;
    P = p;
    chunk = (int)std::min<long long>(batch, cap / p);
    shm = bytes;
    return true;
  }
  return false;
}

}  // namespace

void sym_eigvals(double *A, long long a_bs, int lda, int n, int batch, double *d, double *e, double *refl,
                 double *beta, long long t_bs, double *evals, long long ev_bs, bool clamp, hipStream_t st,
                 double *mwg) {
  JOLT_REQUIRE(n >= 1 && n <= 8192, JOLT_EINVAL, "eigensolver: unsupported size");
  JOLT_REQUIRE(t_bs == n, JOLT_EINVAL, "eigensolver: tridiagonal stride must equal n");
  size_t lds_full = tridiag_lds_bytes(n);
  const size_t lds_cap = 150 * 1024;
  ensure_lds_attrs();
  int P = 0, chunk = 0;
  size_t shm_m = 0;
  const bool blocked = lds_full > lds_cap && mwg != nullptr && n > 64 * TCH && tridiag_blocked_fits(n);
  const bool multi = !blocked && lds_full > lds_cap && mwg != nullptr && mwg_plan(n, batch, P, chunk, shm_m);
  if (lds_full <= lds_cap) {
    hipLaunchKernelGGL(tridiag_values_kernel, dim3(batch), dim3(LT), lds_full, st, A, a_bs, lda, (const int *)nullptr,
                       n, d, e, refl, beta, t_bs, evals, ev_bs, clamp ? 1 : 0, 1);
  } else if (blocked) {
    tridiag_blocked(A, a_bs, lda, n, batch, d, e, refl, beta, t_bs, mwg, st);
  } else if (multi) {
    const long long ms = mwg_doubles(n);
    const WaitPolicy wp = wait_policy();
    hipLaunchKernelGGL(mwg_reset_kernel, dim3((batch + 255) / 256), dim3(256), 0, st, mwg, ms, batch);
    HIP_LAUNCH_CHECK();
    for (int b0 = 0; b0 < batch; b0 += chunk) {
      const int nm = std::min(chunk, batch - b0);
      // cooperative launch: the runtime starts it only if every workgroup of the grid can be resident at
      // once (the per-step exchange waits on all of a matrix's workgroups); if it refuses, the chunk
      // takes the one-workgroup-per-matrix reduction (same reflectors up to rounding order)
      const double *a_ = A + b0 * a_bs;
      double *d_ = d + b0 * t_bs, *e_ = e + b0 * t_bs, *r_ = refl + b0 * t_bs * (long long)n, *be_ = beta + b0 * t_bs;
      double *x_ = mwg + b0 * ms;
      long long a_bs_ = a_bs, t_bs_ = t_bs;
      int lda_ = lda, n_ = n, P_ = P;
      unsigned sl_ = wp.spin_limit, te_ = wp.target_extra;
      void *args[] = {&a_, &a_bs_, &lda_, &n_, &P_, &d_, &e_, &r_, &be_, &t_bs_, &x_, &sl_, &te_};
      if (hipLaunchCooperativeKernel((const void *)tridiag_mwg_kernel, dim3(nm * P), dim3(LT), args, (unsigned)shm_m,
                                     st) == hipSuccess)
        continue;
      (void)hipGetLastError();
      const size_t shm_up = (5 * (size_t)n + 64 * TCH * (LT / 64)) * sizeof(double);
      JOLT_REQUIRE(shm_up <= 150 * 1024, JOLT_EHIP, "eigensolver: cooperative launch refused, no fallback fits");
      hipLaunchKernelGGL(tridiag_fused_kernel<true>, dim3(nm), dim3(LT), shm_up, st, A + b0 * a_bs, a_bs, lda, n, d_, e_,
                         r_, be_, t_bs, evals + b0 * ev_bs, ev_bs, clamp ? 1 : 0);
      HIP_LAUNCH_CHECK();
    }
  } else {
    const size_t shm_up = (5 * (size_t)n + 64 * TCH * (LT / 64)) * sizeof(double);
    if (n <= 64 * TCH && shm_up <= 150 * 1024) {
      hipLaunchKernelGGL(tridiag_fused_kernel<true>, dim3(batch), dim3(LT), shm_up, st, A, a_bs, lda, n, d, e, refl,
                         beta, t_bs, evals, ev_bs, clamp ? 1 : 0);
    } else {
      const size_t shm = 4 * (size_t)n * sizeof(double);
      JOLT_REQUIRE(shm <= 150 * 1024, JOLT_EINVAL, "eigensolver: n too large for LDS staging");
      hipLaunchKernelGGL(tridiag_fused_kernel<false>, dim3(batch), dim3(LT), shm, st, A, a_bs, lda, n, d, e, refl,
                         beta, t_bs, evals, ev_bs, clamp ? 1 : 0);
    }
  }
  HIP_LAUNCH_CHECK();
  // eigenvalues of the tridiagonals: BL lanes per eigenvalue, 256 / BL eigenvalues per block
  const size_t bshm = 2 * (size_t)n * sizeof(double);
  JOLT_REQUIRE(bshm <= 150 * 1024, JOLT_EINVAL, "eigensolver: n too large for the bisection");
  const unsigned *errw = multi ? (const unsigned *)mwg + 1 : nullptr;
  const long long err_bs = multi ? 2 * mwg_doubles(n) : 0LL;
  if ((long long)n * batch >= 4096) {
    dim3 bgrid((unsigned)(((long long)n * 4 + 255) / 256), batch);
    hipLaunchKernelGGL(bisect_kernel<4>, bgrid, dim3(256), bshm, st, d, e, t_bs, n, evals, ev_bs, clamp ? 1 : 0, errw,
                       err_bs);
  } else {
    dim3 bgrid((unsigned)(((long long)n * 16 + 255) / 256), batch);
    hipLaunchKernelGGL(bisect_kernel<16>, bgrid, dim3(256), bshm, st, d, e, t_bs, n, evals, ev_bs, clamp ? 1 : 0, errw,
                       err_bs);
  }
  HIP_LAUNCH_CHECK();
}

// (also the T factors of the WY back-transformation, which runs after inverse iteration)
size_t invit_work_doubles(int n, int kmax) {
  const size_t w = 6ull * n * kmax + ((size_t)n * kmax + 7) / 8 + 8;
  return n > 64 * 9 ? std::max<size_t>(w, (size_t)wy_tfactor_doubles(n)) : w;
}

void sym_eigvecs(const double *d, const double *e, const double *refl, const double *beta, long long t_bs,
                 const double *evals, long long ev_bs, int n, const int *k_dev, int kmax, int batch, double *Zw,
                 long long z_bs, double *work, long long w_bs, double *out64, float *out32, long long out_bs,
                 int out_ld, hipStream_t st) {
  if (kmax <= 0) return;
  hipLaunchKernelGGL(invit_kernel, dim3((kmax + 63) / 64, batch), dim3(64), 2 * (size_t)n * sizeof(double), st, d, e,
                     t_bs, evals, ev_bs, k_dev, (const int *)nullptr, n, Zw, z_bs, work, w_bs, kmax);
  HIP_LAUNCH_CHECK();
  hipLaunchKernelGGL(invit_cluster_kernel, dim3(batch), dim3(IT), 0, st, d, e, t_bs, evals, ev_bs, k_dev,
                     (const int *)nullptr, n, Zw, z_bs);
  HIP_LAUNCH_CHECK();
  if (n <= 64 * 9) {
    // register variant: 4 rows per wave, 4 waves per workgroup
    constexpr int VPW = 4;
    dim3 g2((kmax + 4 * VPW - 1) / (4 * VPW), batch);
    if (n <= 128)
      hipLaunchKernelGGL((backtransform_regs_kernel<2, VPW>), g2, dim3(256), 0, st, Zw, z_bs, refl, beta, t_bs, n, k_dev,
                         out64, out32, out_bs, out_ld);
    else if (n <= 256)
      hipLaunchKernelGGL((backtransform_regs_kernel<4, VPW>), g2, dim3(256), 0, st, Zw, z_bs, refl, beta, t_bs, n, k_dev,
                         out64, out32, out_bs, out_ld);
    else
      hipLaunchKernelGGL((backtransform_regs_kernel<9, VPW>), g2, dim3(256), 0, st, Zw, z_bs, refl, beta, t_bs, n, k_dev,
                         out64, out32, out_bs, out_ld);
    HIP_LAUNCH_CHECK();
    return;
  }
  // larger matrices: reflectors in compact WY blocks (the work array is free again after the
  // inverse iteration and holds the blocks' T factors)
  backtransform_wy(Zw, z_bs, refl, beta, t_bs, n, k_dev, kmax, batch, work, w_bs, out64, out32, out_bs, out_ld, st);
}

long long chol_scratch_doubles(int n) {
  return 2LL * n * n + (long long)((n + CNB - 1) / CNB) * CNB * CNB + 2 * CNB * 33 + 8;
}

void chol_inv(const double *G, long long g_bs, int ldg, int n, int batch, double *Rw, long long r_bs, float *RinvT,
              long long o_bs, int ld_out, float *amax, hipStream_t st) {
  JOLT_REQUIRE(n >= 1 && n <= CHOL_MAXN_LDS, JOLT_EINVAL, "Cholesky QR: panel width above 544 is not supported");
  JOLT_REQUIRE(r_bs >= chol_scratch_doubles(n), JOLT_EINVAL, "Cholesky QR: scratch too small per matrix");
  ensure_lds_attrs();
  {
    const long long nn = (long long)n * n;
    hipLaunchKernelGGL(chol_init_kernel, dim3((unsigned)std::min<long long>((nn + 255) / 256, 1024), batch), dim3(256),
                       0, st, G, g_bs, ldg, n, Rw, r_bs, amax);
    HIP_LAUNCH_CHECK();
    hipLaunchKernelGGL(chol_diag_kernel, dim3(batch), dim3(64), 0, st, n, Rw, r_bs, 0);
    HIP_LAUNCH_CHECK();
    for (int k0 = 0; k0 < n; k0 += CNB) {
      const int rem = n - k0 - std::min(CNB, n - k0);
      if (rem <= 0) break;
      const int ntl = (rem + 31) / 32;
      hipLaunchKernelGGL(chol_update_kernel, dim3(ntl * ntl, batch), dim3(256), 0, st, Rw, r_bs, n, k0);
      HIP_LAUNCH_CHECK();
    }
  }
  const int nblk = (n + CNB - 1) / CNB;  // the diagonal-block inverses were written by chol_diag_kernel
  const int ncb = (n + SW - 1) / SW;
  const size_t tshm = (size_t)nblk * CNB * SW * sizeof(double);
  hipLaunchKernelGGL(tri_inv_kernel, dim3(ncb, batch), dim3(512), tshm, st, Rw, r_bs, n, RinvT, o_bs, ld_out, amax);
  HIP_LAUNCH_CHECK();
}

void gram64(const float *P, long long p_bs, int ldp, int rows, int K, double *H, long long h_bs, int ldh, int batch,
            hipStream_t st) {
  int t = (rows + 63) / 64;
  hipLaunchKernelGGL(gram64_kernel, dim3(t, t, batch), dim3(256), 0, st, P, p_bs, ldp, rows, K, H, h_bs, ldh);
  HIP_LAUNCH_CHECK();
}

}  // namespace jolt
