// Householder tridiagonalisation of symmetric fp64 matrices too large for the LDS- and
// register-resident reductions of linalg.hip (the exact token Gram of long prefills: T x T with T
// in the thousands).  Same reflectors and output format as those (Golub & Van Loan, "Matrix
// Computations", Sec. 8.3.1): d, e, beta per matrix, reflector k stored in row k (v_k[k + 1] = 1
// implicit), and the same formulas for the reflector of a row.
//
// Blocked over panels of kPanel reflectors with the two-sided update deferred to the end of each
// panel (the panel form of Dongarra, Sorensen & Hammarling, "Block reduction of matrices to
// condensed forms", 1989): within a panel the working matrix is the stored one minus
// sum_i (v_i w_i^T + w_i v_i^T) over the panel's earlier steps, applied to the vectors that need
// it, and the stored matrix (upper triangle only) takes the whole panel at once.  Per reflector:
//   symv   many workgroups: partial products of the stored upper triangle with v, in 128 x 128
//          tiles (row sums and column sums into one slot per tile pair, so that every sum is
//          taken in a fixed order), plus the dots of v with the panel's vectors;
//   step   one workgroup per matrix: p = beta (A v - panel terms), w = p - (beta/2)(p.v) v, the
//          next row of the working matrix and its reflector;
//   update at the end of a panel, the rank-2 kPanel update of the stored upper triangle.
// The matrix streams from HBM once per reflector (half of it: the upper triangle) instead of twice,
// and each launch spreads it over the whole GPU.
#include <math.h>

#include "common.hpp"
#include "linalg.hpp"

namespace jolt {

namespace {

constexpr int kPanel = 32;   // reflectors per deferred update
constexpr int kTS = 128;     // symv tile side
constexpr int kStepT = 1024; // threads of the per-matrix step

struct TbArgs {
  double *A;           // [batch] symmetric n x n, row pitch lda (upper triangle kept current)
  long long a_bs;
  int lda, n, nt;      // nt: symv tiles per side
  double *refl;        // [batch][n][n]: row k = reflector k (may be A itself when lda == n)
  double *d, *e, *beta;
  long long t_bs;
  double *scr;         // per matrix s_bs doubles: Vp [2][kPanel][n], Wp [2][kPanel][n],
  long long s_bs;      //   part [nt][nt][kTS], dpart [nt][2 kPanel]
};

__device__ __forceinline__ double *vpan(const TbArgs &a, int b, int P, int i) {
  return a.scr + b * a.s_bs + ((long long)P * kPanel + i) * a.n;
}
__device__ __forceinline__ double *wpan(const TbArgs &a, int b, int P, int i) {
  return a.scr + b * a.s_bs + ((long long)(2 + P) * kPanel + i) * a.n;
}
__device__ __forceinline__ double *slot(const TbArgs &a, int b, int X, int S) {
  return a.scr + b * a.s_bs + 4LL * kPanel * a.n + ((long long)X * a.nt + S) * kTS;
}
__device__ __forceinline__ double *dslot(const TbArgs &a, int b, int t) {
  return a.scr + b * a.s_bs + 4LL * kPanel * a.n + (long long)a.nt * a.nt * kTS + (long long)t * 2 * kPanel;
}
// p = beta_j A_cur v_j and the panel-corrected row r (both [n]), then one partial p . v per step-A block
constexpr int kStepA = 256;
__device__ __forceinline__ double *pvec(const TbArgs &a, int b) {
  return a.scr + b * a.s_bs + 4LL * kPanel * a.n + (long long)a.nt * a.nt * kTS + (long long)a.nt * 2 * kPanel;
}
__device__ __forceinline__ double *xvec(const TbArgs &a, int b) { return pvec(a, b) + a.n; }
__device__ __forceinline__ double *pdots(const TbArgs &a, int b) { return pvec(a, b) + 2LL * a.n; }

// tile (I, J), I <= J, of the upper triangle of an m x m tile grid, row-major
__device__ __forceinline__ void upper_tile(int q, int m, int &I, int &J) {
  int i = 0;
  while (q >= m - i) {
    q -= m - i;
    ++i;
  }
  I = i;
  J = i + q;
}

__device__ double bsum(double v, double *red) {
  v = warp_sum_d(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  double s = 0.0;
  for (int i = 0; i < nw; ++i) s += red[i];
  return s;
}

// Partial products of the stored upper triangle (rows and columns >= r + 1) with v_r: tile (I, J)
// writes its row sums to slot (I, J) and its column sums to slot (J, I); a diagonal tile writes
// both, added, to (I, I).  Diagonal tiles also form their share of the dots of v_r with the
// earlier vectors of its panel (W_i, then V_i).
__global__ void __launch_bounds__(256) tb_symv_kernel(TbArgs a, int r) {
  const int b = blockIdx.y, n = a.n, s = r + 1;
  const int t0 = s / kTS;
  int I, J;
  upper_tile(blockIdx.x, a.nt - t0, I, J);
  I += t0;
  J += t0;
  const bool diag = I == J;
  const int R0 = I * kTS, C0 = J * kTS;
  const int P = (r / kPanel) & 1, c = r % kPanel;
  const double *v = vpan(a, b, P, c);
  const double *Ab = a.A + b * a.a_bs;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ double cs[4][kTS];
  __shared__ double rsum[kTS];
  const int col0 = C0 + lane, col1 = C0 + 64 + lane;
  const bool ok0 = col0 >= s && col0 < n, ok1 = col1 >= s && col1 < n;
  const double vc0 = ok0 ? v[col0] : 0.0, vc1 = ok1 ? v[col1] : 0.0;
  const int cl0 = min(col0, n - 1), cl1 = min(col1, n - 1);
  double ca0 = 0.0, ca1 = 0.0;
  // wave w: rows R0 + 32 w .. + 31, eight rows' loads in flight at a time
  for (int k0 = 0; k0 < 32; k0 += 8) {
    double a0[8], a1[8], vr[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int row = R0 + wave * 32 + k0 + u;
      const bool rv = row >= s && row < n;
      vr[u] = rv ? v[row] : 0.0;
      const double *rp = Ab + (long long)min(row, n - 1) * a.lda;
      a0[u] = (rv && ok0 && (!diag || col0 >= row)) ? rp[cl0] : 0.0;
      a1[u] = (rv && ok1 && (!diag || col1 >= row)) ? rp[cl1] : 0.0;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int row = R0 + wave * 32 + k0 + u;
      const double rs = warp_sum_d(a0[u] * vc0 + a1[u] * vc1);
      if (lane == 0) rsum[row - R0] = rs;
      if (!diag || col0 > row) ca0 += a0[u] * vr[u];
      if (!diag || col1 > row) ca1 += a1[u] * vr[u];
    }
  }
  cs[wave][lane] = ca0;
  cs[wave][64 + lane] = ca1;
  __syncthreads();
  if (tid < kTS) {
    const double col = cs[0][tid] + cs[1][tid] + cs[2][tid] + cs[3][tid];
    if (diag) {
      slot(a, b, I, I)[tid] = rsum[tid] + col;
    } else {
      slot(a, b, I, J)[tid] = rsum[tid];
      slot(a, b, J, I)[tid] = col;
    }
  }
  if (diag && c > 0) {
    // dots over this tile's rows [R0, R0 + 128) intersected with [s, n); entry q < c is W_q . v,
    // entry kPanel + q is V_q . v
    for (int q = wave; q < 2 * c; q += 4) {
      const double *u = q < c ? wpan(a, b, P, q) : vpan(a, b, P, q - c);
      const double x0 = ok0 ? u[col0] : 0.0, x1 = ok1 ? u[col1] : 0.0;
      const double dsum = warp_sum_d(x0 * vc0 + x1 * vc1);
      if (lane == 0) dslot(a, b, I)[q < c ? q : kPanel + q - c] = dsum;
    }
  }
}

// Step A, many workgroups per matrix (j >= 0): for the entries x >= j + 1 of block blockIdx.x,
// p = beta_j (A_cur v_j) with A_cur the stored matrix minus the panel's earlier rank-2 terms (the symv
// slots summed in a fixed order, the panel terms from the dots of the diagonal tiles), the panel-
// corrected row r = j + 1 of the working matrix (without step j's own term), and this block's part
// of p . v_j.
__global__ void __launch_bounds__(kStepA) tb_stepA_kernel(TbArgs a, int j) {
  __shared__ double red[kStepA / 64];
  __shared__ double coef[4 * kPanel];  // W_i . v, V_i . v, V_i[r], W_i[r]
  const int b = blockIdx.y, n = a.n, tid = threadIdx.x, r = j + 1, s = r;
  const int x0 = blockIdx.x * kStepA;
  if (x0 + kStepA <= s) return;  // uniform: the block lies before the support
  const int P = (j / kPanel) & 1, c = j % kPanel, t0 = s / kTS;
  const double *vj = vpan(a, b, P, c);
  if (tid < 2 * c) {
    const int q = tid < c ? tid : kPanel + tid - c;
    double sum = 0.0;
    for (int t = t0; t < a.nt; ++t) sum += dslot(a, b, t)[q];
    coef[q] = sum;
  } else if (tid >= 64 && tid < 64 + c) {
    coef[2 * kPanel + tid - 64] = vpan(a, b, P, tid - 64)[r];
    coef[3 * kPanel + tid - 64] = wpan(a, b, P, tid - 64)[r];
  }
  __syncthreads();
  const double bj = a.beta[b * a.t_bs + j];
  const int xx = x0 + tid;
  double pd = 0.0;
  if (xx >= s && xx < n) {
    const int X = xx / kTS, xo = xx % kTS;
    double y = 0.0;
    for (int S = t0; S < a.nt; ++S) y += slot(a, b, X, S)[xo];
    double pc = 0.0, xc = 0.0;
    for (int i = 0; i < c; ++i) {
      const double Vi = vpan(a, b, P, i)[xx], Wi = wpan(a, b, P, i)[xx];
      pc += Vi * coef[i] + Wi * coef[kPanel + i];
      xc += coef[2 * kPanel + i] * Wi + coef[3 * kPanel + i] * Vi;
    }
    const double p = bj * (y - pc);
    pvec(a, b)[xx] = p;
    xvec(a, b)[xx] = a.A[b * a.a_bs + (long long)r * a.lda + xx] - xc;
    pd = p * vj[xx];
  }
  pd = bsum(pd, red);
  if (tid == 0) pdots(a, b)[blockIdx.x] = pd;
}

// Step B, one workgroup per matrix.  j >= 0: w_j = p - (beta_j / 2)(p . v_j) v_j (the partial dots
// summed in block order), then row r = j + 1 of the working matrix gets step j's own term and yields
// its reflector, or for r = n - 2 the last 2 x 2 block.  j = -1: the reflector of row 0.
__global__ void __launch_bounds__(kStepT) tb_step_kernel(TbArgs a, int j) {
  extern __shared__ double sm[];
  __shared__ double red[kStepT / 64];
  __shared__ double cj_s;
  const int b = blockIdx.x, n = a.n, tid = threadIdx.x;
  double *d = a.d + b * a.t_bs, *e = a.e + b * a.t_bs, *be = a.beta + b * a.t_bs;
  const double *Ab = a.A + b * a.a_bs;
  double *v = sm, *w = sm + n, *x = sm + 2 * n;
  const int r = j + 1;
  int P = 0, c = 0;
  if (j >= 0) {
    P = (j / kPanel) & 1;
    c = j % kPanel;
    const int s = r;
    const double *vj = vpan(a, b, P, c);
    if (tid == 0) {
      const double *pdb = pdots(a, b);
      double sum = 0.0;
      for (int q = s / kStepA; q < (n + kStepA - 1) / kStepA; ++q) sum += pdb[q];
      cj_s = 0.5 * be[j] * sum;
    }
    __syncthreads();
    const double cj = cj_s;
    const double *pv = pvec(a, b), *xv = xvec(a, b);
    double *wj = wpan(a, b, P, c);
    for (int xx = s + tid; xx < n; xx += kStepT) {
      const double vx = vj[xx], wx = pv[xx] - cj * vx;
      v[xx] = vx;
      w[xx] = wx;
      wj[xx] = wx;
    }
    __syncthreads();
    const double vr = v[r], wr = w[r];
    for (int m = r + tid; m < n; m += kStepT) x[m] = xv[m] - (vr * w[m] + wr * v[m]);
    __syncthreads();
  } else {
    for (int m = tid; m < n; m += kStepT) x[m] = Ab[m];
    __syncthreads();
  }
  if (r <= n - 3) {
    double ps = 0.0;
    for (int m = r + 2 + tid; m < n; m += kStepT) ps += x[m] * x[m];
    const double sigma = bsum(ps, red);
    const double alpha = x[r + 1], dr = x[r];
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
    double *vn = vpan(a, b, (r / kPanel) & 1, r % kPanel);
    double *R = a.refl + b * a.t_bs * (long long)n + (long long)r * n;  // may be row r of A: read above
    for (int m = r + 1 + tid; m < n; m += kStepT) {
      const double vm = (m == r + 1) ? 1.0 : x[m] / v0;
      vn[m] = vm;
      R[m] = vm;
    }
    if (tid == 0) {
      d[r] = dr;
      e[r] = (sigma == 0.0) ? alpha : mu;
      be[r] = bet;
    }
  } else if (tid == 0) {
    d[n - 2] = x[n - 2];
    e[n - 2] = x[n - 1];
    be[n - 2] = 0.0;
    double dl = Ab[(long long)(n - 1) * a.lda + (n - 1)];
    if (j >= 0) {
      for (int i = 0; i < c; ++i) dl -= 2.0 * vpan(a, b, P, i)[n - 1] * wpan(a, b, P, i)[n - 1];
      dl -= 2.0 * v[n - 1] * w[n - 1];
    }
    d[n - 1] = dl;
    e[n - 1] = 0.0;
    be[n - 1] = 0.0;
  }
}

// Stored upper triangle, rows and columns >= r + 1: A -= sum_i (V_i W_i^T + W_i V_i^T) over the
// kPanel steps of panel P.  128 x 128 tiles, 8 x 8 outputs per thread (rows 8 ty .. 8 ty + 7, columns
// tx + 16 q: a row's loads and stores coalesce), the panel's vectors staged through LDS 16 at a time.
constexpr int kTU = 128, kUK = 16;
__global__ void __launch_bounds__(256) tb_update_kernel(TbArgs a, int r, int P) {
  const int b = blockIdx.y, n = a.n, s = r + 1;
  const int nu = (n + kTU - 1) / kTU, t0 = s / kTU;
  int I, J;
  upper_tile(blockIdx.x, nu - t0, I, J);
  I += t0;
  J += t0;
  const int R0 = I * kTU, C0 = J * kTU, tid = threadIdx.x;
  __shared__ double Va[kUK][kTU], Wa[kUK][kTU], Vb[kUK][kTU], Wb[kUK][kTU];
  const int ty = tid >> 4, tx = tid & 15;
  double acc[8][8];
#pragma unroll
  for (int u = 0; u < 8; ++u)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[u][q] = 0.0;
  for (int i0 = 0; i0 < kPanel; i0 += kUK) {
    __syncthreads();
    for (int idx = tid; idx < kUK * kTU; idx += 256) {
      const int i = idx / kTU, o = idx % kTU;
      const int ra = R0 + o, cb = C0 + o;
      const bool oa = ra >= s && ra < n, ob = cb >= s && cb < n;
      Va[i][o] = oa ? vpan(a, b, P, i0 + i)[ra] : 0.0;
      Wa[i][o] = oa ? wpan(a, b, P, i0 + i)[ra] : 0.0;
      Vb[i][o] = ob ? vpan(a, b, P, i0 + i)[cb] : 0.0;
      Wb[i][o] = ob ? wpan(a, b, P, i0 + i)[cb] : 0.0;
    }
    __syncthreads();
    for (int i = 0; i < kUK; ++i) {
      double av[8], aw[8], bv[8], bw[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        av[u] = Va[i][ty * 8 + u];
        aw[u] = Wa[i][ty * 8 + u];
        bv[u] = Vb[i][tx + 16 * u];
        bw[u] = Wb[i][tx + 16 * u];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[u][q] += av[u] * bw[q] + aw[u] * bv[q];
    }
  }
  double *Ab = a.A + b * a.a_bs;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int row = R0 + ty * 8 + u;
    if (row < s || row >= n) continue;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int col = C0 + tx + 16 * q;
      if (col < n && col >= row) Ab[(long long)row * a.lda + col] -= acc[u][q];
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Back-transformation z <- H_0 H_1 ... H_{n-3} z of eigenvector rows for large n, kWB reflectors at
// a time as compact WY products (Schreiber & Van Loan, "A storage-efficient WY representation for
// products of Householder transformations", 1989): H_k0 ... H_{k0+kWB-1} = I - V T V^T with T upper
// triangular.  Blocks are applied last to first, each as W = T (V^T Z) and Z -= V W over the rows
// > k0; a workgroup owns kWQ vectors through all blocks, so workgroups never exchange data.
constexpr int kWB = 32, kWQ = 64, kXC = 64;

// T of every block: S = V^T V over the block's rows, then T[i][i] = beta_i and
// T[0:i, i] = -beta_i T[0:i, 0:i] S[0:i, i] (reflectors past n - 3 are zero: beta 0).
__global__ void __launch_bounds__(256) wy_tfactor_kernel(const double *refl, const double *beta, long long t_bs, int n,
                                                         double *Tf, long long tf_bs) {
  const int kb = blockIdx.x, b = blockIdx.y, k0 = kb * kWB, tid = threadIdx.x, nr = n - 2;
  const double *R = refl + b * t_bs * (long long)n;
  const double *be = beta + b * t_bs;
  __shared__ double Vs[kWB][kXC + 1];
  __shared__ double S[kWB][kWB + 1];
  __shared__ double T[kWB][kWB + 1];
  const int i = tid >> 3, l0 = (tid & 7) * 4;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  for (int xb = k0 + 1; xb < n; xb += kXC) {
    __syncthreads();
    for (int idx = tid; idx < kWB * kXC; idx += 256) {
      const int r = idx / kXC, xx = idx % kXC, x = xb + xx, kk = k0 + r;
      Vs[r][xx] = (kk < nr && x >= kk + 1 && x < n) ? R[(long long)kk * n + x] : 0.0;
    }
    __syncthreads();
    for (int xx = 0; xx < kXC; ++xx) {
      const double a = Vs[i][xx];
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[u] += a * Vs[l0 + u][xx];
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) S[i][l0 + u] = acc[u];
  __syncthreads();
  if (tid < kWB) {
    // lane j forms row j of T column by column (its own earlier entries only)
    const int j = tid;
    for (int c = 0; c < kWB; ++c) {
      const double bc = (k0 + c < nr) ? be[k0 + c] : 0.0;
      double t = 0.0;
      if (j == c) {
        t = bc;
      } else if (j < c) {
        double sum = 0.0;
        for (int l = j; l < c; ++l) sum += T[j][l] * S[l][c];
        t = -bc * sum;
      }
      T[j][c] = t;
    }
  }
  __syncthreads();
  double *To = Tf + b * tf_bs + (long long)kb * kWB * kWB;
  for (int idx = tid; idx < kWB * kWB; idx += 256) To[idx] = T[idx / kWB][idx % kWB];
}

__global__ void __launch_bounds__(256) wy_apply_kernel(double *Z, long long z_bs, const double *refl, long long t_bs,
                                                       int n, const int *k_of, const double *Tf, long long tf_bs,
                                                       double *out64, float *out32, long long out_bs, int out_ld) {
  const int b = blockIdx.y, q0 = blockIdx.x * kWQ, tid = threadIdx.x;
  const int k = min(k_of[b], n);
  if (q0 >= k) return;
  const int nq = min(kWQ, k - q0), nr = n - 2, nblk = (nr + kWB - 1) / kWB;
  double *Zb = Z + b * z_bs + (long long)q0 * n;  // the workgroup's vectors, row q at q n
  const double *R = refl + b * t_bs * (long long)n;
  __shared__ double Vs[kWB][kXC + 1];
  __shared__ double Zs[kWQ][kXC + 1];
  __shared__ double Ws[kWB][kWQ + 1];
  __shared__ double Ts[kWB][kWB + 1];
  const int lane = tid & 63, wave = tid >> 6;
  for (int kb = nblk - 1; kb >= 0; --kb) {
    const int k0 = kb * kWB, x0 = k0 + 1;
    const double *Tb = Tf + b * tf_bs + (long long)kb * kWB * kWB;
    for (int idx = tid; idx < kWB * kWB; idx += 256) Ts[idx / kWB][idx % kWB] = Tb[idx];
    // W = V^T Z: two halves of each chunk's rows, 4 reflectors x 4 vectors per thread
    const int h = tid >> 7, ig = (tid & 127) >> 4, qg = tid & 15;
    double acc[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[u][v] = 0.0;
    for (int xb = x0; xb < n; xb += kXC) {
      __syncthreads();
      for (int idx = tid; idx < kWB * kXC; idx += 256) {
        const int r = idx / kXC, xx = idx % kXC, x = xb + xx, kk = k0 + r;
        Vs[r][xx] = (kk < nr && x >= kk + 1 && x < n) ? R[(long long)kk * n + x] : 0.0;
      }
      for (int idx = tid; idx < kWQ * kXC; idx += 256) {
        const int q = idx / kXC, xx = idx % kXC, x = xb + xx;
        Zs[q][xx] = (q < nq && x < n) ? Zb[(long long)q * n + x] : 0.0;
      }
      __syncthreads();
      for (int xx = h * (kXC / 2); xx < (h + 1) * (kXC / 2); ++xx) {
        double a[4], c[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          a[u] = Vs[ig * 4 + u][xx];
          c[u] = Zs[qg + 16 * u][xx];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[u][v] += a[u] * c[v];
      }
    }
    __syncthreads();
    if (h == 1) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) Ws[ig * 4 + u][qg + 16 * v] = acc[u][v];
    }
    __syncthreads();
    if (h == 0) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) Ws[ig * 4 + u][qg + 16 * v] += acc[u][v];
    }
    __syncthreads();
    // W <- T W (T upper triangular)
    {
      const int i = tid >> 3, g = tid & 7;
      double w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) w[u] = 0.0;
      for (int l = i; l < kWB; ++l) {
        const double t = Ts[i][l];
#pragma unroll
        for (int u = 0; u < 8; ++u) w[u] += t * Ws[l][g + 8 * u];
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < 8; ++u) Ws[i][g + 8 * u] = w[u];
      __syncthreads();
    }
    // Z -= V W over rows x >= x0: lane = row within a chunk, wave = 16 vectors
    for (int xb = x0; xb < n; xb += kXC) {
      const int x = xb + lane;
      double vv[kWB];
#pragma unroll
      for (int r = 0; r < kWB; ++r) {
        const int kk = k0 + r;
        vv[r] = (kk < nr && x >= kk + 1 && x < n) ? R[(long long)kk * n + min(x, n - 1)] : 0.0;
      }
      if (x < n) {
        for (int u = 0; u < 16; ++u) {
          const int q = wave * 16 + u;
          if (q >= nq) break;
          double z = Zb[(long long)q * n + x];
#pragma unroll
          for (int r = 0; r < kWB; ++r) z -= vv[r] * Ws[r][q];
          Zb[(long long)q * n + x] = z;
        }
      }
    }
    __syncthreads();
  }
  // sign normalisation (largest-magnitude entry positive, first index on ties) and output
  for (int q = wave; q < nq; q += 4) {
    const double *zq = Zb + (long long)q * n;
    double best = -1.0;
    int bi = 0;
    for (int i = lane; i < n; i += 64) {
      const double a = fabs(zq[i]);
      if (a > best) {
        best = a;
        bi = i;
      }
    }
    for (int o = 32; o > 0; o >>= 1) {
      const double ob = __shfl_xor(best, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ob > best || (ob == best && oi < bi)) {
        best = ob;
        bi = oi;
      }
    }
    const double sg = (zq[bi] < 0.0) ? -1.0 : 1.0;
    for (int i = lane; i < n; i += 64) {
      const double x = sg * zq[i];
      const long long o = b * out_bs + (long long)(q0 + q) * out_ld + i;
      if (out64) out64[o] = x;
      if (out32) out32[o] = (float)x;
    }
  }
}

}  // namespace

long long wy_tfactor_doubles(int n) { return (long long)((n - 2 + kWB - 1) / kWB) * kWB * kWB; }

void backtransform_wy(double *Zw, long long z_bs, const double *refl, const double *beta, long long t_bs, int n,
                      const int *k_dev, int kmax, int batch, double *Tf, long long tf_bs, double *out64, float *out32,
                      long long out_bs, int out_ld, hipStream_t st) {
  JOLT_REQUIRE(n >= 3 && t_bs == n && tf_bs >= wy_tfactor_doubles(n), JOLT_EINVAL, "WY back-transform: bad layout");
  const int nblk = (n - 2 + kWB - 1) / kWB;
  hipLaunchKernelGGL(wy_tfactor_kernel, dim3(nblk, batch), dim3(256), 0, st, refl, beta, t_bs, n, Tf, tf_bs);
  HIP_LAUNCH_CHECK();
  hipLaunchKernelGGL(wy_apply_kernel, dim3((kmax + kWQ - 1) / kWQ, batch), dim3(256), 0, st, Zw, z_bs, refl, t_bs, n,
                     k_dev, (const double *)Tf, tf_bs, out64, out32, out_bs, out_ld);
  HIP_LAUNCH_CHECK();
}

long long tridiag_blocked_doubles(int n) {
  const long long nt = (n + kTS - 1) / kTS;
  const long long raw = 4LL * kPanel * n + nt * nt * kTS + nt * 2 * kPanel + 2LL * n + (n + kStepA - 1) / kStepA;
  return (raw + 31) / 32 * 32;
}

bool tridiag_blocked_fits(int n) { return n >= 3 && 3 * (size_t)n * sizeof(double) <= 150 * 1024; }

void tridiag_blocked(double *A, long long a_bs, int lda, int n, int batch, double *d, double *e, double *refl,
                     double *beta, long long t_bs, double *scr, hipStream_t st) {
  JOLT_REQUIRE(tridiag_blocked_fits(n), JOLT_EINVAL, "blocked tridiagonalisation: unsupported size");
  JOLT_REQUIRE(lda >= n && t_bs == n && scr != nullptr, JOLT_EINVAL, "blocked tridiagonalisation: bad layout");
  static bool attr = false;
  const size_t shm = 3 * (size_t)n * sizeof(double);
  if (!attr) {
    (void)hipFuncSetAttribute((const void *)tb_step_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, 150 * 1024);
    (void)hipGetLastError();
    attr = true;
  }
  TbArgs a;
  a.A = A;
  a.a_bs = a_bs;
  a.lda = lda;
  a.n = n;
  a.nt = (n + kTS - 1) / kTS;
  a.refl = refl;
  a.d = d;
  a.e = e;
  a.beta = beta;
  a.t_bs = t_bs;
  a.scr = scr;
  a.s_bs = tridiag_blocked_doubles(n);
  const int nu = (n + kTU - 1) / kTU;
  hipLaunchKernelGGL(tb_step_kernel, dim3(batch), dim3(kStepT), shm, st, a, -1);
  HIP_LAUNCH_CHECK();
  for (int r = 0; r + 2 < n; ++r) {
    if (r > 0 && r % kPanel == 0) {
      const int m = nu - (r + 1) / kTU;
      hipLaunchKernelGGL(tb_update_kernel, dim3(m * (m + 1) / 2, batch), dim3(256), 0, st, a, r,
                         ((r - 1) / kPanel) & 1);
      HIP_LAUNCH_CHECK();
    }
    const int m = a.nt - (r + 1) / kTS;
    hipLaunchKernelGGL(tb_symv_kernel, dim3(m * (m + 1) / 2, batch), dim3(256), 0, st, a, r);
    HIP_LAUNCH_CHECK();
    hipLaunchKernelGGL(tb_stepA_kernel, dim3((n + kStepA - 1) / kStepA, batch), dim3(kStepA), 0, st, a, r);
    HIP_LAUNCH_CHECK();
    hipLaunchKernelGGL(tb_step_kernel, dim3(batch), dim3(kStepT), shm, st, a, r);
    HIP_LAUNCH_CHECK();
  }
}

}  // namespace jolt
