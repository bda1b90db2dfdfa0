// Small device kernels around the main passes: the FlashJoLT Gaussian test matrix, fills,
// norms and spectra assembly (Sec. 3.1 tail entry), factor rounding into the blob, headers.
#include <math.h>

#include "common.hpp"
#include "misc.hpp"

namespace jolt {

namespace {

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ull;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBull;
  z ^= z >> 31;
  return z;
}
__device__ __forceinline__ double unif(uint64_t w) { return ((double)(w >> 11) + 0.5) * (1.0 / 9007199254740992.0); }

// Omega^T[c][m] = gaussian element (m * ell + c) of the sketch stream (SplitMix64 + Box-Muller),
// rounded to the cache dtype.
__global__ void omega_kernel(void *out, int dtype, int M, int ell, uint64_t key) {
  const long long n = (long long)M * ell;
  for (long long e = blockIdx.x * (long long)blockDim.x + threadIdx.x; e < n; e += (long long)gridDim.x * blockDim.x) {
    const uint64_t k = (uint64_t)e >> 1;
    const double u1 = unif(mix64(key + (2 * k + 1) * 0x9E3779B97F4A7C15ull));
    const double u2 = unif(mix64(key + (2 * k + 2) * 0x9E3779B97F4A7C15ull));
    const double r = sqrt(-2.0 * log(u1));
    const double th = 2.0 * M_PI * u2;
    const double g = (e & 1) ? r * sin(th) : r * cos(th);
    const int m = (int)(e / ell), c = (int)(e % ell);
    const long long o = (long long)c * M + m;
    if (dtype == JOLT_F32) ((float *)out)[o] = (float)g;
    else {
      // one round-to-nearest-even of the fp64 value to 11 (fp16) or 8 (bf16) significant bits
      const int mant = (dtype == JOLT_F16) ? 10 : 7, emin = (dtype == JOLT_F16) ? -14 : -126;
      int ex;
      (void)frexp(g == 0.0 ? 1.0 : g, &ex);
      const int eb = max(ex - 1, emin);
      const double q = ldexp(1.0, eb - mant);
      const double rv = rint(g / q) * q;  // exactly representable in the target format
      if (dtype == JOLT_F16) ((_Float16 *)out)[o] = (_Float16)(float)rv;
      else ((uint16_t *)out)[o] = (uint16_t)(__float_as_uint((float)rv) >> 16);
    }
  }
}

// Cross products of the token bases of consecutive layers: block (l, s) forms the k x k matrix
// S = U_l U_{l+1}^T of sequence s, U_l the first k rows of length T of layer l's key cell (cells
// ordered (sequence, layer, K|V), rows at stride ld, cell stride cs); products summed in fp64.
template <int K>
__global__ void __launch_bounds__(256) pair_cross_kernel(const float *U, long long cs, int ld, int T, int L, double *S) {
  __shared__ double red[4][K * K];
  const int l = blockIdx.x, sq = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float *a = U + (long long)(2 * (sq * L + l)) * cs;
  const float *b = a + 2 * cs;
  double acc[K * K];
#pragma unroll
  for (int i = 0; i < K * K; ++i) acc[i] = 0.0;
  for (int t = tid; t < T; t += 256) {
    double x[K], y[K];
#pragma unroll
    for (int i = 0; i < K; ++i) {
      x[i] = a[(long long)i * ld + t];
      y[i] = b[(long long)i * ld + t];
    }
#pragma unroll
    for (int i = 0; i < K; ++i)
#pragma unroll
      for (int j = 0; j < K; ++j) acc[i * K + j] += x[i] * y[j];
  }
#pragma unroll
  for (int i = 0; i < K * K; ++i) {
    double v = acc[i];
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    if (lane == 0) red[w][i] = v;
  }
  __syncthreads();
  if (tid < K * K) S[((long long)sq * (L - 1) + l) * K * K + tid] = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
}

__global__ void fill_f32_kernel(float *p, long long n, float v) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x) p[i] = v;
}
__global__ void fill_f64_kernel(double *p, long long n, double v) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x) p[i] = v;
}

__global__ void trace_kernel(const double *G, long long g_bs, int n, double *out) {
  if (threadIdx.x != 0) return;
  const double *g = G + blockIdx.x * g_bs;
  double s = 0.0;
  for (int i = 0; i < n; ++i) s += g[(long long)i * n + i];
  out[blockIdx.x] = s;
}

__global__ void flash_spec_kernel(const double *evals, long long ev_bs, int q, const double *norm2, double *specT,
                                  long long sp_bs) {
  const double *ev = evals + blockIdx.x * ev_bs;
  double *sp = specT + blockIdx.x * sp_bs;
  for (int i = threadIdx.x; i < q; i += blockDim.x) sp[i] = ev[i];
  if (threadIdx.x == 0) {
    double s = 0.0;
    for (int i = 0; i < q; ++i) s += ev[i];
    sp[q] = fmax(0.0, norm2[blockIdx.x] - s);
  }
}

template <int S>
__device__ __forceinline__ float round_to(float v) {
  if constexpr (S == SRC_F32) return v;
  else if constexpr (S == SRC_F16) return f16_to_f32(f32_to_f16_rne(v));
  else return bf16_to_f32(f32_to_bf16_rne(v));
}

// U_T (blob, [T][rT] storage dtype) from rows UTt[r][t] (fp32), 32 x 32 LDS transpose.
template <int S>
__global__ void put_ut_kernel(const FactorCell *cells, const float *UTt, long long ut_bs, int ld_in, int T) {
  __shared__ float tile[32][33];
  const FactorCell c = cells[blockIdx.z];
  const int r0 = blockIdx.y * 32, t0 = blockIdx.x * 32;
  if (r0 >= c.rT) return;
  const float *in = UTt + blockIdx.z * ut_bs;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int yy = ty; yy < 32; yy += 8) {
    int r = r0 + yy, t = t0 + tx;
    tile[yy][tx] = (r < c.rT && t < T) ? in[(long long)r * ld_in + t] : 0.f;
  }
  __syncthreads();
  for (int yy = ty; yy < 32; yy += 8) {
    int t = t0 + yy, r = r0 + tx;
    if (t < T && r < c.rT) store_elem<S>(c.UT, (long long)t * c.rT + r, tile[tx][yy]);
  }
}

// U_d [D][rd] and core [GH][rT][rd] into the blob (rounded), plus their rounded fp32 copies
// Udr[kk][d] and Cr[j][r][kk] (uniform strides, zero beyond the ranks).
template <int S>
__global__ void put_small_kernel(const FactorCell *cells, const float *Udrows, long long ud_bs, const float *Cp,
                                 long long cp_bs, int kmax, int kmax_d, int D, int GH, float *Udr, float *Cr) {
  const int cell = blockIdx.y;
  const FactorCell c = cells[cell];
  const float *ud = Udrows + cell * ud_bs;
  const float *cp = Cp + cell * cp_bs;
  float *udr = Udr + (long long)cell * kmax_d * D;
  float *cr = Cr + (long long)cell * GH * kmax * kmax_d;
  const long long n1 = (long long)D * c.rd;
  const long long n2 = (long long)GH * c.rT * c.rd;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n1 + n2; i += (long long)gridDim.x * blockDim.x) {
    if (i < n1) {
      int d = (int)(i / c.rd), kk = (int)(i % c.rd);
      float v = round_to<S>(ud[(long long)kk * D + d]);
      store_elem<S>(c.Ud, i, v);
      udr[(long long)kk * D + d] = v;
    } else {
      long long q = i - n1;
      int j = (int)(q / ((long long)c.rT * c.rd));
      int r = (int)((q / c.rd) % c.rT), kk = (int)(q % c.rd);
      float v = round_to<S>(cp[((long long)r * GH + j) * kmax_d + kk]);
      store_elem<S>(c.core, q, v);
      cr[((long long)j * kmax + r) * kmax_d + kk] = v;
    }
  }
}

// blob -> Udr / Cr (reconstruct side)
template <int S>
__global__ void get_small_kernel(const FactorCell *cells, int kmax, int kmax_d, int D, int GH, float *Udr, float *Cr) {
  const int cell = blockIdx.y;
  const FactorCell c = cells[cell];
  float *udr = Udr + (long long)cell * kmax_d * D;
  float *cr = Cr + (long long)cell * GH * kmax * kmax_d;
  const long long n1 = (long long)D * c.rd;
  const long long n2 = (long long)GH * c.rT * c.rd;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n1 + n2; i += (long long)gridDim.x * blockDim.x) {
    if (i < n1) {
      int d = (int)(i / c.rd), kk = (int)(i % c.rd);
      udr[(long long)kk * D + d] = load_elem<S>(c.Ud, i);
    } else {
      long long q = i - n1;
      int j = (int)(q / ((long long)c.rT * c.rd));
      int r = (int)((q / c.rd) % c.rT), kk = (int)(q % c.rd);
      cr[((long long)j * kmax + r) * kmax_d + kk] = load_elem<S>(c.core, q);
    }
  }
}

__global__ void headers_kernel(const FactorCell *cells, int ncells) {
  const int cell = blockIdx.x;
  if (cell >= ncells) return;
  const FactorCell c = cells[cell];
  // zero the alignment padding after every part of the section (at most 255 bytes each)
  for (int r = 0; r < 5; ++r) {
    uint8_t *p = (uint8_t *)c.pad_ptr[r];
    for (int i = threadIdx.x; i < c.pad_len[r]; i += blockDim.x) p[i] = 0;
  }
  if (threadIdx.x < 64) {
    uint32_t *h = (uint32_t *)c.header;
    h[threadIdx.x] = threadIdx.x < 10 ? c.hdr[threadIdx.x] : 0u;  // 256-byte header
  }
}

// Bcat[cell][j][n][k] = Qt[n][k] for k < D
__global__ void bcat_q_kernel(float *Bcat, int ncells, int GH, int D, int Kb, const float *Qt) {
  const long long per = (long long)GH * D * D;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < per * ncells; i += (long long)gridDim.x * blockDim.x) {
    long long cell = i / per, q = i % per;
    int j = (int)(q / (D * D)), n = (int)((q / D) % D), k = (int)(q % D);
    Bcat[((cell * GH + j) * D + n) * Kb + k] = Qt[(long long)n * D + k];
  }
}

// max |x| of each cell: 16-byte loads where the cell is aligned, one atomic per workgroup (the
// per-wave atomics of a wide grid all hit the same word and serialise in L2)
__global__ void __launch_bounds__(256) amax_kernel(const float *x, long long per, long long bs, float *out) {
  __shared__ float red[4];
  const int cell = blockIdx.y;
  const float *p = x + cell * bs;
  const long long stride = (long long)gridDim.x * 256, i0 = blockIdx.x * 256LL + threadIdx.x;
  float m = 0.f;
  long long tail = 0;
  if ((((uintptr_t)p) & 15) == 0) {
    const long long n4 = per / 4;
    const float4 *p4 = (const float4 *)p;
    for (long long i = i0; i < n4; i += stride) {
      const float4 v = p4[i];
      m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
    tail = n4 * 4;
  }
  for (long long i = tail + i0; i < per; i += stride) m = fmaxf(m, fabsf(p[i]));
  m = warp_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0)
    atomicMax((unsigned int *)(out + cell), __float_as_uint(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]))));
}

int grid_for(long long n) { return (int)std::max<long long>(1, std::min<long long>((n + 255) / 256, 8192)); }

}  // namespace

void gen_omega(void *out, int dtype, int M, int ell, uint64_t key, hipStream_t st) {
  long long n = (long long)M * ell;
  hipLaunchKernelGGL(omega_kernel, dim3(grid_for(n)), dim3(256), 0, st, out, dtype, M, ell, key);
  HIP_LAUNCH_CHECK();
}
void pair_cross(const float *U, long long cell_stride, int ld, int T, int k, int L, int n_seq, double *S,
                hipStream_t st) {
  JOLT_REQUIRE(k == 8, JOLT_EINVAL, "layer grouping: 8 token vectors per layer");
  if (L < 2) return;
  hipLaunchKernelGGL((pair_cross_kernel<8>), dim3(L - 1, n_seq), dim3(256), 0, st, U, cell_stride, ld, T, L, S);
  HIP_LAUNCH_CHECK();
}

void fill_f32(float *p, long long n, float v, hipStream_t st) {
  if (n <= 0) return;
  hipLaunchKernelGGL(fill_f32_kernel, dim3(grid_for(n)), dim3(256), 0, st, p, n, v);
  HIP_LAUNCH_CHECK();
}
void fill_f64(double *p, long long n, double v, hipStream_t st) {
  if (n <= 0) return;
  hipLaunchKernelGGL(fill_f64_kernel, dim3(grid_for(n)), dim3(256), 0, st, p, n, v);
  HIP_LAUNCH_CHECK();
}
void trace_f64(const double *G, long long g_bs, int n, int batch, double *out, hipStream_t st) {
  hipLaunchKernelGGL(trace_kernel, dim3(batch), dim3(64), 0, st, G, g_bs, n, out);
  HIP_LAUNCH_CHECK();
}
void flash_spec(const double *evals, long long ev_bs, int q, const double *norm2, double *specT, long long sp_bs,
                int batch, hipStream_t st) {
  hipLaunchKernelGGL(flash_spec_kernel, dim3(batch), dim3(256), 0, st, evals, ev_bs, q, norm2, specT, sp_bs);
  HIP_LAUNCH_CHECK();
}
void put_ut(int dtype, const FactorCell *cells, int ncells, const float *UTt, long long ut_bs, int ld_in, int T,
            int kmax, hipStream_t st) {
  dim3 grid((T + 31) / 32, (kmax + 31) / 32, ncells);
  if (dtype == JOLT_F16) hipLaunchKernelGGL(put_ut_kernel<SRC_F16>, grid, dim3(256), 0, st, cells, UTt, ut_bs, ld_in, T);
  else if (dtype == JOLT_BF16) hipLaunchKernelGGL(put_ut_kernel<SRC_BF16>, grid, dim3(256), 0, st, cells, UTt, ut_bs, ld_in, T);
  else hipLaunchKernelGGL(put_ut_kernel<SRC_F32>, grid, dim3(256), 0, st, cells, UTt, ut_bs, ld_in, T);
  HIP_LAUNCH_CHECK();
}
void put_small(int dtype, const FactorCell *cells, int ncells, const float *Udrows, long long ud_bs, const float *Cp,
               long long cp_bs, int kmax, int kmax_d, int D, int GH, float *Udr, float *Cr, hipStream_t st) {
  dim3 grid(256, ncells);
  if (dtype == JOLT_F16) hipLaunchKernelGGL(put_small_kernel<SRC_F16>, grid, dim3(256), 0, st, cells, Udrows, ud_bs, Cp, cp_bs, kmax, kmax_d, D, GH, Udr, Cr);
  else if (dtype == JOLT_BF16) hipLaunchKernelGGL(put_small_kernel<SRC_BF16>, grid, dim3(256), 0, st, cells, Udrows, ud_bs, Cp, cp_bs, kmax, kmax_d, D, GH, Udr, Cr);
  else hipLaunchKernelGGL(put_small_kernel<SRC_F32>, grid, dim3(256), 0, st, cells, Udrows, ud_bs, Cp, cp_bs, kmax, kmax_d, D, GH, Udr, Cr);
  HIP_LAUNCH_CHECK();
}
void get_small(int dtype, const FactorCell *cells, int ncells, int kmax, int kmax_d, int D, int GH, float *Udr,
               float *Cr, hipStream_t st) {
  dim3 grid(256, ncells);
  if (dtype == JOLT_F16) hipLaunchKernelGGL(get_small_kernel<SRC_F16>, grid, dim3(256), 0, st, cells, kmax, kmax_d, D, GH, Udr, Cr);
  else if (dtype == JOLT_BF16) hipLaunchKernelGGL(get_small_kernel<SRC_BF16>, grid, dim3(256), 0, st, cells, kmax, kmax_d, D, GH, Udr, Cr);
  else hipLaunchKernelGGL(get_small_kernel<SRC_F32>, grid, dim3(256), 0, st, cells, kmax, kmax_d, D, GH, Udr, Cr);
  HIP_LAUNCH_CHECK();
}
void write_headers(const FactorCell *cells, int ncells, hipStream_t st) {
  hipLaunchKernelGGL(headers_kernel, dim3(ncells), dim3(256), 0, st, cells, ncells);
  HIP_LAUNCH_CHECK();
}
void bcat_q(float *Bcat, int ncells, int GH, int D, int Kb, const float *Qt, hipStream_t st) {
  long long n = (long long)ncells * GH * D * D;
  hipLaunchKernelGGL(bcat_q_kernel, dim3(grid_for(n)), dim3(256), 0, st, Bcat, ncells, GH, D, Kb, Qt);
  HIP_LAUNCH_CHECK();
}
namespace {
struct RopeArgs {
  float inv[64];
  int H2;
  long long n;
};
__global__ void rope_table_kernel(RopeArgs r, float *out) {
  for (long long e = blockIdx.x * (long long)blockDim.x + threadIdx.x; e < r.n; e += (long long)gridDim.x * blockDim.x) {
    const long long p = e / r.H2;
    const int i = (int)(e - p * r.H2);
    const float a = __fmul_rn((float)p, r.inv[i]);
    float sn, cs;
    sincosf(a, &sn, &cs);
    out[2 * e] = cs;
    out[2 * e + 1] = sn;
  }
}
}  // namespace

void rope_table(const float *inv, int H2, int n_pos, float *out, hipStream_t st) {
  JOLT_REQUIRE(H2 >= 1 && H2 <= 64 && n_pos >= 0, JOLT_EINVAL, "rope table: bad shape");
  RopeArgs r;
  for (int i = 0; i < H2; ++i) r.inv[i] = inv[i];
  r.H2 = H2;
  r.n = (long long)n_pos * H2;
  if (r.n == 0) return;
  hipLaunchKernelGGL(rope_table_kernel, dim3(grid_for(r.n)), dim3(256), 0, st, r, out);
  HIP_LAUNCH_CHECK();
}

void amax_cells(const float *x, long long per, long long bs, int ncells, float *out, hipStream_t st) {
  fill_f32(out, ncells, 0.f, st);
  int g = (int)std::min<long long>((per + 4095) / 4096, 128);  // about 16 elements per thread, at most 128 groups per cell
  hipLaunchKernelGGL(amax_kernel, dim3(std::max(g, 1), ncells), dim3(256), 0, st, x, per, bs, out);
  HIP_LAUNCH_CHECK();
}

}  // namespace jolt
