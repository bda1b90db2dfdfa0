// Dense contractions on gfx950 matrix cores (v_mfma_f32_16x16x32_{f16,bf16}).
//
// Every GEMM of the compressor (sketch, power-iteration and projection products against the
// cache, Gram matrices, triangular applies of the thin QR) runs through this kernel.  The
// cache enters at its own 16-bit precision (exact).  fp32 operands are split exactly into
// 16-bit planes inside the LDS store (fp16: hi + lo after a power-of-two scale, 22 bits;
// bf16: three planes, 24 bits) and the cross products that matter are accumulated in fp32,
// which keeps fp32-class accuracy at matrix-core rates.
//
// Tile 128 x 128 x 32, 256 threads (4 waves in 2 x 2, each 64 x 64 = 4 x 4 MFMA tiles).
// LDS holds every plane of the A and B tiles as [row][k] with k contiguous (row pitch 40
// halves).  Sources contiguous along M or N are transposed while being stored.
// Block ids are remapped so that tiles sharing an operand panel run on the same XCD.
#include "common.hpp"
#include "gemm_core.hpp"

namespace jolt {

namespace {

using namespace core;

// Store one raw 8-vector (already in registers) into the LDS tile [plane][row][k], splitting into
// planes.  KC: the 8 values run along k at row r; else along rows r..r+7 at column k.
template <int S, int MF, int P, bool KC>
__device__ __forceinline__ void store_raw8(uint16_t *tile, int rows, int r, int k, const Raw8<S> &x, float scale) {
  if constexpr (KC && S != SRC_F32 && ((S == SRC_F16 && MF == MF_F16) || (S == SRC_BF16 && MF == MF_BF16))) {
    *(uint4 *)(tile + r * LDK + k) = x.v;  // already in the MFMA format
  } else {
    uint16_t pl[8][3];
#pragma unroll
    for (int i = 0; i < 8; ++i) split_planes<S, MF>(raw_elem<S>(x, i), scale, pl[i]);
    lds_store8<P, KC>(tile, rows, r, k, pl);
  }
}

template <int MF, int SA, bool AKC, int SB, bool BKC>
__global__ void __launch_bounds__(NT) gemm_kernel(GemmArgs g) {
  constexpr int PA = Planes<SA, MF>::n, PB = Planes<SB, MF>::n;
  constexpr int MAXO = (MF == MF_F16) ? 1 : 2;  // keep cross products with plane order i+j <= MAXO
  constexpr int ASZ = PA * BM * LDK, BSZ = PB * BN * LDK, STG = ASZ + BSZ;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STG];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int zb = blockIdx.z, split = blockIdx.y;
  const int inner = g.inner > 0 ? g.inner : 1;
  const int batch = zb / inner, bin = zb % inner;
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  const int ntiles = tiles_m * tiles_n;
  // XCD-aware remap: hardware block b runs on XCD b % 8; give each XCD a contiguous range.
  int b = blockIdx.x, t = b;
  {
    int per = ntiles / 8;
    if (b < per * 8) t = (b % 8) * per + b / 8;
  }
  int tm, tn;
  if (g.m_fastest) { tm = t % tiles_m; tn = t / tiles_m; }
  else { tn = t % tiles_n; tm = t / tiles_n; }
  const int m0 = tm * BM, n0 = tn * BN;

  const int kbeg = split * g.k_chunk;
  const int kend = min(g.K, kbeg + g.k_chunk);
  if (kbeg >= kend && split > 0) return;

  const char *Ab = (const char *)g.A + ((long long)batch * g.a_bs + (long long)bin * g.a_bs2) * (SA == SRC_F32 ? 4 : 2);
  const char *Bb = (const char *)g.B + ((long long)batch * g.b_bs + (long long)bin * g.b_bs2) * (SB == SRC_F32 ? 4 : 2);
  float ascale = 1.f, bscale = 1.f;
  if constexpr (SA == SRC_F32 && MF == MF_F16)
    ascale = f16_split_scale(g.a_amax ? g.a_amax[(long long)batch * g.ab_amax_bs] : g.a_amax_c);
  if constexpr (SB == SRC_F32 && MF == MF_F16)
    bscale = f16_split_scale(g.b_amax ? g.b_amax[(long long)batch * g.ab_amax_bs] : g.b_amax_c);

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  Raw8<SA> ra[2];
  Raw8<SB> rb[2];

  auto gload = [&](int k0) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      int v = tid + it * NT;
      if constexpr (AKC) {
        int r = v >> 2, kv = (v & 3) * 8;
        int m = m0 + r;
        load_raw8<SA>(Ab, (long long)m * g.a_ld, k0 + kv, kend, m < g.M, g.a_blk, g.a_blk_stride, ra[it]);
      } else {
        int kr = v >> 4, mv = (v & 15) * 8;
        int k = k0 + kr;
        load_raw8<SA>(Ab, (long long)k * g.a_ld, m0 + mv, g.M, k < kend, g.a_blk, g.a_blk_stride, ra[it]);
      }
      if constexpr (BKC) {
        int r = v >> 2, kv = (v & 3) * 8;
        int n = n0 + r;
        load_raw8<SB>(Bb, (long long)n * g.b_ld, k0 + kv, kend, n < g.N, g.b_blk, g.b_blk_stride, rb[it]);
      } else {
        int kr = v >> 4, nv = (v & 15) * 8;
        int k = k0 + kr;
        load_raw8<SB>(Bb, (long long)k * g.b_ld, n0 + nv, g.N, k < kend, g.b_blk, g.b_blk_stride, rb[it]);
      }
    }
  };
  auto lstore = [&](int buf) {
    uint16_t *As = lds + buf * STG, *Bs = As + ASZ;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      int v = tid + it * NT;
      if constexpr (AKC) store_raw8<SA, MF, PA, true>(As, BM, v >> 2, (v & 3) * 8, ra[it], ascale);
      else store_raw8<SA, MF, PA, false>(As, BM, (v & 15) * 8, v >> 4, ra[it], ascale);
      if constexpr (BKC) store_raw8<SB, MF, PB, true>(Bs, BN, v >> 2, (v & 3) * 8, rb[it], bscale);
      else store_raw8<SB, MF, PB, false>(Bs, BN, (v & 15) * 8, v >> 4, rb[it], bscale);
    }
  };

  const int wm = wave >> 1, wn = wave & 1;
  const int fr = lane & 15, fk = (lane >> 4) * 8;

  if (kbeg < kend) {
    gload(kbeg);
    lstore(0);
    __syncthreads();
    int buf = 0;
    for (int k0 = kbeg; k0 < kend; k0 += BK) {
      const bool more = k0 + BK < kend;
      if (more) gload(k0 + BK);
      const uint16_t *As = lds + buf * STG, *Bs = As + ASZ;
      uint4 af[PA][4], bf[PB][4];
#pragma unroll
      for (int p = 0; p < PA; ++p)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          af[p][i] = *(const uint4 *)(As + p * BM * LDK + (wm * 64 + i * 16 + fr) * LDK + fk);
#pragma unroll
      for (int p = 0; p < PB; ++p)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bf[p][j] = *(const uint4 *)(Bs + p * BN * LDK + (wn * 64 + j * 16 + fr) * LDK + fk);
#pragma unroll
      for (int pa = PA - 1; pa >= 0; --pa)
#pragma unroll
        for (int pb = PB - 1; pb >= 0; --pb)
          if (pa + pb <= MAXO)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int j = 0; j < 4; ++j) acc[i][j] = mfma<MF>(af[pa][i], bf[pb][j], acc[i][j]);
      if (more) lstore(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
  }

  const float cs = g.alpha / (ascale * bscale);
  float *Cb = g.C + (long long)batch * g.c_bs + (long long)bin * g.c_bs2 + (long long)split * g.c_split;
  float *C2b = g.C2 ? g.C2 + (long long)batch * g.c2_bs : nullptr;
  float lmax = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int mb = m0 + wm * 64 + i * 16 + (lane >> 4) * 4;
      const int n = n0 + wn * 64 + j * 16 + fr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = mb + r;
        if (m < g.M && n < g.N) {
          float v = acc[i][j][r] * cs;
          Cb[(long long)m * g.c_ld + n] = v;
          lmax = fmaxf(lmax, fabsf(v));
        }
      }
      if (C2b && n < g.N) {
        if (mb + 4 <= g.M && ((g.c2_ld & 3) == 0)) {
          *(float4 *)(C2b + (long long)n * g.c2_ld + mb) =
              make_float4(acc[i][j][0] * cs, acc[i][j][1] * cs, acc[i][j][2] * cs, acc[i][j][3] * cs);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (mb + r < g.M) C2b[(long long)n * g.c2_ld + mb + r] = acc[i][j][r] * cs;
        }
      }
    }
  if (g.c_amax) {  // one atomic per workgroup
    __shared__ float wred[NT / 64];
    lmax = warp_max(lmax);
    if (lane == 0) wred[threadIdx.x >> 6] = lmax;
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int w = 1; w < NT / 64; ++w) lmax = fmaxf(lmax, wred[w]);
      atomicMax((unsigned int *)(g.c_amax + (long long)batch * g.c_amax_bs), __float_as_uint(lmax));
    }
  }
}

template <int MF, int SA, bool AKC, int SB, bool BKC>
void launch_t(const GemmArgs &g, int batch, int nsplit, hipStream_t st) {
  int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  dim3 grid(tiles, nsplit, batch);
  hipLaunchKernelGGL((gemm_kernel<MF, SA, AKC, SB, BKC>), grid, dim3(NT), 0, st, g);
}

template <int MF, int SA, int SB>
void launch_layout(bool akc, bool bkc, const GemmArgs &g, int batch, int nsplit, hipStream_t st) {
  if (akc && bkc) launch_t<MF, SA, true, SB, true>(g, batch, nsplit, st);
  else if (akc && !bkc) launch_t<MF, SA, true, SB, false>(g, batch, nsplit, st);
  else if (!akc && bkc) launch_t<MF, SA, false, SB, true>(g, batch, nsplit, st);
  else launch_t<MF, SA, false, SB, false>(g, batch, nsplit, st);
}

__global__ void reduce_splits_kernel(const float *part, long long part_bs, long long part_ss, int nsplit,
                                     int rows, int cols, long long ld_in, void *out, int out_f64,
                                     long long out_bs, long long ld_out) {
  const int b = blockIdx.y;
  long long n = (long long)rows * cols;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x) {
    int r = (int)(i / cols), c = (int)(i % cols);
    const float *p = part + b * part_bs + (long long)r * ld_in + c;
    double s = 0.0;
    for (int k = 0; k < nsplit; ++k) s += (double)p[k * part_ss];
    if (out_f64) ((double *)out)[b * out_bs + (long long)r * ld_out + c] = s;
    else ((float *)out)[b * out_bs + (long long)r * ld_out + c] = (float)s;
  }
}

// Split-K partials summed in fixed order (fp64) and written in two layouts, C[r][c] and
// C2[c][r], through a 32 x 32 LDS tile so both stores are coalesced; max |C| per batch is folded
// into amax (float bits, atomic max; the caller clears it).
__global__ void __launch_bounds__(256) reduce_splits_dual_kernel(const float *part, long long part_bs,
                                                                 long long part_ss, int nsplit, int rows, int cols,
                                                                 long long ld_in, float *C, long long c_bs,
                                                                 long long c_ld, float *C2, long long c2_bs,
                                                                 long long c2_ld, float *amax) {
  __shared__ float tile[32][33];
  __shared__ float wmax[4];
  const int b = blockIdx.z, tid = threadIdx.x, tx = tid & 31, ty = tid >> 5;  // 32 x 8 threads
  const int r0 = blockIdx.y * 32, c0 = blockIdx.x * 32;
  const float *pb = part + b * part_bs;
  float lmax = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = r0 + ty + 8 * k, c = c0 + tx;
    float v = 0.f;
    if (r < rows && c < cols) {
      const float *p = pb + (long long)r * ld_in + c;
      double s = 0.0;
      for (int q = 0; q < nsplit; ++q) s += (double)p[q * part_ss];
      v = (float)s;
      C[b * c_bs + (long long)r * c_ld + c] = v;
    }
    tile[ty + 8 * k][tx] = v;
    lmax = fmaxf(lmax, fabsf(v));
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c = c0 + ty + 8 * k, r = r0 + tx;
    if (r < rows && c < cols) C2[b * c2_bs + (long long)c * c2_ld + r] = tile[tx][ty + 8 * k];
  }
  if (amax) {
    lmax = warp_max(lmax);
    if ((tid & 63) == 0) wmax[tid >> 6] = lmax;
    __syncthreads();
    if (tid == 0)
      atomicMax((unsigned int *)(amax + b), __float_as_uint(fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]))));
  }
}

// The same reduction on 64 x 64 tiles with 16-byte accesses on every side (rows, columns and
// leading dimensions multiples of 4 floats): a thread sums four consecutive columns of four rows
// (all split loads in flight together) and stores four consecutive rows of four columns of C2.
// The splits are summed in the same fixed order, so the results equal the scalar kernel's.
__global__ void __launch_bounds__(256) reduce_splits_dual_vec_kernel(const float *part, long long part_bs,
                                                                     long long part_ss, int nsplit, int rows, int cols,
                                                                     long long ld_in, float *C, long long c_bs,
                                                                     long long c_ld, float *C2, long long c2_bs,
                                                                     long long c2_ld, float *amax) {
  __shared__ float tile[64][65];
  __shared__ float wmax[4];
  const int b = blockIdx.z, tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;  // 16 x 16 threads
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const float *pb = part + b * part_bs;
  float lmax = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = r0 + ty + 16 * k, c = c0 + 4 * tx;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r < rows && c < cols) {  // cols % 4 == 0: the four columns are all inside
      const float *p = pb + (long long)r * ld_in + c;
      double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
      int q = 0;
      for (; q + 4 <= nsplit; q += 4) {
        float4 x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) x[u] = *(const float4 *)(p + (q + u) * part_ss);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          s0 += (double)x[u].x;
          s1 += (double)x[u].y;
          s2 += (double)x[u].z;
          s3 += (double)x[u].w;
        }
      }
      for (; q < nsplit; ++q) {
        const float4 x = *(const float4 *)(p + q * part_ss);
        s0 += (double)x.x;
        s1 += (double)x.y;
        s2 += (double)x.z;
        s3 += (double)x.w;
      }
      v = make_float4((float)s0, (float)s1, (float)s2, (float)s3);
      *(float4 *)(C + b * c_bs + (long long)r * c_ld + c) = v;
    }
    const int rr = ty + 16 * k;
    tile[rr][4 * tx] = v.x;
    tile[rr][4 * tx + 1] = v.y;
    tile[rr][4 * tx + 2] = v.z;
    tile[rr][4 * tx + 3] = v.w;
    lmax = fmaxf(lmax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int cc = ty + 16 * k, c = c0 + cc, r = r0 + 4 * tx;
    if (c < cols && r < rows) {
      if (r + 4 <= rows) {
        *(float4 *)(C2 + b * c2_bs + (long long)c * c2_ld + r) =
            make_float4(tile[4 * tx][cc], tile[4 * tx + 1][cc], tile[4 * tx + 2][cc], tile[4 * tx + 3][cc]);
      } else {
        for (int u = 0; r + u < rows; ++u) C2[b * c2_bs + (long long)c * c2_ld + r + u] = tile[4 * tx + u][cc];
      }
    }
  }
  if (amax) {
    lmax = warp_max(lmax);
    if ((tid & 63) == 0) wmax[tid >> 6] = lmax;
    __syncthreads();
    if (tid == 0)
      atomicMax((unsigned int *)(amax + b), __float_as_uint(fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]))));
  }
}

}  // namespace

void gemm(int mf, int sa, bool a_kc, int sb, bool b_kc, const GemmArgs &g, int batch, int nsplit,
          hipStream_t st) {
  JOLT_REQUIRE(g.M > 0 && g.N > 0 && g.K > 0 && batch > 0 && nsplit > 0, JOLT_EINVAL, "gemm: empty shape");
  JOLT_REQUIRE(nsplit == 1 || (g.k_chunk % BK == 0 && (long long)g.k_chunk * nsplit >= g.K), JOLT_EINVAL,
               "gemm: bad split");
  JOLT_REQUIRE(g.a_blk % 8 == 0 && g.b_blk % 8 == 0 && g.a_ld % 8 == 0 && g.b_ld % 8 == 0 &&
                   g.a_blk_stride % 8 == 0 && g.b_blk_stride % 8 == 0 && g.a_bs % 8 == 0 && g.b_bs % 8 == 0 &&
                   g.a_bs2 % 8 == 0 && g.b_bs2 % 8 == 0 && ((uintptr_t)g.A % 16) == 0 && ((uintptr_t)g.B % 16) == 0,
               JOLT_EINVAL, "gemm: operands must be 16-byte aligned with strides in multiples of 8 elements");
  JOLT_REQUIRE(g.inner >= 1 && batch % g.inner == 0, JOLT_EINVAL, "gemm: bad inner batch");
  JOLT_REQUIRE(g.C2 == nullptr || ((uintptr_t)g.C2 % 16) == 0, JOLT_EINVAL, "gemm: C2 must be 16-byte aligned");
  JOLT_REQUIRE(g.tri == 0 || (a_kc && b_kc), JOLT_EINVAL, "gemm: structure flags need K-contiguous operands");
  JOLT_REQUIRE(!(g.tri & 6) || nsplit == 1, JOLT_EINVAL, "gemm: triangular operands need a single split");
  JOLT_REQUIRE(!(g.tri & 1) || g.M == g.N, JOLT_EINVAL, "gemm: upper-triangle output needs a square product");
  JOLT_REQUIRE(g.Cpl == nullptr || (a_kc && b_kc && nsplit == 1 && g.inner <= 1 && g.C2 == nullptr),
               JOLT_EINVAL, "gemm: plane output needs K-contiguous operands, one split, no second output");
  JOLT_REQUIRE(g.Cpl != nullptr || g.C != nullptr, JOLT_EINVAL, "gemm: no output");
  GemmArgs h = g;
  if (nsplit == 1) h.k_chunk = ((g.K + BK - 1) / BK) * BK;
  if (a_kc && b_kc) {
    gemm_kc(mf, sa, sb, h, batch, nsplit, st);
    return;
  }
  if (mf == MF_F16) {
    if (sa == SRC_F16 && sb == SRC_F16) launch_layout<MF_F16, SRC_F16, SRC_F16>(a_kc, b_kc, h, batch, nsplit, st);
    else if (sa == SRC_F16 && sb == SRC_F32) launch_layout<MF_F16, SRC_F16, SRC_F32>(a_kc, b_kc, h, batch, nsplit, st);
    else if (sa == SRC_F32 && sb == SRC_F16) launch_layout<MF_F16, SRC_F32, SRC_F16>(a_kc, b_kc, h, batch, nsplit, st);
    else if (sa == SRC_F32 && sb == SRC_F32) launch_layout<MF_F16, SRC_F32, SRC_F32>(a_kc, b_kc, h, batch, nsplit, st);
    else JOLT_REQUIRE(false, JOLT_EINVAL, "gemm: bad f16 operand types");
  } else {
    if (sa == SRC_BF16 && sb == SRC_BF16) launch_layout<MF_BF16, SRC_BF16, SRC_BF16>(a_kc, b_kc, h, batch, nsplit, st);
    else if (sa == SRC_F32 && sb == SRC_F32) launch_layout<MF_BF16, SRC_F32, SRC_F32>(a_kc, b_kc, h, batch, nsplit, st);
    else if (sa == SRC_BF16 && sb == SRC_F32) launch_layout<MF_BF16, SRC_BF16, SRC_F32>(a_kc, b_kc, h, batch, nsplit, st);
    else if (sa == SRC_F32 && sb == SRC_BF16) launch_layout<MF_BF16, SRC_F32, SRC_BF16>(a_kc, b_kc, h, batch, nsplit, st);
    else JOLT_REQUIRE(false, JOLT_EINVAL, "gemm: bad bf16 operand types");
  }
  HIP_LAUNCH_CHECK();
}

void reduce_splits(const float *part, long long part_bs, long long part_ss, int nsplit, long long n,
                   int rows, int cols, long long ld_in, void *out, bool out_f64, long long out_bs,
                   long long ld_out, int batch, hipStream_t st) {
  (void)n;
  long long tot = (long long)rows * cols;
  int blocks = (int)std::min<long long>((tot + 255) / 256, 4096);
  hipLaunchKernelGGL(reduce_splits_kernel, dim3(blocks, batch), dim3(256), 0, st, part, part_bs, part_ss, nsplit,
                     rows, cols, ld_in, out, out_f64 ? 1 : 0, out_bs, ld_out);
  HIP_LAUNCH_CHECK();
}

void reduce_splits_dual(const float *part, long long part_bs, long long part_ss, int nsplit, int rows, int cols,
                        long long ld_in, float *C, long long c_bs, long long c_ld, float *C2, long long c2_bs,
                        long long c2_ld, float *amax, int batch, hipStream_t st) {
  const bool vec = cols % 4 == 0 && ld_in % 4 == 0 && part_ss % 4 == 0 && part_bs % 4 == 0 && c_ld % 4 == 0 &&
                   c_bs % 4 == 0 && c2_ld % 4 == 0 && c2_bs % 4 == 0 && ((uintptr_t)part & 15) == 0 &&
                   ((uintptr_t)C & 15) == 0 && ((uintptr_t)C2 & 15) == 0;
  if (vec) {
    dim3 grid((cols + 63) / 64, (rows + 63) / 64, batch);
    hipLaunchKernelGGL(reduce_splits_dual_vec_kernel, grid, dim3(256), 0, st, part, part_bs, part_ss, nsplit, rows,
                       cols, ld_in, C, c_bs, c_ld, C2, c2_bs, c2_ld, amax);
  } else {
    dim3 grid((cols + 31) / 32, (rows + 31) / 32, batch);
    hipLaunchKernelGGL(reduce_splits_dual_kernel, grid, dim3(256), 0, st, part, part_bs, part_ss, nsplit, rows, cols,
                       ld_in, C, c_bs, c_ld, C2, c2_bs, c2_ld, amax);
  }
  HIP_LAUNCH_CHECK();
}

}  // namespace jolt
