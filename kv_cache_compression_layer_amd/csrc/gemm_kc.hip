// Dense contractions whose operands are both contiguous along K (every large product of the
// compressor: sketch, power-iteration and projection products against the cache, Gram matrices
// of the tall panels, triangular applies of the thin QR).
//
// Same arithmetic as the general kernel in gemm.hip: 16x16x32 MFMA on 16-bit planes (the cache
// at its own precision, fp32 operands split exactly into planes after a power-of-two scale), the
// same plane-product order inside each 32-deep k step, so every output element sees the same
// sequence of fp32 accumulations.  What differs is the shape of the work:
//   * 4 waves (2 x 2) per block; each wave owns TM x TN output subtiles of 16 x 16 (64 x 128 or
//     128 x 64), so a wave reads 12 fragments from LDS for 32 MFMAs instead of 8 for 16;
//   * LDS tiles are [row][32] without padding; the four 16-byte chunks of a row are XOR-permuted
//     by the row index so that fragment loads and tile stores are free of bank conflicts, which
//     keeps two blocks resident per CU even with two fp32 planes;
//   * the loop is specialised outside the k loop (every subtile live or not; aligned full
//     stages with pointer-increment addressing or the general bounds-checked path);
//   * subtiles entirely outside M or N skip their MFMAs (the ragged last tile of a 522-wide
//     sketch dimension costs its loads, not its matrix-core time).
#include <type_traits>

#include "common.hpp"
#include "gemm_core.hpp"

namespace jolt {

namespace {

using namespace core;

constexpr int KBK = 32;   // k per LDS stage (one MFMA depth)
constexpr int KNT = 256;  // threads per block (4 waves, 2 x 2)

// LDS element offset of chunk `chunk` (8 halves) of row `row` in a [rows][32] tile.  The chunk
// permutation depends on row % 8 only (rows 2i and 2i + 1 share a 128-byte bank row, and the
// four pairs of a fragment's eight rows get the four chunk rotations), which measures free of
// LDS bank conflicts for both the fragment reads and the tile stores; every 16-row fragment of
// a wave shares one pattern, so fragment addresses differ by compile-time constants.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * KBK + ((chunk ^ (row >> 1)) & 3) * 8;
}

// Store one raw 8-vector (8 consecutive k of one row) into every plane of an LDS tile.
template <int S, int MF, int P>
__device__ __forceinline__ void put8(uint16_t *tile, int plane_elems, int off, const Raw8<S> &x, float scale) {
  if constexpr (S != SRC_F32 && ((S == SRC_F16 && MF == MF_F16) || (S == SRC_BF16 && MF == MF_BF16))) {
    *(uint4 *)(tile + off) = x.v;
  } else {
    uint16_t pl[8][3];
#pragma unroll
    for (int i = 0; i < 8; ++i) split_planes<S, MF>(raw_elem<S>(x, i), scale, pl[i]);
#pragma unroll
    for (int p = 0; p < P; ++p) {
      uint4 w;
      w.x = pl[0][p] | ((uint32_t)pl[1][p] << 16);
      w.y = pl[2][p] | ((uint32_t)pl[3][p] << 16);
      w.z = pl[4][p] | ((uint32_t)pl[5][p] << 16);
      w.w = pl[6][p] | ((uint32_t)pl[7][p] << 16);
      *(uint4 *)(tile + p * plane_elems + off) = w;
    }
  }
}

template <int MF, int SA, int SB, int TM, int TN, int W>
__global__ void __launch_bounds__(KNT) __attribute__((amdgpu_waves_per_eu(W, W))) gemm_kc_kernel(GemmArgs g) {
  constexpr int PA = Planes<SA, MF>::n, PB = Planes<SB, MF>::n;
  constexpr int MAXO = (MF == MF_F16) ? 1 : 2;  // keep plane products with order i + j <= MAXO
  constexpr int WM = TM * 16, WN = TN * 16, BM = 2 * WM, BN = 2 * WN;
  constexpr int ASZ = PA * BM * KBK, BSZ = PB * BN * KBK, STG = ASZ + BSZ;
  constexpr int LA = BM * 4 / KNT, LB = BN * 4 / KNT;  // 8-element loads per thread per stage
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STG];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // XCD-aware remap over the whole grid: linear block L is dispatched to XCD L % 8, so give each
  // XCD one contiguous range of (batch, split, tile) -- whole cells where the grid allows -- and
  // every operand panel is streamed through one L2 instead of all eight.
  int t, split, zb;
  {
    const long long gx = gridDim.x, gxy = gx * gridDim.y, total = gxy * gridDim.z;
    long long L = blockIdx.x + gx * blockIdx.y + gxy * blockIdx.z;
    const long long per = total / 8;
    if (L < per * 8) L = (L % 8) * per + L / 8;
    t = (int)(L % gx);
    split = (int)((L / gx) % gridDim.y);
    zb = (int)(L / gxy);
  }
  const int inner = g.inner > 0 ? g.inner : 1;
  const int batch = zb / inner, bin = zb % inner;
  const int tiles_m = (g.M + BM - 1) / BM;
  const int tiles_n = (g.N + BN - 1) / BN;
  int tm, tn;
  if (g.m_fastest) { tm = t % tiles_m; tn = t / tiles_m; }
  else { tn = t % tiles_n; tm = t / tiles_n; }
  const int m0 = tm * BM, n0 = tn * BN;

  const int kbeg = split * g.k_chunk;
  int kend = min(g.K, kbeg + g.k_chunk);
  if (kbeg >= kend && split > 0) return;
  if (g.tri & 2) kend = min(kend, n0 + BN);
  if (g.tri & 4) kend = min(kend, m0 + BM);
  if ((g.tri & 1) && m0 >= n0 + BN) kend = kbeg;  // strictly below the diagonal: zeros

  const char *Ab = (const char *)g.A + ((long long)batch * g.a_bs + (long long)bin * g.a_bs2) * (SA == SRC_F32 ? 4 : 2);
  const char *Bb = (const char *)g.B + ((long long)batch * g.b_bs + (long long)bin * g.b_bs2) * (SB == SRC_F32 ? 4 : 2);
  float ascale = 1.f, bscale = 1.f;
  if constexpr (SA == SRC_F32 && MF == MF_F16)
    ascale = f16_split_scale(g.a_amax ? g.a_amax[(long long)batch * g.ab_amax_bs] : g.a_amax_c);
  if constexpr (SB == SRC_F32 && MF == MF_F16)
    bscale = f16_split_scale(g.b_amax ? g.b_amax[(long long)batch * g.ab_amax_bs] : g.b_amax_c);

  const int wm = wave >> 1, wn = wave & 1;
  const int fr = lane & 15, fc = lane >> 4;
  // live 16-row / 16-column subtiles of this wave (uniform across the wave)
  const int mlive = min(TM, max(0, (g.M - (m0 + wm * WM) + 15) / 16));
  const int nlive = min(TN, max(0, (g.N - (n0 + wn * WN) + 15) / 16));
  const bool full = (mlive == TM) && (nlive == TN);

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  Raw8<SA> ra[LA];
  Raw8<SB> rb[LB];
  // Load slots: thread v of a stage loads 8 consecutive k of row v / 4 at chunk v % 4.  Row
  // pointers are fixed for the whole k loop (rows past the edge read row 0 and are zeroed); the
  // k offset in blocked addressing, (k / blk) * blk_stride + k % blk, is advanced by the stage
  // depth without divisions.  When blk is a multiple of 32 a stage never straddles a block, so a
  // full stage needs no per-lane index arithmetic at all.
  constexpr int ESA = (SA == SRC_F32) ? 4 : 2, ESB = (SB == SRC_F32) ? 4 : 2;
  // (byte offsets of the rows within the batch fit 32 bits: checked by the host)
  uint32_t pa[LA], pb[LB];
  bool oka[LA], okb[LB];
#pragma unroll
  for (int it = 0; it < LA; ++it) {
    const int v = tid + it * KNT, m = m0 + (v >> 2);
    oka[it] = m < g.M;
    pa[it] = (uint32_t)(((long long)(oka[it] ? m : 0) * g.a_ld + (v & 3) * 8) * ESA);
  }
#pragma unroll
  for (int it = 0; it < LB; ++it) {
    const int v = tid + it * KNT, n = n0 + (v >> 2);
    okb[it] = n < g.N;
    pb[it] = (uint32_t)(((long long)(okb[it] ? n : 0) * g.b_ld + (v & 3) * 8) * ESB);
  }
  const bool afast = (g.a_blk % KBK) == 0, bfast = (g.b_blk % KBK) == 0;
  const int nsteps = (kend - kbeg + KBK - 1) / KBK;
  const int nfast = (afast && bfast) ? (kend - kbeg) / KBK : 0;  // leading steps with fast loads
  // fast path state: scalar base pointers of the current stage and the position inside the block
  int ar = kbeg % g.a_blk, br = kbeg % g.b_blk;
  const char *abase = Ab + ((long long)(kbeg / g.a_blk) * g.a_blk_stride + ar) * ESA;
  const char *bbase = Bb + ((long long)(kbeg / g.b_blk) * g.b_blk_stride + br) * ESB;
  auto gload_fast = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < LA; ++it) {
      if constexpr (SA == SRC_F32) {
        const float4 *q = (const float4 *)(abase + pa[it]);
        float4 x = q[0], y = q[1];
        if (!oka[it]) x = y = make_float4(0.f, 0.f, 0.f, 0.f);
        ra[it].a = x;
        ra[it].b = y;
      } else {
        uint4 x = *(const uint4 *)(abase + pa[it]);
        if (!oka[it]) x = make_uint4(0u, 0u, 0u, 0u);
        ra[it].v = x;
      }
    }
#pragma unroll
    for (int it = 0; it < LB; ++it) {
      if constexpr (SB == SRC_F32) {
        const float4 *q = (const float4 *)(bbase + pb[it]);
        float4 x = q[0], y = q[1];
        if (!okb[it]) x = y = make_float4(0.f, 0.f, 0.f, 0.f);
        rb[it].a = x;
        rb[it].b = y;
      } else {
        uint4 x = *(const uint4 *)(bbase + pb[it]);
        if (!okb[it]) x = make_uint4(0u, 0u, 0u, 0u);
        rb[it].v = x;
      }
    }
    // next stage: a block of blocked addressing ends exactly on a stage boundary
    ar += KBK;
    abase += KBK * ESA;
    if (ar == g.a_blk) { ar = 0; abase += (g.a_blk_stride - g.a_blk) * ESA; }
    br += KBK;
    bbase += KBK * ESB;
    if (br == g.b_blk) { br = 0; bbase += (g.b_blk_stride - g.b_blk) * ESB; }
  };
  auto gload_slow = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < LA; ++it) {
      const int v = tid + it * KNT, m = m0 + (v >> 2);
      load_raw8<SA>(Ab, (long long)m * g.a_ld, k0 + (v & 3) * 8, kend, m < g.M, g.a_blk, g.a_blk_stride, ra[it]);
    }
#pragma unroll
    for (int it = 0; it < LB; ++it) {
      const int v = tid + it * KNT, n = n0 + (v >> 2);
      load_raw8<SB>(Bb, (long long)n * g.b_ld, k0 + (v & 3) * 8, kend, n < g.N, g.b_blk, g.b_blk_stride, rb[it]);
    }
  };
  auto lstore = [&](int buf) __attribute__((always_inline)) {
    uint16_t *As = lds + buf * STG, *Bs = As + ASZ;
#pragma unroll
    for (int it = 0; it < LA; ++it) {
      const int v = tid + it * KNT;
      put8<SA, MF, PA>(As, BM * KBK, swz(v >> 2, v & 3), ra[it], ascale);
    }
#pragma unroll
    for (int it = 0; it < LB; ++it) {
      const int v = tid + it * KNT;
      put8<SB, MF, PB>(Bs, BN * KBK, swz(v >> 2, v & 3), rb[it], bscale);
    }
  };

  // fragment i of the wave's A rows sits at aoff + i * 16 rows (same chunk pattern); likewise B
  const int aoff = swz(wm * WM + fr, fc), boff = swz(wn * WN + fr, fc);

  // one 32-deep step from LDS buffer `buf`; FULL: every subtile of the wave is inside M x N
  auto compute = [&](auto FULL, int buf) __attribute__((always_inline)) {
    const uint16_t *As = lds + buf * STG, *Bs = As + ASZ;
    uint4 bf[PB][TN];
#pragma unroll
    for (int p = 0; p < PB; ++p)
#pragma unroll
      for (int j = 0; j < TN; ++j) bf[p][j] = *(const uint4 *)(Bs + p * BN * KBK + j * 16 * KBK + boff);
#pragma unroll
    for (int pa_ = PA - 1; pa_ >= 0; --pa_) {
      uint4 af[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = *(const uint4 *)(As + pa_ * BM * KBK + i * 16 * KBK + aoff);
#pragma unroll
      for (int pb_ = PB - 1; pb_ >= 0; --pb_) {
        if (pa_ + pb_ > MAXO) continue;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            if constexpr (decltype(FULL)::value) acc[i][j] = mfma<MF>(af[i], bf[pb_][j], acc[i][j]);
            else if (i < mlive && j < nlive) acc[i][j] = mfma<MF>(af[i], bf[pb_][j], acc[i][j]);
          }
      }
    }
  };
  auto mainloop = [&](auto FULL) __attribute__((always_inline)) {
    if (nfast > 0) gload_fast();
    else gload_slow(kbeg);
    lstore(0);
    __syncthreads();
    int buf = 0, s = 0;
    // steady state: the next step's loads take the fast path
    for (; s + 1 < nfast; ++s) {
      gload_fast();
      compute(FULL, buf);
      lstore(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
    // remaining steps (the ragged end of K, or every step when blocked addressing is irregular)
    for (; s < nsteps; ++s) {
      const bool more = s + 1 < nsteps;
      if (more) gload_slow(kbeg + (s + 1) * KBK);
      compute(FULL, buf);
      if (more) lstore(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
  };
  if (kbeg < kend) {
    if (full) mainloop(std::integral_constant<bool, true>{});
    else mainloop(std::integral_constant<bool, false>{});
  }

  const float cs = g.alpha / (ascale * bscale);
  float *Cb = g.C ? g.C + (long long)batch * g.c_bs + (long long)bin * g.c_bs2 + (long long)split * g.c_split : nullptr;
  float *C2b = g.C2 ? g.C2 + (long long)batch * g.c2_bs : nullptr;
  uint16_t *Pb = g.Cpl ? g.Cpl + (long long)batch * g.cpl_bs : nullptr;
  const float pscale = f16_split_scale(g.cpl_amax);
  float lmax = 0.f;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int mb = m0 + wm * WM + i * 16 + fc * 4;
      const int n = n0 + wn * WN + j * 16 + fr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = mb + r;
        if (m < g.M && n < g.N) {
          const float v = acc[i][j][r] * cs;
          if (Pb) {
            uint16_t pl[3];
            const long long o = (long long)m * g.c_ld + n;
            if (g.cpl_mf == MF_F16) {
              split_planes<SRC_F32, MF_F16>(v, pscale, pl);
              Pb[o] = pl[0];
              Pb[o + g.cpl_ps] = pl[1];
            } else {
              split_planes<SRC_F32, MF_BF16>(v, 1.f, pl);
              Pb[o] = pl[0];
              Pb[o + g.cpl_ps] = pl[1];
              Pb[o + 2 * g.cpl_ps] = pl[2];
            }
          } else {
            Cb[(long long)m * g.c_ld + n] = v;
          }
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
    __shared__ float wred[KNT / 64];
    lmax = warp_max(lmax);
    if (lane == 0) wred[threadIdx.x >> 6] = lmax;
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int w = 1; w < KNT / 64; ++w) lmax = fmaxf(lmax, wred[w]);
      atomicMax((unsigned int *)(g.c_amax + (long long)batch * g.c_amax_bs), __float_as_uint(lmax));
    }
  }
}

template <int MF, int SA, int SB, int TM, int TN, int W = 2>
void launch_kc(const GemmArgs &g, int batch, int nsplit, hipStream_t st) {
  constexpr int BM = 32 * TM, BN = 32 * TN;
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_kc_kernel<MF, SA, SB, TM, TN, W>), dim3(tiles, nsplit, batch), dim3(KNT), 0, st, g);
}

template <int MF, int SA, int SB>
void launch_shape(const GemmArgs &g, int batch, int nsplit, hipStream_t st) {
  // wide output -> 128 x 256 blocks, tall -> 256 x 128, small or square -> 128 x 128; two fp32
  // operands keep 128 x 128 (the larger tiles would not fit two waves per SIMD)
  if ((SA == SRC_F32 && SB == SRC_F32) || (g.M <= 160 && g.N <= 160) || (g.tri & 1))
    launch_kc<MF, SA, SB, 4, 4>(g, batch, nsplit, st);
  else if (g.N >= g.M) launch_kc<MF, SA, SB, 4, 8>(g, batch, nsplit, st);
  else launch_kc<MF, SA, SB, 8, 4>(g, batch, nsplit, st);
}

}  // namespace

// Both operands contiguous along K; arguments validated by gemm().
void gemm_kc(int mf, int sa, int sb, const GemmArgs &g, int batch, int nsplit, hipStream_t st) {
  const long long esa = sa == SRC_F32 ? 4 : 2, esb = sb == SRC_F32 ? 4 : 2;
  JOLT_REQUIRE(((long long)g.M * g.a_ld + 32) * esa < (1LL << 32) && ((long long)g.N * g.b_ld + 32) * esb < (1LL << 32),
               JOLT_EINVAL, "gemm: row offsets exceed 32 bits");
  if (mf == MF_F16) {
    if (sa == SRC_F16 && sb == SRC_F16) launch_shape<MF_F16, SRC_F16, SRC_F16>(g, batch, nsplit, st);
    else if (sa == SRC_F16 && sb == SRC_F32) launch_shape<MF_F16, SRC_F16, SRC_F32>(g, batch, nsplit, st);
    else if (sa == SRC_F32 && sb == SRC_F16) launch_shape<MF_F16, SRC_F32, SRC_F16>(g, batch, nsplit, st);
    else if (sa == SRC_F32 && sb == SRC_F32) launch_shape<MF_F16, SRC_F32, SRC_F32>(g, batch, nsplit, st);
    else JOLT_REQUIRE(false, JOLT_EINVAL, "gemm: bad f16 operand types");
  } else {
    if (sa == SRC_BF16 && sb == SRC_BF16) launch_shape<MF_BF16, SRC_BF16, SRC_BF16>(g, batch, nsplit, st);
    else if (sa == SRC_F32 && sb == SRC_F32) launch_shape<MF_BF16, SRC_F32, SRC_F32>(g, batch, nsplit, st);
    else if (sa == SRC_BF16 && sb == SRC_F32) launch_shape<MF_BF16, SRC_BF16, SRC_F32>(g, batch, nsplit, st);
    else if (sa == SRC_F32 && sb == SRC_BF16) launch_shape<MF_BF16, SRC_F32, SRC_BF16>(g, batch, nsplit, st);
    else JOLT_REQUIRE(false, JOLT_EINVAL, "gemm: bad bf16 operand types");
  }
  HIP_LAUNCH_CHECK();
}

}  // namespace jolt
