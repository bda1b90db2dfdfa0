// Residual codec of the method (Sec. 3, "Rotated low-bit residual"): fused encode and decode.
//
// Encode, per cell, per head-slice j = (l, h) and 256-token tile:
//   E_rot = (X_j - U_T D_j) Q = [X_j | U_T] [Q ; -D_j Q]     (one MFMA pass, K = d_h + r_T)
//   per row: absmax (wavefront + cross-wave reduction), s = absmax / q_max (fp32),
//   code = clamp(rint(e / s)), packed b bits per element LSB-first, one fp32 scale per row.
// Decode:
//   X_hat_j = s (codes Q^T) + U_T D_j                         (two MFMA passes, one accumulator)
// D_j = C_j U_d^T is the backbone slice; the operand [Q ; -D_j Q] is prepared per cell.
// fp32 operands are split into 16-bit planes exactly as in the GEMM kernel; cache values and
// codes are exact in 16 bits.
#include "common.hpp"
#include "gemm_core.hpp"
#include "codec.hpp"

namespace jolt {

namespace {

using namespace core;

template <int MF, int PA, int PB, int MAXO>
__device__ __forceinline__ void mma_step(const uint16_t *As, const uint16_t *Bs, int wm, int wn, int lane,
                                         f32x4 (&acc)[4][4]) {
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  uint4 af[PA][4], bf[PB][4];
#pragma unroll
  for (int p = 0; p < PA; ++p)
#pragma unroll
    for (int i = 0; i < 4; ++i) af[p][i] = *(const uint4 *)(As + p * BM * LDK + (wm * 64 + i * 16 + fr) * LDK + fk);
#pragma unroll
  for (int p = 0; p < PB; ++p)
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[p][j] = *(const uint4 *)(Bs + p * BN * LDK + (wn * 64 + j * 16 + fr) * LDK + fk);
#pragma unroll
  for (int pa = PA - 1; pa >= 0; --pa)
#pragma unroll
    for (int pb = PB - 1; pb >= 0; --pb)
      if (pa + pb <= MAXO)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = mfma<MF>(af[pa][i], bf[pb][j], acc[i][j]);
}

// Store a raw 8-vector into an LDS tile along k (row r, column k), splitting into planes.
template <int S, int MF, int P, int NB16>
__device__ __forceinline__ void put8(uint16_t *tile, int rows, int r, int k, const Raw8<S> &x, float scale) {
  if constexpr (S != SRC_F32 && ((S == SRC_F16 && MF == MF_F16) || (S == SRC_BF16 && MF == MF_BF16))) {
    *(uint4 *)(tile + r * LDK + k) = x.v;
  } else {
    uint16_t pl[8][3];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (S == SRC_F32 && MF == MF_F16 && NB16 == 3) split3_f16(raw_elem<S>(x, i), scale, pl[i]);
      else split_planes<S, MF>(raw_elem<S>(x, i), scale, pl[i]);
    }
    lds_store8<P, true>(tile, rows, r, k, pl);
  }
}

// 16-bit plane count of a source under the MFMA type; for fp32 with f16 MFMA the B operand of
// the codec uses NB16 planes (hi, lo[, lo2]).
template <int S, int MF, int NB16>
struct CPlanes {
  static constexpr int n = (S == SRC_F32) ? (MF == MF_F16 ? NB16 : 3) : 1;
};

template <int S, int MF, int NB16>
__device__ __forceinline__ void csplit(float x, float scale, uint16_t (&p)[3]) {
  if constexpr (S == SRC_F32 && MF == MF_F16 && NB16 == 3) split3_f16(x, scale, p);
  else split_planes<S, MF>(x, scale, p);
}

// ------------------------------------------------------------------------------------------ encode
// Tile: 256 rows (4 waves x 64 rows, each wave holding whole rows) x all D columns; the k loop runs
// over [X_j | U_T] (D + r_T).  LDS tiles are [row][32] with the 16-byte chunks XOR-permuted by
// (row / 2) % 4 (free of bank conflicts for fragment loads and tile stores); row pointers are fixed
// for the k loop, full stages load without index arithmetic, the ragged last stage is bounds-checked.
constexpr int EBM = 256, EKB = 32, ENT = 256;

__device__ __forceinline__ int eswz(int row, int chunk) { return row * EKB + ((chunk ^ (row >> 1)) & 3) * 8; }

template <int S, int MF, int P>
__device__ __forceinline__ void eput8(uint16_t *tile, int plane_elems, int off, const Raw8<S> &x, float scale) {
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

template <int S>
__device__ __forceinline__ void eload8(const char *p, bool ok, Raw8<S> &r) {
  if constexpr (S == SRC_F32) {
    const float4 *q = (const float4 *)p;
    float4 x = q[0], y = q[1];
    if (!ok) x = y = make_float4(0.f, 0.f, 0.f, 0.f);
    r.a = x;
    r.b = y;
  } else {
    uint4 x = *(const uint4 *)p;
    if (!ok) x = make_uint4(0u, 0u, 0u, 0u);
    r.v = x;
  }
}

// W waves per SIMD: 2 for 16-bit caches; fp32 caches carry three planes per operand and run at 1.
// B = [Q ; -D_j Q] arrives as 16-bit planes (split once per cell by the host sequence).  The MFMA
// takes B as its first operand, so lane l holds output columns 4 (l / 16) + r (r = 0..3) of token
// row l % 16 in every 16 x 16 subtile: four consecutive codes of one row per lane.
template <int MF, int SX, int TN, int W = (SX == SRC_F32 ? 1 : 2)>
__global__ void __launch_bounds__(ENT) __attribute__((amdgpu_waves_per_eu(W, W)))
encode_kernel(EncArgs ea, int T, int ttiles, int GHmax) {
  constexpr int D = TN * 16;
  constexpr int PA = Planes<SX, MF>::n, PB = Planes<SRC_F32, MF>::n;
  constexpr int MAXO = (MF == MF_F16) ? 1 : 2;
  constexpr int ASZ = PA * EBM * EKB, BSZ = PB * D * EKB, STG = ASZ + BSZ;
  constexpr int LA = EBM * 4 / ENT, LB = D * 4 / ENT;  // 8-element chunks per thread per stage (B: per plane)
  constexpr int ESX = (SX == SRC_F32) ? 4 : 2;
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];  // 2 * STG halves
  __shared__ float srow[EBM];
  uint32_t *rowbits = (uint32_t *)lds;  // [EBM][D * bits / 32] packed codes, reuses the tiles
  static_assert(2 * STG * 2 >= EBM * D, "packed codes must fit in the tile buffers");

  // XCD-aware order over the whole grid: consecutive (cell, slice, tile) on one XCD, so the
  // tiles of one slice share its B panel in that XCD's L2
  int tt, j, cz;
  {
    const long long gx = gridDim.x, total = gx * gridDim.z;
    long long L = blockIdx.x + gx * blockIdx.z;
    const long long per = total / 8;
    if (L < per * 8) L = (L % 8) * per + L / 8;
    cz = (int)(L / gx);
    const int x = (int)(L % gx);
    j = x / ttiles;
    tt = x % ttiles;
  }
  const EncCell c = ea.cells[cz];
  if (j >= c.GH) return;
  const int tid = threadIdx.x, lane = tid & 63, wm = tid >> 6;
  const int fr = lane & 15, fc = lane >> 4;
  const int t0 = tt * EBM;
  const int rT = c.rT, K = D + rT;
  const char *xbase = (c.kv ? ea.xv : ea.xk) + c.x_off + (long long)j * T * D * ESX;
  const char *utbase = ea.utb + c.ut_off;
  const char *bj = ea.bcat + c.bcat_off + (long long)j * D * c.Kb * 2;  // plane 0 of slice j
  const float bscale = (MF == MF_F16) ? f16_split_scale(ea.bamax[c.am_idx]) : 1.f;

  f32x4 acc[4][TN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < TN; ++q) acc[i][q] = f32x4{0.f, 0.f, 0.f, 0.f};

  // load slots: A rows t0 + v / 4 (X then U_T), B rows n = v / 4 of each plane of B_j, chunk v % 4
  Raw8<SX> ra[LA];
  uint4 rb[PB][LB];
  int trow[LA];  // token row of each load slot (row 0 past the end; zeroed on load)
  bool oka[LA];
#pragma unroll
  for (int it = 0; it < LA; ++it) {
    const int v = tid + it * ENT, t = t0 + (v >> 2);
    oka[it] = t < T;
    trow[it] = oka[it] ? t : 0;
  }
  auto bload = [&](int k0, bool check) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < PB; ++p)
#pragma unroll
      for (int it = 0; it < LB; ++it) {
        const int v = tid + it * ENT, k = k0 + (v & 3) * 8;
        uint4 x = make_uint4(0u, 0u, 0u, 0u);
        if (!check || k < K) x = *(const uint4 *)(bj + (p * ea.b_ps + (long long)(v >> 2) * c.Kb + k) * 2);
        rb[p][it] = x;
      }
  };
  auto gload_fast = [&](int k0) __attribute__((always_inline)) {
    // (row offsets formed per stage: 64-bit offsets held per slot would cost registers)
    if (k0 < D) {
#pragma unroll
      for (int it = 0; it < LA; ++it) {
        const int c = ((tid + it * ENT) & 3) * 8 + k0;
        eload8<SX>(xbase + ((long long)trow[it] * D + c) * ESX, oka[it], ra[it]);
      }
    } else {
#pragma unroll
      for (int it = 0; it < LA; ++it) {
        const int c = ((tid + it * ENT) & 3) * 8 + (k0 - D);
        eload8<SX>(utbase + ((long long)trow[it] * rT + c) * ESX, oka[it], ra[it]);
      }
    }
    bload(k0, false);
  };
  auto gload_slow = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < LA; ++it) {
      const int v = tid + it * ENT, t = t0 + (v >> 2), k = k0 + (v & 3) * 8;
      if (k < D) load_raw8<SX>(xbase, (long long)t * D, k, D, t < T, 1 << 30, 0, ra[it]);
      else load_raw8<SX>(utbase, (long long)t * rT, k - D, rT, t < T, 1 << 30, 0, ra[it]);
    }
    bload(k0, true);
  };
  auto lstore = [&](int buf) __attribute__((always_inline)) {
    uint16_t *As = lds + buf * STG, *Bs = As + ASZ;
#pragma unroll
    for (int it = 0; it < LA; ++it) {
      const int v = tid + it * ENT;
      eput8<SX, MF, PA>(As, EBM * EKB, eswz(v >> 2, v & 3), ra[it], 1.f);
    }
#pragma unroll
    for (int p = 0; p < PB; ++p)
#pragma unroll
      for (int it = 0; it < LB; ++it) {
        const int v = tid + it * ENT;
        *(uint4 *)(Bs + p * D * EKB + eswz(v >> 2, v & 3)) = rb[p][it];
      }
  };
  const int aoff = eswz(wm * 64 + fr, fc), boff = eswz(fr, fc);
  // plane products in the order (pa, pb) descending, as in the GEMM kernels; B fragments are
  // loaded per plane so only one plane is live
  auto compute = [&](int buf) __attribute__((always_inline)) {
    const uint16_t *As = lds + buf * STG, *Bs = As + ASZ;
#pragma unroll
    for (int pa = PA - 1; pa >= 0; --pa) {
      uint4 af[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = *(const uint4 *)(As + pa * EBM * EKB + i * 16 * EKB + aoff);
#pragma unroll
      for (int pb = PB - 1; pb >= 0; --pb) {
        if (pa + pb > MAXO) continue;
        // B fragments in two halves of the columns (fewer live registers)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uint4 bf[TN / 2];
#pragma unroll
          for (int q = 0; q < TN / 2; ++q) bf[q] = *(const uint4 *)(Bs + pb * D * EKB + (h * TN / 2 + q) * 16 * EKB + boff);
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q = 0; q < TN / 2; ++q) acc[i][h * TN / 2 + q] = mfma<MF>(bf[q], af[i], acc[i][h * TN / 2 + q]);
        }
      }
    }
  };

  const int nsteps = (K + EKB - 1) / EKB, nfull = K / EKB;
  if (nfull > 0) gload_fast(0);
  else gload_slow(0);
  lstore(0);
  __syncthreads();
  int buf = 0, s = 0;
  for (; s + 1 < nfull; ++s) {
    gload_fast((s + 1) * EKB);
    compute(buf);
    lstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
  for (; s < nsteps; ++s) {
    const bool more = s + 1 < nsteps;
    if (more) gload_slow((s + 1) * EKB);
    compute(buf);
    if (more) lstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  // ---- quantisation and packing ---------------------------------------------------------------
  // Row m = wm * 64 + 16 i + fr of the tile lives in the four lanes fr + 16 fc, each holding its
  // columns 16 q + 4 fc + r.  The code of e is rint(e / s) in fp32 (IEEE quotient); it is formed
  // from e * (1 / s), whose distance from the quotient (< 2e-5 for |e / s| <= 127) only matters
  // within 1e-4 of a rounding boundary, where the quotient itself is taken.  Each lane ORs the
  // 4 b bits of its four codes into the row's words in LDS (LSB-first), then the tile's rows are
  // copied out whole.
  const float inv = 1.f / bscale;  // a power of two
  const int b = c.bits;
  const int qm = (b >= 2) ? ((1 << (b - 1)) - 1) : 1;
  const int wpr = D * b / 32;  // 32-bit words per row (D in {64, 128}: integral)
  for (int w = tid; w < EBM * wpr; w += ENT) rowbits[w] = 0u;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float m = 0.f;
#pragma unroll
    for (int q = 0; q < TN; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = acc[i][q][r] * inv;
        acc[i][q][r] = v;
        m = fmaxf(m, fabsf(v));
      }
    m = fmaxf(m, __shfl_xor(m, 16, 64));
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    const int row = wm * 64 + i * 16 + fr;
    const float sc = (b == 1) ? m : m / (float)qm;
    if (fc == 0) srow[row] = sc;
    const float rinv = sc > 0.f ? 1.f / sc : 0.f;
#pragma unroll
    for (int q = 0; q < TN; ++q) {
      uint32_t chunk = 0u;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = acc[i][q][r];
        uint32_t u;
        if (b == 1) u = (v >= 0.f) ? 1u : 0u;
        else if (sc > 0.f) {
          const float t = v * rinv;
          float qv = rintf(t);
          if (__builtin_expect(fabsf(fabsf(t - qv) - 0.5f) < 1e-4f, 0)) qv = rintf(v / sc);
          qv = fminf(fmaxf(qv, (float)-qm), (float)qm);
          u = (uint32_t)((int)qv + qm);
        } else u = (uint32_t)qm;
        chunk |= u << (r * b);
      }
      const int bit = (q * 16 + fc * 4) * b, wd = bit >> 5, sh = bit & 31;
      atomicOr(&rowbits[row * wpr + wd], chunk << sh);
      if (sh + 4 * b > 32) atomicOr(&rowbits[row * wpr + wd + 1], chunk >> (32 - sh));
    }
  }
  __syncthreads();
  const long long row0 = (long long)j * T + t0;
  const int nrows = min(EBM, T - t0);
  float *scales = (float *)(ea.scb + c.sc_off);
  for (int rr = tid; rr < nrows; rr += ENT) scales[row0 + rr] = srow[rr];
  uint32_t *out = (uint32_t *)(ea.cdb + c.cd_off + row0 * (D * b / 8));
  for (int w = tid; w < nrows * wpr; w += ENT) out[w] = rowbits[w];
}

// ------------------------------------------------------------------------------------------ decode
// unpack 8 codes (elements k0..k0+7 of row) to their signed values
__device__ __forceinline__ void unpack8(const uint8_t *rowp, int k0, int b, float (&v)[8]) {
  const uint8_t *p = rowp + (k0 * b) / 8;
  uint64_t w = 0;
  for (int i = 0; i < b; ++i) w |= (uint64_t)p[i] << (8 * i);
  const int qm = (b >= 2) ? ((1 << (b - 1)) - 1) : 1;
  const uint64_t mask = (1ull << b) - 1ull;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int u = (int)((w >> (i * b)) & mask);
    v[i] = (b == 1) ? (u ? 1.f : -1.f) : (float)(u - qm);
  }
}

template <int MF, int SX, int NB16>
__global__ void __launch_bounds__(NT) decode_kernel(const DecCell *cells, int T, int D, int ttiles) {
  constexpr int PA = CPlanes<SX, MF, NB16>::n;  // U_T part; the codes part uses one plane
  constexpr int PB = CPlanes<SRC_F32, MF, NB16>::n;
  constexpr int MAXO = (MF == MF_F16) ? (NB16 - 1) : 2;
  constexpr int ASZ = PA * BM * LDK, BSZ = PB * BN * LDK, STG = ASZ + BSZ;
  constexpr int SC = (MF == MF_F16) ? SRC_F16 : SRC_BF16;  // small integer codes are exact
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STG];
  __shared__ float srow[BM];

  const DecCell c = cells[blockIdx.z];
  const int j = blockIdx.x / ttiles, tt = blockIdx.x % ttiles;
  if (j >= c.GH) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int t0 = tt * BM;
  const int fr = lane & 15;
  const float qscale = (MF == MF_F16) ? f16_split_scale(1.f) : 1.f;
  const float dscale = (MF == MF_F16) ? f16_split_scale(*c.d_amax) : 1.f;
  const int b = c.bits;
  const int rowbytes = D * b / 8;

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[i][q] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- phase 1: codes Q^T, then scale rows ---------------------------------------------------
  if (b > 0) {
    float ca[2][8];
    Raw8<SRC_F32> rb[2];
    auto gload = [&](int k0) {
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        int v = tid + it * NT;
        int r = v >> 2, kv = (v & 3) * 8;
        int t = t0 + r;
        if (t < T) unpack8(c.codes + ((long long)j * T + t) * rowbytes, k0 + kv, b, ca[it]);
        else
#pragma unroll
          for (int i = 0; i < 8; ++i) ca[it][i] = 0.f;
        load_raw8<SRC_F32>(c.Q, (long long)r * D, k0 + kv, D, r < D, 1 << 30, 0, rb[it]);
      }
    };
    auto lstore = [&](int buf) {
      uint16_t *As = lds + buf * STG, *Bs = As + ASZ;
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        int v = tid + it * NT;
        uint16_t pa[8][3];
#pragma unroll
        for (int i = 0; i < 8; ++i) split_planes<SC, MF>(ca[it][i], 1.f, pa[i]);
        lds_store8<1, true>(As, BM, v >> 2, (v & 3) * 8, pa);
        put8<SRC_F32, MF, PB, NB16>(Bs, BN, v >> 2, (v & 3) * 8, rb[it], qscale);
      }
    };
    gload(0);
    lstore(0);
    __syncthreads();
    int buf = 0;
    for (int k0 = 0; k0 < D; k0 += BK) {
      const bool more = k0 + BK < D;
      if (more) gload(k0 + BK);
      mma_step<MF, 1, PB, MAXO>(lds + buf * STG, lds + buf * STG + ASZ, wm, wn, lane, acc);
      if (more) lstore(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
    for (int rr = tid; rr < BM; rr += NT) srow[rr] = (t0 + rr < T) ? c.scales[(long long)j * T + t0 + rr] : 0.f;
    __syncthreads();
    // rows scaled by s and moved into the dscale frame of phase 2
    const float f = dscale / qscale;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float sr = srow[wm * 64 + i * 16 + (lane >> 4) * 4 + r] * f;
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][q][r] *= sr;
      }
  }
  // ---- phase 2: + U_T D_j ------------------------------------------------------------------
  {
    const float *Dj = c.Dm + (long long)j * D * c.Kd;
    Raw8<SX> ra[2];
    Raw8<SRC_F32> rb[2];
    auto gload = [&](int k0) {
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        int v = tid + it * NT;
        int r = v >> 2, kv = (v & 3) * 8;
        int t = t0 + r;
        load_raw8<SX>(c.UT, (long long)t * c.rT, k0 + kv, c.rT, t < T, 1 << 30, 0, ra[it]);
        load_raw8<SRC_F32>(Dj, (long long)r * c.Kd, k0 + kv, c.rT, r < D, 1 << 30, 0, rb[it]);
      }
    };
    auto lstore = [&](int buf) {
      uint16_t *As = lds + buf * STG, *Bs = As + ASZ;
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        int v = tid + it * NT;
        put8<SX, MF, PA, NB16>(As, BM, v >> 2, (v & 3) * 8, ra[it], 1.f);
        put8<SRC_F32, MF, PB, NB16>(Bs, BN, v >> 2, (v & 3) * 8, rb[it], dscale);
      }
    };
    __syncthreads();
    gload(0);
    lstore(0);
    __syncthreads();
    int buf = 0;
    for (int k0 = 0; k0 < c.rT; k0 += BK) {
      const bool more = k0 + BK < c.rT;
      if (more) gload(k0 + BK);
      mma_step<MF, PA, PB, MAXO>(lds + buf * STG, lds + buf * STG + ASZ, wm, wn, lane, acc);
      if (more) lstore(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
  }
  const float inv = 1.f / dscale;
  const long long obase = (long long)j * T * D;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + wm * 64 + i * 16 + (lane >> 4) * 4 + r;
      if (t >= T) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = wn * 64 + q * 16 + fr;
        if (n < D) store_elem<SX>(c.out, obase + (long long)t * D + n, acc[i][q][r] * inv);
      }
    }
}

template <int MF, int SX, int TN>
void launch_enc(const EncArgs &a, int ncells, int T, int GHmax, hipStream_t st) {
  constexpr int D = TN * 16;
  constexpr int PA = Planes<SX, MF>::n, PB = Planes<SRC_F32, MF>::n;
  constexpr size_t shm = 2 * (size_t)(PA * EBM * EKB + PB * D * EKB) * 2;
  static bool attr = false;  // allow the dynamic LDS size once
  if (!attr) {
    (void)hipFuncSetAttribute((const void *)encode_kernel<MF, SX, TN>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)shm);
    (void)hipGetLastError();
    attr = true;
  }
  const int tt = (T + EBM - 1) / EBM;
  hipLaunchKernelGGL((encode_kernel<MF, SX, TN>), dim3(tt * GHmax, 1, ncells), dim3(ENT), shm, st, a, T, tt, GHmax);
}
template <int MF, int SX, int NB16>
void launch_dec(const DecCell *cells, int ncells, int T, int D, int GHmax, hipStream_t st) {
  int tt = (T + BM - 1) / BM;
  hipLaunchKernelGGL((decode_kernel<MF, SX, NB16>), dim3(tt * GHmax, 1, ncells), dim3(NT), 0, st, cells, T, D, tt);
}

}  // namespace

void encode_cells(int dtype, const EncArgs &a, int ncells, int T, int D, int GHmax, hipStream_t st) {
  JOLT_REQUIRE(D == 64 || D == 128, JOLT_EINVAL, "codec: d_head must be 64 or 128");
  if (ncells <= 0) return;
  if (D == 128) {
    if (dtype == JOLT_F16) launch_enc<MF_F16, SRC_F16, 8>(a, ncells, T, GHmax, st);
    else if (dtype == JOLT_BF16) launch_enc<MF_BF16, SRC_BF16, 8>(a, ncells, T, GHmax, st);
    else launch_enc<MF_BF16, SRC_F32, 8>(a, ncells, T, GHmax, st);
  } else {
    if (dtype == JOLT_F16) launch_enc<MF_F16, SRC_F16, 4>(a, ncells, T, GHmax, st);
    else if (dtype == JOLT_BF16) launch_enc<MF_BF16, SRC_BF16, 4>(a, ncells, T, GHmax, st);
    else launch_enc<MF_BF16, SRC_F32, 4>(a, ncells, T, GHmax, st);
  }
  HIP_LAUNCH_CHECK();
}

void decode_cells(int dtype, const DecCell *d_cells, int ncells, int T, int D, int GHmax, hipStream_t st) {
  JOLT_REQUIRE(D == 64 || D == 128, JOLT_EINVAL, "codec: d_head must be 64 or 128");
  if (dtype == JOLT_F16) launch_dec<MF_F16, SRC_F16, 2>(d_cells, ncells, T, D, GHmax, st);
  else if (dtype == JOLT_BF16) launch_dec<MF_BF16, SRC_BF16, 2>(d_cells, ncells, T, D, GHmax, st);
  else launch_dec<MF_BF16, SRC_F32, 2>(d_cells, ncells, T, D, GHmax, st);
  HIP_LAUNCH_CHECK();
}

}  // namespace jolt
