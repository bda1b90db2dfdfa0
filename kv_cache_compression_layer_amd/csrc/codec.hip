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
#include "dma.hpp"
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


// ------------------------------------------------------------------------------- encode (DMA-fed)
// 16-bit caches.  One block of 2 NWR waves takes 128 NWR token rows of one (cell, slice) and all D
// output columns; wave (wr, wc) owns rows 128 wr .. 128 wr + 127 and columns (D / 2) wc .. (D / 2) wc +
// D / 2 - 1 (the wave tile that needs the fewest fragment reads per MFMA with B in PB planes).
// Operand tiles go global -> LDS by DMA with NS stages in flight: A = [X_j | U_T] rows (X_j for k < D,
// U_T after; the buffer descriptors bound each source, so rows past T and the U_T columns past r_T in
// the last 32-deep stage read zero), B = the PB 16-bit planes of [Q ; -D_j Q] (rows past D + r_T are
// zero).  Each stage multiplies in the order of encode_kernel (B plane descending), so every
// accumulator sees the same fp32 sequence and the codes are the same.  The block's LDS (at most 80 KB)
// leaves room for a second block per CU, whose main loop covers this one's prologue and epilogue.
// Row |max| is combined across the two column halves through LDS; codes are ORed into LDS row words
// (row pitch padded by four words against bank conflicts) and copied out with 16-byte stores.
// Block order: 8 slices x 8 token tiles of a cell run as one group on one XCD, so each U_T tile and
// each slice's B planes are fetched from HBM once per group and reused from that XCD's L2.

__device__ __forceinline__ long long uniform64(long long v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (long long)(((uint64_t)hi << 32) | lo);
}

template <int MF, int TN, int NS, int NWR>
struct XCfg {
  static constexpr int D = TN * 16, NW = 2 * NWR, NT = 64 * NW, ROWS = 128 * NWR;
  static constexpr int PB = (MF == MF_F16) ? 2 : 3;     // planes of B
  static constexpr int MAXO = (MF == MF_F16) ? 1 : 2;   // plane products kept: pb <= MAXO (A has one plane)
  static constexpr int WR = 128, WC = D / 2, TI = WR / 16, TQ = WC / 16;
  static constexpr int ASZ = ROWS * dma::DK, BSZ = PB * D * dma::DK, STG = ASZ + BSZ;  // halves per stage
  // DMA slots per wave and stage: NA of A (16-row groups w, w + NW, ...) and NBS of B (B group w + NW i;
  // a wave past the last B group repeats group w % NGB: the same bytes to the same place as the wave
  // that owns it)
  static constexpr int NGA = ROWS / 16, NGB = PB * D / 16, NA = NGA / NW, NBS = (NGB + NW - 1) / NW;
  static constexpr int ND = NA + NBS;
  static constexpr int RP = D * 8 / 32 + 4;  // LDS row pitch of the packed codes (words; b <= 8)
  static_assert(NGA % NW == 0, "A groups split evenly over the waves");
  static_assert(NS * STG * 2 <= 80 * 1024, "two blocks per CU");
  static_assert((ROWS * RP + 3 * ROWS) * 4 <= NS * STG * 2, "epilogue fits in the stage buffers");
  static_assert((NS - 2) * ND < 64, "vmcnt range");
};

// one stage of DMA requests of this wave into stage buffer dst: A from X_j (k < D) or U_T, then B
template <int D, int NW, int NA, int NBS>
__device__ __forceinline__ void enc_issue(dma::lds16 *__restrict__ dst, int k, dma::i32x4 rsx, dma::i32x4 rsu,
                                          dma::i32x4 rsb, const uint32_t (&gx)[NA], const uint32_t (&gu)[NA],
                                          const uint32_t (&gb)[NBS], int wave, const int (&bslot)[NBS]) {
  using namespace dma;
  if (k < D) {
#pragma unroll
    for (int i = 0; i < NA; ++i)
      raw_buffer_load_lds(rsx, (__attribute__((address_space(3))) uint32_t *)(dst + (i * NW + wave) * 16 * DK), 16,
                          (int)gx[i], k * 2, 0, 0);
  } else {
#pragma unroll
    for (int i = 0; i < NA; ++i)
      raw_buffer_load_lds(rsu, (__attribute__((address_space(3))) uint32_t *)(dst + (i * NW + wave) * 16 * DK), 16,
                          (int)gu[i], (k - D) * 2, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < NBS; ++i)
    raw_buffer_load_lds(rsb, (__attribute__((address_space(3))) uint32_t *)(dst + bslot[i] * 16 * DK), 16, (int)gb[i],
                        k * 2, 0, 0);
}

// (slice, tile) of block index `rem` of a cell with GH slices and tt tiles: groups of SG slices x TG
// tiles, tile-major inside a group (consecutive blocks share the U_T tile)
__device__ __forceinline__ void enc_order(int rem, int GH, int tt, int &j, int &tile) {
  constexpr int SG = 8, TG = 8;
  const int sg = rem / (SG * tt), ns = min(SG, GH - sg * SG);
  const int rem2 = rem - sg * SG * tt;
  const int tg = rem2 / (ns * TG);
  const int rem3 = rem2 - tg * ns * TG;
  j = sg * SG + rem3 % ns;
  tile = tg * TG + rem3 / ns;
}

template <int MF, int TN, int NS, int NWR>
__global__ void __launch_bounds__(128 * NWR) __attribute__((amdgpu_waves_per_eu(2, 2)))
encode_dma_kernel(EncArgs ea, int T, int ttiles, int GHmax) {
  using C = XCfg<MF, TN, NS, NWR>;
  using namespace dma;
  constexpr int D = C::D, PB = C::PB, TI = C::TI, TQ = C::TQ, ND = C::ND, NGA = C::NGA, NW = C::NW, NT = C::NT;
  constexpr int ROWS = C::ROWS, RP = C::RP;
  __shared__ __attribute__((aligned(1024))) uint16_t lds_raw[NS * C::STG];
  lds16 *const L0 = (lds16 *)lds_raw, *const Llast = L0 + (NS - 1) * C::STG;

  // XCD-aware order: consecutive blocks of the remapped index run on one XCD; inside a cell, groups of
  // slices x tiles (enc_order)
  int tt, j, cz;
  {
    const long long gx = gridDim.x, total = gx * gridDim.z;
    long long L = blockIdx.x + gx * blockIdx.z;
    const long long per = total / 8;
    if (L < per * 8) L = (L % 8) * per + L / 8;
    cz = (int)(L / gx);
    const int x = (int)(L % gx);
    if (x >= GHmax * ttiles) return;
    enc_order(x, GHmax, ttiles, j, tt);
  }
  // the cell record is read with vector loads (the compiler cannot prove it invariant); its fields are
  // block-uniform, so they are moved to scalar registers: buffer descriptors built from vector
  // registers would make every DMA request a serialising waterfall loop
  EncCell c = ea.cells[cz];
  c.x_off = uniform64(c.x_off);
  c.ut_off = uniform64(c.ut_off);
  c.sc_off = uniform64(c.sc_off);
  c.cd_off = uniform64(c.cd_off);
  c.bcat_off = uniform64(c.bcat_off);
  c.kv = __builtin_amdgcn_readfirstlane(c.kv);
  c.am_idx = __builtin_amdgcn_readfirstlane(c.am_idx);
  c.GH = __builtin_amdgcn_readfirstlane(c.GH);
  c.rT = __builtin_amdgcn_readfirstlane(c.rT);
  c.bits = __builtin_amdgcn_readfirstlane(c.bits);
  c.Kb = __builtin_amdgcn_readfirstlane(c.Kb);
  if (j >= c.GH) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1;
  const int fr = lane & 15, fc = lane >> 4;
  const int t0 = tt * ROWS;
  const int rT = c.rT, K = D + rT, Kb = c.Kb;
  const int nsteps = (K + DK - 1) / DK;

  // sources: X_j [T][D], U_T [T][rT] (cache dtype), B planes [plane][n][Kb] of slice j
  const char *xj = (c.kv ? ea.xv : ea.xk) + c.x_off + (long long)j * T * D * 2;
  const char *ut = ea.utb + c.ut_off;
  const char *bj = ea.bcat + c.bcat_off + (long long)j * D * Kb * 2;
  const i32x4 rsx = make_rsrc(xj, (uint32_t)((long long)T * D * 2));
  const i32x4 rsu = make_rsrc(ut, (uint32_t)((long long)T * rT * 2));
  const i32x4 rsb = make_rsrc(bj, 0xFFFFFFFFu);
  const float bscale = (MF == MF_F16) ? f16_split_scale(ea.bamax[c.am_idx]) : 1.f;

  // DMA slots of this wave: lane -> row lane / 4 of a 16-row group, logical chunk
  // (lane % 4) ^ ((row / 2) % 4) (the tile's XOR permutation)
  constexpr int NA = C::NA, NBS = C::NBS;
  uint32_t gx_[NA], gu_[NA], gb_[NBS];
  int bslot[NBS];
  {
    const int r = lane >> 2, p = lane & 3;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int row = (i * NW + wave) * 16 + r, ch = (p ^ (row >> 1)) & 3;
      const long long t = (long long)t0 + row;  // past T: out of the descriptor's range, reads zero
      gx_[i] = (uint32_t)min((t * D + ch * 8) * 2, 0xFFFFFFF0LL);
      gu_[i] = (uint32_t)min((t * rT + ch * 8) * 2, 0xFFFFFFF0LL);
    }
#pragma unroll
    for (int i = 0; i < NBS; ++i) {
      int Gb = i * NW + wave;
      if (Gb >= C::NGB) Gb = wave % C::NGB;
      bslot[i] = NGA + Gb;
      const int plane = Gb / (D / 16), row = (Gb % (D / 16)) * 16 + r, ch = (p ^ (row >> 1)) & 3;
      gb_[i] = (uint32_t)((plane * ea.b_ps + (long long)row * Kb + ch * 8) * 2);
    }
  }

  const int aoff = dswz(wr * C::WR + fr, fc), boff = C::ASZ + dswz(wc * C::WC + fr, fc);
  f32x4 acc[TI][TQ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int q = 0; q < TQ; ++q) acc[i][q] = f32x4{0.f, 0.f, 0.f, 0.f};

  {
    lds16 *far = L0;
#pragma unroll
    for (int q = 0; q < NS - 1; ++q)
      if (q < nsteps) {
        enc_issue<D, NW, NA, NBS>(far, q * DK, rsx, rsu, rsb, gx_, gu_, gb_, wave, bslot);
        far += C::STG;
      }
    lds16 *cur = L0;
    for (int s = 0; s < nsteps; ++s) {
      const int later = min(NS - 2, nsteps - 1 - s);
      wait_stages<ND, NS - 2>(later);
      wait_lgkm0();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (s + NS - 1 < nsteps)
        enc_issue<D, NW, NA, NBS>(far, (s + NS - 1) * DK, rsx, rsu, rsb, gx_, gu_, gb_, wave, bslot);
      u32x4 af[TI];
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        af[i] = *(const lds_u32x4 *)(cur + aoff + i * 16 * DK);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int pb = PB - 1; pb >= 0; --pb) {
        if (pb > C::MAXO) continue;
        u32x4 bf[TQ];
#pragma unroll
        for (int q = 0; q < TQ; ++q) {
          bf[q] = *(const lds_u32x4 *)(cur + boff + pb * D * DK + q * 16 * DK);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int q = 0; q < TQ; ++q) acc[i][q] = mfma16<MF>(bf[q], af[i], acc[i][q]);
        __builtin_amdgcn_sched_barrier(0);
      }
      cur = cur == Llast ? L0 : cur + C::STG;
      far = far == Llast ? L0 : far + C::STG;
    }
  }
  __syncthreads();  // every wave is done with the stage buffers: the epilogue reuses them

  // ---- quantisation and packing (the rules of encode_kernel) -------------------------------------
  // lane (fr, fc) of wave (wr, wc) holds, per 16-row group i and column group q, the columns
  // D/2 wc + 16 q + 4 fc + r (r = 0..3) of token row 128 wr + 16 i + fr.  The accumulators carry the
  // power-of-two split scale of B: e = acc / bscale exactly, so |max| and the code decisions are taken
  // on acc with the scale folded into their factors (the same fp32 values as on e).
  const int b = c.bits;
  const int qm = (b >= 2) ? ((1 << (b - 1)) - 1) : 1;
  uint32_t *rowbits = (uint32_t *)lds_raw;            // [ROWS][RP]
  float *rmax = (float *)(rowbits + ROWS * RP);       // [2][ROWS]
  float *srow = rmax + 2 * ROWS;                      // [ROWS]
  const float inv = 1.f / bscale;  // a power of two
  for (int w = tid; w < ROWS * RP; w += NT) rowbits[w] = 0u;
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    float m = 0.f;
#pragma unroll
    for (int q = 0; q < TQ; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(acc[i][q][r]));
    m = fmaxf(m, __shfl_xor(m, 16, 64));
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    if (fc == 0) rmax[wc * ROWS + wr * C::WR + i * 16 + fr] = m * inv;
  }
  __syncthreads();
  auto put = [&](int row, int q, uint32_t chunk) __attribute__((always_inline)) {
    const int bit = (wc * C::WC + q * 16 + fc * 4) * b, wd = bit >> 5, sh = bit & 31;
    atomicOr(&rowbits[row * RP + wd], chunk << sh);
    if (sh + 4 * b > 32) atomicOr(&rowbits[row * RP + wd + 1], chunk >> (32 - sh));
  };
  if (b == 1) {  // sign code, scale = |max|
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int row = wr * C::WR + i * 16 + fr;
      if (wc == 0 && fc == 0) srow[row] = fmaxf(rmax[row], rmax[ROWS + row]);
#pragma unroll
      for (int q = 0; q < TQ; ++q) {
        uint32_t chunk = 0u;
#pragma unroll
        for (int r = 0; r < 4; ++r) chunk |= (acc[i][q][r] >= 0.f ? 1u : 0u) << r;
        put(row, q, chunk);
      }
    }
  } else {
    const float qmf = (float)qm;
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int row = wr * C::WR + i * 16 + fr;
      const float m = fmaxf(rmax[row], rmax[ROWS + row]);
      const float sc = m / qmf;  // IEEE quotient, as the scale is defined
      if (wc == 0 && fc == 0) srow[row] = sc;
      // code = rint(e / sc): formed from e * (1 / sc), which differs from the IEEE quotient by far less
      // than 1e-4 for |e / sc| <= 127, so only values within 1e-4 of a rounding boundary can round
      // differently; if any of the lane's values is that close, the lane takes the quotient for all of them
      const float rs = sc > 0.f ? __builtin_amdgcn_rcpf(sc) * inv : 0.f;  // zero row: every code is q_max (0)
      uint32_t chunk[TQ];
      bool near = false;
#pragma unroll
      for (int q = 0; q < TQ; ++q) {
        chunk[q] = 0u;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float t = acc[i][q][r] * rs;
          const float qv = rintf(t);
          near |= fabsf(fabsf(t - qv) - 0.5f) < 1e-4f;
          const float cq = __builtin_amdgcn_fmed3f(qv, -qmf, qmf) + qmf;
          chunk[q] |= (uint32_t)cq << (r * b);
        }
      }
      if (near) {
#pragma unroll
        for (int q = 0; q < TQ; ++q) {
          chunk[q] = 0u;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float qv = rintf((acc[i][q][r] * inv) / sc);
            chunk[q] |= (uint32_t)(__builtin_amdgcn_fmed3f(qv, -qmf, qmf) + qmf) << (r * b);
          }
        }
      }
#pragma unroll
      for (int q = 0; q < TQ; ++q) put(row, q, chunk[q]);
    }
  }
  __syncthreads();
  const int wpr = D * b / 32;
  const long long row0 = (long long)j * T + t0;
  const int nrows = min(ROWS, T - t0);
  float *scales = (float *)(ea.scb + c.sc_off);
  for (int rr = tid; rr < nrows; rr += NT) scales[row0 + rr] = srow[rr];
  // codes: wpr words per row (D b / 8 bytes, a multiple of 8); 16-byte stores when aligned
  char *outb = ea.cdb + c.cd_off + row0 * (D * b / 8);
  if ((((uintptr_t)outb) & 15) == 0 && (wpr & 3) == 0) {
    const int q4 = wpr / 4;
    for (int w = tid; w < nrows * q4; w += NT) {
      const int rr = w / q4, k4 = w - rr * q4;
      *(uint4 *)(outb + ((long long)rr * wpr + 4 * k4) * 4) = *(const uint4 *)(rowbits + rr * RP + 4 * k4);
    }
  } else {
    for (int w = tid; w < nrows * wpr; w += NT) {
      const int rr = w / wpr, k = w - rr * wpr;
      ((uint32_t *)outb)[(long long)rr * wpr + k] = rowbits[rr * RP + k];
    }
  }
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
struct DecCfg {
  static constexpr int PA = CPlanes<SX, MF, NB16>::n;  // U_T part; the codes part uses one plane
  static constexpr int PB = CPlanes<SRC_F32, MF, NB16>::n;
  static constexpr int MAXO = (MF == MF_F16) ? (NB16 - 1) : 2;
  static constexpr int ASZ = PA * BM * LDK, BSZ = PB * BN * LDK, STG = ASZ + BSZ;
};

// Rebuild rows t0 .. t0 + 127 of head slice j of a cell, X_hat_j = s (codes Q^T) + U_T D_j, into the
// calling wave's accumulators (row wm 64 + 16 i + 4 (lane / 16) + r, column wn 64 + 16 q + lane % 16
// for wave (wm, wn)), in real units; rows past T come out zero.  lds: 2 STG halves of staging,
// srow: BM floats.  Every thread of the block calls it (it synchronises the block).
// QP: planes of Q taken in the codes phase (every caller takes all of them: with the leading plane
// alone, small elements of a 16-bit reconstruction move by more than their own rounding step)
template <int MF, int SX, int NB16, int QP>
__device__ __forceinline__ void rebuild_tile(const DecCell &c, int j, int t0, int T, int D, uint16_t *lds, float *srow,
                                             f32x4 (&acc)[4][4]) {
  using C = DecCfg<MF, SX, NB16>;
  constexpr int PA = C::PA, PB = C::PB, MAXO = C::MAXO, ASZ = C::ASZ, STG = C::STG;
  static_assert(QP >= 1 && QP <= PB, "planes of Q");
  constexpr int SC = (MF == MF_F16) ? SRC_F16 : SRC_BF16;  // small integer codes are exact
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const float qscale = (MF == MF_F16) ? f16_split_scale(1.f) : 1.f;
  const float dscale = (MF == MF_F16) ? f16_split_scale(*c.d_amax) : 1.f;
  const int b = c.bits;
  const int rowbytes = D * b / 8;

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[i][q] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- phase 1: codes Q^T, then scale rows ---------------------------------------------------
  if (b > 0) {
    float ca[2][8];
    Raw8<SRC_F16> rb[2][QP];  // Q's planes, raw 16-bit
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
#pragma unroll
        for (int p = 0; p < QP; ++p)
          load_raw8<SRC_F16>(c.Qpl + p * c.qpl_ps, (long long)r * D, k0 + kv, D, r < D, 1 << 30, 0, rb[it][p]);
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
#pragma unroll
        for (int p = 0; p < QP; ++p)
          *(uint4 *)(Bs + p * BN * LDK + (v >> 2) * LDK + (v & 3) * 8) = rb[it][p].v;
      }
    };
    gload(0);
    lstore(0);
    __syncthreads();
    int buf = 0;
    for (int k0 = 0; k0 < D; k0 += BK) {
      const bool more = k0 + BK < D;
      if (more) gload(k0 + BK);
      mma_step<MF, 1, QP, MAXO>(lds + buf * STG, lds + buf * STG + ASZ, wm, wn, lane, acc);
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
    const uint16_t *Dj = c.Dpl + (long long)j * D * c.Kd;
    Raw8<SX> ra[2];
    Raw8<SRC_F16> rb[2][PB];  // D_j's planes, raw 16-bit
    auto gload = [&](int k0) {
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        int v = tid + it * NT;
        int r = v >> 2, kv = (v & 3) * 8;
        int t = t0 + r;
        load_raw8<SX>(c.UT, (long long)t * c.rT, k0 + kv, c.rT, t < T, 1 << 30, 0, ra[it]);
#pragma unroll
        for (int p = 0; p < PB; ++p)
          load_raw8<SRC_F16>(Dj + p * c.dpl_ps, (long long)r * c.Kd, k0 + kv, c.rT, r < D, 1 << 30, 0, rb[it][p]);
      }
    };
    auto lstore = [&](int buf) {
      uint16_t *As = lds + buf * STG, *Bs = As + ASZ;
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        int v = tid + it * NT;
        put8<SX, MF, PA, NB16>(As, BM, v >> 2, (v & 3) * 8, ra[it], 1.f);
#pragma unroll
        for (int p = 0; p < PB; ++p)
          *(uint4 *)(Bs + p * BN * LDK + (v >> 2) * LDK + (v & 3) * 8) = rb[it][p].v;
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
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][q][r] *= inv;
}

template <int MF, int SX, int NB16>
__global__ void __launch_bounds__(NT) decode_kernel(const DecCell *cells, int T, int D, int ttiles) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * DecCfg<MF, SX, NB16>::STG];
  __shared__ float srow[BM];
  const DecCell c = cells[blockIdx.z];
  const int j = blockIdx.x / ttiles, tt = blockIdx.x % ttiles;
  if (j >= c.GH) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1, fr = lane & 15;
  const int t0 = tt * BM;
  f32x4 acc[4][4];
  rebuild_tile<MF, SX, NB16, DecCfg<MF, SX, NB16>::PB>(c, j, t0, T, D, lds, srow, acc);
  // the tile goes through LDS (rounded to the output type, rows padded by 16 bytes) so that every
  // global store is a whole 16 bytes of a row
  constexpr int ES = SX == SRC_F32 ? 4 : 2;
  const int pitch = D * ES + 16;  // bytes
  char *ob = (char *)lds;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = wm * 64 + i * 16 + (lane >> 4) * 4 + r;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = wn * 64 + q * 16 + fr;
        if (n < D) {
          if constexpr (SX == SRC_F32) *(float *)(ob + row * pitch + n * 4) = acc[i][q][r];
          else if constexpr (SX == SRC_F16) *(uint16_t *)(ob + row * pitch + n * 2) = f32_to_f16_rne(acc[i][q][r]);
          else *(uint16_t *)(ob + row * pitch + n * 2) = f32_to_bf16_rne(acc[i][q][r]);
        }
      }
    }
  __syncthreads();
  const int cpr = D * ES / 16;  // 16-byte chunks per row
  char *out = (char *)c.out + ((long long)j * T + t0) * D * ES;
  for (int w = threadIdx.x; w < BM * cpr; w += NT) {
    const int row = w / cpr, ch = w - row * cpr;
    if (t0 + row < T) *(uint4 *)(out + (long long)row * D * ES + ch * 16) = *(const uint4 *)(ob + row * pitch + ch * 16);
  }
}

// ------------------------------------------------------------------------------- decode (DMA-fed)
// 16-bit caches.  X_hat_j = s o (C_j Q^T) + U_T D_j as one loop of 32-deep stages over k in
// [0, D + r_T): B = the planes of Q (k < D, shared by every slice) and then of D_j (k >= D, rows zero
// from r_T up to the padded pitch), global -> LDS by DMA; A = the codes for k < D (the stage's packed
// code words go to LDS by DMA and each lane unpacks its fragments: small integers, exact in 16 bits)
// and the U_T rows for k >= D (DMA; columns past r_T meet the zero rows of B).  After the last codes
// stage the rows are scaled by s and moved into D_j's split frame, as in rebuild_tile.  Block: 256
// token rows of one (cell, slice) on four waves of 128 rows x D/2 columns (the encode's tile and block
// order); each lane stores its four consecutive columns of a row straight from the accumulators.
template <int MF, int TN>
struct YCfg {
  static constexpr int NS = 2, NWR = 2;
  static constexpr int D = TN * 16, NW = 2 * NWR, NT = 64 * NW, ROWS = 128 * NWR;
  static constexpr int PB = (MF == MF_F16) ? 2 : 3;    // planes of B
  static constexpr int MAXO = (MF == MF_F16) ? 1 : 2;  // plane products kept: pb <= MAXO (A has one plane)
  static constexpr int WR = 128, WC = D / 2, TI = WR / 16, TQ = WC / 16;
  static constexpr int ASZ = ROWS * dma::DK, BSZ = PB * D * dma::DK, STG = ASZ + BSZ;  // halves per stage
  static constexpr int NGA = ROWS / 16, NGB = PB * D / 16, NA = NGA / NW, NBS = (NGB + NW - 1) / NW;
  static_assert(NGA % NW == 0, "A groups split evenly over the waves");
  static_assert(ROWS * 8 * 4 + 12 <= ASZ * 2, "a stage's code words fit in its A area");
  static_assert(NS * STG * 2 <= 80 * 1024, "two blocks per CU");
};

template <int MF, int TN>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
decode_dma_kernel(const DecCell *cells, int T, int ttiles, int GHmax) {
  using C = YCfg<MF, TN>;
  using namespace dma;
  constexpr int D = C::D, PB = C::PB, TI = C::TI, TQ = C::TQ, NW = C::NW, NA = C::NA, NBS = C::NBS;
  constexpr int NGA = C::NGA, ROWS = C::ROWS;
  __shared__ __attribute__((aligned(1024))) uint16_t lds_raw[C::NS * C::STG];
  lds16 *const L0 = (lds16 *)lds_raw, *const L1 = L0 + C::STG;

  int tt, j, cz;
  {
    const long long gx = gridDim.x, total = gx * gridDim.z;
    long long L = blockIdx.x + gx * blockIdx.z;
    const long long per = total / 8;
    if (L < per * 8) L = (L % 8) * per + L / 8;
    cz = (int)(L / gx);
    const int x = (int)(L % gx);
    if (x >= GHmax * ttiles) return;
    enc_order(x, GHmax, ttiles, j, tt);
  }
  // block-uniform fields in scalar registers (descriptors built from them stay scalar)
  const DecCell cv = cells[cz];
  const int GH = __builtin_amdgcn_readfirstlane(cv.GH), rT = __builtin_amdgcn_readfirstlane(cv.rT);
  const int b = __builtin_amdgcn_readfirstlane(cv.bits), Kd = __builtin_amdgcn_readfirstlane(cv.Kd);
  if (j >= GH) return;
  const char *ut = (const char *)uniform64((long long)cv.UT);
  const char *dpl = (const char *)uniform64((long long)cv.Dpl);
  const char *qpl = (const char *)uniform64((long long)cv.Qpl);
  const long long dpl_ps = uniform64(cv.dpl_ps), qpl_ps = uniform64(cv.qpl_ps);
  const uint8_t *codes = (const uint8_t *)uniform64((long long)cv.codes);
  const float *scales = (const float *)uniform64((long long)cv.scales);
  char *out = (char *)uniform64((long long)cv.out);
  const float qscale = (MF == MF_F16) ? f16_split_scale(1.f) : 1.f;
  const float dscale = (MF == MF_F16) ? f16_split_scale(*(const float *)uniform64((long long)cv.d_amax)) : 1.f;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1, fr = lane & 15, fc = lane >> 4;
  const int t0 = tt * ROWS;
  const int kbeg = b > 0 ? 0 : D, kend = D + rT;
  const int nsteps = (kend - kbeg + DK - 1) / DK;

  const i32x4 rsu = make_rsrc(ut, (uint32_t)((long long)T * rT * 2));
  const i32x4 rsq = make_rsrc(qpl, 0xFFFFFFFFu);
  const i32x4 rsd = make_rsrc(dpl + (long long)j * D * Kd * 2, 0xFFFFFFFFu);
  const long long rowbytes = (long long)D * b / 8;  // packed codes per row
  const i32x4 rsc = make_rsrc(codes + (long long)j * T * rowbytes, (uint32_t)(T * rowbytes));
  // DMA requests of one stage (offsets formed per request: fewer live registers).  A: lane -> row
  // lane / 4 of a 16-row group, logical chunk (lane % 4) ^ ((row / 2) % 4); B: group w + NW i of this
  // wave (past the last group it repeats group w % NGB: the same bytes to the same place as the wave
  // that owns it).  Codes: request m of wave w covers rows 8 (m NW + w) .. + 7, lane -> row lane / 8,
  // word lane % 8 of the row's bytes from (k / 8) b on.
  const int lr = lane >> 2, lp = lane & 3;
  auto issue = [&](lds16 *dst, int k) __attribute__((always_inline)) {
    if (k < D) {
#pragma unroll
      for (int m = 0; m < ROWS / 8 / NW; ++m) {
        const int rq = m * NW + wave, row = rq * 8 + (lane >> 3);
        const long long off = (long long)(t0 + row) * rowbytes + (k / 8) * b + 4 * (lane & 7);
        raw_buffer_load_lds(rsc, (__attribute__((address_space(3))) uint32_t *)dst + rq * 64, 4,
                            (int)min(off, 0xFFFFFFF0LL), 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const int row = (i * NW + wave) * 16 + lr, ch = (lp ^ (row >> 1)) & 3;
        const long long t = (long long)t0 + row;  // past T: out of the descriptor's range, reads zero
        const uint32_t go = (uint32_t)min((t * rT + ch * 8) * 2, 0xFFFFFFF0LL);
        raw_buffer_load_lds(rsu, (__attribute__((address_space(3))) uint32_t *)(dst + (i * NW + wave) * 16 * DK), 16,
                            (int)go, (k - D) * 2, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < NBS; ++i) {
      int Gb = i * NW + wave;
      if (Gb >= C::NGB) Gb = wave % C::NGB;
      const int plane = Gb / (D / 16), n = (Gb % (D / 16)) * 16 + lr, ch = (lp ^ (n >> 1)) & 3;
      auto *ld = (__attribute__((address_space(3))) uint32_t *)(dst + (NGA + Gb) * 16 * DK);
      if (k >= D)
        raw_buffer_load_lds(rsd, ld, 16, (int)((plane * dpl_ps + (long long)n * Kd + ch * 8) * 2), (k - D) * 2, 0, 0);
      else
        raw_buffer_load_lds(rsq, ld, 16, (int)((plane * qpl_ps + (long long)n * D + ch * 8) * 2), k * 2, 0, 0);
    }
  };
  // A fragment of codes: rows 128 wr + 16 i + fr, chunk fc (8 codes, b bytes) from the stage's words
  // (bits fc 8 b .. of the row; words past the row's b hold bits no code reads)
  const int qm = (b >= 2) ? ((1 << (b - 1)) - 1) : 1;
  const int cbit = fc * 8 * b, cdw = cbit >> 5, csh = cbit & 31;
  const uint64_t cmask = (b >= 8) ? 0xFFull : ((1ull << b) - 1ull);
  auto cfrag = [&](const lds16 *stage, int i) __attribute__((always_inline)) -> u32x4 {
    const __attribute__((address_space(3))) uint32_t *cl =
        (const __attribute__((address_space(3))) uint32_t *)stage + (wr * C::WR + i * 16 + fr) * 8 + cdw;
    const uint32_t w0 = cl[0], w1 = cl[1], w2 = cl[2];
    const uint64_t lo = ((uint64_t)w1 << 32) | w0;
    const uint64_t w = csh ? ((lo >> csh) | ((uint64_t)w2 << (64 - csh))) : lo;
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int u = (int)((w >> (e * b)) & cmask);
      const float v = (b == 1) ? (u ? 1.f : -1.f) : (float)(u - qm);
      h[e] = (MF == MF_F16) ? (uint32_t)f32_to_f16_rne(v) : (uint32_t)f32_to_bf16_rne(v);
    }
    u32x4 r;
    r[0] = h[0] | (h[1] << 16);
    r[1] = h[2] | (h[3] << 16);
    r[2] = h[4] | (h[5] << 16);
    r[3] = h[6] | (h[7] << 16);
    return r;
  };

  const int aoff = dswz(wr * C::WR + fr, fc), boff = C::ASZ + dswz(wc * C::WC + fr, fc);
  f32x4 acc[TI][TQ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int q = 0; q < TQ; ++q) acc[i][q] = f32x4{0.f, 0.f, 0.f, 0.f};

  issue(L0, kbeg);
  for (int s = 0; s < nsteps; ++s) {
    const int k = kbeg + s * DK;
    lds16 *cur = (s & 1) ? L1 : L0;
    wait_vm<0>();
    wait_lgkm0();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const bool last_codes = k + DK == D;
    float srow[TI];
    if (last_codes) {  // the row scales, needed after this stage's products
#pragma unroll
      for (int i = 0; i < TI; ++i) srow[i] = scales[(long long)j * T + min(t0 + wr * C::WR + i * 16 + fr, T - 1)];
    }
    u32x4 af[TI];
    if (k < D) {
#pragma unroll
      for (int i = 0; i < TI; ++i) af[i] = cfrag(cur, i);
    } else {
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        af[i] = *(const lds_u32x4 *)(cur + aoff + i * 16 * DK);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (s + 1 < nsteps) issue((s & 1) ? L0 : L1, k + DK);
#pragma unroll
    for (int pb = PB - 1; pb >= 0; --pb) {
      if (pb > C::MAXO) continue;
      u32x4 bf[TQ];
#pragma unroll
      for (int q = 0; q < TQ; ++q) {
        bf[q] = *(const lds_u32x4 *)(cur + boff + pb * D * DK + q * 16 * DK);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int q = 0; q < TQ; ++q) acc[i][q] = mfma16<MF>(bf[q], af[i], acc[i][q]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (last_codes) {  // rows times s, into the frame of D_j's planes
      const float f = dscale / qscale;
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const float si = srow[i] * f;
#pragma unroll
        for (int q = 0; q < TQ; ++q)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][q][r] *= si;
      }
    }
  }
  // lane (fr, fc): columns D/2 wc + 16 q + 4 fc + r (r = 0..3) of token row 128 wr + 16 i + fr
  const float inv = 1.f / dscale;
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    const int t = t0 + wr * C::WR + i * 16 + fr;
    if (t >= T) continue;
    char *orow = out + ((long long)j * T + t) * D * 2;
#pragma unroll
    for (int q = 0; q < TQ; ++q) {
      const int n = wc * C::WC + q * 16 + fc * 4;
      uint32_t h[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = acc[i][q][r] * inv;
        h[r] = (MF == MF_F16) ? (uint32_t)f32_to_f16_rne(v) : (uint32_t)f32_to_bf16_rne(v);
      }
      uint2 w2;
      w2.x = h[0] | (h[1] << 16);
      w2.y = h[2] | (h[3] << 16);
      *(uint2 *)(orow + n * 2) = w2;
    }
  }
}

// ------------------------------------------------------------------------------------------ fused decode
// four consecutive elements of a cache-dtype array as floats (one 8- or 16-byte load; idx a multiple of 4)
template <int SX>
__device__ __forceinline__ void load4(const void *base, long long idx, float (&v)[4]) {
  if constexpr (SX == SRC_F32) {
    const float4 f = *(const float4 *)((const float *)base + idx);
    v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
  } else {
    const uint2 w = *(const uint2 *)((const uint16_t *)base + idx);
    const uint32_t h[4] = {w.x & 0xFFFFu, w.x >> 16, w.y & 0xFFFFu, w.y >> 16};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (SX == SRC_F16) v[e] = (float)__builtin_bit_cast(_Float16, (uint16_t)h[e]);
      else v[e] = __builtin_bit_cast(float, h[e] << 16);
    }
  }
}

// The tile rebuild on the DMA pipeline (16-bit caches): rows t0 .. t0 + 127 of head slice j in
// rebuild_tile's accumulator layout (row wm 64 + 16 i + 4 (lane / 16) + r, column wn 64 + 16 q +
// lane % 16 for wave (wm, wn)), real units.  Stages as decode_dma_kernel: the codes' words with Q's
// planes, then U_T rows with D_j's planes (padded pitch, zero past r_T), two stage buffers of
// RCfg::STG halves in lds; srow: BM floats.  Every thread of the block calls it (it synchronises the
// block and leaves lds free).
template <int MF, int D>
struct RCfg {
  static constexpr int NS = 2, ROWS = BM, NW = 4;
  static constexpr int PB = (MF == MF_F16) ? 2 : 3;
  static constexpr int MAXO = (MF == MF_F16) ? 1 : 2;
  static constexpr int ASZ = ROWS * dma::DK, BSZ = PB * D * dma::DK, STG = ASZ + BSZ;
  static constexpr int NGA = ROWS / 16, NGB = PB * D / 16, NA = NGA / NW, NBS = (NGB + NW - 1) / NW;
  static_assert(NGA % NW == 0, "A groups split evenly over the waves");
  static_assert(ROWS * 8 * 4 + 12 <= ASZ * 2, "a stage's code words fit in its A area");
};

template <int MF, int D>
__device__ __forceinline__ void rebuild_tile_dma(const DecCell &c, int j, int t0, int T, uint16_t *lds, float *srow,
                                                 f32x4 (&acc)[4][4]) {
  using C = RCfg<MF, D>;
  using namespace dma;
  constexpr int PB = C::PB, NW = C::NW, NA = C::NA, NBS = C::NBS, NGA = C::NGA, ROWS = C::ROWS;
  lds16 *const L0 = (lds16 *)lds, *const L1 = L0 + C::STG;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1, fr = lane & 15, fc = lane >> 4;
  const int rT = c.rT, b = c.bits, Kd = c.Kd;
  const float qscale = (MF == MF_F16) ? f16_split_scale(1.f) : 1.f;
  const float dscale = (MF == MF_F16) ? f16_split_scale(*c.d_amax) : 1.f;
  const int kbeg = b > 0 ? 0 : D, kend = D + rT;
  const int nsteps = (kend - kbeg + DK - 1) / DK;
  const long long rowbytes = (long long)D * b / 8;
  const i32x4 rsu = make_rsrc(c.UT, (uint32_t)((long long)T * rT * 2));
  const i32x4 rsq = make_rsrc(c.Qpl, 0xFFFFFFFFu);
  const i32x4 rsd = make_rsrc(c.Dpl + (long long)j * D * Kd, 0xFFFFFFFFu);
  const i32x4 rsc = make_rsrc(c.codes + (long long)j * T * rowbytes, (uint32_t)(T * rowbytes));
  const int lr = lane >> 2, lp = lane & 3;
  auto issue = [&](lds16 *dst, int k) __attribute__((always_inline)) {
    if (k < D) {
#pragma unroll
      for (int m = 0; m < ROWS / 8 / NW; ++m) {
        const int rq = m * NW + wave, row = rq * 8 + (lane >> 3);
        const long long off = (long long)(t0 + row) * rowbytes + (k / 8) * b + 4 * (lane & 7);
        raw_buffer_load_lds(rsc, (__attribute__((address_space(3))) uint32_t *)dst + rq * 64, 4,
                            (int)min(off, 0xFFFFFFF0LL), 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const int row = (i * NW + wave) * 16 + lr, ch = (lp ^ (row >> 1)) & 3;
        const long long t = (long long)t0 + row;
        const uint32_t go = (uint32_t)min((t * rT + ch * 8) * 2, 0xFFFFFFF0LL);
        raw_buffer_load_lds(rsu, (__attribute__((address_space(3))) uint32_t *)(dst + (i * NW + wave) * 16 * DK), 16,
                            (int)go, (k - D) * 2, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < NBS; ++i) {
      int Gb = i * NW + wave;
      if (Gb >= C::NGB) Gb = wave % C::NGB;
      const int plane = Gb / (D / 16), n = (Gb % (D / 16)) * 16 + lr, ch = (lp ^ (n >> 1)) & 3;
      auto *ld = (__attribute__((address_space(3))) uint32_t *)(dst + (NGA + Gb) * 16 * DK);
      if (k >= D)
        raw_buffer_load_lds(rsd, ld, 16, (int)((plane * c.dpl_ps + (long long)n * Kd + ch * 8) * 2), (k - D) * 2, 0, 0);
      else
        raw_buffer_load_lds(rsq, ld, 16, (int)((plane * c.qpl_ps + (long long)n * D + ch * 8) * 2), k * 2, 0, 0);
    }
  };
  const int qm = (b >= 2) ? ((1 << (b - 1)) - 1) : 1;
  const int cbit = fc * 8 * b, cdw = cbit >> 5, csh = cbit & 31;
  const uint64_t cmask = (b >= 8) ? 0xFFull : ((1ull << b) - 1ull);
  auto cfrag = [&](const lds16 *stage, int i) __attribute__((always_inline)) -> u32x4 {
    const __attribute__((address_space(3))) uint32_t *cl =
        (const __attribute__((address_space(3))) uint32_t *)stage + (wm * 64 + i * 16 + fr) * 8 + cdw;
    const uint32_t w0 = cl[0], w1 = cl[1], w2 = cl[2];
    const uint64_t lo = ((uint64_t)w1 << 32) | w0;
    const uint64_t w = csh ? ((lo >> csh) | ((uint64_t)w2 << (64 - csh))) : lo;
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int u = (int)((w >> (e * b)) & cmask);
      const float v = (b == 1) ? (u ? 1.f : -1.f) : (float)(u - qm);
      h[e] = (MF == MF_F16) ? (uint32_t)f32_to_f16_rne(v) : (uint32_t)f32_to_bf16_rne(v);
    }
    u32x4 r;
    r[0] = h[0] | (h[1] << 16);
    r[1] = h[2] | (h[3] << 16);
    r[2] = h[4] | (h[5] << 16);
    r[3] = h[6] | (h[7] << 16);
    return r;
  };
  for (int rr = tid; rr < ROWS; rr += NT) srow[rr] = (b > 0 && t0 + rr < T) ? c.scales[(long long)j * T + t0 + rr] : 0.f;
  const int aoff = dswz(wm * 64 + fr, fc), boff = C::ASZ + dswz(wn * 64 + fr, fc);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[i][q] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();  // the caller's last use of lds is over
  issue(L0, kbeg);
  for (int s = 0; s < nsteps; ++s) {
    const int k = kbeg + s * DK;
    lds16 *cur = (s & 1) ? L1 : L0;
    wait_vm<0>();
    wait_lgkm0();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    u32x4 af[4];
    if (k < D) {
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = cfrag(cur, i);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        af[i] = *(const lds_u32x4 *)(cur + aoff + i * 16 * DK);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (s + 1 < nsteps) issue((s & 1) ? L0 : L1, k + DK);
    if (wn * 64 < D) {  // (d_h = 64: the second column wave has no columns)
#pragma unroll
      for (int pb = PB - 1; pb >= 0; --pb) {
        if (pb > C::MAXO) continue;
        u32x4 bf[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          bf[q] = *(const lds_u32x4 *)(cur + boff + pb * D * DK + q * 16 * DK);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[i][q] = mfma16<MF>(af[i], bf[q], acc[i][q]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (k + DK == D) {  // rows times s, into the frame of D_j's planes
      const float f = dscale / qscale;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float si = srow[wm * 64 + i * 16 + fc * 4 + r] * f;
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[i][q][r] *= si;
        }
    }
  }
  const float inv = 1.f / dscale;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][q][r] *= inv;
  __syncthreads();  // every wave is done with the stage buffers
}

// Code of element n of a packed row (b bits, LSB-first, offset binary) as its signed value; reads the
// second byte only when the element reaches into it.
__device__ __forceinline__ float code_at(const uint8_t *rowp, int n, int b) {
  const int bit = n * b, by = bit >> 3, sh = bit & 7;
  unsigned w = rowp[by];
  if (sh + b > 8) w |= (unsigned)rowp[by + 1] << 8;
  const int u = (int)((w >> sh) & ((1u << b) - 1u));
  const int qm = (b >= 2) ? ((1 << (b - 1)) - 1) : 1;
  return (b == 1) ? (u ? 1.f : -1.f) : (float)(u - qm);
}

__device__ __forceinline__ float warp_sum_f(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Attention of one decode step over a token chunk of one KV head (Sec. 4.5): per 128-token tile the
// key rows are rebuilt on chip (rebuild_tile: codes de-rotated plus U_T D_h), rotated by RoPE at their
// positions and scored against the head's G queries; an online softmax state (max m, sum l) is carried
// over the tiles.  Values stay compressed: the weights are accumulated against the value token factor
// (z = sum p U_T^V[t], rank space) and against the scaled value codes (w = sum p s_t u_t, rotated frame);
// the merge expands both once per head.  The block writes its chunk's (m, l, z, w) per query head.
template <int MF, int SX, int NB16, int D, int G8>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(G8 <= 4 ? 2 : 1, G8 <= 4 ? 2 : 1))) attend_kernel(AttnArgs a) {
  constexpr int KP = D + 1, H2 = D / 2, ZU = kAttnMaxRank / NT;
  constexpr int STGB = SX == SRC_F32 ? 2 * DecCfg<MF, SX, NB16>::STG * 2 : RCfg<MF, D>::NS * RCfg<MF, D>::STG * 2;
  constexpr int KTB = BM * KP * 4;
  constexpr int SMB = STGB > KTB ? STGB : KTB;
  // the staging of the tile rebuild and the key tile share the memory (one is done when the other starts)
  __shared__ __attribute__((aligned(1024))) char smem[SMB];
  __shared__ float srow[BM];
  __shared__ float qs[G8 * D];
  __shared__ float ps[G8 * BM];
  __shared__ float alpha_s[G8], m_s[G8], l_s[G8];
  uint16_t *lds = (uint16_t *)smem;
  float *kt = (float *)smem;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, fr = lane & 15;
  const int h = blockIdx.y, ch = blockIdx.x, G = a.G, T = a.T;
  const int tbeg = ch * a.chunk, tend = min(T, tbeg + a.chunk);
  for (int i = tid; i < G * D; i += NT) qs[i] = a.q[(long long)h * G * D + i];
  if (tid < G) {
    m_s[tid] = -INFINITY;
    l_s[tid] = 0.f;
  }
  const int rTv = a.v.rT, bv = a.v.bits, rbv = D * bv / 8;
  // running state: z[g][k] for k = tid + NT u in zr; w[g][n] for n = tid < D in wr
  float zr[ZU][G8], wr[G8];
#pragma unroll
  for (int g = 0; g < G8; ++g) {
    wr[g] = 0.f;
#pragma unroll
    for (int u = 0; u < ZU; ++u) zr[u][g] = 0.f;
  }
  __syncthreads();
  for (int t0 = tbeg; t0 < tend; t0 += BM) {
    f32x4 acc[4][4];
    if constexpr (SX == SRC_F32) rebuild_tile<MF, SX, NB16, DecCfg<MF, SX, NB16>::PB>(a.k, h, t0, T, D, lds, srow, acc);
    else rebuild_tile_dma<MF, D>(a.k, h, t0, T, lds, srow, acc);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wm * 64 + i * 16 + (lane >> 4) * 4 + r;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = wn * 64 + q * 16 + fr;
          if (n < D) kt[row * KP + n] = acc[i][q][r];
        }
      }
    __syncthreads();
    // RoPE: the pair (i, i + D/2) of row t turns by the angle of (t, i).  Thread: pair i = tid % H2 of
    // rows tid / H2 + RS k; the table entries of 8 rows are requested together
    {
      constexpr int RS = NT / H2, RR = BM / RS, RB2 = 8;
      const int i = tid % H2, rbase = tid / H2;
      const float2 *tab = (const float2 *)a.rope;
#pragma unroll
      for (int k0 = 0; k0 < RR; k0 += RB2) {
        float2 cs[RB2];
#pragma unroll
        for (int k = 0; k < RB2; ++k) {
          const int t = min(t0 + rbase + RS * (k0 + k), tend - 1);
          cs[k] = tab[(long long)t * H2 + i];
        }
#pragma unroll
        for (int k = 0; k < RB2; ++k) {
          float *kr = kt + (rbase + RS * (k0 + k)) * KP;
          const float x0 = kr[i], x1 = kr[i + H2];
          kr[i] = x0 * cs[k].x - x1 * cs[k].y;
          kr[i + H2] = x1 * cs[k].x + x0 * cs[k].y;
        }
      }
    }
    __syncthreads();
    // scores: thread pair (2 row, 2 row + 1) takes row `row`, each half of the columns for every head
    // (the key row is read once for all heads; the query reads are the same address across the wave)
    {
      const int row = tid >> 1, half = tid & 1;
      const float *kr = kt + row * KP + half * H2, *qh = qs + half * H2;
      float d[G8];
#pragma unroll
      for (int g = 0; g < G8; ++g) d[g] = 0.f;
#pragma unroll 4
      for (int n = 0; n < H2; ++n) {
        const float kv = kr[n];
#pragma unroll
        for (int g = 0; g < G8; ++g)
          if (g < G) d[g] = fmaf(kv, qh[g * D + n], d[g]);
      }
      const bool live = t0 + row < tend;
#pragma unroll
      for (int g = 0; g < G8; ++g) {
        const float v = d[g] + __shfl_xor(d[g], 1, 64);
        if (g < G && half == 0) ps[g * BM + row] = live ? v * a.scale : -INFINITY;
      }
    }
    __syncthreads();
    // online softmax per query head (every tile holds at least one token of the chunk)
    for (int g = wave; g < G; g += NT / 64) {
      const float v0 = ps[g * BM + lane], v1 = ps[g * BM + 64 + lane];
      const float mo = m_s[g], mn = fmaxf(mo, warp_max(fmaxf(v0, v1)));
      const float p0 = expf(v0 - mn), p1 = expf(v1 - mn);
      ps[g * BM + lane] = p0;
      ps[g * BM + 64 + lane] = p1;
      const float sm = warp_sum_f(p0 + p1);
      if (lane == 0) {
        const float al = expf(mo - mn);
        alpha_s[g] = al;
        l_s[g] = fmaf(l_s[g], al, sm);
        m_s[g] = mn;
      }
    }
    __syncthreads();
    float al[G8];
#pragma unroll
    for (int g = 0; g < G8; ++g) al[g] = g < G ? alpha_s[g] : 0.f;
    const int nrow = min(BM, tend - t0);
    // The tile's value sums, each as one batch of independent wide loads per thread, then reduced in a
    // fixed order (lanes by shuffles, waves through the dead key tile).
    float *vpart = kt;  // [4 waves][G8][128]
    const int lane6 = tid & 63, wv = tid >> 6;
    // value token factor, rank space: z[g][k] += sum_t p[g][t] U_T^V[t][k]; lane (q4, row group rg):
    // ranks kb + 4 q4 .. + 3, rows rg + 8 i (i < 16)
    {
      const int q4 = tid & 31, rg = tid >> 5;
#pragma unroll
      for (int u = 0; u < ZU; ++u)
#pragma unroll
        for (int g = 0; g < G8; ++g) zr[u][g] *= al[g];
      for (int kb = 0; kb < rTv; kb += 128) {
        const int k4 = kb + 4 * q4;
        float za[G8][4];
#pragma unroll
        for (int g = 0; g < G8; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e) za[g][e] = 0.f;
        if (k4 < rTv) {
          float uv[16][4];
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row = rg + 8 * i;
            if (row < nrow) load4<SX>(a.v.UT, (long long)(t0 + row) * rTv + k4, uv[i]);
            else uv[i][0] = uv[i][1] = uv[i][2] = uv[i][3] = 0.f;
          }
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row = rg + 8 * i;
#pragma unroll
            for (int g = 0; g < G8; ++g) {
              if (g >= G) continue;
              const float pg = ps[g * BM + row];
#pragma unroll
              for (int e = 0; e < 4; ++e) za[g][e] = fmaf(pg, uv[i][e], za[g][e]);
            }
          }
        }
#pragma unroll
        for (int g = 0; g < G8; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e) za[g][e] += __shfl_xor(za[g][e], 32, 64);
        if (lane6 < 32 && k4 < rTv)
#pragma unroll
          for (int g = 0; g < G8; ++g)
            if (g < G)
#pragma unroll
              for (int e = 0; e < 4; ++e) vpart[(wv * G8 + g) * 128 + 4 * q4 + e] = za[g][e];
        __syncthreads();
        // owner of rank k = kb + c: thread k % NT, slot k / NT
        const int c = tid - (kb % NT);
        if (c >= 0 && c < 128 && kb + c < rTv) {
          const int u = kb / NT;
#pragma unroll
          for (int uu = 0; uu < ZU; ++uu)
            if (uu == u)
#pragma unroll
              for (int g = 0; g < G8; ++g)
                if (g < G)
                  zr[uu][g] += ((vpart[(0 * G8 + g) * 128 + c] + vpart[(1 * G8 + g) * 128 + c]) +
                                vpart[(2 * G8 + g) * 128 + c]) + vpart[(3 * G8 + g) * 128 + c];
        }
        __syncthreads();
      }
    }
    // value residual, rotated frame: w[g][n] += sum_t p[g][t] s_t c_t[n]; lane (c8, row group rg):
    // columns 8 c8 .. + 7 (b bytes of a packed row), rows rg + 16 i (i < 8)
#pragma unroll
    for (int g = 0; g < G8; ++g) wr[g] *= al[g];
    if (bv > 0) {
      const int c8 = tid & 15, rg = tid >> 4;
      const int qmv = (bv >= 2) ? ((1 << (bv - 1)) - 1) : 1;
      const uint64_t cmask = (bv >= 8) ? 0xFFull : ((1ull << bv) - 1ull);
      const int off = c8 * bv, a0 = off & ~3, sh = (off & 3) * 8;
      float wa[G8][8];
#pragma unroll
      for (int g = 0; g < G8; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) wa[g][e] = 0.f;
      if (c8 < D / 8) {
        uint32_t cw[8][3];
        float sv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int row = rg + 16 * i;
          if (row < nrow) {
            const long long vr = (long long)h * T + t0 + row;
            const uint32_t *w = (const uint32_t *)(a.v.codes + vr * rbv + a0);
            sv[i] = a.v.scales[vr];
            cw[i][0] = w[0];
            cw[i][1] = (a0 + 4 < rbv) ? w[1] : 0u;
            cw[i][2] = (a0 + 8 < rbv) ? w[2] : 0u;
          } else {
            sv[i] = 0.f;
            cw[i][0] = cw[i][1] = cw[i][2] = 0u;
          }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int row = min(rg + 16 * i, BM - 1);
          const uint64_t lo = ((uint64_t)cw[i][1] << 32) | cw[i][0];
          const uint64_t wbits = sh ? ((lo >> sh) | ((uint64_t)cw[i][2] << (64 - sh))) : lo;
          float cv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int u = (int)((wbits >> (e * bv)) & cmask);
            cv[e] = (bv == 1) ? (u ? 1.f : -1.f) : (float)(u - qmv);
          }
#pragma unroll
          for (int g = 0; g < G8; ++g) {
            if (g >= G) continue;
            const float pg = ps[g * BM + row] * sv[i];
#pragma unroll
            for (int e = 0; e < 8; ++e) wa[g][e] = fmaf(pg, cv[e], wa[g][e]);
          }
        }
      }
#pragma unroll
      for (int g = 0; g < G8; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          wa[g][e] += __shfl_xor(wa[g][e], 16, 64);
          wa[g][e] += __shfl_xor(wa[g][e], 32, 64);
        }
      if (lane6 < 16 && c8 < D / 8)
#pragma unroll
        for (int g = 0; g < G8; ++g)
          if (g < G)
#pragma unroll
            for (int e = 0; e < 8; ++e) vpart[(wv * G8 + g) * 128 + 8 * c8 + e] = wa[g][e];
      __syncthreads();
      if (tid < D)
#pragma unroll
        for (int g = 0; g < G8; ++g)
          if (g < G)
            wr[g] += ((vpart[(0 * G8 + g) * 128 + tid] + vpart[(1 * G8 + g) * 128 + tid]) +
                      vpart[(2 * G8 + g) * 128 + tid]) + vpart[(3 * G8 + g) * 128 + tid];
    }
    __syncthreads();
  }
  // the chunk's state
  float *P = a.part + (long long)(ch * a.H + h) * G * a.PS;
  if (tid < D)
#pragma unroll
    for (int g = 0; g < G8; ++g)
      if (g < G) P[(long long)g * a.PS + 2 + a.rtv_ld + tid] = wr[g];
#pragma unroll
  for (int u = 0; u < ZU; ++u) {
    const int k = tid + NT * u;
    if (k < rTv)
#pragma unroll
      for (int g = 0; g < G8; ++g)
        if (g < G) P[(long long)g * a.PS + 2 + k] = zr[u][g];
  }
  if (tid < G) {
    P[(long long)tid * a.PS] = m_s[tid];
    P[(long long)tid * a.PS + 1] = l_s[tid];
  }
}

// Merge of the chunk states of one query head (fixed chunk order), with the dense tail (its keys
// rotated at positions T ..), then the expansion out = (z D_h^V + w Q^T + sum_tail p v) / l.
template <int SX>
__global__ void __launch_bounds__(256) attend_merge_kernel(AttnMergeArgs a) {
  __shared__ float wc[kAttnMaxChunks];
  __shared__ float ts[kAttnMaxTail];
  __shared__ float zs[kAttnMaxRank];
  __shared__ float wsum[128];
  __shared__ float Ls;
  const int hg = blockIdx.x, h = hg / a.G, g = hg - h * a.G;
  const int tid = threadIdx.x, D = a.D, H2 = D / 2;
  const float *qg = a.q + (long long)hg * D;
  for (int i = tid; i < a.n_tail; i += 256) {
    const long long base = ((long long)h * a.n_tail + i) * D;
    const long long t = a.T + i;
    float d = 0.f;
    for (int n = 0; n < H2; ++n) {
      const float cs = a.rope[(t * H2 + n) * 2], sn = a.rope[(t * H2 + n) * 2 + 1];
      const float x0 = load_elem<SX>(a.k_tail, base + n), x1 = load_elem<SX>(a.k_tail, base + n + H2);
      d = fmaf(x0 * cs - x1 * sn, qg[n], d);
      d = fmaf(x1 * cs + x0 * sn, qg[n + H2], d);
    }
    ts[i] = d * a.scale;
  }
  __syncthreads();
  auto part = [&](int c) { return a.part + ((long long)(c * a.H + h) * a.G + g) * a.PS; };
  if (tid == 0) {
    float M = -INFINITY;
    for (int c = 0; c < a.n_chunks; ++c) M = fmaxf(M, part(c)[0]);
    for (int i = 0; i < a.n_tail; ++i) M = fmaxf(M, ts[i]);
    float L = 0.f;
    for (int c = 0; c < a.n_chunks; ++c) {
      const float e = expf(part(c)[0] - M);
      wc[c] = e;
      L = fmaf(e, part(c)[1], L);
    }
    for (int i = 0; i < a.n_tail; ++i) {
      const float e = expf(ts[i] - M);
      ts[i] = e;
      L += e;
    }
    Ls = L;
  }
  __syncthreads();
  for (int k = tid; k < a.rTv; k += 256) {
    float z = 0.f;
    for (int c = 0; c < a.n_chunks; ++c) z = fmaf(wc[c], part(c)[2 + k], z);
    zs[k] = z;
  }
  for (int n = tid; n < D; n += 256) {
    float w = 0.f;
    if (a.bits_v > 0)
      for (int c = 0; c < a.n_chunks; ++c) w = fmaf(wc[c], part(c)[2 + a.rtv_ld + n], w);
    wsum[n] = w;
  }
  __syncthreads();
  for (int n = tid; n < D; n += 256) {
    const float *dm = a.DmV + ((long long)h * D + n) * a.Kd;
    float o = 0.f;
    for (int k = 0; k < a.rTv; ++k) o = fmaf(zs[k], dm[k], o);
    if (a.bits_v > 0)
      for (int k = 0; k < D; ++k) o = fmaf(wsum[k], a.Q[(long long)n * D + k], o);
    for (int i = 0; i < a.n_tail; ++i) o = fmaf(ts[i], load_elem<SX>(a.v_tail, ((long long)h * a.n_tail + i) * D + n), o);
    a.out[(long long)hg * D + n] = o / Ls;
  }
}

// G8: the number of query heads per KV head the kernel is built for (its registers hold that many
// states); up to 4 (grouped-query models) or up to 8
template <int MF, int SX, int NB16>
void launch_attend(const AttnArgs &a, hipStream_t st) {
  const dim3 grid(a.n_chunks, a.H);
  if (a.G <= 4) {
    if (a.D == 128) hipLaunchKernelGGL((attend_kernel<MF, SX, NB16, 128, 4>), grid, dim3(NT), 0, st, a);
    else hipLaunchKernelGGL((attend_kernel<MF, SX, NB16, 64, 4>), grid, dim3(NT), 0, st, a);
  } else {
    if (a.D == 128) hipLaunchKernelGGL((attend_kernel<MF, SX, NB16, 128, 8>), grid, dim3(NT), 0, st, a);
    else hipLaunchKernelGGL((attend_kernel<MF, SX, NB16, 64, 8>), grid, dim3(NT), 0, st, a);
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
template <int MF, int TN, int NS>
void launch_enc_dma(const EncArgs &a, int ncells, int T, int GHmax, hipStream_t st) {
  using C = XCfg<MF, TN, NS, 2>;
  const int tt = (T + C::ROWS - 1) / C::ROWS;
  hipLaunchKernelGGL((encode_dma_kernel<MF, TN, NS, 2>), dim3(tt * GHmax, 1, ncells), dim3(C::NT), 0, st, a, T, tt,
                     GHmax);
}

template <int MF, int TN>
void launch_dec_dma(const DecCell *cells, int ncells, int T, int GHmax, hipStream_t st) {
  using C = YCfg<MF, TN>;
  const int tt = (T + C::ROWS - 1) / C::ROWS;
  hipLaunchKernelGGL((decode_dma_kernel<MF, TN>), dim3(tt * GHmax, 1, ncells), dim3(C::NT), 0, st, cells, T, tt, GHmax);
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
  // 16-bit caches: the DMA-fed kernel (B rows padded with zeros to a multiple of 32); fp32 caches carry
  // A in three planes split while loading and keep the register-staged kernel
  if (D == 128) {
    if (dtype == JOLT_F16) launch_enc_dma<MF_F16, 8, 2>(a, ncells, T, GHmax, st);
    else if (dtype == JOLT_BF16) launch_enc_dma<MF_BF16, 8, 2>(a, ncells, T, GHmax, st);
    else launch_enc<MF_BF16, SRC_F32, 8>(a, ncells, T, GHmax, st);
  } else {
    if (dtype == JOLT_F16) launch_enc_dma<MF_F16, 4, 3>(a, ncells, T, GHmax, st);
    else if (dtype == JOLT_BF16) launch_enc_dma<MF_BF16, 4, 2>(a, ncells, T, GHmax, st);
    else launch_enc<MF_BF16, SRC_F32, 4>(a, ncells, T, GHmax, st);
  }
  HIP_LAUNCH_CHECK();
}

void attend_cells(int dtype, const AttnArgs &a, hipStream_t st) {
  JOLT_REQUIRE(a.D == 64 || a.D == 128, JOLT_EINVAL, "attention: d_head must be 64 or 128");
  JOLT_REQUIRE(a.G >= 1 && a.G <= kAttnMaxG && a.v.rT <= kAttnMaxRank && a.n_chunks >= 1 &&
                   a.n_chunks <= kAttnMaxChunks && a.chunk % BM == 0,
               JOLT_EINVAL, "attention: launch shape out of range");
  if (dtype == JOLT_F16) launch_attend<MF_F16, SRC_F16, 2>(a, st);
  else if (dtype == JOLT_BF16) launch_attend<MF_BF16, SRC_BF16, 2>(a, st);
  else launch_attend<MF_BF16, SRC_F32, 2>(a, st);
  HIP_LAUNCH_CHECK();
}

void attend_merge(int dtype, const AttnMergeArgs &m, hipStream_t st) {
  JOLT_REQUIRE(m.n_chunks >= 1 && m.n_chunks <= kAttnMaxChunks && m.n_tail >= 0 && m.n_tail <= kAttnMaxTail &&
                   m.rTv <= kAttnMaxRank && m.D <= 128,
               JOLT_EINVAL, "attention merge: shape out of range");
  const dim3 grid(m.H * m.G);
  if (dtype == JOLT_F16) hipLaunchKernelGGL(attend_merge_kernel<SRC_F16>, grid, dim3(256), 0, st, m);
  else if (dtype == JOLT_BF16) hipLaunchKernelGGL(attend_merge_kernel<SRC_BF16>, grid, dim3(256), 0, st, m);
  else hipLaunchKernelGGL(attend_merge_kernel<SRC_F32>, grid, dim3(256), 0, st, m);
  HIP_LAUNCH_CHECK();
}

void decode_cells(int dtype, const DecCell *d_cells, int ncells, int T, int D, int GHmax, hipStream_t st) {
  JOLT_REQUIRE(D == 64 || D == 128, JOLT_EINVAL, "codec: d_head must be 64 or 128");
  // 16-bit caches: the DMA-fed kernel (D_j planes zero-padded to a multiple of 32 columns); fp32
  // caches keep the register-staged tile rebuild
  if (dtype == JOLT_F16) {
    if (D == 128) launch_dec_dma<MF_F16, 8>(d_cells, ncells, T, GHmax, st);
    else launch_dec_dma<MF_F16, 4>(d_cells, ncells, T, GHmax, st);
  } else if (dtype == JOLT_BF16) {
    if (D == 128) launch_dec_dma<MF_BF16, 8>(d_cells, ncells, T, GHmax, st);
    else launch_dec_dma<MF_BF16, 4>(d_cells, ncells, T, GHmax, st);
  } else {
    launch_dec<MF_BF16, SRC_F32, 2>(d_cells, ncells, T, D, GHmax, st);
  }
  HIP_LAUNCH_CHECK();
}

}  // namespace jolt
