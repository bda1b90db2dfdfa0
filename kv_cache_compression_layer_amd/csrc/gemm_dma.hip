// Dense contractions on 16-bit planes that sit in memory, both operands contiguous along K,
// fed by the gfx950 global->LDS DMA path (global_load_lds_dwordx4).
//
// Arithmetic is that of gemm_kc.hip: 16x16x32 MFMA over the planes of each operand (fp32 values
// pre-split into hi/lo fp16 planes after the same power-of-two scale, or into three bf16 planes),
// plane products taken in the same order inside each 32-deep k step, so every output element
// sees the same sequence of fp32 accumulations as there.  What differs is how the matrix cores
// are fed:
//   * eight waves per block (4 x 2), two per SIMD, each owning TM x TN 16 x 16 subtiles (48 x 128
//     for the fp32-plane products: 192 x 256 blocks) with the accumulators in registers;
//   * operand tiles go from global memory straight into LDS (no staging registers, no VALU):
//     lane l of a DMA instruction writes bytes [16 l, 16 l + 16) of a 1 KB run, i.e. chunk l % 4
//     of row l / 4 of a 16-row group, so the lane loads whichever logical chunk the row's XOR
//     permutation puts there and the fragment reads stay free of bank conflicts;
//   * NS LDS stages: stage s + NS - 1 is requested before stage s is multiplied, so global
//     latency is covered by NS - 1 stages of matrix-core work;
//   * fragment reads are issued in the order the MFMAs consume them (pinned by scheduling
//     barriers), so a wave's first MFMAs start after two reads instead of after the whole stage.
// Operands are zero-padded along K to a multiple of 32 in memory; rows past M (N) read a valid
// row and their results are dropped.
//
// B may instead be contiguous along N (BKC = false: B(k, n) at k * b_ld + n, n blocked by b_blk /
// b_blk_stride), as a token-major cache is for a product that contracts over tokens.  Its stage is
// then 32 k-rows of the block's 256 columns, each row 16 slots of 16 columns whose order is XOR-
// permuted by the row (rowswz), and each fragment of 8 consecutive k for one column comes from two
// transposing LDS reads (ds_read_b64_tr_b16: in every 16-lane group, lane i receives element i % 4
// of the 64 bits addressed by lane 4 q + i / 4 as its q-th value).  The 16 rows one such read
// touches sit in 16 different slots, so the reads are free of bank conflicts.
#include <type_traits>

#include "common.hpp"
#include "gemm_core.hpp"
#include "dma.hpp"

namespace jolt {

namespace {

using namespace core;
using namespace dma;

template <int MF, int PA, int PB, int TM, int TN, int NS, int NWM, int NWN>
struct Cfg {
  static constexpr int NW = NWM * NWN, NT = 64 * NW;  // waves (NWM x NWN) and threads per block
  static constexpr int WM = TM * 16, WN = TN * 16, BM = NWM * WM, BN = NWN * WN;
  static constexpr int ASZ = PA * BM * DK, BSZ = PB * BN * DK, STG = ASZ + BSZ;  // halves per stage
  // 16-row groups of a stage: A planes' groups then B planes' (the LDS stage holds them in that
  // order, 1 KB each); wave w requests groups w, w + NW, ... -- ND per wave, a wave without a last
  // group repeats its first one (same bytes to the same place)
  static constexpr int NGA = PA * BM / 16, NG = NGA + PB * BN / 16;
  static constexpr int ND = (NG + NW - 1) / NW;
  static constexpr int MAXO = (MF == MF_F16) ? 1 : 2;  // plane products with order pa + pb <= MAXO
  static_assert(NW <= NG, "every wave needs a group of its own");
  static_assert(NS >= 2 && NS <= 6, "LDS stage count");
  static_assert(NS * STG * 2 <= 160 * 1024, "the stages must fit in LDS");
  static_assert((NS - 2) * ND < 64, "vmcnt range");
};

// one stage of DMA requests of this wave into stage buffer `dst`: slot i loads group gi[i] from
// operand A (isa bit i) or B at per-lane offset go[i] plus the stage's k position ak / bk
template <class C>
__device__ __forceinline__ void issue(lds16 *__restrict__ dst, i32x4 ra, i32x4 rb, uint32_t ak, uint32_t bk,
                                      const uint32_t (&go)[C::ND], const int (&gi)[C::ND], uint32_t isa) {
#pragma unroll
  for (int i = 0; i < C::ND; ++i) {
    const bool a = (isa >> i) & 1;
    raw_buffer_load_lds(a ? ra : rb, (__attribute__((address_space(3))) uint32_t *)(dst + gi[i] * 16 * DK), 16,
                        (int)go[i], (int)(a ? ak : bk), 0, 0);
  }
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// slot permutation of k-row r of an N-contiguous B stage: any 16 rows {8 g + q + 4 h : g, q < 4}
// (fixed h) get 16 different values
__device__ __forceinline__ int rowswz(int r) { return (r & 3) | ((r >> 3) << 2); }

template <class C, int PA, int PB, int TM, int TN>
struct Frags {
  u32x4 a[PA][TM];
  u32x4 b[PB][TN];
};

// fragment reads in the order the MFMAs consume them (the first A fragment, the B plane of the
// first plane product, the rest of that A plane, then the other planes), so the in-order LDS
// return lets the first MFMAs start after a few reads
template <class C, int PA, int PB, int TM, int TN, bool BKC>
__device__ __forceinline__ void read_frags(const lds16 *__restrict__ src, int aoff, int boff, const int (&btr)[TN],
                                           Frags<C, PA, PB, TM, TN> &f) {
  constexpr int PB0 = (PB - 1 < C::MAXO - (PA - 1)) ? PB - 1 : (C::MAXO - (PA - 1) > 0 ? C::MAXO - (PA - 1) : 0);
  // (a scheduling barrier after each read pins the issue order, which the scheduler would otherwise
  // regroup by address so that the first MFMA waits for nearly every read of the stage)
  auto ra = [&](int p, int i) __attribute__((always_inline)) {
    f.a[p][i] = *(const lds_u32x4 *)(src + p * C::BM * DK + i * 16 * DK + aoff);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto rb = [&](int p, int j) __attribute__((always_inline)) {
    if constexpr (BKC) {
      f.b[p][j] = *(const lds_u32x4 *)(src + C::ASZ + p * C::BN * DK + j * 16 * DK + boff);
    } else {
      // k rows r and r + 4 of the lane's 16-lane group (8 consecutive k in all)
      const lds16 *q = src + C::ASZ + p * C::BN * DK + btr[j];
      const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)q));
      const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(q + 4 * C::BN)));
      f.b[p][j] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  ra(PA - 1, 0);
#pragma unroll
  for (int j = 0; j < TN; ++j) rb(PB0, j);
#pragma unroll
  for (int i = 1; i < TM; ++i) ra(PA - 1, i);
#pragma unroll
  for (int p = PB - 1; p >= 0; --p)
    if (p != PB0)
#pragma unroll
      for (int j = 0; j < TN; ++j) rb(p, j);
#pragma unroll
  for (int p = PA - 2; p >= 0; --p)
#pragma unroll
    for (int i = 0; i < TM; ++i) ra(p, i);
}

// MFMAs of one stage over the output columns [J0, J1) of the wave; the plane products of each
// output element run in the order of gemm_kc.hip (A plane descending, then B plane descending).
template <int MF, class C, int PA, int PB, int TM, int TN, int J0, int J1, bool FULL>
__device__ __forceinline__ void mfmas(const Frags<C, PA, PB, TM, TN> &f, f32x4 (&acc)[TM][TN], int mlive, int nlive) {
  // each plane product is one group of independent MFMAs (one per accumulator); the scheduling
  // barrier between groups keeps the scheduler from interleaving two products of one accumulator,
  // which makes the register allocator copy accumulators instead of updating them in place
#pragma unroll
  for (int pa = PA - 1; pa >= 0; --pa)
#pragma unroll
    for (int pb = PB - 1; pb >= 0; --pb) {
      if (pa + pb > C::MAXO) continue;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = J0; j < J1; ++j) {
          if constexpr (FULL) acc[i][j] = mfma16<MF>(f.a[pa][i], f.b[pb][j], acc[i][j]);
          else if (i < mlive && j < nlive) acc[i][j] = mfma16<MF>(f.a[pa][i], f.b[pb][j], acc[i][j]);
        }
      __builtin_amdgcn_sched_barrier(0);
    }
}

template <int MF, int PA, int PB, int TM, int TN, int NS, int NWM, int NWN, bool BKC, bool OPL>
__global__ void __launch_bounds__(64 * NWM * NWN) __attribute__((amdgpu_waves_per_eu(NWM * NWN / 4, NWM * NWN / 4)))
gemm_dma_kernel(GemmArgs g) {
  using C = Cfg<MF, PA, PB, TM, TN, NS, NWM, NWN>;
  static_assert(BKC || C::BN == 256, "an N-contiguous B stage is 16 slots of 16 columns per k-row");
  using F = Frags<C, PA, PB, TM, TN>;
  constexpr int BM = C::BM, BN = C::BN, WM = C::WM, WN = C::WN;
  __shared__ __attribute__((aligned(1024))) uint16_t lds_raw[NS * C::STG];
  lds16 *const L0 = (lds16 *)lds_raw, *const Llast = L0 + (NS - 1) * C::STG;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // XCD-aware remap over the whole grid (linear block L runs on XCD L % 8): each XCD gets one
  // contiguous range of (batch, split, tile), so operand panels stream through one L2.
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
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  int tm, tn;
  if (g.m_fastest) { tm = t % tiles_m; tn = t / tiles_m; }
  else { tn = t % tiles_n; tm = t / tiles_n; }
  const int m0 = tm * BM, n0 = tn * BN;

  const int kbeg = split * g.k_chunk;
  int kend = min(g.K, kbeg + g.k_chunk);
  if (kbeg >= kend && split > 0) return;
  if (g.tri & 2) kend = min(kend, n0 + BN);
  if (g.tri & 4) kend = min(kend, m0 + BM);         // A lower triangular: A(m, k) = 0 for k > m
  if ((g.tri & 1) && m0 >= n0 + BN) kend = kbeg;  // strictly below the diagonal: zeros
  const int nsteps = max(0, (kend - kbeg + DK - 1) / DK);

  const char *Ab = (const char *)g.A + (batch * g.a_bs + bin * g.a_bs2) * 2;
  const char *Bb = (const char *)g.B + (batch * g.b_bs + bin * g.b_bs2) * 2;
  float ascale = 1.f, bscale = 1.f;
  if constexpr (PA > 1 && MF == MF_F16)
    ascale = f16_split_scale(g.a_amax ? g.a_amax[(long long)batch * g.ab_amax_bs] : g.a_amax_c);
  if constexpr (PB > 1 && MF == MF_F16)
    bscale = f16_split_scale(g.b_amax ? g.b_amax[(long long)batch * g.ab_amax_bs] : g.b_amax_c);

  // per-lane byte offsets of the DMA sources (row part and permuted chunk), fixed over k
  constexpr int ND = C::ND, NGA = C::NGA, NG = C::NG;
  uint32_t go[ND];
  int gi[ND];
  uint32_t isa = 0;
  {
    const int r = lane >> 2, p = lane & 3;
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      int G = i * C::NW + wave;
      if (G >= NG) G = wave;
      gi[i] = G;
      if (G < NGA) {
        isa |= 1u << i;
        const int plane = G / (BM / 16), row = (G % (BM / 16)) * 16 + r;
        const int c = (p ^ (row >> 1)) & 3;
        const int m = min(m0 + row, g.M - 1);
        go[i] = (uint32_t)((plane * g.a_ps + (long long)m * g.a_ld + c * 8) * 2);
      } else if constexpr (BKC) {
        const int Gb = G - NGA, plane = Gb / (BN / 16), row = (Gb % (BN / 16)) * 16 + r;
        const int c = (p ^ (row >> 1)) & 3;
        const int n = min(n0 + row, g.N - 1);
        go[i] = (uint32_t)((plane * g.b_ps + (long long)n * g.b_ld + c * 8) * 2);
      } else {
        // group = k-rows 2 gb and 2 gb + 1 (512 bytes each); lane l fills 16-byte chunk l % 32 of
        // row l / 32, i.e. half (l & 1) of physical slot (l % 32) / 2, which holds logical slot
        // (l % 32) / 2 ^ rowswz(row); columns past N read the last valid chunk (results dropped)
        const int Gb = G - NGA, plane = Gb / (BN / 16), kr = (Gb % (BN / 16)) * 2 + (lane >> 5);
        const int ch = lane & 31, slot = (ch >> 1) ^ rowswz(kr);
        const int n = min(n0 + slot * 16 + (ch & 1) * 8, g.N - 8);
        const long long nb = (long long)(n / g.b_blk) * g.b_blk_stride + n % g.b_blk;
        go[i] = (uint32_t)((plane * g.b_ps + (long long)kr * g.b_ld + nb) * 2);
      }
    }
  }
  // byte offset (from the batch base) of the next stage to request, in blocked addressing
  // (k -> (k / blk) * stride + k % blk); descriptors cover the whole 32-bit offset range, every
  // offset formed here is inside the operand (checked by the host)
  const i32x4 rsa = make_rsrc(Ab, 0xFFFFFFFFu), rsb = make_rsrc(Bb, 0xFFFFFFFFu);
  // (an N-contiguous B advances by 32 rows of b_ld per stage; its blocking is along N)
  int ak = kbeg % g.a_blk, bk = BKC ? kbeg % g.b_blk : 0;
  uint32_t aso = (uint32_t)(((long long)(kbeg / g.a_blk) * g.a_blk_stride + ak) * 2);
  uint32_t bso = BKC ? (uint32_t)(((long long)(kbeg / g.b_blk) * g.b_blk_stride + bk) * 2)
                     : (uint32_t)((long long)kbeg * g.b_ld * 2);
  const uint32_t ajump = (uint32_t)((g.a_blk_stride - g.a_blk) * 2), bjump = (uint32_t)((g.b_blk_stride - g.b_blk) * 2);
  const uint32_t bstep = BKC ? DK * 2 : (uint32_t)(DK * g.b_ld * 2);
  auto advance = [&]() __attribute__((always_inline)) {
    ak += DK;
    aso += DK * 2;
    if (ak == g.a_blk) { ak = 0; aso += ajump; }
    bso += bstep;
    if constexpr (BKC) {
      bk += DK;
      if (bk == g.b_blk) { bk = 0; bso += bjump; }
    }
  };

  const int wm = wave / NWN, wn = wave % NWN;
  const int fr = lane & 15, fc = lane >> 4;
  const int aoff = dswz(wm * WM + fr, fc), boff = dswz(wn * WN + fr, fc);
  // N-contiguous B: half offset of the first transposing read of subtile j (rows 8 (lane / 16) +
  // (lane / 4) % 4, whose slot permutation is lane / 4; columns 4 (lane % 4) of the slot)
  int btr[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j)
    btr[j] = BKC ? 0
                 : (8 * (lane >> 4) + ((lane >> 2) & 3)) * BN + (((wn * TN + j) ^ (lane >> 2)) << 4) + 4 * (lane & 3);

  // Stage q's requests.  An N-contiguous B with fewer valid rows than K (b_krows): in the stage that
  // holds the last valid row, lanes whose k-row lies past it load that row instead (A is zero in
  // those columns, so the products add exact zeros and no request leaves B).
  // (only a B in planes -- a basis, ell rows -- can be ragged; the cache always fills its stages)
  constexpr bool KCLAMP = !BKC && PB > 1;
  const int kvalid = (KCLAMP && g.b_krows > 0) ? g.b_krows : 0x7FFFFFFF;
  const uint32_t brow = (uint32_t)(g.b_ld * 2);
  auto issue_q = [&](lds16 *dst, int q) __attribute__((always_inline)) {
    if constexpr (KCLAMP) {
      const int krem = kvalid - (kbeg + q * DK);  // valid rows in this stage (wave-uniform)
      if (krem < DK) {
        uint32_t gt[ND];
#pragma unroll
        for (int i = 0; i < ND; ++i) {
          gt[i] = go[i];
          if (!((isa >> i) & 1)) {
            const int kr = ((gi[i] - NGA) % (BN / 16)) * 2 + (lane >> 5);
            if (kr >= krem) gt[i] -= (uint32_t)(kr - (krem - 1)) * brow;
          }
        }
        issue<C>(dst, rsa, rsb, aso, bso, gt, gi, isa);
        return;
      }
    }
    issue<C>(dst, rsa, rsb, aso, bso, go, gi, isa);
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Every subtile is multiplied, also those past M or N (their rows read a valid row and their
  // results are not stored): in a tile that is partly outside, the other wave of the same rows or
  // columns is fully inside and sets the block's time anyway.
  // Stage s: once stage s has landed everywhere (which also means every wave is done reading
  // stage s - 1), request stage s + 2 into stage s - 1's buffer, then read and multiply stage s.
  if (nsteps > 0) {
    {
      F fx;
      // prologue: stages 0 .. NS - 2 in flight
      lds16 *far = L0;
#pragma unroll
      for (int q = 0; q < NS - 1; ++q)
        if (q < nsteps) {
          issue_q(far, q);
          advance();
          far += C::STG;
        }
      lds16 *cur = L0;
      for (int s = 0; s < nsteps; ++s) {
        // stage s is complete once at most min(NS - 2, nsteps - 1 - s) later stages are in flight
        const int later = min(NS - 2, nsteps - 1 - s);
        wait_stages<C::ND, NS - 2>(later);
        wait_lgkm0();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (s + NS - 1 < nsteps) {
          issue_q(far, s + NS - 1);
          advance();
        }
        read_frags<C, PA, PB, TM, TN, BKC>(cur, aoff, boff, btr, fx);
        __builtin_amdgcn_sched_barrier(0);
        mfmas<MF, C, PA, PB, TM, TN, 0, TN, true>(fx, acc, 0, 0);
        cur = cur == Llast ? L0 : cur + C::STG;
        far = far == Llast ? L0 : far + C::STG;
      }
    }
  }

  const float cs = g.alpha / (ascale * bscale);
  if constexpr (OPL) {
    // Output as two fp16 planes (the split of split_planes, scale of the bound cpl_amax).  The tile is
    // staged through LDS as fp32 rows (pitch BN + 4: the four rows a store instruction touches fall
    // in different banks) so that each thread splits 8 consecutive columns of a row and writes 16
    // bytes to each plane.
    constexpr int CP = BN + 4;
    static_assert(BM * CP * 4 <= NS * C::STG * 2, "the output tile fits in the stage buffers");
    float *ct = (float *)lds_raw;
    __syncthreads();  // every wave is done reading the last stage
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          ct[(wm * WM + i * 16 + fc * 4 + r) * CP + wn * WN + j * 16 + fr] = acc[i][j][r] * cs;
    __syncthreads();
    uint16_t *Pb = g.Cpl + (long long)batch * g.cpl_bs;
    const float pscale = f16_split_scale(g.cpl_amax);
    for (int w = tid; w < BM * BN / 8; w += C::NT) {
      const int row = w / (BN / 8), c8 = (w % (BN / 8)) * 8;
      const int m = m0 + row, n = n0 + c8;
      if (m < g.M && n < g.N) {  // (N is a multiple of 8)
        const float4 x0 = *(const float4 *)(ct + row * CP + c8), x1 = *(const float4 *)(ct + row * CP + c8 + 4);
        const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        uint16_t h[8][3];
#pragma unroll
        for (int e = 0; e < 8; ++e) split_planes<SRC_F32, MF_F16>(v[e], pscale, h[e]);
        uint16_t *o = Pb + (long long)m * g.c_ld + n;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          uint4 u;
          u.x = h[0][p] | ((uint32_t)h[1][p] << 16);
          u.y = h[2][p] | ((uint32_t)h[3][p] << 16);
          u.z = h[4][p] | ((uint32_t)h[5][p] << 16);
          u.w = h[6][p] | ((uint32_t)h[7][p] << 16);
          *(uint4 *)(o + p * g.cpl_ps) = u;
        }
      }
    }
    return;
  }
  float *Cb = g.C ? g.C + (long long)batch * g.c_bs + (long long)bin * g.c_bs2 + (long long)split * g.c_split : nullptr;
  float *C2b = g.C2 ? g.C2 + (long long)batch * g.c2_bs : nullptr;
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
  if (g.c_amax) {
    // one atomic per wave: a second LDS object here would cost the main loop its alias-free
    // LDS accesses (the compiler then waits for every DMA before each fragment read)
    lmax = warp_max(lmax);
    if (lane == 0) atomicMax((unsigned int *)(g.c_amax + (long long)batch * g.c_amax_bs), __float_as_uint(lmax));
  }
}

// Gram C = X^T X of a row-major 16-bit matrix X [rows][128] (one cell of the cache: its slices'
// token rows one after another), K split over blocks: C[b][s][m][n] = sum over the rows k of split
// s of X[k][m] X[k][n].  The product contracts over rows, along which X is strided, and both
// operands are X: each 32-row stage goes global->LDS by DMA once and the fragments of both come
// from it through transposing LDS reads (as for an N-contiguous B above).  Stage row k keeps its 16
// chunks of 8 columns with chunk c at position c ^ (2 xsw(k)): the 16 rows one read touches then
// take 32 different 16-byte positions of a 512-byte window (no bank conflicts).  Rows past `rows`
// read zero (descriptor bound).  Four waves of 64 x 64 outputs; four stages of 8 KB.
constexpr int kXgStages = 4;
__device__ __forceinline__ int xsw(int k) { return ((k >> 1) & 1) | (((k >> 3) & 3) << 1); }

template <int MF>
__global__ void __launch_bounds__(256) xgram_kernel(const uint16_t *X, long long x_bs, int rows, int k_chunk, float *C,
                                                    long long c_bs) {
  constexpr int D = 128, STG = DK * D, NS = kXgStages;  // halves per stage
  __shared__ __attribute__((aligned(1024))) uint16_t lds_raw[NS * STG];
  lds16 *const L0 = (lds16 *)lds_raw, *const Llast = L0 + (NS - 1) * STG;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int split = blockIdx.x, b = blockIdx.y;
  const int kbeg = split * k_chunk, kend = min(rows, kbeg + k_chunk);
  const int nsteps = max(0, (kend - kbeg + DK - 1) / DK);
  const i32x4 rs = make_rsrc(X + b * x_bs, (uint32_t)((long long)rows * D * 2));
  // DMA instruction i of a stage (this wave issues i = wave and wave + 4) fills rows 4 i .. 4 i + 3:
  // lane l writes position l % 16 of row 4 i + l / 16
  uint32_t go[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int k = 4 * (wave + 4 * u) + (lane >> 4), c = (lane & 15) ^ (2 * xsw(k));
    go[u] = (uint32_t)(k * D * 2 + c * 16);
  }
  uint32_t so = (uint32_t)((long long)kbeg * D * 2);
  auto issue = [&](lds16 *dst) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
      raw_buffer_load_lds(rs, (__attribute__((address_space(3))) uint32_t *)(dst + (wave + 4 * u) * 4 * D), 16,
                          (int)go[u], (int)so, 0, 0);
    so += DK * D * 2;
  };
  // fragment of 16-column slot s: rows 8 (lane / 16) + (lane / 4) % 4 and 4 below (xsw of both is
  // lane / 8), columns 4 (lane % 4) .. + 3 of the slot
  const int wm = wave >> 1, wn = wave & 1;
  const int rbase = (8 * (lane >> 4) + ((lane >> 2) & 3)) * D + 4 * (lane & 1);
  int ao[4], bo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ao[i] = rbase + 8 * (2 * ((4 * wm + i) ^ (lane >> 3)) + ((lane >> 1) & 1));
    bo[i] = rbase + 8 * (2 * ((4 * wn + i) ^ (lane >> 3)) + ((lane >> 1) & 1));
  }
  auto frag = [&](const lds16 *q) __attribute__((always_inline)) {
    const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)q));
    const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(q + 4 * D)));
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (nsteps > 0) {
    lds16 *far = L0;
#pragma unroll
    for (int q = 0; q < NS - 1; ++q)
      if (q < nsteps) {
        issue(far);
        far += STG;
      }
    lds16 *cur = L0;
    for (int s = 0; s < nsteps; ++s) {
      wait_stages<2, NS - 2>(min(NS - 2, nsteps - 1 - s));
      wait_lgkm0();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (s + NS - 1 < nsteps) issue(far);
      u32x4 a[4], bb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = frag(cur + ao[i]);
#pragma unroll
      for (int j = 0; j < 4; ++j) bb[j] = frag(cur + bo[j]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16<MF>(a[i], bb[j], acc[i][j]);
      cur = cur == Llast ? L0 : cur + STG;
      far = far == Llast ? L0 : far + STG;
    }
  }
  float *Cb = C + b * c_bs + (long long)split * D * D;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = 64 * wm + 16 * i + 4 * (lane >> 4), n = 64 * wn + 16 * j + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) Cb[(long long)(m + r) * D + n] = acc[i][j][r];
    }
}

template <int MF, int PA, int PB, int TM, int TN, int NS, int NWM, int NWN, bool BKC = true, bool OPL = false>
void launch_dma(const GemmArgs &g, int batch, int nsplit, hipStream_t st) {
  using C = Cfg<MF, PA, PB, TM, TN, NS, NWM, NWN>;
  const int tiles = ((g.M + C::BM - 1) / C::BM) * ((g.N + C::BN - 1) / C::BN);
  hipLaunchKernelGGL((gemm_dma_kernel<MF, PA, PB, TM, TN, NS, NWM, NWN, BKC, OPL>), dim3(tiles, nsplit, batch),
                     dim3(C::NT), 0, st, g);
}

// fp32 rows -> P 16-bit planes with the split of the fp32 GEMM operands (power-of-two scale from
// the batch's |x| bound for fp16; three bf16 planes otherwise); columns [cols, cols_pad) become 0.
// Thread: SPT runs of 8 consecutive columns of one row, 2048 columns apart (the block's loads of one
// run are contiguous); the loads of all runs are issued before the first split.
constexpr int kSplitRuns = 4;
template <int MF, int P>
__global__ void __launch_bounds__(256) split_planes_kernel(const float *src, long long s_bs, long long s_ld, int rows,
                                                           int cols, int cols_pad, uint16_t *dst, long long d_bs,
                                                           long long d_ps, long long d_ld, const float *amax,
                                                           int amax_bs) {
  const int b = blockIdx.z, row = blockIdx.y;
  if (row >= rows) return;
  float scale = 1.f;
  if constexpr (MF == MF_F16) scale = f16_split_scale(amax ? amax[(long long)b * amax_bs] : 1.f);
  const float *xr = src + b * s_bs + row * s_ld;
  uint16_t *dr = dst + b * d_bs + row * d_ld;
  float v[kSplitRuns][8];
#pragma unroll
  for (int u = 0; u < kSplitRuns; ++u) {
    const int c0 = ((blockIdx.x * kSplitRuns + u) * 256 + threadIdx.x) * 8;
    const float *x = xr + c0;
    if (c0 + 8 <= cols) {
      const float4 p = *(const float4 *)x, q = *(const float4 *)(x + 4);
      v[u][0] = p.x; v[u][1] = p.y; v[u][2] = p.z; v[u][3] = p.w;
      v[u][4] = q.x; v[u][5] = q.y; v[u][6] = q.z; v[u][7] = q.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[u][i] = c0 + i < cols ? x[i] : 0.f;
    }
  }
#pragma unroll
  for (int u = 0; u < kSplitRuns; ++u) {
    const int c0 = ((blockIdx.x * kSplitRuns + u) * 256 + threadIdx.x) * 8;
    if (c0 >= cols_pad) continue;
    uint16_t pl[8][3];
#pragma unroll
    for (int i = 0; i < 8; ++i) split_planes<SRC_F32, MF>(v[u][i], scale, pl[i]);
#pragma unroll
    for (int p = 0; p < P; ++p) {
      uint4 w;
      w.x = pl[0][p] | ((uint32_t)pl[1][p] << 16);
      w.y = pl[2][p] | ((uint32_t)pl[3][p] << 16);
      w.z = pl[4][p] | ((uint32_t)pl[5][p] << 16);
      w.w = pl[6][p] | ((uint32_t)pl[7][p] << 16);
      *(uint4 *)(dr + c0 + p * d_ps) = w;
    }
  }
}

}  // namespace

void split_planes(int mf, const float *src, long long s_bs, long long s_ld, int rows, int cols, int cols_pad,
                  uint16_t *dst, long long d_bs, long long d_ps, long long d_ld, const float *amax, int amax_bs,
                  int batch, hipStream_t st) {
  JOLT_REQUIRE(cols_pad % 8 == 0 && s_ld % 4 == 0 && d_ld % 8 == 0 && d_ps % 8 == 0 && d_bs % 8 == 0 &&
                   ((uintptr_t)src & 15) == 0 && ((uintptr_t)dst & 15) == 0,
               JOLT_EINVAL, "split_planes: misaligned operand");
  if (rows <= 0 || cols_pad <= 0 || batch <= 0) return;
  dim3 grid((cols_pad / 8 + 256 * kSplitRuns - 1) / (256 * kSplitRuns), rows, batch);
  if (mf == MF_F16)
    hipLaunchKernelGGL((split_planes_kernel<MF_F16, 2>), grid, dim3(256), 0, st, src, s_bs, s_ld, rows, cols,
                       cols_pad, dst, d_bs, d_ps, d_ld, amax, amax_bs);
  else
    hipLaunchKernelGGL((split_planes_kernel<MF_BF16, 3>), grid, dim3(256), 0, st, src, s_bs, s_ld, rows, cols,
                       cols_pad, dst, d_bs, d_ps, d_ld, amax, amax_bs);
  HIP_LAUNCH_CHECK();
}

// Returns false (launching nothing) when the product does not fit this path: K ranges must be
// whole 32-deep stages, every source offset of a batch must fit 32 bits, and only the plane
// layouts used by the compressor are instantiated.  b_kc = false: B(k, n) at k * b_ld plus n
// blocked by b_blk / b_blk_stride (N a multiple of 8, blocks of whole 8-column chunks).
bool gemm_dma(int mf, int pa, int pb, const GemmArgs &g0, int batch, int nsplit, hipStream_t st, bool b_kc) {
  GemmArgs g = g0;
  if (nsplit == 1) g.k_chunk = g.K;  // one split covers K (callers leave k_chunk unset then)
  if (g.M <= 0 || g.N <= 0 || batch <= 0 || nsplit <= 0) return true;
  if (g.K % DK != 0 || g.k_chunk <= 0 || g.k_chunk % DK != 0 || (long long)g.k_chunk * nsplit < g.K) return false;
  if (g.inner > 1 || ((g.tri & 4) && nsplit != 1)) return false;
  if (g.a_blk % DK != 0 || g.b_blk % (b_kc ? DK : 8) != 0) return false;
  if (!b_kc && (g.N % 8 != 0 || (g.tri & ~4) != 0)) return false;
  // ragged B rows: N-contiguous B, one split, K the valid rows rounded up to one stage
  if (g.b_krows != 0 && (b_kc || pb < 2 || nsplit != 1 || g.b_krows < 1 || g.b_krows > g.K || g.K - g.b_krows >= DK))
    return false;
  // plane output: only the N-contiguous fp16 two-plane x two-plane product writes it
  if (g.Cpl && (g.C2 || g.c_amax || nsplit != 1 || g.cpl_mf != MF_F16 || b_kc || mf != MF_F16 || pa != 2 || pb != 2 ||
                g.c_ld % 8 != 0 || g.cpl_ps % 8 != 0 || g.cpl_bs % 8 != 0 || ((uintptr_t)g.Cpl & 15)))
    return false;
  if (!g.Cpl && !g.C) return false;
  if ((g.a_ld * 2) % 16 != 0 || (g.b_ld * 2) % 16 != 0 || (g.a_ps * 2) % 16 != 0 || (g.b_ps * 2) % 16 != 0) return false;
  if (!b_kc && (g.b_blk_stride * 2) % 16 != 0) return false;
  auto extent = [](long long rows, long long ld, long long planes, long long ps, long long K, int blk,
                   long long bstride) {
    const long long kmax = (K - 1) / blk * bstride + (K - 1) % blk + 1;
    return ((planes - 1) * ps + (rows - 1) * ld + kmax) * 2;
  };
  // (an N-contiguous B is the same extent with the roles of rows and K exchanged)
  const long long bext = b_kc ? extent(g.N, g.b_ld, pb, g.b_ps, g.K, g.b_blk, g.b_blk_stride)
                              : extent(g.K, g.b_ld, pb, g.b_ps, g.N, g.b_blk, g.b_blk_stride);
  if (extent(g.M, g.a_ld, pa, g.a_ps, g.K, g.a_blk, g.a_blk_stride) >= (1LL << 32) || bext >= (1LL << 32))
    return false;
  if (((uintptr_t)g.A & 15) || ((uintptr_t)g.B & 15)) return false;
  // 8 waves (4 x 2) of 48 x 128 output each: 192 x 256 blocks; Grams of fp32 rows (both operands
  // in planes) on 48 x 96 wave tiles: 192 x 192 blocks, which tile a 522-row Gram with less padding
  if (!b_kc) {
    // (fp32 x fp32 products whose B is the basis planes, e.g. R^{-T} Y^T: 128 x 256 blocks, 4 x 2 waves
    // of 32 x 128, so that three stages of both operands' two planes fit in LDS)
    if (mf == MF_F16 && pa == 2 && pb == 1) launch_dma<MF_F16, 2, 1, 3, 8, 3, 4, 2, false>(g, batch, nsplit, st);
    else if (mf == MF_F16 && pa == 2 && pb == 2 && g.Cpl)
      launch_dma<MF_F16, 2, 2, 2, 8, 3, 4, 2, false, true>(g, batch, nsplit, st);
    else if (mf == MF_F16 && pa == 2 && pb == 2) launch_dma<MF_F16, 2, 2, 2, 8, 3, 4, 2, false>(g, batch, nsplit, st);
    else if (mf == MF_BF16 && pa == 3 && pb == 1) launch_dma<MF_BF16, 3, 1, 3, 8, 3, 4, 2, false>(g, batch, nsplit, st);
    else return false;
    HIP_LAUNCH_CHECK();
    return true;
  }
  if (mf == MF_F16 && pa == 2 && pb == 1) launch_dma<MF_F16, 2, 1, 3, 12, 3, 4, 2>(g, batch, nsplit, st);
  else if (mf == MF_F16 && pa == 2 && pb == 2) launch_dma<MF_F16, 2, 2, 3, 6, 3, 4, 2>(g, batch, nsplit, st);
  else if (mf == MF_BF16 && pa == 3 && pb == 3) launch_dma<MF_BF16, 3, 3, 3, 6, 2, 4, 2>(g, batch, nsplit, st);
  else if (mf == MF_F16 && pa == 1 && pb == 1) launch_dma<MF_F16, 1, 1, 3, 12, 4, 4, 2>(g, batch, nsplit, st);
  else if (mf == MF_BF16 && pa == 3 && pb == 1) launch_dma<MF_BF16, 3, 1, 3, 8, 3, 4, 2>(g, batch, nsplit, st);
  else if (mf == MF_BF16 && pa == 1 && pb == 1) launch_dma<MF_BF16, 1, 1, 3, 8, 4, 4, 2>(g, batch, nsplit, st);
  else return false;
  HIP_LAUNCH_CHECK();
  return true;
}


// Gram partials of 16-bit row-major [rows][128] matrices (see xgram_kernel): C[b][s] at
// b * c_bs + s * 128 * 128, fp32 [128][128].  False (nothing launched) when the shape does not fit.
bool xgram_dma(int mf, const void *X, long long x_bs, int rows, int D, float *C, long long c_bs, int k_chunk,
               int nsplit, int batch, hipStream_t st) {
  if (D != 128 || rows <= 0 || batch <= 0 || nsplit <= 0) return false;
  if (k_chunk <= 0 || k_chunk % DK != 0 || (long long)k_chunk * nsplit < rows) return false;
  if ((long long)rows * D * 2 >= (1LL << 31) || ((uintptr_t)X & 15) || (x_bs * 2) % 16 != 0) return false;
  if (mf == MF_F16)
    hipLaunchKernelGGL(xgram_kernel<MF_F16>, dim3(nsplit, batch), dim3(256), 0, st, (const uint16_t *)X, x_bs, rows,
                       k_chunk, C, c_bs);
  else
    hipLaunchKernelGGL(xgram_kernel<MF_BF16>, dim3(nsplit, batch), dim3(256), 0, st, (const uint16_t *)X, x_bs, rows,
                       k_chunk, C, c_bs);
  HIP_LAUNCH_CHECK();
  return true;
}

}  // namespace jolt
