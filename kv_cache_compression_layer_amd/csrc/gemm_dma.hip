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
#include <type_traits>

#include "common.hpp"
#include "gemm_core.hpp"

namespace jolt {

namespace {

using namespace core;

typedef __attribute__((address_space(3))) uint16_t lds16;
typedef __attribute__((address_space(3))) void ldsv;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

template <int MF>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (MF == MF_F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a), __builtin_bit_cast(half8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf168, a), __builtin_bit_cast(bf168, b), c, 0, 0, 0);
}

constexpr int DK = 32;  // k per stage (one MFMA depth)

// LDS half offset of logical chunk `chunk` of row `row` in a [rows][32] tile (XOR permutation by
// row / 2, measured free of bank conflicts for fragment reads).
__device__ __forceinline__ int dswz(int row, int chunk) { return row * DK + ((chunk ^ (row >> 1)) & 3) * 8; }

// s_waitcnt with vmcnt = n and the other counters left open
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4)); }
// wait until at most `later` stages of ND requests each are outstanding (later <= MAXL, uniform)
template <int ND, int MAXL>
__device__ __forceinline__ void wait_stages(int later) {
  if constexpr (MAXL <= 0) {
    wait_vm<0>();
  } else {
    if (later >= MAXL) wait_vm<MAXL * ND>();
    else wait_stages<ND, MAXL - 1>(later);
  }
}

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

// raw buffer load of 16 bytes per lane straight into LDS (M0 = wave-uniform LDS base; lane l
// writes bytes [16 l, 16 l + 16) after it); address = descriptor base + voffset + soffset
__device__ void raw_buffer_load_lds(i32x4 rsrc, __attribute__((address_space(3))) uint32_t *lds, int size, int voffset,
                                    int soffset, int offset, int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

// buffer descriptor of a raw byte range (stride 0, no swizzle; loads past num_records read zero)
__device__ __forceinline__ i32x4 make_rsrc(const void *base, uint32_t num_records) {
  const uint64_t a = (uint64_t)base;
  i32x4 r;
  r[0] = (int)(uint32_t)a;
  r[1] = (int)((uint32_t)(a >> 32) & 0xFFFFu);
  r[2] = (int)num_records;
  r[3] = 0x00020000;
  return r;
}

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

template <class C, int PA, int PB, int TM, int TN>
struct Frags {
  u32x4 a[PA][TM];
  u32x4 b[PB][TN];
};

// fragment reads in the order the MFMAs consume them (the first A fragment, the B plane of the
// first plane product, the rest of that A plane, then the other planes), so the in-order LDS
// return lets the first MFMAs start after a few reads
template <class C, int PA, int PB, int TM, int TN>
__device__ __forceinline__ void read_frags(const lds16 *__restrict__ src, int aoff, int boff,
                                           Frags<C, PA, PB, TM, TN> &f) {
  constexpr int PB0 = (PB - 1 < C::MAXO - (PA - 1)) ? PB - 1 : (C::MAXO - (PA - 1) > 0 ? C::MAXO - (PA - 1) : 0);
  // (a scheduling barrier after each read pins the issue order, which the scheduler would otherwise
  // regroup by address so that the first MFMA waits for nearly every read of the stage)
  auto ra = [&](int p, int i) __attribute__((always_inline)) {
    f.a[p][i] = *(const lds_u32x4 *)(src + p * C::BM * DK + i * 16 * DK + aoff);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto rb = [&](int p, int j) __attribute__((always_inline)) {
    f.b[p][j] = *(const lds_u32x4 *)(src + C::ASZ + p * C::BN * DK + j * 16 * DK + boff);
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

template <int MF, int PA, int PB, int TM, int TN, int NS, int NWM, int NWN>
__global__ void __launch_bounds__(64 * NWM * NWN) __attribute__((amdgpu_waves_per_eu(NWM * NWN / 4, NWM * NWN / 4)))
gemm_dma_kernel(GemmArgs g) {
  using C = Cfg<MF, PA, PB, TM, TN, NS, NWM, NWN>;
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
      } else {
        const int Gb = G - NGA, plane = Gb / (BN / 16), row = (Gb % (BN / 16)) * 16 + r;
        const int c = (p ^ (row >> 1)) & 3;
        const int n = min(n0 + row, g.N - 1);
        go[i] = (uint32_t)((plane * g.b_ps + (long long)n * g.b_ld + c * 8) * 2);
      }
    }
  }
  // byte offset (from the batch base) of the next stage to request, in blocked addressing
  // (k -> (k / blk) * stride + k % blk); descriptors cover the whole 32-bit offset range, every
  // offset formed here is inside the operand (checked by the host)
  const i32x4 rsa = make_rsrc(Ab, 0xFFFFFFFFu), rsb = make_rsrc(Bb, 0xFFFFFFFFu);
  int ak = kbeg % g.a_blk, bk = kbeg % g.b_blk;
  uint32_t aso = (uint32_t)(((long long)(kbeg / g.a_blk) * g.a_blk_stride + ak) * 2);
  uint32_t bso = (uint32_t)(((long long)(kbeg / g.b_blk) * g.b_blk_stride + bk) * 2);
  const uint32_t ajump = (uint32_t)((g.a_blk_stride - g.a_blk) * 2), bjump = (uint32_t)((g.b_blk_stride - g.b_blk) * 2);
  auto advance = [&]() __attribute__((always_inline)) {
    ak += DK;
    aso += DK * 2;
    if (ak == g.a_blk) { ak = 0; aso += ajump; }
    bk += DK;
    bso += DK * 2;
    if (bk == g.b_blk) { bk = 0; bso += bjump; }
  };

  const int wm = wave / NWN, wn = wave % NWN;
  const int fr = lane & 15, fc = lane >> 4;
  const int aoff = dswz(wm * WM + fr, fc), boff = dswz(wn * WN + fr, fc);

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
          issue<C>(far, rsa, rsb, aso, bso, go, gi, isa);
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
          issue<C>(far, rsa, rsb, aso, bso, go, gi, isa);
          advance();
        }
        read_frags<C, PA, PB, TM, TN>(cur, aoff, boff, fx);
        __builtin_amdgcn_sched_barrier(0);
        mfmas<MF, C, PA, PB, TM, TN, 0, TN, true>(fx, acc, 0, 0);
        cur = cur == Llast ? L0 : cur + C::STG;
        far = far == Llast ? L0 : far + C::STG;
      }
    }
  }

  const float cs = g.alpha / (ascale * bscale);
  float *Cb = g.C + (long long)batch * g.c_bs + (long long)bin * g.c_bs2 + (long long)split * g.c_split;
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

template <int MF, int PA, int PB, int TM, int TN, int NS, int NWM, int NWN>
void launch_dma(const GemmArgs &g, int batch, int nsplit, hipStream_t st) {
  using C = Cfg<MF, PA, PB, TM, TN, NS, NWM, NWN>;
  const int tiles = ((g.M + C::BM - 1) / C::BM) * ((g.N + C::BN - 1) / C::BN);
  hipLaunchKernelGGL((gemm_dma_kernel<MF, PA, PB, TM, TN, NS, NWM, NWN>), dim3(tiles, nsplit, batch), dim3(C::NT), 0, st, g);
}

// fp32 rows -> P 16-bit planes with the split of the fp32 GEMM operands (power-of-two scale from
// the batch's |x| bound for fp16; three bf16 planes otherwise); columns [cols, cols_pad) become 0.
// Thread: 8 consecutive columns of one row.
template <int MF, int P>
__global__ void __launch_bounds__(256) split_planes_kernel(const float *src, long long s_bs, long long s_ld, int rows,
                                                           int cols, int cols_pad, uint16_t *dst, long long d_bs,
                                                           long long d_ps, long long d_ld, const float *amax,
                                                           int amax_bs) {
  const int b = blockIdx.z, row = blockIdx.y;
  const int c0 = (blockIdx.x * 256 + threadIdx.x) * 8;
  if (row >= rows || c0 >= cols_pad) return;
  float scale = 1.f;
  if constexpr (MF == MF_F16) scale = f16_split_scale(amax ? amax[(long long)b * amax_bs] : 1.f);
  const float *x = src + b * s_bs + row * s_ld + c0;
  float v[8];
  if (c0 + 8 <= cols) {
    const float4 p = *(const float4 *)x, q = *(const float4 *)(x + 4);
    v[0] = p.x; v[1] = p.y; v[2] = p.z; v[3] = p.w; v[4] = q.x; v[5] = q.y; v[6] = q.z; v[7] = q.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = c0 + i < cols ? x[i] : 0.f;
  }
  uint16_t pl[8][3];
#pragma unroll
  for (int i = 0; i < 8; ++i) split_planes<SRC_F32, MF>(v[i], scale, pl[i]);
  uint16_t *d = dst + b * d_bs + row * d_ld + c0;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    uint4 w;
    w.x = pl[0][p] | ((uint32_t)pl[1][p] << 16);
    w.y = pl[2][p] | ((uint32_t)pl[3][p] << 16);
    w.z = pl[4][p] | ((uint32_t)pl[5][p] << 16);
    w.w = pl[6][p] | ((uint32_t)pl[7][p] << 16);
    *(uint4 *)(d + p * d_ps) = w;
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
  dim3 grid((cols_pad / 8 + 255) / 256, rows, batch);
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
// layouts used by the compressor are instantiated.
bool gemm_dma(int mf, int pa, int pb, const GemmArgs &g0, int batch, int nsplit, hipStream_t st) {
  GemmArgs g = g0;
  if (nsplit == 1) g.k_chunk = g.K;  // one split covers K (callers leave k_chunk unset then)
  if (g.M <= 0 || g.N <= 0 || batch <= 0 || nsplit <= 0) return true;
  if (g.K % DK != 0 || g.k_chunk <= 0 || g.k_chunk % DK != 0 || (long long)g.k_chunk * nsplit < g.K) return false;
  if (g.inner > 1 || (g.tri & 1)) return false;
  if (g.a_blk % DK != 0 || g.b_blk % DK != 0) return false;
  if ((g.a_ld * 2) % 16 != 0 || (g.b_ld * 2) % 16 != 0 || (g.a_ps * 2) % 16 != 0 || (g.b_ps * 2) % 16 != 0) return false;
  auto extent = [](long long rows, long long ld, long long planes, long long ps, long long K, int blk,
                   long long bstride) {
    const long long kmax = (K - 1) / blk * bstride + (K - 1) % blk + 1;
    return ((planes - 1) * ps + (rows - 1) * ld + kmax) * 2;
  };
  if (extent(g.M, g.a_ld, pa, g.a_ps, g.K, g.a_blk, g.a_blk_stride) >= (1LL << 32) ||
      extent(g.N, g.b_ld, pb, g.b_ps, g.K, g.b_blk, g.b_blk_stride) >= (1LL << 32))
    return false;
  if (((uintptr_t)g.A & 15) || ((uintptr_t)g.B & 15)) return false;
  // 8 waves (4 x 2) of 48 x 128 output each: 192 x 256 blocks
  if (mf == MF_F16 && pa == 2 && pb == 1) launch_dma<MF_F16, 2, 1, 3, 8, 3, 4, 2>(g, batch, nsplit, st);
  else if (mf == MF_F16 && pa == 1 && pb == 1) launch_dma<MF_F16, 1, 1, 3, 8, 4, 4, 2>(g, batch, nsplit, st);
  else if (mf == MF_BF16 && pa == 3 && pb == 1) launch_dma<MF_BF16, 3, 1, 3, 8, 3, 4, 2>(g, batch, nsplit, st);
  else if (mf == MF_BF16 && pa == 1 && pb == 1) launch_dma<MF_BF16, 1, 1, 3, 8, 4, 4, 2>(g, batch, nsplit, st);
  else return false;
  HIP_LAUNCH_CHECK();
  return true;
}

}  // namespace jolt
