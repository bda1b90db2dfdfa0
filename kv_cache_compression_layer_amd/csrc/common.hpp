// Shared definitions of libjolt (host and device).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>
#include <string>

#include "../../include/jolt.h"

namespace jolt {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf168 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

enum Src { SRC_F16 = 0, SRC_BF16 = 1, SRC_F32 = 2 };
enum Mf { MF_F16 = 0, MF_BF16 = 1 };

inline int dtype_bytes(int dt) { return dt == JOLT_F32 ? 4 : 2; }

// ---------------------------------------------------------------------------------------------
// error reporting (thread-local message; the status is the return value)
// ---------------------------------------------------------------------------------------------
void set_error(const std::string &msg);
const char *get_error();

struct Fail {
  int status;
};

#define JOLT_REQUIRE(cond, status, msg)                                                         \
  do {                                                                                          \
    if (!(cond)) {                                                                              \
      ::jolt::set_error(std::string(msg));                                                      \
      throw ::jolt::Fail{status};                                                               \
    }                                                                                           \
  } while (0)

#define HIP_TRY(expr)                                                                           \
  do {                                                                                          \
    hipError_t e_ = (expr);                                                                     \
    if (e_ != hipSuccess) {                                                                     \
      ::jolt::set_error(std::string(#expr) + ": " + hipGetErrorString(e_));                    \
      throw ::jolt::Fail{JOLT_EHIP};                                                            \
    }                                                                                           \
  } while (0)

#define HIP_LAUNCH_CHECK() HIP_TRY(hipGetLastError())

// Bounded cross-workgroup waits (the per-cell allocation and the multi-workgroup
// tridiagonalisation): each wait polls a step counter at most spin_limit times, for a target count
// raised by target_extra.  target_extra is 0 except under jolt_test_wait_policy(), where it makes
// every wait lapse so that the lapse reporting can be exercised while every kernel still ends.
struct WaitPolicy {
  unsigned spin_limit;
  unsigned target_extra;
};
WaitPolicy wait_policy();

// ---------------------------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t r = 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)((u + r) >> 16);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }
__device__ __forceinline__ uint16_t f32_to_f16_rne(float f) {
  _Float16 h = (_Float16)f;
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

template <int S>
__device__ __forceinline__ float load_elem(const void *p, long long i) {
  if constexpr (S == SRC_F32) return ((const float *)p)[i];
  else if constexpr (S == SRC_F16) return f16_to_f32(((const uint16_t *)p)[i]);
  else return bf16_to_f32(((const uint16_t *)p)[i]);
}

template <int S>
__device__ __forceinline__ void store_elem(void *p, long long i, float v) {
  if constexpr (S == SRC_F32) ((float *)p)[i] = v;
  else if constexpr (S == SRC_F16) ((uint16_t *)p)[i] = f32_to_f16_rne(v);
  else ((uint16_t *)p)[i] = f32_to_bf16_rne(v);
}

// power-of-two scale that maps amax into [2^14, 2^15) (fp16 split of fp32 operands)
__device__ __forceinline__ float f16_split_scale(float amax) {
  if (!(amax > 0.f) || !isfinite(amax)) return 1.f;
  int e = ilogbf(amax);
  return ldexpf(1.f, 14 - e);
}

__device__ __forceinline__ float warp_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
// Sum over the 64 lanes of a wave, returned to every lane (every lane must be active): pairs and
// quads by DPP quad permutes, half rows and rows by the mirror permutes, then rows 1 and 3 take
// row 0's and row 2's sums (row_bcast15) and rows 2 and 3 take row 1's (row_bcast31), so lane 63
// ends with the total, which is broadcast.  Registers only (no LDS permutes), fixed order.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ double dpp_f64(double v) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, ROWMASK, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, ROWMASK, 0xF, false);
  return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double warp_sum_d(double v) {
  v += dpp_f64<0xB1, 0xF>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp_f64<0x4E, 0xF>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp_f64<0x141, 0xF>(v);  // row_half_mirror
  v += dpp_f64<0x140, 0xF>(v);  // row_mirror
  v += dpp_f64<0x142, 0xA>(v);  // row_bcast15 into rows 1 and 3
  v += dpp_f64<0x143, 0xC>(v);  // row_bcast31 into rows 2 and 3
  const int lo = __builtin_amdgcn_readlane(__double2loint(v), 63);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(v), 63);
  return __hiloint2double(hi, lo);
}

// ---------------------------------------------------------------------------------------------
// GEMM on MFMA with exact splitting of fp32 operands into 16-bit planes
// C[b](m, n) = c_scale * sum_k A[b](m, k) B[b](k, n), fp32 output.
// ---------------------------------------------------------------------------------------------
struct GemmArgs {
  const void *A;
  const void *B;
  float *C;
  int M, N, K;
  long long a_bs, b_bs, c_bs;  // batch strides (elements)
  long long a_ld;              // stride of A's strided dim
  long long a_blk_stride;      // A's contiguous dim: index i -> (i / a_blk) * a_blk_stride + i % a_blk
  int a_blk;
  long long b_ld;
  long long b_blk_stride;
  int b_blk;
  long long c_ld;
  long long c_split;  // stride between split-K partial outputs (elements)
  int k_chunk;        // K per split, multiple of 32
  const float *a_amax;  // per-batch |A| bound for the fp16 split (device), or null -> a_amax_c
  float a_amax_c;
  const float *b_amax;
  float b_amax_c;
  float *c_amax;  // optional per-batch running max |C| (float bits, atomic max)
  int m_fastest;  // tile order: m tiles adjacent (else n tiles adjacent)
  // two-level batch: grid z = outer * inner + in; offsets outer*x_bs + in*x_bs2; amax pointers
  // are indexed by outer * (ab_amax_bs | c_amax_bs)
  int inner;
  long long a_bs2, b_bs2, c_bs2;
  int ab_amax_bs, c_amax_bs;
  float alpha;  // output multiplier
  // optional second, transposed output: C2[n][m] (row pitch c2_ld, batch stride c2_bs)
  float *C2;
  long long c2_ld, c2_bs;
  // structure flags: 1 = only tiles touching the upper triangle (m < n) are needed; the others
  // are written as zeros without work; 2 = B(k, n) = 0 for k > n (an upper triangular factor),
  // so each column tile stops its k loop at its last column (single split only); 4 = A(m, k) = 0
  // for k > m (a lower triangular factor), so each row tile stops its k loop at its last row
  // (single split, K-contiguous kernel only)
  int tri;
  // operands stored as 16-bit planes (plane-GEMM path): element stride between planes
  long long a_ps, b_ps;
  // optional (K-contiguous kernel): C written as its 16-bit planes instead of fp32, [plane][M][c_ld]
  // at plane stride cpl_ps and batch stride cpl_bs, split as split_planes does (type cpl_mf; fp16
  // planes after the power-of-two scale of the bound cpl_amax on |C|)
  uint16_t *Cpl;
  long long cpl_ps, cpl_bs;
  float cpl_amax;
  int cpl_mf;
  // (plane-GEMM path, B contiguous along N) rows of B that hold data: 0 = all K rows; else K is that
  // count rounded up to a whole 32-deep stage, A is zero in the columns past it, and the k-rows of B
  // past it are read from its last valid row instead (so they never leave B)
  int b_krows;
};

// a_kc: A contiguous along K (else along M); b_kc: B contiguous along K (else along N)
void gemm(int mf, int sa, bool a_kc, int sb, bool b_kc, const GemmArgs &g, int batch, int nsplit,
          hipStream_t st);

// the same product for operands that are both contiguous along K (larger wave tiles); called by
// gemm() after validation
void gemm_kc(int mf, int sa, int sb, const GemmArgs &g, int batch, int nsplit, hipStream_t st);
// Products of operands stored as 16-bit planes (pa planes of A at stride a_ps, pb of B), A
// contiguous along K, B along K (b_kc) or along N, fed through LDS by DMA; false (nothing
// launched) when the shape does not fit.
bool gemm_dma(int mf, int pa, int pb, const GemmArgs &g, int batch, int nsplit, hipStream_t st, bool b_kc = true);
// Split-K partials of X^T X for 16-bit row-major X [rows][D] (D = 128; batch stride x_bs elements):
// C[b][s][m][n] (fp32, batch stride c_bs, split stride D * D) over rows [s k_chunk, (s + 1) k_chunk).
// False (nothing launched) when the shape does not fit.
bool xgram_dma(int mf, const void *X, long long x_bs, int rows, int D, float *C, long long c_bs, int k_chunk,
               int nsplit, int batch, hipStream_t st);
// fp32 rows [batch][rows][s_ld] -> planes [batch][plane][rows][d_ld] (2 fp16 planes after the
// power-of-two scale of amax[b * amax_bs], or 3 bf16 planes); columns [cols, cols_pad) zeroed.
void split_planes(int mf, const float *src, long long s_bs, long long s_ld, int rows, int cols, int cols_pad,
                  uint16_t *dst, long long d_bs, long long d_ps, long long d_ld, const float *amax, int amax_bs,
                  int batch, hipStream_t st);

// split-K partials summed in fixed order (fp64) into C [rows][cols] (row pitch c_ld) and its
// transpose C2 [cols][rows] (row pitch c2_ld); optional per-batch max |C| into amax (atomic max)
void reduce_splits_dual(const float *part, long long part_bs, long long part_ss, int nsplit, int rows, int cols,
                        long long ld_in, float *C, long long c_bs, long long c_ld, float *C2, long long c2_bs,
                        long long c2_ld, float *amax, int batch, hipStream_t st);

// sum of split-K partials in fixed order: out[b][i] = sum_s part[b][s][i] (fp64 accumulate)
void reduce_splits(const float *part, long long part_bs, long long part_ss, int nsplit, long long n,
                   int rows, int cols, long long ld_in, void *out, bool out_f64, long long out_bs,
                   long long ld_out, int batch, hipStream_t st);

}  // namespace jolt
