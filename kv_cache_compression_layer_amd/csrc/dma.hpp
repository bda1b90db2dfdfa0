// Global->LDS DMA helpers of gfx950 (buffer_load ... lds), shared by the plane GEMM (gemm_dma.hip)
// and the residual encode (codec.hip).
#pragma once
#include "common.hpp"

namespace jolt {
namespace dma {

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

}  // namespace dma
}  // namespace jolt
