// MFMA building blocks shared by the GEMM and codec kernels (16-bit planes of fp32 values,
// 8-element vector loads with blocked addressing, LDS tile stores, 16x16x32 MFMA).
#pragma once
#include "common.hpp"

namespace jolt {
namespace core {

constexpr int BM = 128, BN = 128, BK = 32, LDK = 40, NT = 256;

template <int S, int MF>
struct Planes {
  static constexpr int n = (S == SRC_F32) ? (MF == MF_F16 ? 2 : 3) : 1;
};

// fp32 -> three fp16 planes (hi, lo, lo2) after a power-of-two scale: used where 22 bits
// are not enough.
__device__ __forceinline__ void split3_f16(float x, float scale, uint16_t (&p)[3]) {
  float y = x * scale;
  uint16_t h = f32_to_f16_rne(y);
  float r = y - f16_to_f32(h);
  uint16_t l = f32_to_f16_rne(r);
  p[0] = h;
  p[1] = l;
  p[2] = f32_to_f16_rne(r - f16_to_f32(l));
}

__device__ __forceinline__ long long blk_idx(long long i, int blk, long long bstride) {
  return (i / blk) * bstride + (i % blk);
}

// Load 8 consecutive elements (along the contiguous dim) as fp32; zero outside [0, lim).
template <int S>
__device__ __forceinline__ void load8(const void *base, long long off, int c0, int lim, bool row_ok,
                                      int blk, long long bstride, float (&v)[8]) {
  if (row_ok && c0 + 8 <= lim) {
    long long o = off + blk_idx(c0, blk, bstride);
    if constexpr (S == SRC_F32) {
      const float4 *p = (const float4 *)((const float *)base + o);
      float4 x = p[0], y = p[1];
      v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
      v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
    } else {
      uint4 x = *(const uint4 *)((const uint16_t *)base + o);
      uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint16_t lo = (uint16_t)(w[i] & 0xFFFF), hi = (uint16_t)(w[i] >> 16);
        if constexpr (S == SRC_F16) { v[2 * i] = f16_to_f32(lo); v[2 * i + 1] = f16_to_f32(hi); }
        else { v[2 * i] = bf16_to_f32(lo); v[2 * i + 1] = bf16_to_f32(hi); }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int c = c0 + i;
      v[i] = (row_ok && c < lim) ? load_elem<S>(base, off + blk_idx(c, blk, bstride)) : 0.f;
    }
  }
}

// Split one fp32 value into the 16-bit planes of the MFMA type.
template <int S, int MF>
__device__ __forceinline__ void split_planes(float x, float scale, uint16_t (&p)[3]) {
  if constexpr (S != SRC_F32) {
    if constexpr (MF == MF_F16) p[0] = f32_to_f16_rne(x);
    else p[0] = f32_to_bf16_rne(x);
  } else if constexpr (MF == MF_F16) {
    float y = x * scale;
    uint16_t h = f32_to_f16_rne(y);
    p[0] = h;
    p[1] = f32_to_f16_rne(y - f16_to_f32(h));
  } else {
    uint16_t a = f32_to_bf16_rne(x);
    float r1 = x - bf16_to_f32(a);
    uint16_t b = f32_to_bf16_rne(r1);
    float r2 = r1 - bf16_to_f32(b);
    p[0] = a; p[1] = b; p[2] = f32_to_bf16_rne(r2);
  }
}

// Raw 8-element vector of a source (no conversion): 16-bit -> one uint4, fp32 -> two float4.
template <int S>
struct Raw8 {
  uint4 v;
};
template <>
struct Raw8<SRC_F32> {
  float4 a, b;
};

template <int S>
__device__ __forceinline__ void load_raw8(const void *base, long long off, int c0, int lim, bool row_ok, int blk,
                                          long long bstride, Raw8<S> &r) {
  if (row_ok && c0 + 8 <= lim) {
    long long o = off + blk_idx(c0, blk, bstride);
    if constexpr (S == SRC_F32) {
      const float4 *p = (const float4 *)((const float *)base + o);
      r.a = p[0];
      r.b = p[1];
    } else {
      r.v = *(const uint4 *)((const uint16_t *)base + o);
    }
  } else {
    if constexpr (S == SRC_F32) {
      float t[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        int c = c0 + i;
        t[i] = (row_ok && c < lim) ? ((const float *)base)[off + blk_idx(c, blk, bstride)] : 0.f;
      }
      r.a = make_float4(t[0], t[1], t[2], t[3]);
      r.b = make_float4(t[4], t[5], t[6], t[7]);
    } else {
      uint16_t t[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        int c = c0 + i;
        t[i] = (row_ok && c < lim) ? ((const uint16_t *)base)[off + blk_idx(c, blk, bstride)] : (uint16_t)0;
      }
      r.v.x = t[0] | ((uint32_t)t[1] << 16);
      r.v.y = t[2] | ((uint32_t)t[3] << 16);
      r.v.z = t[4] | ((uint32_t)t[5] << 16);
      r.v.w = t[6] | ((uint32_t)t[7] << 16);
    }
  }
}

template <int S>
__device__ __forceinline__ float raw_elem(const Raw8<S> &r, int i) {
  if constexpr (S == SRC_F32) {
    const float t[8] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w};
    return t[i];
  } else {
    const uint32_t w[4] = {r.v.x, r.v.y, r.v.z, r.v.w};
    uint16_t h = (uint16_t)((i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFF));
    if constexpr (S == SRC_F16) return f16_to_f32(h);
    else return bf16_to_f32(h);
  }
}

template <int MF>
__device__ __forceinline__ f32x4 mfma(const uint4 &a, const uint4 &b, f32x4 c) {
  if constexpr (MF == MF_F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a), __builtin_bit_cast(half8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf168, a), __builtin_bit_cast(bf168, b), c, 0, 0, 0);
}

// Store 8 values (already split to planes) into the LDS tile [plane][row][k].
template <int P, bool KC>
__device__ __forceinline__ void lds_store8(uint16_t *tile, int rows, int r, int k, const uint16_t (&pl)[8][3]) {
  // KC: the 8 values run along k at row r; else they run along rows r..r+7 at column k.
#pragma unroll
  for (int p = 0; p < P; ++p) {
    uint16_t *t = tile + p * rows * LDK;
    if constexpr (KC) {
      uint4 w;
      w.x = pl[0][p] | ((uint32_t)pl[1][p] << 16);
      w.y = pl[2][p] | ((uint32_t)pl[3][p] << 16);
      w.z = pl[4][p] | ((uint32_t)pl[5][p] << 16);
      w.w = pl[6][p] | ((uint32_t)pl[7][p] << 16);
      *(uint4 *)(t + r * LDK + k) = w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) t[(r + i) * LDK + k] = pl[i][p];
    }
  }
}

}  // namespace core
}  // namespace jolt
