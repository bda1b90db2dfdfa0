// Host-side descriptors and launchers of the residual codec kernels (codec.hip).
#pragma once
#include "common.hpp"

namespace jolt {

// One cell of the encode pass, as byte offsets from the bases in EncArgs (so that every address
// the kernel forms derives from a kernel argument and compiles to global memory instructions).
// Bcat[j][n][k] (fp32, row pitch Kb, a multiple of 32): k < D -> Q[k][n]; D <= k < D + rT ->
// -(D_j Q)[k - D][n]; k >= D + rT -> 0.
struct EncCell {
  long long x_off;     // cache slice [GH][T][D] (cache dtype) in xk (kv == 0) or xv (kv == 1)
  long long ut_off;    // U_T [T][rT] (cache dtype) in utb
  long long sc_off;    // fp32 scales [GH*T] in scb
  long long cd_off;    // codes [GH*T][D*bits/8] in cdb
  long long bcat_off;  // B = [Q ; -D_j Q] as 16-bit planes [plane][GH][D][Kb] in bcat (bytes)
  int kv, am_idx;      // cache selector; index of max |Bcat| in bamax (fp16 split scale)
  int GH, rT, bits, Kb;
};

struct EncArgs {
  const char *xk, *xv, *utb;
  char *scb, *cdb;
  const char *bcat;   // 16-bit planes of B, plane stride b_ps elements
  long long b_ps;
  const float *bamax;
  const EncCell *cells;
};

// One cell of the decode pass.  Dm[j][n][r] = D_j[r][n] (fp32, row pitch Kd); Q row-major.  The
// tile rebuild reads both as 16-bit planes split once beforehand (split_planes with the decode's
// matrix-core type: Dm after the scale of d_amax, Q after the scale of 1).
struct DecCell {
  const void *UT;      // [T][rT] storage dtype
  const float *Dm;     // [GH][D][Kd]
  const float *Q;      // [D][D] rotation
  const uint16_t *Dpl; // planes of Dm: [plane][GH][D][Kd], plane stride dpl_ps
  const uint16_t *Qpl; // planes of Q: [plane][D][D], plane stride qpl_ps
  long long dpl_ps, qpl_ps;
  const float *d_amax; // device max |Dm|
  const float *scales;
  const uint8_t *codes;
  void *out;           // [GH][T][D] cache dtype
  int GH, rT, bits, Kd;
};

// One decode step of one layer over its compressed K and V cells (fused decode).  Slice j of either
// cell is KV head j of the layer (codes, scales and Dm start at the layer's first head).
constexpr int kAttnMaxG = 8;          // query heads per KV head
constexpr int kAttnMaxRank = 512;     // value token rank
constexpr int kAttnMaxChunks = 2048;  // token chunks of the split
constexpr int kAttnMaxTail = 1024;    // dense tail tokens
struct AttnArgs {
  DecCell k, v;
  const float *q;     // [H G][D] queries, rotated at their position
  const float *rope;  // [positions][D/2][2] cosine, sine
  float *part;        // [n_chunks][H][G][PS]: m, l, z[rtv_ld], w[D]
  int T, D, H, G, chunk, n_chunks, rtv_ld, PS;
  float scale;        // 1 / sqrt(d_h)
};
struct AttnMergeArgs {
  const float *part;
  int n_chunks, H, G, D, T, rTv, rtv_ld, PS, bits_v, Kd;
  const float *DmV;  // [H][D][Kd]: D_h^T of the value backbone
  const float *Q;    // [D][D] rotation
  const void *k_tail, *v_tail;  // [H][n_tail][D] cache dtype, keys before RoPE
  int n_tail;
  const float *q, *rope;
  float scale;
  float *out;  // [H G][D]
};
void attend_cells(int dtype, const AttnArgs &a, hipStream_t st);
void attend_merge(int dtype, const AttnMergeArgs &m, hipStream_t st);

void encode_cells(int dtype, const EncArgs &a, int ncells, int T, int D, int GHmax, hipStream_t st);
void decode_cells(int dtype, const DecCell *d_cells, int ncells, int T, int D, int GHmax, hipStream_t st);

}  // namespace jolt
