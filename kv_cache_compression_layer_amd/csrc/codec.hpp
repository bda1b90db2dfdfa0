// Host-side descriptors and launchers of the residual codec kernels (codec.hip).
#pragma once
#include "common.hpp"

namespace jolt {

// One cell of the encode pass.  Bcat[j][n][k] (fp32, row pitch Kb): k < D -> Q[k][n];
// D <= k < D + rT -> -(D_j Q)[k - D][n].  b_amax: device max |Bcat| (fp16 split scale).
struct EncCell {
  const void *X;      // [GH][T][D] cache dtype
  const void *UT;     // [T][rT] storage dtype
  const float *Bcat;  // [GH][D][Kb]
  const float *b_amax;
  float *scales;      // [GH*T]
  uint8_t *codes;     // [GH*T][D*bits/8]
  int GH, rT, bits, Kb;
};

// One cell of the decode pass.  Dm[j][n][r] = D_j[r][n] (fp32, row pitch Kd); Q row-major.
struct DecCell {
  const void *UT;      // [T][rT] storage dtype
  const float *Dm;     // [GH][D][Kd]
  const float *Q;      // [D][D] rotation
  const float *d_amax; // device max |Dm|
  const float *scales;
  const uint8_t *codes;
  void *out;           // [GH][T][D] cache dtype
  int GH, rT, bits, Kd;
};

void encode_cells(int dtype, const EncCell *d_cells, int ncells, int T, int D, int GHmax, hipStream_t st);
void decode_cells(int dtype, const DecCell *d_cells, int ncells, int T, int D, int GHmax, hipStream_t st);

}  // namespace jolt
