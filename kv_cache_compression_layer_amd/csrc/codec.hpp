// Host-side descriptors and launchers of the residual codec kernels (codec.hip).
#pragma once
#include "common.hpp"

namespace jolt {

// One cell of the encode pass, as byte offsets from the bases in EncArgs (so that every address
// the kernel forms derives from a kernel argument and compiles to global memory instructions).
// Bcat[j][n][k] (fp32, row pitch Kb): k < D -> Q[k][n]; D <= k < D + rT -> -(D_j Q)[k - D][n].
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

void encode_cells(int dtype, const EncArgs &a, int ncells, int T, int D, int GHmax, hipStream_t st);
void decode_cells(int dtype, const DecCell *d_cells, int ncells, int T, int D, int GHmax, hipStream_t st);

}  // namespace jolt
