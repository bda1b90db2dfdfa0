// Allocation kernel interface (alloc.hip).
#pragma once
#include "common.hpp"

namespace jolt {

struct AllocOut {
  int status;
  int iters;
  double lambda;
  long long S;
  double E;
  unsigned sync;  // step counter of the one-workgroup-per-cell kernel (cleared before it runs)
  unsigned err;   // set when one of its bounded waits ran out
};

// status of an allocation whose workgroups could not all be scheduled together
constexpr int kAllocEsync = -100;
constexpr const char *kAllocEsyncMsg =
    "allocation: its workgroups could not all be scheduled together (other work on the device)";

struct AllocArgs {
  static constexpr int kMaxCells = 4096;
  int n_cells;
  const int *shape;           // device [n_cells][4] = {G, H, T, D}
  int elem_bytes;
  const double *specT;        // device
  const long long *specT_off; // device [n_cells+1]
  const double *specD;
  const long long *specD_off;
  const double *norm2;        // device [n_cells]
  const int *rT_grid;         // device
  int n_rT;
  const int *rd_grid;
  int n_rd;
  const int *bits;            // device [n_bits], ascending, bits[0] == 0
  int n_bits;
  const double *eps2;         // device [9]
  double budget;
  int greedy;                 // per-cell minimiser: 0 exact argmin over the grid, 1 the greedy rank search
  int cell_first, cell_step;  // cell k of this run is cell cell_first + k * cell_step of shape, the
                              // spectra, norm2, out_pick and out_err (scratch is indexed by k)
  double *tailT;              // scratch [n_cells][n_rT]
  double *tailD;              // scratch [n_cells][n_rd]
  double *e;                  // scratch [n_cells][n_bits*n_rT*n_rd]
  long long *s;               // scratch, same shape
  int *out_pick;              // [n_cells] grid index (b-major, then r_T, then r_d)
  double *out_err;            // [n_cells] table distortion e of each pick (may be null)
  AllocOut *out;
};

void run_alloc(const AllocArgs &a, hipStream_t st);

}  // namespace jolt
