// Small device kernels (misc.hip).
#pragma once
#include "common.hpp"

namespace jolt {

// Per-cell blob pointers for the factor writers/readers and the header writer.
struct FactorCell {
  void *header;
  void *UT;    // [T][rT]
  void *Ud;    // [D][rd]
  void *core;  // [GH][rT][rd]
  int rT, rd, bits, pad;
  uint32_t hdr[10];
  void *pad_ptr[5];  // alignment padding after U_T, U_d, core, scales, codes (zeroed by the header writer)
  int pad_len[5];
};

void gen_omega(void *out, int dtype, int M, int ell, uint64_t key, hipStream_t st);
void fill_f32(float *p, long long n, float v, hipStream_t st);
// S[s][l] = U_l U_{l+1}^T (k x k, fp64) for consecutive layers of each sequence; U holds k rows of
// length T (pitch ld) per cell, cells (sequence, layer, K|V) at stride cell_stride
void pair_cross(const float *U, long long cell_stride, int ld, int T, int k, int L, int n_seq, double *S,
                hipStream_t st);
void fill_f64(double *p, long long n, double v, hipStream_t st);
void trace_f64(const double *G, long long g_bs, int n, int batch, double *out, hipStream_t st);
void flash_spec(const double *evals, long long ev_bs, int q, const double *norm2, double *specT, long long sp_bs,
                int batch, hipStream_t st);
void put_ut(int dtype, const FactorCell *cells, int ncells, const float *UTt, long long ut_bs, int ld_in, int T,
            int kmax, hipStream_t st);
void put_small(int dtype, const FactorCell *cells, int ncells, const float *Udrows, long long ud_bs, const float *Cp,
               long long cp_bs, int kmax, int kmax_d, int D, int GH, float *Udr, float *Cr, hipStream_t st);
void get_small(int dtype, const FactorCell *cells, int ncells, int kmax, int kmax_d, int D, int GH, float *Udr,
               float *Cr, hipStream_t st);
void write_headers(const FactorCell *cells, int ncells, hipStream_t st);
void bcat_q(float *Bcat, int ncells, int GH, int D, int Kb, const float *Qt, hipStream_t st);
void amax_cells(const float *x, long long per, long long bs, int ncells, float *out, hipStream_t st);
// RoPE cosine / sine table: out[p][i] = {cos a, sin a}, a = fp32(p) * inv[i] rounded to fp32, for
// p < n_pos and i < H2 (inv: host array of H2 <= 64 inverse frequencies)
void rope_table(const float *inv, int H2, int n_pos, float *out, hipStream_t st);

}  // namespace jolt
