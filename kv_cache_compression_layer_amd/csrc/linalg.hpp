// Host launchers of the fp64 dense linear algebra kernels (linalg.hip).
#pragma once
#include "common.hpp"

namespace jolt {

// Eigenvalues (descending) of `batch` symmetric n x n fp64 matrices A[b] (overwritten).
// d, e, beta: [batch][n]; refl: [batch][n][n]; t_bs must equal n.  mwg (optional, 8-byte
// aligned, tridiag_mwg_bytes(n, batch) bytes) lets matrices too large for one workgroup's LDS be
// reduced by several workgroups each: up to 576 wide with their rows spread over those
// workgroups' LDS, wider ones by the blocked reduction of tridiag_blk.hip.
size_t tridiag_mwg_bytes(int n, int batch);

// Blocked Householder tridiagonalisation (tridiag_blk.hip) for 576 < n with 3 n doubles of LDS:
// scratch of tridiag_blocked_doubles(n) doubles per matrix; same outputs as sym_eigvals' reduction.
long long tridiag_blocked_doubles(int n);
bool tridiag_blocked_fits(int n);
void tridiag_blocked(double *A, long long a_bs, int lda, int n, int batch, double *d, double *e, double *refl,
                     double *beta, long long t_bs, double *scr, hipStream_t st);

// Eigenvector back-transformation for large n in compact WY blocks (tridiag_blk.hip): Zw rows as
// for sym_eigvecs (updated in place), Tf: wy_tfactor_doubles(n) doubles per matrix of scratch.
long long wy_tfactor_doubles(int n);
void backtransform_wy(double *Zw, long long z_bs, const double *refl, const double *beta, long long t_bs, int n,
                      const int *k_dev, int kmax, int batch, double *Tf, long long tf_bs, double *out64, float *out32,
                      long long out_bs, int out_ld, hipStream_t st);
void sym_eigvals(double *A, long long a_bs, int lda, int n, int batch, double *d, double *e, double *refl,
                 double *beta, long long t_bs, double *evals, long long ev_bs, bool clamp, hipStream_t st,
                 double *mwg = nullptr);

// Eigenvectors of the k_dev[b] largest eigenvalues (after sym_eigvals), as rows
// out[b][j][0..n) (fp64 and/or fp32; out_ld >= n).  Zw: [batch][kmax][n] scratch,
// work: invit_work_doubles(n, kmax) per batch.
size_t invit_work_doubles(int n, int kmax);
void sym_eigvecs(const double *d, const double *e, const double *refl, const double *beta, long long t_bs,
                 const double *evals, long long ev_bs, int n, const int *k_dev, int kmax, int batch, double *Zw,
                 long long z_bs, double *work, long long w_bs, double *out64, float *out32, long long out_bs,
                 int out_ld, hipStream_t st);

// G[b] (fp64, n x n SPD) = R^T R; writes (R^{-1})^T as fp32 [n][ld_out] and its max |entry|.
// Rw: [batch][chol_scratch_doubles(n)] fp64 scratch (R, then the inverses of its 32 x 32
// diagonal blocks).
long long chol_scratch_doubles(int n);
void chol_inv(const double *G, long long g_bs, int ldg, int n, int batch, double *Rw, long long r_bs, float *RinvT,
              long long o_bs, int ld_out, float *amax, hipStream_t st);

// H[b] = P[b] P[b]^T in fp64 for fp32 rows P[b] [rows][ldp] (K columns used).
void gram64(const float *P, long long p_bs, int ldp, int rows, int K, double *H, long long h_bs, int ldh, int batch,
            hipStream_t st);

}  // namespace jolt
