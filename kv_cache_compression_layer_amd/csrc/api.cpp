// C ABI of libjolt: argument validation, workspace carving and stage sequencing.  Work is ordered on
// the caller's stream; the spectra stages of disjoint cell ranges fork onto library-owned side
// streams (default priority) and join back before the allocation reads them.
//
// Pipeline of jolt_compress (Krishnan & Schulz, "A JoLT for the KV Cache", Sec. 3 and 3.1):
//   spectra   feature Gram -> ||X||^2, unprojected feature spectrum;
//             FlashJoLT: Y = X_(T) Omega, Cholesky-QR, power iteration, B = Q^T X_(T),
//             eig(B B^T) -> q_cap values + tail entry;  exact: eig(X_(T) X_(T)^T)
//   allocate  distortion/byte table + Lagrangian bisection (one stream sync for the picks)
//   fit       token factor, token projection, projected feature Gram -> U_d, core,
//             rounding into the blob
//   residual  [X | U_T][Q ; -D_j Q] -> per-row b-bit codes and fp32 scales
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <functional>
#include <mutex>
#include <string>
#include <vector>

#include "alloc.hpp"
#include "codec.hpp"
#include "common.hpp"
#include "linalg.hpp"
#include "misc.hpp"
#include "setup.hpp"

namespace jolt {

static thread_local std::string g_err;
void set_error(const std::string &msg) { g_err = msg; }
const char *get_error() { return g_err.c_str(); }

// Spin limit of the bounded cross-workgroup waits (about 2M polls of s_sleep 1: well beyond any
// wait of co-resident workgroups) and the test-only target offset.
static std::atomic<unsigned> g_spin_limit{1u << 21};
static std::atomic<unsigned> g_target_extra{0u};
WaitPolicy wait_policy() { return WaitPolicy{g_spin_limit.load(), g_target_extra.load()}; }

// ------------------------------------------------------------------------------------ profiler
// Optional per-stage timing with HIP events recorded on the caller's stream (off by default).
struct StageRec {
  const char *name;
  hipEvent_t a, b;
};
static std::vector<StageRec> g_recs;
static bool g_prof = false;

struct Stage {
  hipStream_t st;
  StageRec rec;
  bool on;
  Stage(const char *name, hipStream_t s) : st(s), on(g_prof) {
    if (!on) return;
    rec.name = name;
    HIP_TRY(hipEventCreate(&rec.a));
    HIP_TRY(hipEventCreate(&rec.b));
    HIP_TRY(hipEventRecord(rec.a, st));
  }
  void end() {
    if (!on) return;
    on = false;
    if (hipEventRecord(rec.b, st) == hipSuccess) g_recs.push_back(rec);
  }
  ~Stage() { end(); }
};

namespace {

constexpr int BIG = 1 << 30;

inline long long rup(long long x, long long a) { return (x + a - 1) / a * a; }

// ------------------------------------------------------------------------------------ workspace
struct Arena {
  char *base = nullptr;
  size_t cap = 0, off = 0;
  bool dry = true;
  template <class T>
  T *take(long long count) {
    size_t bytes = (size_t)rup(std::max<long long>(count, 1) * (long long)sizeof(T), 256);
    T *p = dry ? nullptr : (T *)(base + off);
    off += bytes;
    if (!dry && off > cap) {
      set_error("workspace too small: need more than " + std::to_string(cap) + " bytes");
      throw Fail{JOLT_EWORKSPACE};
    }
    return p;
  }
};

// ------------------------------------------------------------------------------------ plan
struct Plan {
  int n_seq, L, H, T, D, dtype, n_groups, G, GH, M, n_cells, c;
  int mode, q, ell, ell_ld, T_ld, power_iters, nT;
  std::vector<int> rT, rd, bits;
  double eps2[9];
  double C;
  uint64_t rot_seed, sketch_seed;
  long long cell_elems() const { return (long long)GH * T * D; }
  int xmf() const { return dtype == JOLT_F16 ? MF_F16 : MF_BF16; }
  int fp32_planes() const { return xmf() == MF_F16 ? 2 : 3; }  // planes of an fp32 operand
  long long pln_cell() const { return (long long)fp32_planes() * ell * std::max<long long>(T_ld, M); }
  long long apl_cell() const { return (long long)fp32_planes() * ell * rup(ell, 32); }
  // FlashJoLT keeps its bases' row layout ([T][ell_ld]) only when some product reads it: with fp16
  // planes and at least one power iteration, every such product runs on the basis planes instead
  bool rows_layout() const {
    return !(xsrc() != SRC_F32 && xmf() == MF_F16 && fp32_planes() == 2 && T % 32 == 0 && power_iters >= 1);
  }
  int xsrc() const { return dtype == JOLT_F16 ? SRC_F16 : (dtype == JOLT_BF16 ? SRC_BF16 : SRC_F32); }
};

void check_grid(const int32_t *g, int n, const char *name, std::vector<int> &out) {
  JOLT_REQUIRE(g != nullptr && n > 0, JOLT_EINVAL, std::string(name) + ": empty grid");
  out.assign(g, g + n);
  for (int i = 0; i < n; ++i) {
    JOLT_REQUIRE(out[i] >= 8 && out[i] % 8 == 0, JOLT_EINVAL, std::string(name) + ": ranks must be positive multiples of 8");
    if (i) JOLT_REQUIRE(out[i] > out[i - 1], JOLT_EINVAL, std::string(name) + ": grid must be strictly ascending");
  }
}

void fill_bits_eps(const jolt_params *p, int D, Plan &pl) {
  std::vector<int> b;
  if (p->bits && p->n_bits > 0) b.assign(p->bits, p->bits + p->n_bits);
  JOLT_REQUIRE(p->n_bits >= 0, JOLT_EINVAL, "bits: negative count");
  b.push_back(0);
  for (int v : b) JOLT_REQUIRE(v >= 0 && v <= 8, JOLT_EINVAL, "bits must lie in 0..8");
  std::sort(b.begin(), b.end());
  b.erase(std::unique(b.begin(), b.end()), b.end());
  pl.bits = b;
  if (p->eps2) {
    JOLT_REQUIRE(p->eps2[0] == 1.0, JOLT_EINVAL, "eps2[0] must be 1");
    for (int v : b) JOLT_REQUIRE(isfinite(p->eps2[v]) && p->eps2[v] >= 0.0, JOLT_EINVAL, "eps2 must be finite and >= 0");
    for (int i = 0; i < 9; ++i) pl.eps2[i] = p->eps2[i];
  } else {
    const std::vector<double> &t = eps2_table(D);
    for (int i = 0; i < 9; ++i) pl.eps2[i] = t[i];
  }
}

// jolt_alloc_variant flags: known ones only, uniform ranks alone
void check_variant(int v) {
  JOLT_REQUIRE(v >= 0 && (v & ~(JOLT_ALLOC_GREEDY | JOLT_ALLOC_KV_DECOUPLED | JOLT_ALLOC_UNIFORM_RANKS)) == 0 &&
                   (!(v & JOLT_ALLOC_UNIFORM_RANKS) || v == JOLT_ALLOC_UNIFORM_RANKS),
               JOLT_EINVAL, "alloc_variant: unknown flags, or uniform ranks combined with another variant");
}

Plan make_plan(const jolt_cache_desc *d, const jolt_params *p) {
  JOLT_REQUIRE(d && p, JOLT_EINVAL, "null descriptor or params");
  Plan pl;
  pl.n_seq = d->n_seq;
  pl.L = d->n_layers;
  pl.H = d->n_heads;
  pl.T = d->n_tokens;
  pl.D = d->d_head;
  pl.dtype = d->dtype;
  JOLT_REQUIRE(pl.n_seq >= 1 && pl.L >= 1 && pl.H >= 1 && pl.T >= 1, JOLT_EINVAL, "cache shape must be positive");
  JOLT_REQUIRE(pl.D == 64 || pl.D == 128, JOLT_EINVAL, "d_head must be 64 or 128");
  JOLT_REQUIRE(pl.dtype == JOLT_F16 || pl.dtype == JOLT_BF16 || pl.dtype == JOLT_F32, JOLT_EINVAL, "bad dtype");
  JOLT_REQUIRE(d->n_groups >= 1 && d->group_start, JOLT_EINVAL, "no layer groups");
  pl.n_groups = d->n_groups;
  JOLT_REQUIRE(d->group_start[0] == 0 && d->group_start[pl.n_groups] == pl.L, JOLT_EINVAL,
               "group_start must run from 0 to n_layers");
  pl.G = d->group_start[1] - d->group_start[0];
  for (int g = 0; g < pl.n_groups; ++g) {
    JOLT_REQUIRE(d->group_start[g + 1] > d->group_start[g], JOLT_EINVAL, "group_start must be increasing");
    JOLT_REQUIRE(d->group_start[g + 1] - d->group_start[g] == pl.G, JOLT_EINVAL,
                 "this entry point needs layer groups of one size (jolt_compress and jolt_reconstruct take any)");
  }
  pl.GH = pl.G * pl.H;
  pl.M = pl.GH * pl.D;
  pl.n_cells = pl.n_seq * pl.n_groups * 2;
  JOLT_REQUIRE(pl.n_cells <= AllocArgs::kMaxCells, JOLT_EINVAL, "too many cells");
  pl.c = dtype_bytes(pl.dtype);
  pl.mode = p->mode;
  JOLT_REQUIRE(pl.mode == JOLT_EXACT || pl.mode == JOLT_FLASH, JOLT_EINVAL, "bad mode");
  check_variant(p->alloc_variant);
  JOLT_REQUIRE(p->target_ratio > 1.0 && isfinite(p->target_ratio), JOLT_EINVAL, "target_ratio must exceed 1");
  pl.C = p->target_ratio;
  check_grid(p->rT_grid, p->n_rT, "rT_grid", pl.rT);
  check_grid(p->rd_grid, p->n_rd, "rd_grid", pl.rd);
  JOLT_REQUIRE(pl.rd.back() <= pl.D, JOLT_EINVAL, "rd_grid exceeds d_head");
  fill_bits_eps(p, pl.D, pl);
  pl.rot_seed = p->rot_seed;
  pl.sketch_seed = p->sketch_seed;
  pl.T_ld = (int)rup(pl.T, 8);
  if (pl.mode == JOLT_FLASH) {
    JOLT_REQUIRE(p->oversample >= 0 && p->power_iters >= 0, JOLT_EINVAL, "oversample / power_iters must be >= 0");
    int q = p->qcap > 0 ? p->qcap : std::min(std::max(pl.C <= 4.0 ? 32 : 64, (pl.T + 31) / 32), 512);
    int ell = std::min({q + p->oversample, pl.T, pl.M});
    q = std::min(q, ell);
    pl.q = q;
    pl.ell = ell;
    pl.power_iters = p->power_iters;
    pl.nT = q + 1;
    JOLT_REQUIRE(pl.rT.back() <= q, JOLT_EINVAL, "rT_grid exceeds q_cap");
    JOLT_REQUIRE(ell <= 544, JOLT_EINVAL, "q_cap + oversample must not exceed 544");
  } else {
    JOLT_REQUIRE(pl.T <= pl.M, JOLT_EINVAL, "exact mode needs T <= |g| n_h d_h");
    pl.q = pl.T;
    pl.ell = pl.T;
    pl.power_iters = 0;
    pl.nT = pl.T;
    JOLT_REQUIRE(pl.rT.back() <= pl.T, JOLT_EINVAL, "rT_grid exceeds min(T, M)");
  }
  pl.ell_ld = (int)rup(pl.ell, 16);
  return pl;
}

// ------------------------------------------------------------------------------------ buffers
struct Bufs {
  // common
  float *part;
  float *fpart;  // feature Gram partials (own region: that stage may run beside the token stages)
  double *perr;  // [n_cells] table distortion of each pick (read back with the picks)
  long long fpart_elems;
  double *Gd64, *dD, *eD, *betaD, *evD;
  double *specT, *specD, *norm2;
  // flash / exact token stage
  void *omegaT;
  // tall panels, each in two layouts: rows of length T ([ell][T_ld]) and rows of length ell
  // ([T][ell_ld]); P likewise ([ell][M] and [M][ell_ld]); Z only as Z^T ([ell][M])
  float *bufA, *bufB, *bufA2, *bufB2, *Pt, *P2, *Zt, *RinvT, *YpT;
  double *G64, *Rw, *dT, *eT, *betaT, *evT;
  double *mwg;  // exchange scratch of the multi-workgroup tridiagonalisation (FlashJoLT B B^T)
  float *amax;  // [9][n_cells]: slot k of cell c at amax[k * am_ld + c]
  int am_ld;
  // FlashJoLT keeps the final basis implicit (Q = Y R^{-1} is never formed).  The fit then reads Y
  // ([T][ell_ld], bufA2) with its |max| basis_am, R^{-T} (RinvT) and P' = Y^T X (P2); Wt holds
  // W~ = R^{-1} W as rows.  basis_implicit = 0: bufA2 holds an orthonormal Q.
  int basis_implicit;
  float *basis_am;
  float *Wt;
  // whether the bases' row layout ([T][ell_ld], bufA2 / bufB2) exists (Plan::rows_layout)
  int rows_layout;
  // fit
  float *Wrows, *Udrows, *Cp, *Udr, *Cr, *Vt, *Bcat, *bamax, *Qf, *Qtf;
  uint16_t *Bpl;  // 16-bit planes of Bcat, [cell][plane][GH][D][Kb]
  double *Zw, *work, *ZwD, *workD;
  // alloc
  double *tailT, *tailD, *tab_e;
  long long *tab_s;
  int *pick;
  AllocOut *aout;
  // 16-bit planes of an fp32 operand of the plane GEMM: Q^T for the projection, Z^T for the
  // power-iteration sketch (used one after the other), [cell][plane][ell][max(T_ld, M)]
  uint16_t *pln;
  // 16-bit planes of a small fp32 left factor whose product runs on the basis planes (R^{-T} of a
  // Cholesky-QR apply, the factor rows of U_T): [cell][plane][ell][rup(ell, 32)], columns past ell zero
  uint16_t *apl;
  // device parameter area
  char *params;
  size_t params_bytes;
  long long part_elems;
};

int nsplit_for(long long K, long long tiles, int batch, long long min_chunk) {
  long long want = (2048 + tiles * batch - 1) / (tiles * batch);
  long long maxs = std::max<long long>(1, K / min_chunk);
  return (int)std::max<long long>(1, std::min<long long>(want, std::min<long long>(maxs, 256)));
}

long long tiles_of(long long M, long long N) { return ((M + 127) / 128) * ((N + 127) / 128); }

// K splits of a Gram of `rows` rows on the DMA plane kernel (192 x 192 tiles, the upper triangle's
// tiles working): about 2048 working blocks, K chunks of at least 1024
int gram_plane_splits(long long rows, long long K, int batch) {
  const long long t = (rows + 191) / 192;
  return nsplit_for(K, t * (t + 1) / 2, batch, 1024);
}

// The spectra of the cells can run as kViews independent chains of consecutive cells on their own
// streams, each with its own split-K scratch.  Measured on the 8B shape, two chains gained nothing
// over one (the matrix-core launches of one chain already fill the GPU, and the fp64 stages of a
// chain lose their CUs to the other's), so one chain is used.
constexpr int kViews = 1;

// Exact mode: token Grams wider than the register-resident one-workgroup reduction take the blocked
// multi-launch reduction (its panels and partial products need a scratch per cell).
bool exact_blocked(const Plan &pl) { return pl.mode != JOLT_FLASH && pl.T > 576 && tridiag_blocked_fits((int)pl.T); }

int n_views(const Plan &pl) {
  int v = kViews;
  while (v > 1 && (pl.n_cells % (2 * v) != 0)) --v;  // views hold whole (group, K|V) pairs
  return v;
}

struct Sizes {
  int kmax, kmax_d, Kb;
  long long part_elems;    // whole split-K scratch
  long long part_view;     // per spectra view (the first n_views of them are disjoint slices)
};

// K splits of the FlashJoLT projection: one per 16384 tokens, at most 4 (K = T is the long side).
// Measured on the 8B shape (3 x 16 output tiles per cell): 4 splits beat 8 and 16, whose extra
// partial sums cost more write and reduction traffic than the shorter blocks gain.
int project_splits(const Plan &pl) { return (int)std::min<long long>(4, std::max<long long>(1, pl.T / 16384)); }

// split-K partials of the unprojected feature Gram (K = GH T_ld, padding included)
long long feature_part_elems(const Plan &pl, int nb) {
  const int ns = nsplit_for((long long)pl.GH * pl.T, 1, nb, 8192);
  return rup((long long)nb * ns * pl.D * pl.D, 64);
}

long long part_elems_for(const Plan &pl, int kmax, int nb) {
  long long pe = 0;
  {  // feature Gram partials
    int ns = nsplit_for((long long)pl.GH * pl.T, 1, nb, 8192);  // K of the feature Gram
    pe = std::max(pe, (long long)nb * ns * pl.D * pl.D);
    int ns2 = nsplit_for((long long)kmax * pl.GH, 1, nb, 1024);
    pe = std::max(pe, (long long)nb * ns2 * pl.D * pl.D);
  }
  if (pl.mode == JOLT_FLASH) {
    const int ps = project_splits(pl);
    if (ps > 1) pe = std::max(pe, (long long)nb * ps * pl.ell * pl.M);
    int ns = nsplit_for(pl.T, tiles_of(pl.ell, pl.ell), nb, 1024);
    pe = std::max(pe, (long long)nb * ns * pl.ell * pl.ell_ld);
    int ns2 = nsplit_for(pl.M, tiles_of(pl.ell, pl.ell), nb, 1024);
    pe = std::max(pe, (long long)nb * ns2 * pl.ell * pl.ell_ld);
    int ns3 = gram_plane_splits(pl.ell, pl.T, nb);
    pe = std::max(pe, (long long)nb * ns3 * pl.ell * rup(pl.ell, 16));
  } else {
    int ns = nsplit_for(pl.M, tiles_of(pl.T, pl.T), nb, 1024);
    pe = std::max(pe, (long long)nb * ns * pl.T * pl.T_ld);
  }
  return rup(pe, 64);
}

Sizes sizes_for(const Plan &pl, int kmax, int kmax_d) {
  Sizes s;
  s.kmax = kmax;
  s.kmax_d = kmax_d;
  s.Kb = (int)rup(pl.D + kmax, 32);  // the encode's 32-deep stages read whole rows of B (zero padded)
  const int nv = n_views(pl);
  s.part_view = part_elems_for(pl, kmax, pl.n_cells / nv);
  s.part_elems = std::max(part_elems_for(pl, kmax, pl.n_cells), nv * s.part_view);
  return s;
}

Bufs carve(Arena &ar, const Plan &pl, const Sizes &sz) {
  Bufs b{};
  const int nb = pl.n_cells, D = pl.D;
  const long long ell = pl.ell, ld = pl.ell_ld;
  b.part = ar.take<float>(sz.part_elems);
  {
    const int nv = n_views(pl);
    Plan pv = pl;
    pv.n_cells = nb / nv;
    b.fpart_elems = std::max(feature_part_elems(pl, nb), nv * feature_part_elems(pv, pv.n_cells));
    b.fpart = ar.take<float>(b.fpart_elems);
  }
  b.Gd64 = ar.take<double>((long long)nb * D * D);
  b.dD = ar.take<double>((long long)nb * D);
  b.eD = ar.take<double>((long long)nb * D);
  b.betaD = ar.take<double>((long long)nb * D);
  b.evD = ar.take<double>((long long)nb * D);
  b.specT = ar.take<double>((long long)nb * pl.nT);
  b.specD = ar.take<double>((long long)nb * D);
  b.norm2 = ar.take<double>(nb);
  b.amax = ar.take<float>(9LL * nb);
  b.am_ld = nb;
  const long long n_tok = pl.mode == JOLT_FLASH ? ell : pl.T;  // size of the token-side eigenproblem
  b.G64 = ar.take<double>((long long)nb * n_tok * n_tok);
  b.dT = ar.take<double>((long long)nb * n_tok);
  b.eT = ar.take<double>((long long)nb * n_tok);
  b.betaT = ar.take<double>((long long)nb * n_tok);
  b.evT = ar.take<double>((long long)nb * n_tok);
  if (pl.mode == JOLT_FLASH) {
    b.omegaT = ar.take<char>(ell * pl.M * pl.c);
    b.bufA = ar.take<float>((long long)nb * ell * pl.T_ld);
    b.bufB = ar.take<float>((long long)nb * ell * pl.T_ld);
    b.rows_layout = pl.rows_layout();
    b.bufA2 = b.rows_layout ? ar.take<float>((long long)nb * pl.T * ld) : nullptr;
    b.bufB2 = b.rows_layout ? ar.take<float>((long long)nb * pl.T * ld) : nullptr;
    b.Pt = ar.take<float>((long long)nb * ell * pl.M);
    b.P2 = ar.take<float>((long long)nb * pl.M * ld);
    b.Zt = ar.take<float>((long long)nb * ell * pl.M);
    b.Rw = ar.take<double>((long long)nb * chol_scratch_doubles((int)ell));
    b.mwg = ar.take<double>((long long)(tridiag_mwg_bytes((int)ell, nb) / sizeof(double)));
    b.RinvT = ar.take<float>((long long)nb * ell * ld);
    b.Wrows = ar.take<float>((long long)nb * sz.kmax * ld);
    b.Wt = ar.take<float>((long long)nb * sz.kmax * ld);
    b.pln = pl.xsrc() == SRC_F32 ? nullptr : ar.take<uint16_t>((long long)nb * pl.pln_cell());
    b.apl = pl.xsrc() == SRC_F32 ? nullptr : ar.take<uint16_t>((long long)nb * pl.apl_cell());
  } else {
    b.bufB = ar.take<float>((long long)nb * sz.kmax * pl.T_ld);  // token factor rows
    b.Zt = ar.take<float>((long long)nb * sz.kmax * pl.M);       // token-projected tensor
    if (exact_blocked(pl)) b.mwg = ar.take<double>((long long)(tridiag_mwg_bytes((int)pl.T, nb) / sizeof(double)));
  }
  b.Zw = ar.take<double>((long long)nb * sz.kmax * n_tok);
  b.work = ar.take<double>((long long)nb * invit_work_doubles((int)n_tok, sz.kmax));
  b.ZwD = ar.take<double>((long long)nb * sz.kmax_d * D);
  b.workD = ar.take<double>((long long)nb * invit_work_doubles(D, sz.kmax_d));
  b.YpT = ar.take<float>((long long)nb * pl.M * sz.kmax);
  b.Udrows = ar.take<float>((long long)nb * sz.kmax_d * D);
  b.Cp = ar.take<float>((long long)nb * sz.kmax * pl.GH * sz.kmax_d);
  b.Udr = ar.take<float>((long long)nb * sz.kmax_d * D);
  b.Cr = ar.take<float>((long long)nb * pl.GH * sz.kmax * sz.kmax_d);
  b.Vt = ar.take<float>((long long)nb * D * sz.kmax_d);
  b.Bcat = ar.take<float>((long long)nb * pl.GH * D * sz.Kb);
  b.Bpl = ar.take<uint16_t>((long long)nb * pl.fp32_planes() * pl.GH * D * sz.Kb);
  b.bamax = ar.take<float>(nb);
  b.Qf = ar.take<float>((long long)D * D);
  b.Qtf = ar.take<float>((long long)D * D);
  const long long per = (long long)pl.bits.size() * pl.rT.size() * pl.rd.size();
  b.tailT = ar.take<double>((long long)nb * pl.rT.size());
  b.tailD = ar.take<double>((long long)nb * pl.rd.size());
  b.tab_e = ar.take<double>(nb * per);
  b.tab_s = ar.take<long long>(nb * per);
  b.pick = ar.take<int>(nb);
  b.perr = ar.take<double>(nb);
  b.aout = ar.take<AllocOut>(1);
  b.params_bytes = (size_t)rup(64 * 1024 + 2LL * D * D * 4 +
                                   (long long)nb * (sizeof(EncCell) + sizeof(DecCell) + sizeof(FactorCell) + 64) +
                                   (pl.rT.size() + pl.rd.size() + 16) * 4,
                               256);
  b.params = ar.take<char>((long long)b.params_bytes);
  b.part_elems = sz.part_elems;
  return b;
}

// ------------------------------------------------------------------------------------ helpers
GemmArgs ga() {
  GemmArgs g;
  memset(&g, 0, sizeof(g));
  g.a_blk = g.b_blk = BIG;
  g.a_amax_c = g.b_amax_c = 1.f;
  g.ab_amax_bs = g.c_amax_bs = 1;
  g.inner = 1;
  g.alpha = 1.f;
  return g;
}

// Run the same X-operand GEMM for the K cells (t = 0) and the V cells (t = 1): cells are
// c = 2 i + t, so per-cell outputs use stride 2 and offset t.
template <class F>
void for_kv(const void *K, const void *V, F f) {
  f(0, K);
  f(1, V);
}

struct Upload {
  std::vector<char> host;
  size_t add(const void *p, size_t n) {
    size_t o = (host.size() + 255) / 256 * 256;
    host.resize(o + n);
    memcpy(host.data() + o, p, n);
    return o;
  }
};

void upload(Bufs &b, Upload &u, hipStream_t st) {
  JOLT_REQUIRE(u.host.size() <= b.params_bytes, JOLT_EWORKSPACE, "parameter area too small");
  if (!u.host.empty()) HIP_TRY(hipMemcpyAsync(b.params, u.host.data(), u.host.size(), hipMemcpyHostToDevice, st));
}

void gram_f32(const Plan &pl, Bufs &b, const float *X, long long ldx, long long xbs, int rows, int K, const float *amax,
              double *out, long long out_bs, int ldo, int batch, hipStream_t st) {
  // out[b] (fp64, rows x rows) = X[b] X[b]^T for fp32 rows X[b] [rows][ldx] (K columns)
  GemmArgs g = ga();
  g.A = X; g.B = X;
  g.M = rows; g.N = rows; g.K = K;
  g.a_ld = ldx; g.b_ld = ldx; g.a_bs = xbs; g.b_bs = xbs;
  g.a_amax = amax; g.b_amax = amax; g.ab_amax_bs = 1;
  int ns = nsplit_for(K, tiles_of(rows, rows), batch, 1024);
  g.k_chunk = (int)rup((K + ns - 1) / ns, 32);
  ns = (int)((K + g.k_chunk - 1) / g.k_chunk);
  const long long rl = rup(rows, 16);
  JOLT_REQUIRE((long long)batch * ns * rows * rl <= b.part_elems, JOLT_EWORKSPACE, "split-K buffer too small");
  g.C = b.part; g.c_ld = rl; g.c_split = (long long)rows * rl; g.c_bs = (long long)ns * rows * rl;
  g.m_fastest = 1;
  g.tri = 1;  // the Cholesky factorisation reads the upper triangle only
  gemm(MF_F16, SRC_F32, true, SRC_F32, true, g, batch, ns, st);
  reduce_splits(b.part, g.c_bs, g.c_split, ns, 0, rows, rows, rl, out, true, out_bs, ldo, batch, st);
}

// gram_f32 on rows already split into their 16-bit planes (P planes [rows][ld] at plane stride ps, batch
// stride bs, split with the scale of amax): the same products on the DMA plane kernel.  False (nothing
// launched) when that kernel does not take the shape.
bool gram_planes(const Plan &pl, Bufs &b, const uint16_t *P, long long ld, long long ps, long long bs, int rows, int K,
                 const float *amax, double *out, long long out_bs, int ldo, int batch, hipStream_t st) {
  const int np = pl.fp32_planes();
  GemmArgs g = ga();
  g.A = P; g.B = P;
  g.M = rows; g.N = rows; g.K = K;
  g.a_ld = g.b_ld = ld; g.a_ps = g.b_ps = ps; g.a_bs = g.b_bs = bs;
  g.a_amax = amax; g.b_amax = amax; g.ab_amax_bs = 1;
  int ns = gram_plane_splits(rows, K, batch);
  g.k_chunk = (int)rup((K + ns - 1) / ns, 32);
  ns = (int)((K + g.k_chunk - 1) / g.k_chunk);
  const long long rl = rup(rows, 16);
  JOLT_REQUIRE((long long)batch * ns * rows * rl <= b.part_elems, JOLT_EWORKSPACE, "split-K buffer too small");
  g.C = b.part; g.c_ld = rl; g.c_split = (long long)rows * rl; g.c_bs = (long long)ns * rows * rl;
  g.m_fastest = 1;
  g.tri = 1;
  if (!gemm_dma(pl.xmf(), np, np, g, batch, ns, st)) return false;
  reduce_splits(b.part, g.c_bs, g.c_split, ns, 0, rows, rows, rl, out, true, out_bs, ldo, batch, st);
  return true;
}

// --------------------------------------------------------------------------- spectra stage
void stage_feature(const Plan &pl, Bufs &b, const void *K, const void *V, hipStream_t st) {
  Stage prof("feature_gram", st);
  const int D = pl.D;
  const long long Kdim = (long long)pl.GH * pl.T;
  int ns = nsplit_for(Kdim, 1, pl.n_cells, 8192);
  GemmArgs g = ga();
  g.M = D; g.N = D; g.K = (int)Kdim;
  g.k_chunk = (int)rup((Kdim + ns - 1) / ns, 32);
  ns = (int)((Kdim + g.k_chunk - 1) / g.k_chunk);
  // A(m = d, k = (j, t)) = B(k, n = d) = X_j[t][d]: a cell's slices follow one another, so k runs
  // over the rows of the cache, each contiguous along d
  g.a_ld = D; g.b_ld = D;
  g.a_bs = g.b_bs = pl.cell_elems();
  g.c_ld = D; g.c_split = (long long)D * D; g.c_bs = 2LL * ns * D * D;
  JOLT_REQUIRE((long long)pl.n_cells * ns * D * D <= b.fpart_elems, JOLT_EWORKSPACE, "split-K buffer too small");
  for_kv(K, V, [&](int t, const void *X) {
    GemmArgs h = g;
    h.A = X; h.B = X;
    h.C = b.fpart + (long long)t * ns * D * D;
    if (pl.c == 2 && xgram_dma(pl.xmf(), X, h.a_bs, (int)Kdim, D, h.C, h.c_bs, g.k_chunk, ns, pl.n_cells / 2, st))
      return;
    gemm(pl.xmf(), pl.xsrc(), false, pl.xsrc(), false, h, pl.n_cells / 2, ns, st);
  });
  reduce_splits(b.fpart, (long long)ns * D * D, (long long)D * D, ns, 0, D, D, D, b.Gd64, true, (long long)D * D, D,
                pl.n_cells, st);
  trace_f64(b.Gd64, (long long)D * D, D, pl.n_cells, b.norm2, st);
  sym_eigvals(b.Gd64, (long long)D * D, D, D, pl.n_cells, b.dD, b.eD, b.Gd64, b.betaD, D, b.specD, D, true, st);
}

// FlashJoLT token spectrum (Sec. 3.1): randomized subspace iteration with Cholesky QR.
// The cache is read as it is: the sketches contract over its contiguous d (K-contiguous), the
// projections over tokens (B contiguous along d, fed to the matrix cores by transposing LDS reads);
// tall fp32 panels are written in both layouts by the GEMM epilogue so the next consumer never
// transposes while loading.
// mark (optional) is recorded on st once the first orthonormal basis Q_0 exists; the next spectra
// chain waits for it, which puts the chains out of phase.
// side_work (optional): enqueues the feature stage on another stream and returns the event that
// marks its end; it is called once the Gaussian sketch is queued, and st waits for the event
// before it forms the spectrum, the first use of the feature stage's ||X||^2.
void stage_flash(const Plan &pl, Bufs &b, const void *K, const void *V, hipStream_t st, hipEvent_t mark = nullptr,
                 const std::function<hipEvent_t()> &side_work = {}) {
  hipEvent_t xready = nullptr;
  const int nb = pl.n_cells, nkv = nb / 2;
  const long long ell = pl.ell, ld = pl.ell_ld, Tld = pl.T_ld, Mf = pl.M, T = pl.T;
  const long long cellX = pl.cell_elems();
  const int am = b.am_ld;
  float *amY = b.amax, *amR = b.amax + am, *amQ = b.amax + 2 * am, *amP = b.amax + 3 * am, *amZ = b.amax + 4 * am;
  // (Omega is generated and the amax slots are cleared once for all cells by spectra_all)

  // Y^T = A X_(T)^T with A = Omega^T (cache dtype) or Z^T (fp32); also Y = (Y^T)^T when the row layout
  // is kept.  On the plane path an fp32 A is first split into its 16-bit planes (the split the GEMM
  // would make on the fly).
  const int P32 = pl.fp32_planes();
  JOLT_REQUIRE(b.rows_layout || (b.pln && b.apl), JOLT_EINVAL, "basis planes missing");
  const bool dma_ok = b.pln != nullptr;
  auto sketch = [&](const void *A, int a_src, long long a_bs, const float *a_amax, float *outT, float *outR,
                    float *c_amax) {
    bool planes = dma_ok && a_src == SRC_F32 && Mf % 32 == 0;
    if (planes) {
      Stage prof_s("split_planes", st);
      split_planes(pl.xmf(), (const float *)A, ell * Mf, Mf, (int)ell, (int)Mf, (int)Mf, b.pln, P32 * ell * Mf,
                   ell * Mf, Mf, a_amax, 1, nb, st);
    }
    Stage prof("sketch_gemm", st);
    for_kv(K, V, [&](int t, const void *X) {
      GemmArgs g = ga();
      g.A = (const char *)A + (a_bs ? t * a_bs * (a_src == SRC_F32 ? 4 : 2) : 0);
      g.B = X; g.M = (int)ell; g.N = (int)T; g.K = (int)Mf;
      g.a_ld = Mf; g.a_bs = 2 * a_bs;
      g.a_amax = a_amax ? a_amax + t : nullptr; g.ab_amax_bs = 2;
      g.b_ld = pl.D; g.b_blk = pl.D; g.b_blk_stride = T * pl.D; g.b_bs = cellX;
      g.C = outT + t * ell * Tld; g.c_ld = Tld; g.c_bs = 2 * ell * Tld;
      if (b.rows_layout) {
        g.C2 = outR + t * T * ld; g.c2_ld = ld; g.c2_bs = 2 * T * ld;
      }
      g.c_amax = c_amax ? c_amax + t : nullptr; g.c_amax_bs = 2;
      g.m_fastest = 1;
      if (planes) {
        GemmArgs h = g;
        h.A = b.pln + t * P32 * ell * Mf;
        h.a_bs = 2 * P32 * ell * Mf;
        h.a_ps = ell * Mf;
        if (gemm_dma(pl.xmf(), P32, 1, h, nkv, 1, st)) return;
      } else if (dma_ok && a_src != SRC_F32) {
        if (gemm_dma(pl.xmf(), 1, 1, g, nkv, 1, st)) return;
      }
      gemm(pl.xmf(), a_src, true, pl.xsrc(), true, g, nkv, 1, st);
    });
  };
  // The 16-bit planes of a basis Y^T (fp32 [ell][T_ld]), read by its Gram and its projection.
  const bool tplanes = dma_ok && T % 32 == 0;
  auto split_basis = [&](const float *Yt, const float *am) {
    if (!tplanes) return;
    Stage prof_s("split_planes", st);
    split_planes(pl.xmf(), Yt, ell * Tld, Tld, (int)ell, (int)T, (int)T, b.pln, P32 * ell * Tld, ell * Tld, Tld, am, 1,
                 nb, st);
  };
  // P'^T = Y^T X_(T) (ell x M) and P' = (P'^T)^T, from the planes of Y^T when they are in b.pln.  K = T
  // is long: the product is split along K (more, shorter blocks fill the last wave of the grid) and
  // the partials are summed in fixed order by the reduction, which writes both layouts and max |P'|.
  // A basis formed explicitly writes its planes directly (below), split with the scale of this bound:
  // an orthonormal basis has entries of magnitude at most 1, the bound leaves room for the loss of
  // orthogonality of one Cholesky-QR pass (a larger entry overflows the fp16 plane and the spectrum
  // comes out non-finite, reported).
  constexpr float kBasisBound = 2.f;
  const int pns = project_splits(pl);
  // q_amax null: Q^T's planes were split with the scale of kBasisBound; qpl: where they are
  auto project = [&](const float *Qt, const float *q_amax, float *c_amax, const uint16_t *qpl) {
    const bool planes = tplanes;
    Stage prof("project_gemm", st);
    GemmArgs g = ga();
    g.M = (int)ell; g.N = (int)Mf; g.K = (int)T;
    g.a_ld = Tld; g.a_bs = 2 * ell * Tld; g.ab_amax_bs = 2;
    if (!q_amax) g.a_amax_c = kBasisBound;
    // B(k = t, n = (j, d)) = X_j[t][d]: the cache as it is, contiguous along d within a slice
    g.b_ld = pl.D; g.b_blk = pl.D; g.b_blk_stride = T * pl.D; g.b_bs = cellX;
    g.m_fastest = 1;
    int ns = 1;
    if (pns > 1) {
      g.k_chunk = (int)rup((T + pns - 1) / pns, 32);
      ns = (int)((T + g.k_chunk - 1) / g.k_chunk);
      JOLT_REQUIRE((long long)nb * ns * ell * Mf <= b.part_elems, JOLT_EWORKSPACE, "split-K buffer too small");
    }
    const long long part_bs = (long long)ns * ell * Mf;
    for_kv(K, V, [&](int t, const void *X) {
      GemmArgs h = g;
      h.B = X;
      h.a_amax = q_amax ? q_amax + t : nullptr;
      if (ns <= 1) {
        h.C = b.Pt + t * ell * Mf; h.c_ld = Mf; h.c_bs = 2 * ell * Mf;
        h.C2 = b.P2 + t * Mf * ld; h.c2_ld = ld; h.c2_bs = 2 * Mf * ld;
        h.c_amax = c_amax + t; h.c_amax_bs = 2;
      } else {
        h.C = b.part + t * part_bs; h.c_ld = Mf; h.c_split = ell * Mf; h.c_bs = 2 * part_bs;
      }
      if (planes) {
        GemmArgs q = h;
        q.A = qpl + t * P32 * ell * Tld; q.a_bs = 2 * P32 * ell * Tld; q.a_ps = ell * Tld;
        if (gemm_dma(pl.xmf(), P32, 1, q, nkv, ns, st, false)) return;
      }
      // (planes written by the apply over Q's buffer have no fp32 copy to fall back on)
      JOLT_REQUIRE(!planes || qpl == b.pln, JOLT_EINVAL, "projection: the plane product was refused");
      h.A = Qt + t * ell * Tld;
      gemm(pl.xmf(), SRC_F32, true, pl.xsrc(), false, h, nkv, ns, st);
    });
    if (ns <= 1) return;
    prof.end();
    Stage prof_r("project_reduce", st);
    reduce_splits_dual(b.part, part_bs, ell * Mf, ns, (int)ell, (int)Mf, Mf, b.Pt, ell * Mf, Mf, b.P2, Mf * ld, ld,
                       c_amax, nb, st);
  };
  struct Pair {
    float *T, *R, *am;
  };
  Pair pa{b.bufA, b.bufA2, amY}, pb{b.bufB, b.bufB2, amQ};
  // R^{-T} and max |R^{-T}| (b.RinvT, amR) from the Gram of the rows of Y^T (on its planes when split)
  auto chol_only = [&](Pair y) {
    Stage prof("cholqr_tall", st);
    if (!(tplanes && gram_planes(pl, b, b.pln, Tld, ell * Tld, P32 * ell * Tld, (int)ell, (int)T, y.am, b.G64,
                                 ell * ell, (int)ell, nb, st)))
      gram_f32(pl, b, y.T, Tld, ell * Tld, (int)ell, (int)T, y.am, b.G64, ell * ell, (int)ell, nb, st);
    chol_inv(b.G64, ell * ell, (int)ell, (int)ell, nb, b.Rw, chol_scratch_doubles((int)ell), b.RinvT, ell * ld, (int)ld,
             amR, st);
  };
  // An intermediate basis is orthonormalised explicitly, Q^T = R^{-T} Y^T (one Cholesky-QR pass; A =
  // R^{-T} is lower triangular: each row tile stops its k loop at its last row), and only Q^T is
  // written unless `rows` asks for Q = (Q^T)^T too: the next projection reads nothing else.
  // (Projecting Y and applying R^{-1} afterwards would save this product but amplifies the
  // projection's rounding by the condition of Y.)
  // With the basis planes in use and no row layout asked for, Q^T goes straight into 16-bit planes
  // as the projection's operand (scale of kBasisBound) instead of fp32: on the fp16 plane path the
  // product reads Y^T from its planes (b.pln) and writes Q^T's planes over q's fp32 buffer (the same
  // bytes per cell); otherwise it reads Y (fp32) and writes them into b.pln.  Returns where Q^T's
  // planes are (null: Q^T was written as fp32 to q).
  auto orthonormalise = [&](Pair y, Pair q, bool rows) -> const uint16_t * {
    chol_only(y);
    Stage prof("cholqr_tall", st);
    const bool to_planes = tplanes && !rows;
    if (to_planes && pl.xmf() == MF_F16 && P32 == 2 && b.apl) {
      // A = R^{-T} as planes with K padded to a whole stage (zero columns), B = Y^T's planes (rows past
      // ell read as its last row, against those zero columns)
      const long long Kp = rup(ell, 32);
      split_planes(MF_F16, b.RinvT, ell * ld, ld, (int)ell, (int)ell, (int)Kp, b.apl, 2 * ell * Kp, ell * Kp, Kp, amR,
                   1, nb, st);
      uint16_t *qpl = (uint16_t *)q.T;
      GemmArgs g = ga();
      g.A = b.apl; g.a_ld = Kp; g.a_ps = ell * Kp; g.a_bs = 2 * ell * Kp; g.a_amax = amR;
      g.B = b.pln; g.b_ld = Tld; g.b_ps = ell * Tld; g.b_bs = 2 * ell * Tld; g.b_amax = y.am; g.b_krows = (int)ell;
      g.ab_amax_bs = 1;
      g.M = (int)ell; g.N = (int)T; g.K = (int)Kp;
      g.c_ld = Tld;
      g.Cpl = qpl; g.cpl_ps = ell * Tld; g.cpl_bs = 2 * ell * Tld; g.cpl_amax = kBasisBound; g.cpl_mf = MF_F16;
      g.m_fastest = 1;
      g.tri = 4;
      if (gemm_dma(MF_F16, 2, 2, g, nb, 1, st, false)) return qpl;
    }
    JOLT_REQUIRE(b.rows_layout, JOLT_EINVAL, "basis apply: the plane product was refused and no row layout exists");
    GemmArgs g = ga();
    g.A = b.RinvT; g.a_ld = ld; g.a_bs = ell * ld; g.a_amax = amR;
    g.B = y.R; g.b_ld = ld; g.b_bs = T * ld; g.b_amax = y.am;
    g.ab_amax_bs = 1;
    g.M = (int)ell; g.N = (int)T; g.K = (int)ell;
    g.c_ld = Tld; g.c_bs = ell * Tld;
    if (to_planes) {
      g.Cpl = b.pln; g.cpl_ps = ell * Tld; g.cpl_bs = P32 * ell * Tld;
      g.cpl_amax = kBasisBound; g.cpl_mf = pl.xmf();
    } else {
      fill_f32(q.am, nb, 0.f, st);
      g.C = q.T;
      g.c_amax = q.am;
      if (rows) {
        g.C2 = q.R; g.c2_ld = ld; g.c2_bs = T * ld;
      }
    }
    g.m_fastest = 1;
    g.tri = 4;
    gemm(MF_F16, SRC_F32, true, SRC_F32, true, g, nb, 1, st);
    return to_planes ? b.pln : nullptr;
  };
  // The final basis stays implicit: Q = Y R^{-1} is never formed.  Its Gram gives R, the projection
  // runs on Y (P' = Y^T X_(T)), B = Q^T X_(T) = R^{-T} P'^T, and the fit reads Y and R^{-1} instead of
  // Q (U_T = Y (R^{-1} W), Y_p = (R^{-1} W)^T P'), so no second pass is needed for orthogonality.
  b.basis_implicit = 1;
  sketch(b.omegaT, pl.xsrc(), 0, nullptr, pa.T, pa.R, pa.am);
  if (side_work) xready = side_work();
  Pair Y = pa;
  split_basis(Y.T, Y.am);
  for (int it = 0; it < pl.power_iters; ++it) {
    Pair Q = (Y.T == pa.T) ? pb : pa;
    const uint16_t *qpl = orthonormalise(Y, Q, false);
    if (it == 0 && mark) HIP_TRY(hipEventRecord(mark, st));
    if (!qpl) split_basis(Q.T, Q.am);
    fill_f32(amP, nb, 0.f, st);
    project(Q.T, qpl ? nullptr : Q.am, amP, qpl ? qpl : b.pln);
    {
      // Z = orth(P) by Cholesky QR; Z^T feeds the next sketch
      Stage prof_z("cholqr_z", st);
      gram_f32(pl, b, b.Pt, Mf, ell * Mf, (int)ell, (int)Mf, amP, b.G64, ell * ell, (int)ell, nb, st);
      chol_inv(b.G64, ell * ell, (int)ell, (int)ell, nb, b.Rw, chol_scratch_doubles((int)ell), b.RinvT, ell * ld, (int)ld, amR, st);
      fill_f32(amZ, nb, 0.f, st);
      // Z^T = R^{-T} P^T (the sketch reads only Z^T)
      GemmArgs g = ga();
      g.A = b.RinvT; g.a_ld = ld; g.a_bs = ell * ld; g.a_amax = amR;
      g.B = b.P2; g.b_ld = ld; g.b_bs = Mf * ld; g.b_amax = amP;
      g.ab_amax_bs = 1;
      g.M = (int)ell; g.N = (int)Mf; g.K = (int)ell;
      g.C = b.Zt; g.c_ld = Mf; g.c_bs = ell * Mf;
      g.c_amax = amZ;
      g.m_fastest = 1;
      g.tri = 4;
      gemm(MF_F16, SRC_F32, true, SRC_F32, true, g, nb, 1, st);
    }
    // the next sketch overwrites Y's pair (Q's is read no more)
    fill_f32(Y.am, nb, 0.f, st);
    sketch(b.Zt, SRC_F32, ell * Mf, amZ, Y.T, Y.R, Y.am);
    split_basis(Y.T, Y.am);
  }
  if (pl.power_iters == 0) {
    // the raw sketch is orthonormalised once explicitly before it becomes the implicit final basis (a
    // second Cholesky-QR pass, R close to the identity), as its condition is not reduced by an iteration
    Pair Q = pb;
    orthonormalise(Y, Q, true);
    if (mark) HIP_TRY(hipEventRecord(mark, st));
    Y = Q;
    split_basis(Y.T, Y.am);
  }
  chol_only(Y);
  b.basis_am = Y.am;
  // B = Q^T X_(T) = R^{-T} P'^T -> H = B B^T (fp64) -> eigenvalues; spectrum = top q + tail entry
  float *amP1 = b.amax + 5 * am;
  fill_f32(amP1, nb, 0.f, st);
  project(Y.T, Y.am, amP1, b.pln);
  const float *Bp = b.Zt;
  {
    // B = R^{-T} P'^T ([ell][M]; R^{-T} is lower triangular), into the free Z^T buffer
    Stage prof("basis_apply", st);
    GemmArgs g = ga();
    g.A = b.RinvT; g.a_ld = ld; g.a_bs = ell * ld; g.a_amax = amR;
    g.B = b.P2; g.b_ld = ld; g.b_bs = Mf * ld; g.b_amax = amP1;
    g.ab_amax_bs = 1;
    g.M = (int)ell; g.N = (int)Mf; g.K = (int)ell;
    g.C = b.Zt; g.c_ld = Mf; g.c_bs = ell * Mf;
    g.m_fastest = 1;
    g.tri = 4;
    gemm(MF_F16, SRC_F32, true, SRC_F32, true, g, nb, 1, st);
  }
  {
    Stage prof("gram64", st);
    gram64(Bp, ell * Mf, (int)Mf, (int)ell, (int)Mf, b.G64, ell * ell, (int)ell, nb, st);
  }
  {
    Stage prof("eigvals_B", st);
    sym_eigvals(b.G64, ell * ell, (int)ell, (int)ell, nb, b.dT, b.eT, b.G64, b.betaT, ell, b.evT, ell, true, st,
                b.mwg);
  }
  // ||X||^2 comes from the feature stage (on the side stream when it runs there)
  if (xready) {
    HIP_TRY(hipStreamWaitEvent(st, xready, 0));
    xready = nullptr;
  }
  flash_spec(b.evT, ell, pl.q, b.norm2, b.specT, pl.nT, nb, st);
  // the fit reads the final basis Y (both layouts) from bufA / bufA2: report it by swapping this
  // view's pointers
  if (Y.T != b.bufA) {
    std::swap(b.bufA, b.bufB);
    std::swap(b.bufA2, b.bufB2);
  }
}

void stage_exact(const Plan &pl, Bufs &b, const void *K, const void *V, hipStream_t st) {
  Stage prof("token_gram_eig", st);
  const int nb = pl.n_cells, nkv = nb / 2;
  const long long T = pl.T, Tld = pl.T_ld, Mf = pl.M;
  int ns = nsplit_for(Mf, tiles_of(T, T), nb, 1024);
  GemmArgs g = ga();
  g.M = (int)T; g.N = (int)T; g.K = (int)Mf;
  g.k_chunk = (int)rup((Mf + ns - 1) / ns, 32);
  ns = (int)((Mf + g.k_chunk - 1) / g.k_chunk);
  g.a_ld = pl.D; g.a_blk = pl.D; g.a_blk_stride = T * pl.D; g.a_bs = pl.cell_elems();
  g.b_ld = pl.D; g.b_blk = pl.D; g.b_blk_stride = T * pl.D; g.b_bs = pl.cell_elems();
  g.c_ld = Tld; g.c_split = T * Tld; g.c_bs = 2LL * ns * T * Tld;
  JOLT_REQUIRE((long long)nb * ns * T * Tld <= b.part_elems, JOLT_EWORKSPACE, "split-K buffer too small");
  for_kv(K, V, [&](int t, const void *X) {
    GemmArgs h = g;
    h.A = X; h.B = X;
    h.C = b.part + (long long)t * ns * T * Tld;
    gemm(pl.xmf(), pl.xsrc(), true, pl.xsrc(), true, h, nkv, ns, st);
  });
  reduce_splits(b.part, (long long)ns * T * Tld, T * Tld, ns, 0, (int)T, (int)T, Tld, b.G64, true, T * T, (int)T, nb,
                st);
  sym_eigvals(b.G64, T * T, (int)T, (int)T, nb, b.dT, b.eT, b.G64, b.betaT, T, b.specT, pl.nT, true, st, b.mwg);
}

// ----------------------------------------------------------------------------- layer grouping
// Per layer, the top kGroupVecs token-mode singular vectors of the key cache, by the FlashJoLT
// pipeline with one layer per cell (oversampling and power iterations enough to converge the leading
// subspace well below the scores' resolution); value cells ride along (the pipeline pairs K and V)
// and are not used.
constexpr int kGroupVecs = 8, kGroupOversample = 24, kGroupPowerIters = 3;

struct LayerSetup {
  std::vector<int32_t> starts;
  int32_t grid[1] = {kGroupVecs};
  double eps2[9] = {1, 1, 1, 1, 1, 1, 1, 1, 1};
  jolt_cache_desc d1;
  jolt_params p1;
};

void layer_setup(const jolt_cache_desc *desc, uint64_t seed, LayerSetup &ls) {
  JOLT_REQUIRE(desc != nullptr && desc->n_layers >= 1, JOLT_EINVAL, "layer grouping: bad cache descriptor");
  ls.d1 = *desc;
  ls.starts.resize(desc->n_layers + 1);
  for (int l = 0; l <= desc->n_layers; ++l) ls.starts[l] = l;
  ls.d1.n_groups = desc->n_layers;
  ls.d1.group_start = ls.starts.data();
  memset(&ls.p1, 0, sizeof(ls.p1));
  ls.p1.mode = JOLT_FLASH;
  ls.p1.oversample = kGroupOversample;
  ls.p1.power_iters = kGroupPowerIters;
  ls.p1.qcap = kGroupVecs;
  ls.p1.rT_grid = ls.grid; ls.p1.n_rT = 1;
  ls.p1.rd_grid = ls.grid; ls.p1.n_rd = 1;
  ls.p1.bits = nullptr; ls.p1.n_bits = 0;
  ls.p1.eps2 = ls.eps2;
  ls.p1.target_ratio = 2.0;
  ls.p1.sketch_seed = seed;
}

// numpy's median: the middle value, or the mean of the two middle values of an even count
double median_of(std::vector<double> v) {
  if (v.empty()) return 0.0;
  std::sort(v.begin(), v.end());
  const size_t n = v.size();
  return (n % 2) ? v[n / 2] : 0.5 * (v[n / 2 - 1] + v[n / 2]);
}

// Sec. 3 "Method": a new group where the score of consecutive layers falls below the median of all
// scores; size bounds first: a group opens only once the current one has two layers, closes at
// eight, and a trailing single layer joins its predecessor
std::vector<int32_t> groups_from_scores(const std::vector<double> &sc, int L) {
  const double med = median_of(sc);
  std::vector<int> sizes{1};
  for (int l = 1; l < L; ++l) {
    if (sizes.back() >= 8 || (sc[l - 1] < med && sizes.back() >= 2)) sizes.push_back(1);
    else ++sizes.back();
  }
  if (sizes.size() > 1 && sizes.back() == 1) {
    sizes.pop_back();
    ++sizes.back();
  }
  std::vector<int32_t> starts{0};
  for (int v : sizes) starts.push_back(starts.back() + v);
  return starts;
}

// ----------------------------------------------------------------------------- allocation
struct AllocDev {
  int *shape, *rT, *rd, *bits;
  long long *offT, *offD;
  double *eps2;
};

// One bisection run over n cells (cell k is cell first + k * step of the tables; its pick lands there).
void run_allocation(int n, int first, int step, int greedy, const AllocDev &ad, int n_rT, int n_rd, int n_bits,
                    int elem_bytes, const double *specT, const double *specD, const double *norm2, double budget,
                    Bufs &b, hipStream_t st) {
  AllocArgs a;
  a.n_cells = n;
  a.shape = ad.shape;
  a.elem_bytes = elem_bytes;
  a.specT = specT; a.specT_off = ad.offT;
  a.specD = specD; a.specD_off = ad.offD;
  a.norm2 = norm2;
  a.rT_grid = ad.rT; a.n_rT = n_rT;
  a.rd_grid = ad.rd; a.n_rd = n_rd;
  a.bits = ad.bits; a.n_bits = n_bits;
  a.eps2 = ad.eps2;
  a.budget = budget;
  a.greedy = greedy;
  a.cell_first = first;
  a.cell_step = step;
  a.tailT = b.tailT; a.tailD = b.tailD; a.e = b.tab_e; a.s = b.tab_s;
  a.out_pick = b.pick; a.out_err = b.perr; a.out = b.aout;
  run_alloc(a, st);
}

// An allocation read back: per cell the full-table index (b-major, then r_T, then r_d) and its
// distortion e, the multiplier(s) and the status.
struct AllocHost {
  std::vector<int> pick;
  std::vector<double> perr;
  double lambda[2] = {0.0, 0.0};  // K/V-decoupled: the keys' and the values' multipliers
  int status = 0;                  // 0 or JOLT_EINFEASIBLE
};

// The allocation variant v (jolt_alloc_variant flags) over the nc cells whose spectra, norms and
// shapes (shape: host copy of the device table) are given, read back to the host.  Joint and greedy:
// one bisection.  K/V-decoupled: one bisection over the even (key) cells and one over the odd (value)
// cells, each under the budget's share of their dense bytes |g| n_h T d_h c.  Uniform ranks: one
// bisection over the bit-widths per (r_T, r_d) grid pair (every cell at that pair); the feasible pair of
// smallest total error wins, ties to fewer bytes, then the earlier pair.
AllocHost allocate_cells(int v, int nc, const AllocDev &ad, const std::vector<int> &shape, int n_rT, int n_rd,
                         int n_bits, int elem_bytes, const double *specT, const double *specD, const double *norm2,
                         double budget, Bufs &b, hipStream_t st) {
  check_variant(v);
  const int greedy = (v & JOLT_ALLOC_GREEDY) ? 1 : 0;
  AllocHost r;
  r.pick.resize(nc);
  r.perr.resize(nc);
  auto read_out = [&](AllocOut &ao) {
    HIP_TRY(hipMemcpyAsync(&ao, b.aout, sizeof(ao), hipMemcpyDeviceToHost, st));
    HIP_TRY(hipStreamSynchronize(st));
    // a lapsed wait in any workgroup (not only the one that writes the status) voids the picks
    JOLT_REQUIRE(ao.status != kAllocEsync && ao.err == 0u, JOLT_EHIP, kAllocEsyncMsg);
  };
  auto read_picks = [&]() {
    HIP_TRY(hipMemcpyAsync(r.pick.data(), b.pick, (size_t)nc * 4, hipMemcpyDeviceToHost, st));
    HIP_TRY(hipMemcpyAsync(r.perr.data(), b.perr, (size_t)nc * 8, hipMemcpyDeviceToHost, st));
    HIP_TRY(hipStreamSynchronize(st));
  };
  if (v & JOLT_ALLOC_UNIFORM_RANKS) {
    bool found = false;
    double bestE = 0.0;
    long long bestS = 0;
    r.status = JOLT_EINFEASIBLE;
    for (int iT = 0; iT < n_rT; ++iT)
      for (int iD = 0; iD < n_rd; ++iD) {
        AllocDev one = ad;
        one.rT += iT;
        one.rd += iD;
        run_allocation(nc, 0, 1, 0, one, 1, 1, n_bits, elem_bytes, specT, specD, norm2, budget, b, st);
        AllocOut ao;
        read_out(ao);
        if (ao.status != 0) continue;
        if (found && !(ao.E < bestE || (ao.E == bestE && ao.S < bestS))) continue;
        found = true;
        bestE = ao.E;
        bestS = ao.S;
        r.lambda[0] = r.lambda[1] = ao.lambda;
        r.status = 0;
        read_picks();
        for (int c = 0; c < nc; ++c) r.pick[c] = (r.pick[c] * n_rT + iT) * n_rd + iD;  // bit index -> table
      }
    return r;
  }
  if (v & JOLT_ALLOC_KV_DECOUPLED) {
    JOLT_REQUIRE(nc >= 2, JOLT_EINVAL, "alloc_variant: K/V-decoupled allocation needs a key and a value cell");
    long long dense[2] = {0, 0};
    for (int c = 0; c < nc; ++c)
      dense[c & 1] += (long long)shape[4 * c] * shape[4 * c + 1] * shape[4 * c + 2] * shape[4 * c + 3] * elem_bytes;
    const double total = (double)(dense[0] + dense[1]);
    for (int kind = 0; kind < 2; ++kind) {
      const int n = (nc - kind + 1) / 2;
      run_allocation(n, kind, 2, greedy, ad, n_rT, n_rd, n_bits, elem_bytes, specT, specD, norm2,
                     budget * ((double)dense[kind] / total), b, st);
      AllocOut ao;
      read_out(ao);
      r.lambda[kind] = ao.lambda;
      if (ao.status != 0) r.status = ao.status;
    }
    read_picks();
    return r;
  }
  run_allocation(nc, 0, 1, greedy, ad, n_rT, n_rd, n_bits, elem_bytes, specT, specD, norm2, budget, b, st);
  AllocOut ao;
  read_out(ao);
  r.lambda[0] = r.lambda[1] = ao.lambda;
  r.status = ao.status;
  read_picks();
  return r;
}

// The multiplier(s) to the caller: one double, two (keys', values') for a K/V-decoupled allocation.
void put_lambda(double *h_lambda, int variant, const AllocHost &r) {
  if (!h_lambda) return;
  h_lambda[0] = r.lambda[0];
  if (variant & JOLT_ALLOC_KV_DECOUPLED) h_lambda[1] = r.lambda[1];
}

struct Section {
  long long off_UT, off_Ud, off_core, off_scales, off_codes, end;
};
Section layout(int G, int H, int T, int D, int c, int rT, int rd, int bits) {
  Section s;
  s.off_UT = 256;
  s.off_Ud = s.off_UT + rup((long long)T * rT * c, 256);
  s.off_core = s.off_Ud + rup((long long)D * rd * c, 256);
  s.off_scales = s.off_core + rup((long long)G * H * rT * rd * c, 256);
  if (bits > 0) {
    s.off_codes = s.off_scales + rup((long long)G * H * T * 4, 256);
    s.end = s.off_codes + rup((long long)G * H * T * D * bits / 8, 256);
  } else {
    s.off_codes = s.end = s.off_scales;
  }
  return s;
}

long long eq1_bytes(int G, int H, int T, int D, int c, int rT, int rd, int b) {
  long long s = ((long long)G * H * rT * rd + (long long)T * rT + (long long)D * rd) * c;
  if (b > 0) s += (long long)G * H * T * (b * D / 8 + 4);
  return s;
}

AllocDev upload_alloc_tables(Upload &u, const Plan &pl, const std::vector<int> &shape, const std::vector<long long> &offT,
                             const std::vector<long long> &offD, std::vector<size_t> &offs) {
  offs.push_back(u.add(shape.data(), shape.size() * 4));
  offs.push_back(u.add(pl.rT.data(), pl.rT.size() * 4));
  offs.push_back(u.add(pl.rd.data(), pl.rd.size() * 4));
  offs.push_back(u.add(pl.bits.data(), pl.bits.size() * 4));
  offs.push_back(u.add(offT.data(), offT.size() * 8));
  offs.push_back(u.add(offD.data(), offD.size() * 8));
  offs.push_back(u.add(pl.eps2, 9 * 8));
  return AllocDev{};
}

AllocDev bind_alloc(char *base, const std::vector<size_t> &o) {
  AllocDev a;
  a.shape = (int *)(base + o[0]);
  a.rT = (int *)(base + o[1]);
  a.rd = (int *)(base + o[2]);
  a.bits = (int *)(base + o[3]);
  a.offT = (long long *)(base + o[4]);
  a.offD = (long long *)(base + o[5]);
  a.eps2 = (double *)(base + o[6]);
  return a;
}

void upload_rotation(const Plan &pl, Bufs &b, Upload &u, std::vector<size_t> &offs) {
  const std::vector<double> &Q = rotation(pl.D, pl.rot_seed);
  std::vector<float> qf(Q.size()), qt(Q.size());
  for (int i = 0; i < pl.D; ++i)
    for (int j = 0; j < pl.D; ++j) {
      qf[(size_t)i * pl.D + j] = (float)Q[(size_t)i * pl.D + j];
      qt[(size_t)j * pl.D + i] = (float)Q[(size_t)i * pl.D + j];
    }
  offs.push_back(u.add(qf.data(), qf.size() * 4));
  offs.push_back(u.add(qt.data(), qt.size() * 4));
}

// ----------------------------------------------------------------------------- fit + residual
struct CellPick {
  int rT, rd, bits;
  long long off;
  Section sec;
};

// Token factor columns 0..kmax-1 of every FlashJoLT cell as rows of length T (U_T^T, [nb][kmax][Tld],
// the first m rows computed) from the eigenvector rows W of B B^T (b.Wrows): U_T = Q W, or
// U_T = Y (R^{-1} W) when the final basis is implicit.  Returns the rows applied to the basis (W, or
// R^{-1} W in b.Wt) and their |max| slot (null: |entries| <= 1), which the token projection reuses.
struct FactorRows {
  const float *rows;
  const float *amax;
};
FactorRows flash_factor_rows(const Plan &pl, Bufs &b, long long kmax, int m, float *UTt, hipStream_t st) {
  const int nb = pl.n_cells;
  const long long ell = pl.ell, ld = pl.ell_ld, Tld = pl.T_ld;
  FactorRows fr{b.Wrows, nullptr};
  if (b.basis_implicit) {
    // W~ rows = W rows R^{-T}: W~[r][k] = sum_j W[r][j] RinvT[j][k] (B contiguous along N)
    float *amW = b.amax + 8 * b.am_ld;
    fill_f32(amW, nb, 0.f, st);
    fill_f32(b.Wt, (long long)nb * kmax * ld, 0.f, st);
    GemmArgs w = ga();
    w.A = b.Wrows; w.a_ld = ld; w.a_bs = kmax * ld; w.a_amax_c = 1.f;
    w.B = b.RinvT; w.b_ld = ld; w.b_bs = ell * ld; w.b_amax = b.amax + b.am_ld;
    w.ab_amax_bs = 1;
    w.M = (int)kmax; w.N = (int)ell; w.K = (int)ell;
    w.C = b.Wt; w.c_ld = ld; w.c_bs = kmax * ld; w.c_amax = amW; w.c_amax_bs = 1; w.m_fastest = 1;
    gemm(MF_F16, SRC_F32, true, SRC_F32, false, w, nb, 1, st);
    fr = FactorRows{b.Wt, amW};
  }
  // U_T^T = rows^T basis^T (rows of length T).  On the fp16 plane path the implicit basis Y is read
  // from its planes (Y^T in b.pln, split with the scale of b.basis_am) and the rows are split into
  // planes with K padded to a whole stage (zero columns; Y^T rows past ell read as its last row).
  if (b.basis_implicit && b.pln && b.apl && fr.amax && pl.xmf() == MF_F16 && pl.fp32_planes() == 2 &&
      pl.T % 32 == 0 && n_views(pl) == 1 && kmax <= ell) {
    const long long Kp = rup(ell, 32);
    split_planes(MF_F16, fr.rows, kmax * ld, ld, m, (int)ell, (int)Kp, b.apl, 2 * kmax * Kp, kmax * Kp, Kp, fr.amax,
                 1, nb, st);
    GemmArgs g = ga();
    g.A = b.apl; g.a_ld = Kp; g.a_ps = kmax * Kp; g.a_bs = 2 * kmax * Kp; g.a_amax = fr.amax;
    g.B = b.pln; g.b_ld = Tld; g.b_ps = ell * Tld; g.b_bs = 2 * ell * Tld; g.b_amax = b.basis_am;
    g.b_krows = (int)ell;
    g.ab_amax_bs = 1;
    g.M = m; g.N = pl.T; g.K = (int)Kp;
    g.C = UTt; g.c_ld = Tld; g.c_bs = kmax * Tld; g.m_fastest = 1;
    if (gemm_dma(MF_F16, 2, 2, g, nb, 1, st, false)) return fr;
  }
  // otherwise from the fp32 basis, [T][ell_ld] in bufA2
  JOLT_REQUIRE(b.rows_layout, JOLT_EINVAL, "token factor: the plane product was refused and no row layout exists");
  GemmArgs g = ga();
  g.A = fr.rows; g.a_ld = ld; g.a_bs = kmax * ld; g.a_amax = fr.amax; g.a_amax_c = 1.f;
  g.B = b.bufA2; g.b_ld = ld; g.b_bs = (long long)pl.T * ld;
  g.b_amax = b.basis_implicit ? b.basis_am : nullptr;  // an orthonormal Q has |entries| <= 1
  g.b_amax_c = 1.f;
  g.ab_amax_bs = 1;
  g.M = m; g.N = pl.T; g.K = (int)ell;
  g.C = UTt; g.c_ld = Tld; g.c_bs = kmax * Tld; g.m_fastest = 1;
  gemm(MF_F16, SRC_F32, true, SRC_F32, true, g, nb, 1, st);
  return fr;
}

void stage_fit(const Plan &pl, Bufs &b, const Sizes &sz, const void *K, const void *V, char *out,
               const std::vector<CellPick> &picks, hipStream_t st) {
  const int nb = pl.n_cells, nkv = nb / 2, D = pl.D, GH = pl.GH;
  const long long Mf = pl.M, Tld = pl.T_ld, kmax = sz.kmax, kmd = sz.kmax_d;
  const long long cellX = pl.cell_elems();
  // ---- per-cell tables
  Upload u;
  std::vector<int> rTv(nb), rdv(nb);
  std::vector<FactorCell> fc(nb);
  for (int c = 0; c < nb; ++c) {
    const CellPick &p = picks[c];
    rTv[c] = p.rT;
    rdv[c] = p.rd;
    FactorCell &f = fc[c];
    f.header = out + p.off;
    f.UT = out + p.off + p.sec.off_UT;
    f.Ud = out + p.off + p.sec.off_Ud;
    f.core = out + p.off + p.sec.off_core;
    f.rT = p.rT; f.rd = p.rd; f.bits = p.bits; f.pad = 0;
    uint32_t h[10] = {0x544C4F4Au, 1u, (uint32_t)pl.G, (uint32_t)pl.H, (uint32_t)pl.T, (uint32_t)D,
                      (uint32_t)p.rT, (uint32_t)p.rd, (uint32_t)p.bits, (uint32_t)pl.dtype};
    memcpy(f.hdr, h, sizeof(h));
    // padding after each part: [start + bytes, next part)
    const long long R = (long long)GH * pl.T;
    const long long part_start[5] = {p.sec.off_UT, p.sec.off_Ud, p.sec.off_core, p.sec.off_scales, p.sec.off_codes};
    const long long part_bytes[5] = {(long long)pl.T * p.rT * pl.c, (long long)D * p.rd * pl.c,
                                     (long long)GH * p.rT * p.rd * pl.c,
                                     p.bits > 0 ? R * 4 : 0, p.bits > 0 ? R * D * p.bits / 8 : 0};
    const long long part_end[5] = {p.sec.off_Ud, p.sec.off_core, p.sec.off_scales,
                                   p.bits > 0 ? p.sec.off_codes : p.sec.off_scales, p.sec.end};
    for (int r = 0; r < 5; ++r) {
      const long long a = part_start[r] + part_bytes[r];
      f.pad_ptr[r] = out + p.off + a;
      f.pad_len[r] = (int)std::max<long long>(0, part_end[r] - a);
    }
  }
  std::vector<size_t> offs;
  size_t o_rT = u.add(rTv.data(), nb * 4), o_rd = u.add(rdv.data(), nb * 4), o_fc = u.add(fc.data(), nb * sizeof(FactorCell));
  std::vector<size_t> rot_offs;
  upload_rotation(pl, b, u, rot_offs);
  upload(b, u, st);
  int *d_rT = (int *)(b.params + o_rT), *d_rd = (int *)(b.params + o_rd);
  FactorCell *d_fc = (FactorCell *)(b.params + o_fc);
  const float *Qf = (const float *)(b.params + rot_offs[0]);
  const float *Qtf = (const float *)(b.params + rot_offs[1]);

  float *amYp = b.amax + 6 * b.am_ld, *amCr = b.amax + 7 * b.am_ld;
  Stage prof_vec("fit_token_factor", st);
  float *UTt = b.bufB;  // [nb][kmax][Tld]
  float *Yp = b.Zt;     // [nb][kmax][Mf]
  fill_f32(amYp, nb, 0.f, st);
  if (pl.mode == JOLT_FLASH) {
    const long long ell = pl.ell, ld = pl.ell_ld;
    fill_f32(b.Wrows, (long long)nb * kmax * ld, 0.f, st);
    sym_eigvecs(b.dT, b.eT, b.G64, b.betaT, ell, b.evT, ell, (int)ell, d_rT, (int)kmax, nb, b.Zw, kmax * ell, b.work,
                (long long)invit_work_doubles((int)ell, (int)kmax), nullptr, b.Wrows, kmax * ld, (int)ld, st);
    const FactorRows fr = flash_factor_rows(pl, b, kmax, (int)kmax, UTt, st);
    // token-projected tensor Y_p = W^T B = rows^T P2^T (kmax x M): P2 holds P = Q^T X, or P' = Y^T X
    // when the basis is implicit (then rows = R^{-1} W)
    GemmArgs h = ga();
    h.A = fr.rows; h.a_ld = ld; h.a_bs = kmax * ld; h.a_amax = fr.amax; h.a_amax_c = 1.f;
    h.B = b.P2; h.b_ld = ld; h.b_bs = Mf * ld; h.b_amax = b.amax + 5 * b.am_ld; h.ab_amax_bs = 1;
    h.M = (int)kmax; h.N = (int)Mf; h.K = (int)ell;
    h.C = Yp; h.c_ld = Mf; h.c_bs = kmax * Mf; h.c_amax = amYp; h.c_amax_bs = 1; h.m_fastest = 1;
    h.C2 = b.YpT; h.c2_ld = kmax; h.c2_bs = Mf * kmax;
    gemm(MF_F16, SRC_F32, true, SRC_F32, true, h, nb, 1, st);
  } else {
    const long long T = pl.T;
    fill_f32(UTt, (long long)nb * kmax * Tld, 0.f, st);
    sym_eigvecs(b.dT, b.eT, b.G64, b.betaT, T, b.specT, pl.nT, (int)T, d_rT, (int)kmax, nb, b.Zw, kmax * T, b.work,
                (long long)invit_work_doubles((int)T, (int)kmax), nullptr, UTt, kmax * Tld, (int)Tld, st);
    // B(k = t, n = (j, d)) = X_j[t][d], the cache as it is (K and V cells in two launches)
    for_kv(K, V, [&](int t, const void *X) {
      GemmArgs g = ga();
      g.A = UTt + t * kmax * Tld; g.a_ld = Tld; g.a_bs = 2 * kmax * Tld; g.a_amax_c = 1.f;
      g.B = X; g.b_ld = D; g.b_blk = D; g.b_blk_stride = T * D; g.b_bs = pl.cell_elems();
      g.M = (int)kmax; g.N = (int)Mf; g.K = (int)T;
      g.C = Yp + t * kmax * Mf; g.c_ld = Mf; g.c_bs = 2 * kmax * Mf;
      g.C2 = b.YpT + t * Mf * kmax; g.c2_ld = kmax; g.c2_bs = 2 * Mf * kmax;
      g.c_amax = amYp + t; g.c_amax_bs = 2; g.m_fastest = 1;
      gemm(pl.xmf(), SRC_F32, true, pl.xsrc(), false, g, nb / 2, 1, st);
    });
  }
  prof_vec.end();
  // ---- projected feature Gram -> U_d
  {
    Stage prof("fit_feature_factor", st);
    const long long Kd = kmax * GH;
    int ns = nsplit_for(Kd, 1, nb, 1024);
    // A(m = d, k = (j, r)) = B(k, n = d) = Y_p^T[(j D + d)][r]
    GemmArgs g = ga();
    g.A = b.YpT; g.B = b.YpT; g.M = D; g.N = D; g.K = (int)Kd;
    g.a_ld = kmax; g.a_blk = (int)kmax; g.a_blk_stride = (long long)D * kmax;
    g.b_ld = kmax; g.b_blk = (int)kmax; g.b_blk_stride = (long long)D * kmax;
    g.a_bs = g.b_bs = Mf * kmax;
    g.a_amax = amYp; g.b_amax = amYp; g.ab_amax_bs = 1;
    g.k_chunk = (int)rup((Kd + ns - 1) / ns, 32);
    ns = (int)((Kd + g.k_chunk - 1) / g.k_chunk);
    JOLT_REQUIRE((long long)nb * ns * D * D <= b.part_elems, JOLT_EWORKSPACE, "split-K buffer too small");
    g.C = b.part; g.c_ld = D; g.c_split = (long long)D * D; g.c_bs = (long long)ns * D * D;
    gemm(MF_F16, SRC_F32, true, SRC_F32, true, g, nb, ns, st);
    reduce_splits(b.part, g.c_bs, g.c_split, ns, 0, D, D, D, b.Gd64, true, (long long)D * D, D, nb, st);
    sym_eigvals(b.Gd64, (long long)D * D, D, D, nb, b.dD, b.eD, b.Gd64, b.betaD, D, b.evD, D, true, st);
    fill_f32(b.Udrows, (long long)nb * kmd * D, 0.f, st);
    sym_eigvecs(b.dD, b.eD, b.Gd64, b.betaD, D, b.evD, D, D, d_rd, (int)kmd, nb, b.ZwD, kmd * D, b.workD,
                (long long)invit_work_doubles(D, (int)kmd), nullptr, b.Udrows, kmd * D, D, st);
  }
  // ---- core: Cp[(r, j)][kk] = Y_p[r][j][:] . U_d[:, kk]
  {
    Stage prof("fit_core", st);
    GemmArgs g = ga();
    g.A = Yp; g.a_ld = D; g.a_bs = kmax * Mf; g.a_amax = amYp; g.ab_amax_bs = 1;
    g.B = b.Udrows; g.b_ld = D; g.b_bs = kmd * D;
    g.M = (int)(kmax * GH); g.N = (int)kmd; g.K = D;
    g.C = b.Cp; g.c_ld = kmd; g.c_bs = kmax * GH * kmd; g.m_fastest = 0;
    gemm(MF_F16, SRC_F32, true, SRC_F32, true, g, nb, 1, st);
  }
  // ---- factors into the blob (rounded) + rounded copies for the residual
  Stage prof_put("put_factors", st);
  fill_f32(b.Udr, (long long)nb * kmd * D, 0.f, st);
  fill_f32(b.Cr, (long long)nb * GH * kmax * kmd, 0.f, st);
  put_ut(pl.dtype, d_fc, nb, UTt, kmax * Tld, (int)Tld, pl.T, (int)kmax, st);
  put_small(pl.dtype, d_fc, nb, b.Udrows, kmd * D, b.Cp, kmax * GH * kmd, (int)kmax, (int)kmd, D, GH, b.Udr, b.Cr, st);
  write_headers(d_fc, nb, st);
  prof_put.end();

  // ---- residual: Bcat = [Q^T | -(D_j Q)^T] per (cell, j), then the fused encode
  bool any = false;
  for (int c = 0; c < nb; ++c) any |= picks[c].bits > 0;
  if (!any) return;
  {
    // Vt[n][kk] = sum_d Q[d][n] Udr[kk][d]
    Stage prof("residual_operand", st);
    GemmArgs g = ga();
    g.A = Qtf; g.a_ld = D; g.a_bs = 0; g.a_amax_c = 1.f;
    g.B = b.Udr; g.b_ld = D; g.b_bs = kmd * D; g.b_amax_c = 1.f;
    g.M = D; g.N = (int)kmd; g.K = D;
    g.C = b.Vt; g.c_ld = kmd; g.c_bs = D * kmd;
    gemm(MF_F16, SRC_F32, true, SRC_F32, true, g, nb, 1, st);
    amax_cells(b.Cr, GH * kmax * kmd, GH * kmax * kmd, nb, amCr, st);
    fill_f32(b.Bcat, (long long)nb * GH * D * sz.Kb, 0.f, st);  // columns past D + r_T stay zero
    bcat_q(b.Bcat, nb, GH, D, sz.Kb, Qtf, st);
    GemmArgs h = ga();
    h.A = b.Vt; h.a_ld = kmd; h.a_bs = D * kmd; h.a_bs2 = 0; h.a_amax_c = 1.f;
    h.B = b.Cr; h.b_ld = kmd; h.b_bs = GH * kmax * kmd; h.b_bs2 = kmax * kmd; h.b_amax = amCr; h.ab_amax_bs = 1;
    h.inner = GH;
    h.M = D; h.N = (int)kmax; h.K = (int)kmd;
    h.C = b.Bcat + D; h.c_ld = sz.Kb; h.c_bs = (long long)GH * D * sz.Kb; h.c_bs2 = (long long)D * sz.Kb;
    h.alpha = -1.f;
    gemm(MF_F16, SRC_F32, true, SRC_F32, true, h, nb * GH, 1, st);
    amax_cells(b.Bcat, (long long)GH * D * sz.Kb, (long long)GH * D * sz.Kb, nb, b.bamax, st);
    const long long per = (long long)GH * D * sz.Kb;
    split_planes(pl.xmf(), b.Bcat, per, sz.Kb, (int)(GH * D), sz.Kb, sz.Kb, b.Bpl, pl.fp32_planes() * per, per,
                 sz.Kb, b.bamax, 1, nb, st);
  }
  std::vector<EncCell> ec;
  for (int c = 0; c < nb; ++c) {
    const CellPick &p = picks[c];
    if (p.bits == 0) continue;
    const int s = c / (2 * pl.n_groups), g = (c / 2) % pl.n_groups, t = c % 2;
    EncCell e;
    e.x_off = ((long long)s * pl.n_groups + g) * cellX * pl.c;
    e.kv = t;
    e.ut_off = p.off + p.sec.off_UT;
    e.sc_off = p.off + p.sec.off_scales;
    e.cd_off = p.off + p.sec.off_codes;
    e.bcat_off = (long long)c * pl.fp32_planes() * GH * D * sz.Kb * 2;
    e.am_idx = c;
    e.GH = GH; e.rT = p.rT; e.bits = p.bits; e.Kb = sz.Kb;
    ec.push_back(e);
  }
  Upload u2;
  size_t o_ec = u2.add(ec.data(), ec.size() * sizeof(EncCell));
  // second upload goes after the first one in the parameter area
  char *dst = b.params + rup((long long)u.host.size(), 256);
  JOLT_REQUIRE(rup((long long)u.host.size(), 256) + (long long)u2.host.size() <= (long long)b.params_bytes,
               JOLT_EWORKSPACE, "parameter area too small");
  HIP_TRY(hipMemcpyAsync(dst, u2.host.data(), u2.host.size(), hipMemcpyHostToDevice, st));
  {
    Stage prof("residual_encode", st);
    EncArgs ea;
    ea.xk = (const char *)K; ea.xv = (const char *)V; ea.utb = out; ea.scb = out; ea.cdb = out;
    ea.bcat = (const char *)b.Bpl; ea.b_ps = (long long)GH * D * sz.Kb;
    ea.bamax = b.bamax; ea.cells = (const EncCell *)(dst + o_ec);
    encode_cells(pl.dtype, ea, (int)ec.size(), pl.T, D, GH, st);
  }
}

// ----------------------------------------------------------------------------- entry helpers
hipStream_t S(void *s) { return (hipStream_t)s; }

template <class F>
int guarded(F f) {
  try {
    g_err.clear();
    return f();
  } catch (const Fail &e) {
    return e.status;
  } catch (const std::exception &e) {
    set_error(std::string("internal error: ") + e.what());
    return JOLT_EINVAL;
  }
}

Sizes sizes_worst(const Plan &pl) { return sizes_for(pl, pl.rT.back(), pl.rd.back()); }

// Side streams (default priority) for the spectra views, created once per device.
hipStream_t side_stream(int i) {
  static std::mutex mu;
  static std::vector<std::vector<hipStream_t>> per_dev;
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lk(mu);
  if ((int)per_dev.size() <= dev) per_dev.resize(dev + 1);
  auto &v = per_dev[dev];
  while ((int)v.size() <= i) {
    hipStream_t s = nullptr;
    HIP_TRY(hipStreamCreateWithFlags(&s, hipStreamNonBlocking));
    v.push_back(s);
  }
  return v[i];
}

// Buffers of cells [c0, c0 + nc) for the spectra stages: every per-cell buffer offset to the first
// cell (same per-cell strides as carve), the split-K scratch slice `slot`, amax slots with the full
// stride.  Only the buffers the spectra stages touch are offset.
Bufs cell_view(const Bufs &b, const Plan &pl, const Sizes &sz, int c0, int slot) {
  Bufs v = b;
  const long long D = pl.D, ell = pl.ell, ld = pl.ell_ld, Tld = pl.T_ld, T = pl.T, M = pl.M;
  const long long n_tok = pl.mode == JOLT_FLASH ? ell : T;
  v.part = b.part + (long long)slot * sz.part_view;
  v.part_elems = sz.part_view;
  {
    Plan pv = pl;
    pv.n_cells = pl.n_cells / n_views(pl);
    v.fpart_elems = feature_part_elems(pv, pv.n_cells);
    v.fpart = b.fpart + (long long)slot * v.fpart_elems;
  }
  v.Gd64 = b.Gd64 + c0 * D * D;
  v.dD = b.dD + c0 * D;
  v.eD = b.eD + c0 * D;
  v.betaD = b.betaD + c0 * D;
  v.evD = b.evD + c0 * D;
  v.specT = b.specT + (long long)c0 * pl.nT;
  v.specD = b.specD + c0 * D;
  v.norm2 = b.norm2 + c0;
  v.amax = b.amax + c0;
  v.G64 = b.G64 + c0 * n_tok * n_tok;
  v.dT = b.dT + c0 * n_tok;
  v.eT = b.eT + c0 * n_tok;
  v.betaT = b.betaT + c0 * n_tok;
  v.evT = b.evT + c0 * n_tok;
  if (pl.mode == JOLT_FLASH) {
    v.bufA = b.bufA + c0 * ell * Tld;
    v.bufB = b.bufB + c0 * ell * Tld;
    v.bufA2 = b.bufA2 ? b.bufA2 + c0 * T * ld : nullptr;
    v.bufB2 = b.bufB2 ? b.bufB2 + c0 * T * ld : nullptr;
    v.Pt = b.Pt + c0 * ell * M;
    v.P2 = b.P2 + c0 * M * ld;
    v.Zt = b.Zt + c0 * ell * M;
    v.Rw = b.Rw + c0 * chol_scratch_doubles((int)ell);
    v.mwg = b.mwg + c0 * (long long)(tridiag_mwg_bytes((int)ell, 1) / sizeof(double));
    v.RinvT = b.RinvT + c0 * ell * ld;
    if (b.pln) v.pln = b.pln + c0 * pl.pln_cell();
    if (b.apl) v.apl = b.apl + c0 * pl.apl_cell();
  } else if (b.mwg) {
    v.mwg = b.mwg + c0 * (long long)(tridiag_mwg_bytes((int)T, 1) / sizeof(double));
  }
  return v;
}

void spectra_all(const Plan &pl, Bufs &b, const Sizes &sz, const void *K, const void *V, hipStream_t st) {
  JOLT_REQUIRE(K && V, JOLT_EINVAL, "null cache pointer");
  const int nv = n_views(pl), nc = pl.n_cells / nv;
  std::vector<hipEvent_t> evs;
  auto new_event = [&]() {
    hipEvent_t e;
    HIP_TRY(hipEventCreateWithFlags(&e, hipEventDisableTiming));
    evs.push_back(e);
    return e;
  };
  // FlashJoLT with one spectra chain: the feature stage (bandwidth-heavy) runs on a side stream
  // beside the first Cholesky QR of the token chain (whose factorisation and triangular-inverse
  // launches leave most of the GPU idle); the token chain waits for it before it forms the spectrum.
  const bool side = pl.mode == JOLT_FLASH && nv == 1;
  hipEvent_t xready = nullptr;
  std::function<hipEvent_t()> side_work;
  if (side) {
    side_work = [&]() -> hipEvent_t {
      hipEvent_t start = new_event();
      HIP_TRY(hipEventRecord(start, st));
      hipStream_t sx = side_stream(0);
      HIP_TRY(hipStreamWaitEvent(sx, start, 0));
      stage_feature(pl, b, K, V, sx);
      xready = new_event();
      HIP_TRY(hipEventRecord(xready, sx));
      return xready;
    };
  }
  if (pl.mode == JOLT_FLASH) {
    gen_omega(b.omegaT, pl.dtype, pl.M, pl.ell, stream_key(pl.sketch_seed, 2), st);
    fill_f32(b.amax, 9LL * b.am_ld, 0.f, st);
  }
  Plan pv = pl;
  pv.n_cells = nc;
  // fork: every view starts after the common prologue; view i > 0 also waits until view i - 1 has
  // formed its first basis
  hipEvent_t fork = new_event();
  HIP_TRY(hipEventRecord(fork, st));
  hipEvent_t prev_mark = nullptr;
  std::vector<hipStream_t> streams(nv);
  bool swapped = false;
  for (int v = 0; v < nv; ++v) {
    hipStream_t sv = v == 0 ? st : side_stream(v - 1);
    streams[v] = sv;
    if (v > 0) HIP_TRY(hipStreamWaitEvent(sv, fork, 0));
    if (prev_mark) HIP_TRY(hipStreamWaitEvent(sv, prev_mark, 0));
    const int c0 = v * nc;
    Bufs bv = cell_view(b, pl, sz, c0, v);
    const long long xoff = (long long)(c0 / 2) * pl.cell_elems() * pl.c;
    const void *Kv = (const char *)K + xoff, *Vv = (const char *)V + xoff;
    if (!side) stage_feature(pv, bv, Kv, Vv, sv);
    hipEvent_t mark = (pl.mode == JOLT_FLASH && v + 1 < nv) ? new_event() : nullptr;
    if (pl.mode == JOLT_FLASH) {
      float *bufA0 = bv.bufA;
      stage_flash(pv, bv, Kv, Vv, sv, mark, side_work);
      swapped = bv.bufA != bufA0;
      if (v == 0) {  // every view takes the same path; the amax slot pointers of view 0 span all cells
        b.basis_implicit = bv.basis_implicit;
        b.basis_am = bv.basis_am;
        b.rows_layout = bv.rows_layout;
      }
    } else {
      stage_exact(pv, bv, Kv, Vv, sv);
    }
    prev_mark = mark;
  }
  // join
  if (xready) HIP_TRY(hipStreamWaitEvent(st, xready, 0));  // (already waited for before the spectrum)
  for (int v = 1; v < nv; ++v) {
    hipEvent_t j = new_event();
    HIP_TRY(hipEventRecord(j, streams[v]));
    HIP_TRY(hipStreamWaitEvent(st, j, 0));
  }
  for (hipEvent_t e : evs) (void)hipEventDestroy(e);  // released once the recorded work completes
  // the fit reads Q (both layouts) from b.bufA / b.bufA2
  if (swapped) {
    std::swap(b.bufA, b.bufB);
    std::swap(b.bufA2, b.bufB2);
  }
}

// Buffers of an allocation alone (jolt_allocate, jolt_allocate_static): the per-cell tables, the
// picks and the parameter area.
Bufs carve_alloc(Arena &ar, const Plan &pl, int n_cells) {
  const long long per = (long long)pl.bits.size() * pl.rT.size() * pl.rd.size();
  Bufs b{};
  b.tailT = ar.take<double>((long long)n_cells * pl.rT.size());
  b.tailD = ar.take<double>((long long)n_cells * pl.rd.size());
  b.tab_e = ar.take<double>(n_cells * per);
  b.tab_s = ar.take<long long>(n_cells * per);
  b.pick = ar.take<int>(n_cells);
  b.perr = ar.take<double>(n_cells);
  b.aout = ar.take<AllocOut>(1);
  b.params_bytes = (size_t)rup(4096 + (long long)n_cells * 40 + (pl.rT.size() + pl.rd.size()) * 4, 256);
  b.params = ar.take<char>((long long)b.params_bytes);
  return b;
}

// Lagrangian allocation on given spectra with the workspace d_ws (ws_bytes; ws_what names it in errors).
int allocate_on(int32_t n_cells, const int32_t *h_cell_shape, int32_t elem_bytes, const double *d_specT,
                const int64_t *h_specT_off, const double *d_specD, const int64_t *h_specD_off, const double *d_norm2,
                const jolt_params *params, double budget_bytes, jolt_pick *h_picks, double *h_lambda, void *d_ws,
                size_t ws_bytes, const char *ws_what, void *stream) {
    JOLT_REQUIRE(n_cells >= 1 && n_cells <= AllocArgs::kMaxCells, JOLT_EINVAL, "n_cells out of range");
    JOLT_REQUIRE(h_cell_shape && d_specT && h_specT_off && d_specD && h_specD_off && d_norm2 && params && h_picks,
                 JOLT_EINVAL, "null argument");
    JOLT_REQUIRE(elem_bytes == 2 || elem_bytes == 4, JOLT_EINVAL, "elem_bytes must be 2 or 4");
    JOLT_REQUIRE(budget_bytes > 0 && isfinite(budget_bytes), JOLT_EINVAL, "budget must be positive");
    check_variant(params->alloc_variant);
    hipStream_t st = S(stream);
    Plan pl;
    check_grid(params->rT_grid, params->n_rT, "rT_grid", pl.rT);
    check_grid(params->rd_grid, params->n_rd, "rd_grid", pl.rd);
    int Dmax = 0;
    for (int c = 0; c < n_cells; ++c) {
      const int32_t *s = h_cell_shape + 4 * c;
      JOLT_REQUIRE(s[0] > 0 && s[1] > 0 && s[2] > 0 && s[3] > 0 && (s[3] * 1) % 8 == 0, JOLT_EINVAL, "bad cell shape");
      JOLT_REQUIRE(h_specT_off[c + 1] > h_specT_off[c] && h_specD_off[c + 1] - h_specD_off[c] == s[3], JOLT_EINVAL,
                   "bad spectrum offsets");
      JOLT_REQUIRE(pl.rT.back() <= h_specT_off[c + 1] - h_specT_off[c], JOLT_EINVAL, "rT_grid exceeds a token spectrum");
      JOLT_REQUIRE(pl.rd.back() <= s[3], JOLT_EINVAL, "rd_grid exceeds d_head");
      Dmax = std::max(Dmax, (int)s[3]);
    }
    fill_bits_eps(params, Dmax, pl);
    pl.n_cells = n_cells;
    // workspace: tables + parameter area (sized first, so that a fixed scratch can refuse cleanly)
    {
      Arena dry;
      carve_alloc(dry, pl, n_cells);
      JOLT_REQUIRE(dry.off <= ws_bytes, JOLT_EWORKSPACE,
                   std::string(ws_what) + " too small: the allocation needs " + std::to_string(dry.off) +
                       " bytes, " + std::to_string(ws_bytes) + " available");
    }
    Arena ar;
    ar.dry = false;
    ar.base = (char *)d_ws;
    ar.cap = ws_bytes;
    JOLT_REQUIRE(d_ws != nullptr, JOLT_EWORKSPACE, "null workspace");
    Bufs b = carve_alloc(ar, pl, n_cells);
    std::vector<int> shape(h_cell_shape, h_cell_shape + 4 * n_cells);
    std::vector<long long> offT(h_specT_off, h_specT_off + n_cells + 1), offD(h_specD_off, h_specD_off + n_cells + 1);
    Upload u;
    std::vector<size_t> o;
    upload_alloc_tables(u, pl, shape, offT, offD, o);
    upload(b, u, st);
    AllocDev ad = bind_alloc(b.params, o);
    AllocHost r = allocate_cells(params->alloc_variant, n_cells, ad, shape, (int)pl.rT.size(), (int)pl.rd.size(),
                                 (int)pl.bits.size(), elem_bytes, d_specT, d_specD, d_norm2, budget_bytes, b, st);
    const std::vector<int> &pick = r.pick;
    const std::vector<double> &perr = r.perr;
    const int nT = (int)pl.rT.size(), nD = (int)pl.rd.size();
    long long off = 0;
    for (int c = 0; c < n_cells; ++c) {
      const int i = pick[c];
      const int bi = i / (nT * nD), ti = (i / nD) % nT, di = i % nD;
      const int32_t *s = h_cell_shape + 4 * c;
      jolt_pick &p = h_picks[c];
      p.rT = pl.rT[ti]; p.rd = pl.rd[di]; p.bits = pl.bits[bi]; p.pad = 0;
      p.bytes = eq1_bytes(s[0], s[1], s[2], s[3], elem_bytes, p.rT, p.rd, p.bits);
      p.err_pred = perr[c];
      Section sec = layout(s[0], s[1], s[2], s[3], elem_bytes, p.rT, p.rd, p.bits);
      p.offset = off;
      p.section_bytes = sec.end;
      off += sec.end;
    }
    put_lambda(h_lambda, params->alloc_variant, r);
    if (r.status != 0) {
      set_error("allocation infeasible: the smallest picks exceed the budget");
      return r.status;
    }
    return 0;
}

// ----------------------------------------------------------------------------- unequal layer groups
// A cache whose layer groups differ in size is compressed partition by partition: the groups of one
// size, staged contiguously, form a cache with equal groups that the batched stages take as it is;
// the allocation runs once over all cells.  Parts are ordered by first appearance of their size.
struct Part {
  int G = 0;
  std::vector<int> groups;      // indices of the original groups, ascending
  std::vector<int32_t> starts;  // 0, G, 2G, ... of the staged cache
  jolt_cache_desc d;
};

std::vector<Part> split_parts(const jolt_cache_desc *d) {
  JOLT_REQUIRE(d && d->n_groups >= 1 && d->group_start && d->n_seq >= 1 && d->n_layers >= 1, JOLT_EINVAL,
               "bad cache descriptor");
  JOLT_REQUIRE(d->group_start[0] == 0 && d->group_start[d->n_groups] == d->n_layers, JOLT_EINVAL,
               "group_start must run from 0 to n_layers");
  std::vector<Part> parts;
  for (int g = 0; g < d->n_groups; ++g) {
    const int G = d->group_start[g + 1] - d->group_start[g];
    JOLT_REQUIRE(G >= 1, JOLT_EINVAL, "group_start must be increasing");
    size_t i = 0;
    while (i < parts.size() && parts[i].G != G) ++i;
    if (i == parts.size()) {
      parts.emplace_back();
      parts.back().G = G;
    }
    parts[i].groups.push_back(g);
  }
  for (Part &p : parts) {
    p.starts.resize(p.groups.size() + 1);
    for (size_t i = 0; i <= p.groups.size(); ++i) p.starts[i] = (int32_t)(i * p.G);
    p.d = *d;
    p.d.n_layers = (int32_t)(p.G * p.groups.size());
    p.d.n_groups = (int32_t)p.groups.size();
    p.d.group_start = p.starts.data();
  }
  return parts;
}

bool equal_groups(const jolt_cache_desc *d) { return split_parts(d).size() == 1; }

// Dense reconstruction of the given cells (all of one group size, as pl describes them)
// The matrix-core type of the residual decode for a cache dtype (fp32 caches decode on bf16 planes).
int dec_mf(int dtype) { return dtype == JOLT_F16 ? MF_F16 : MF_BF16; }

struct RecCell {
  const jolt_pick *p;
  char *out;  // [G][H][T][D] in the cache dtype
};

void reconstruct_cells(const Plan &pl, const std::vector<RecCell> &cells, const char *blob, Arena &ar, hipStream_t st) {
  const int nb = (int)cells.size(), D = pl.D, GH = pl.GH;
  int kmax = 8, kmd = 8;
  for (const RecCell &rc : cells) {
    const jolt_pick &p = *rc.p;
    JOLT_REQUIRE(p.rT >= 8 && p.rT % 8 == 0 && p.rT <= pl.T && p.rd >= 8 && p.rd % 8 == 0 && p.rd <= D &&
                     p.bits >= 0 && p.bits <= 8 && p.offset >= 0 && p.offset % 256 == 0,
                 JOLT_EINVAL, "bad pick");
    kmax = std::max(kmax, p.rT);
    kmd = std::max(kmd, p.rd);
  }
  const int Kd = (int)rup(kmax, 32);  // whole 32-deep stages of D_j's rows (zero past each cell's r_T)
  float *Udr = ar.take<float>((long long)nb * kmd * D);
  float *Cr = ar.take<float>((long long)nb * GH * kmax * kmd);
  float *Dm = ar.take<float>((long long)nb * GH * D * Kd);
  float *am = ar.take<float>(2LL * nb);
  const int dmf = dec_mf(pl.dtype), np = dmf == MF_F16 ? 2 : 3;  // the decode's matrix-core type and planes
  uint16_t *Dpl = ar.take<uint16_t>((long long)np * nb * GH * D * Kd);
  uint16_t *Qpl = ar.take<uint16_t>((long long)np * D * D);
  char *params_area = ar.take<char>(64 * 1024 + (long long)nb * (sizeof(FactorCell) + sizeof(DecCell)) + 2LL * D * D * 4);
  Upload u;
  std::vector<FactorCell> fc(nb);
  std::vector<DecCell> dc(nb);
  std::vector<size_t> rot_offs;
  {
    const std::vector<double> &Q = rotation(D, pl.rot_seed);
    std::vector<float> qf(Q.size());
    for (size_t i = 0; i < Q.size(); ++i) qf[i] = (float)Q[i];
    rot_offs.push_back(u.add(qf.data(), qf.size() * 4));
  }
  for (int c = 0; c < nb; ++c) {
    const jolt_pick &p = *cells[c].p;
    Section sec = layout(pl.G, pl.H, pl.T, D, pl.c, p.rT, p.rd, p.bits);
    FactorCell &f = fc[c];
    memset(&f, 0, sizeof(f));
    f.UT = (void *)(blob + p.offset + sec.off_UT);
    f.Ud = (void *)(blob + p.offset + sec.off_Ud);
    f.core = (void *)(blob + p.offset + sec.off_core);
    f.rT = p.rT; f.rd = p.rd; f.bits = p.bits;
    DecCell &d = dc[c];
    d.UT = f.UT;
    d.Dm = Dm + (long long)c * GH * D * Kd;
    d.Dpl = Dpl + (long long)c * np * GH * D * Kd;
    d.dpl_ps = (long long)GH * D * Kd;
    d.Qpl = Qpl;
    d.qpl_ps = (long long)D * D;
    d.Q = nullptr;  // bound after upload
    d.d_amax = nullptr;
    d.scales = (const float *)(blob + p.offset + sec.off_scales);
    d.codes = (const uint8_t *)(blob + p.offset + sec.off_codes);
    d.out = cells[c].out;
    d.GH = GH; d.rT = p.rT; d.bits = p.bits; d.Kd = Kd;
  }
  size_t o_fc = u.add(fc.data(), nb * sizeof(FactorCell));
  const float *Qdev = (const float *)(params_area + rot_offs[0]);
  for (int c = 0; c < nb; ++c) {
    dc[c].Q = Qdev;
    dc[c].d_amax = am + c;
  }
  size_t o_dc = u.add(dc.data(), nb * sizeof(DecCell));
  HIP_TRY(hipMemcpyAsync(params_area, u.host.data(), u.host.size(), hipMemcpyHostToDevice, st));
  FactorCell *d_fc = (FactorCell *)(params_area + o_fc);
  fill_f32(Udr, (long long)nb * kmd * D, 0.f, st);
  fill_f32(Cr, (long long)nb * GH * kmax * kmd, 0.f, st);
  get_small(pl.dtype, d_fc, nb, kmax, kmd, D, GH, Udr, Cr, st);
  amax_cells(Cr, (long long)GH * kmax * kmd, (long long)GH * kmax * kmd, nb, am + nb, st);
  fill_f32(Dm, (long long)nb * GH * D * Kd, 0.f, st);  // the product writes columns < kmax
  // Dm[cell][j][n][r] = sum_kk Udr[kk][n] Cr[j][r][kk]
  GemmArgs g = ga();
  g.A = Udr; g.a_ld = D; g.a_bs = (long long)kmd * D; g.a_bs2 = 0; g.a_amax_c = 1.f;
  g.B = Cr; g.b_ld = kmd; g.b_bs = (long long)GH * kmax * kmd; g.b_bs2 = (long long)kmax * kmd;
  g.b_amax = am + nb; g.ab_amax_bs = 1;
  g.inner = GH;
  g.M = D; g.N = kmax; g.K = kmd;
  g.C = Dm; g.c_ld = Kd; g.c_bs = (long long)GH * D * Kd; g.c_bs2 = (long long)D * Kd;
  gemm(MF_F16, SRC_F32, false, SRC_F32, true, g, nb * GH, 1, st);
  amax_cells(Dm, (long long)GH * D * Kd, (long long)GH * D * Kd, nb, am, st);
  // the 16-bit planes the tile rebuild reads: D_j after the scale of its cell's |max|, Q after that of 1
  split_planes(dmf, Dm, (long long)GH * D * Kd, Kd, GH * D, Kd, Kd, Dpl, (long long)np * GH * D * Kd,
               (long long)GH * D * Kd, Kd, am, 1, nb, st);
  split_planes(dmf, Qdev, 0, D, D, D, D, Qpl, 0, (long long)D * D, D, nullptr, 0, 1, st);
  Stage prof("residual_decode", st);
  decode_cells(pl.dtype, (const DecCell *)(params_area + o_dc), nb, pl.T, D, GH, st);
}

// Buffers of a compress call over unequal groups: per part the staged K and V and the part's own
// carving; then the spectra of all cells packed in cell order and the allocation's buffers.
struct PartBufs {
  char *K, *V;
  Bufs b;
  Sizes sz;
};
struct PartsLayout {
  std::vector<Plan> pl;
  std::vector<PartBufs> pb;
  double *specT, *specD, *norm2;
  Bufs ab;
  long long nT_total;
};

PartsLayout carve_parts(Arena &ar, const std::vector<Part> &parts, const jolt_params *params) {
  PartsLayout L;
  long long nT_total = 0;
  int nc = 0;
  for (const Part &pt : parts) {
    Plan pl = make_plan(&pt.d, params);
    PartBufs pb;
    const long long bytes = (long long)pl.n_seq * pl.L * pl.H * pl.T * pl.D * pl.c;
    pb.K = ar.take<char>(bytes);
    pb.V = ar.take<char>(bytes);
    pb.sz = sizes_worst(pl);
    pb.b = carve(ar, pl, pb.sz);
    nT_total += (long long)pl.n_cells * pl.nT;
    nc += pl.n_cells;
    L.pl.push_back(pl);
    L.pb.push_back(pb);
  }
  const int D = L.pl[0].D;
  L.specT = ar.take<double>(nT_total);
  L.specD = ar.take<double>((long long)nc * D);
  L.norm2 = ar.take<double>(nc);
  Plan all = L.pl[0];
  all.n_cells = nc;
  L.ab = carve_alloc(ar, all, nc);
  L.nT_total = nT_total;
  return L;
}

int compress_parts(const void *d_K, const void *d_V, const jolt_cache_desc *desc, const jolt_params *params,
                   void *d_out, size_t out_bytes, void *d_ws, size_t ws_bytes, jolt_pick *h_picks, double *h_lambda,
                   hipStream_t st) {
  const std::vector<Part> parts = split_parts(desc);
  Arena ar;
  ar.dry = false;
  ar.base = (char *)d_ws;
  ar.cap = ws_bytes;
  PartsLayout L = carve_parts(ar, parts, params);
  const int n_groups = desc->n_groups, nc = 2 * desc->n_seq * n_groups;
  const Plan &p0 = L.pl[0];
  const int H = p0.H, T = p0.T, D = p0.D, c = p0.c;
  const long long layer = (long long)H * T * D * c;  // bytes of one layer of one sequence
  // global cell c = 2 (s n_groups + g) + t: its part, and its cell index inside the part
  std::vector<int> part_of(nc), local_of(nc);
  std::vector<long long> offT(nc + 1, 0), offD(nc + 1, 0);
  std::vector<int> shape(4 * nc);
  for (size_t q = 0; q < parts.size(); ++q)
    for (int s = 0; s < desc->n_seq; ++s)
      for (size_t gl = 0; gl < parts[q].groups.size(); ++gl)
        for (int t = 0; t < 2; ++t) {
          const int cg = 2 * (s * n_groups + parts[q].groups[gl]) + t;
          part_of[cg] = (int)q;
          local_of[cg] = 2 * (s * (int)parts[q].groups.size() + (int)gl) + t;
        }
  for (int cg = 0; cg < nc; ++cg) {
    const Plan &pl = L.pl[part_of[cg]];
    offT[cg + 1] = offT[cg] + pl.nT;
    offD[cg + 1] = offD[cg] + D;
    shape[4 * cg] = pl.G; shape[4 * cg + 1] = H; shape[4 * cg + 2] = T; shape[4 * cg + 3] = D;
  }
  // stage each part's layers contiguously
  for (size_t q = 0; q < parts.size(); ++q) {
    const Part &pt = parts[q];
    for (int s = 0; s < desc->n_seq; ++s)
      for (size_t gl = 0; gl < pt.groups.size(); ++gl) {
        const long long src = ((long long)s * desc->n_layers + desc->group_start[pt.groups[gl]]) * layer;
        const long long dst = ((long long)s * pt.d.n_layers + (long long)gl * pt.G) * layer;
        HIP_TRY(hipMemcpyAsync(L.pb[q].K + dst, (const char *)d_K + src, pt.G * layer, hipMemcpyDeviceToDevice, st));
        HIP_TRY(hipMemcpyAsync(L.pb[q].V + dst, (const char *)d_V + src, pt.G * layer, hipMemcpyDeviceToDevice, st));
      }
  }
  // spectra per part, packed in cell order
  for (size_t q = 0; q < parts.size(); ++q) {
    spectra_all(L.pl[q], L.pb[q].b, L.pb[q].sz, L.pb[q].K, L.pb[q].V, st);
    const Bufs &b = L.pb[q].b;
    const int nT = L.pl[q].nT;
    for (int cg = 0; cg < nc; ++cg) {
      if (part_of[cg] != (int)q) continue;
      const int cl = local_of[cg];
      HIP_TRY(hipMemcpyAsync(L.specT + offT[cg], b.specT + (long long)cl * nT, nT * 8, hipMemcpyDeviceToDevice, st));
      HIP_TRY(hipMemcpyAsync(L.specD + offD[cg], b.specD + (long long)cl * D, D * 8, hipMemcpyDeviceToDevice, st));
      HIP_TRY(hipMemcpyAsync(L.norm2 + cg, b.norm2 + cl, 8, hipMemcpyDeviceToDevice, st));
    }
  }
  // one allocation over all cells
  Upload u;
  std::vector<size_t> o;
  upload_alloc_tables(u, p0, shape, offT, offD, o);
  upload(L.ab, u, st);
  AllocDev ad = bind_alloc(L.ab.params, o);
  long long dense = 0;
  for (int cg = 0; cg < nc; ++cg) dense += (long long)shape[4 * cg] * H * T * D * c;
  const double budget = (double)dense / p0.C;
  AllocHost r;
  {
    Stage prof("allocate", st);
    r = allocate_cells(params->alloc_variant, nc, ad, shape, (int)p0.rT.size(), (int)p0.rd.size(), (int)p0.bits.size(), c,
                       L.specT, L.specD, L.norm2, budget, L.ab, st);
  }
  const std::vector<int> &pick = r.pick;
  std::vector<double> n2(nc);
  HIP_TRY(hipMemcpyAsync(n2.data(), L.norm2, nc * 8, hipMemcpyDeviceToHost, st));
  HIP_TRY(hipStreamSynchronize(st));
  for (int cg = 0; cg < nc; ++cg) JOLT_REQUIRE(isfinite(n2[cg]), JOLT_ENONFINITE, "non-finite ||X||^2 in a cell");
  for (int cg = 0; cg < nc; ++cg) JOLT_REQUIRE(isfinite(r.perr[cg]), JOLT_ENONFINITE, "non-finite spectrum in a cell");
  put_lambda(h_lambda, params->alloc_variant, r);
  JOLT_REQUIRE(r.status == 0, JOLT_EINFEASIBLE, "allocation infeasible: the smallest picks exceed the budget");
  const int nTg = (int)p0.rT.size(), nDg = (int)p0.rd.size();
  std::vector<CellPick> cp(nc);
  long long off = 0;
  for (int cg = 0; cg < nc; ++cg) {
    const int i = pick[cg], G = shape[4 * cg];
    CellPick &p = cp[cg];
    p.bits = p0.bits[i / (nTg * nDg)];
    p.rT = p0.rT[(i / nDg) % nTg];
    p.rd = p0.rd[i % nDg];
    p.sec = layout(G, H, T, D, c, p.rT, p.rd, p.bits);
    p.off = off;
    off += p.sec.end;
    jolt_pick &h = h_picks[cg];
    h.rT = p.rT; h.rd = p.rd; h.bits = p.bits; h.pad = 0;
    h.bytes = eq1_bytes(G, H, T, D, c, p.rT, p.rd, p.bits);
    h.err_pred = r.perr[cg];
    h.offset = p.off;
    h.section_bytes = p.sec.end;
  }
  JOLT_REQUIRE((size_t)off <= out_bytes, JOLT_EBUFFER, "output buffer too small for the blob");
  // fit and residual per part (blob offsets are the global ones)
  for (size_t q = 0; q < parts.size(); ++q) {
    const Plan &pl = L.pl[q];
    std::vector<CellPick> cpl(pl.n_cells);
    int kmax = 8, kmax_d = 8;
    for (int cg = 0; cg < nc; ++cg) {
      if (part_of[cg] != (int)q) continue;
      cpl[local_of[cg]] = cp[cg];
      kmax = std::max(kmax, cp[cg].rT);
      kmax_d = std::max(kmax_d, cp[cg].rd);
    }
    Sizes fsz = sizes_for(pl, kmax, kmax_d);
    Sizes use = L.pb[q].sz;
    use.kmax = fsz.kmax;
    use.kmax_d = fsz.kmax_d;
    use.Kb = fsz.Kb;
    stage_fit(pl, L.pb[q].b, use, L.pb[q].K, L.pb[q].V, (char *)d_out, cpl, st);
  }
  return 0;
}

}  // namespace
}  // namespace jolt

using namespace jolt;

// Device scratch of jolt_allocate_static, for callers that cannot allocate device memory: the
// allocation's tables, exchange slots and parameter area.  Every device the library runs on holds its
// own copy for the life of the process; its address is looked up once per device (host code never
// passes the array's name itself to a kernel or copy: on the host that name is only a stand-in).
constexpr size_t kStaticScratchBytes = 16u << 20;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {
// Device address of this device's scratch (hipGetSymbolAddress on the first call per device, with that
// device current).
char *static_scratch() {
  static std::mutex mu;
  static std::vector<char *> per_dev;
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lk(mu);
  if ((int)per_dev.size() <= dev) per_dev.resize(dev + 1, nullptr);
  if (per_dev[dev] == nullptr) {
    void *ptr = nullptr;
    HIP_TRY(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
    JOLT_REQUIRE(ptr != nullptr && ((uintptr_t)ptr % 256) == 0, JOLT_EHIP, "static scratch: bad device address");
    per_dev[dev] = (char *)ptr;
  }
  return per_dev[dev];
}
}  // namespace

extern "C" {

const char *jolt_last_error(void) { return get_error(); }

int jolt_profile(int32_t enable) {
  return guarded([&]() {
    g_prof = enable != 0;
    return 0;
  });
}

int32_t jolt_profile_read(char *h_names, int32_t names_bytes, double *h_ms, int32_t *h_count, int32_t max_stages) {
  return guarded([&]() {
    std::vector<std::string> names;
    std::vector<double> ms;
    std::vector<int> cnt;
    for (auto &r : g_recs) {
      HIP_TRY(hipEventSynchronize(r.b));
      float t = 0.f;
      HIP_TRY(hipEventElapsedTime(&t, r.a, r.b));
      size_t i = 0;
      while (i < names.size() && names[i] != r.name) ++i;
      if (i == names.size()) {
        names.push_back(r.name);
        ms.push_back(0.0);
        cnt.push_back(0);
      }
      ms[i] += t;
      cnt[i] += 1;
      (void)hipEventDestroy(r.a);
      (void)hipEventDestroy(r.b);
    }
    g_recs.clear();
    std::string joined;
    int n = 0;
    for (size_t i = 0; i < names.size() && (int)i < max_stages; ++i, ++n) {
      joined += names[i] + "\n";
      h_ms[i] = ms[i];
      h_count[i] = cnt[i];
    }
    JOLT_REQUIRE((int)joined.size() < names_bytes, JOLT_EBUFFER, "profile: name buffer too small");
    memcpy(h_names, joined.c_str(), joined.size() + 1);
    return n;
  });
}

size_t jolt_workspace_bytes(const jolt_cache_desc *desc, const jolt_params *params) {
  size_t out = 0;
  int st = guarded([&]() {
    Arena ar;
    if (equal_groups(desc)) {
      Plan pl = make_plan(desc, params);
      Sizes sz = sizes_worst(pl);
      carve(ar, pl, sz);
    } else {
      carve_parts(ar, split_parts(desc), params);
    }
    out = ar.off + 4096;
    return 0;
  });
  return st == 0 ? out : 0;
}

size_t jolt_output_bytes(const jolt_cache_desc *desc, const jolt_params *params) {
  size_t out = 0;
  int st = guarded([&]() {
    const std::vector<Part> parts = split_parts(desc);
    long long dense = 0, n_cells = 0;
    double C = 0.0;
    for (const Part &pt : parts) {
      Plan pl = make_plan(&pt.d, params);
      dense += (long long)pl.n_cells * pl.cell_elems() * pl.c;
      n_cells += pl.n_cells;
      C = pl.C;
    }
    double B = (double)dense / C;
    // every section: header + up to 5 parts padded to 256 bytes
    out = (size_t)ceil(B) + (size_t)n_cells * (256 + 5 * 256) + 256;
    return 0;
  });
  return st == 0 ? out : 0;
}

int64_t jolt_token_spectrum_len(const jolt_cache_desc *desc, const jolt_params *params) {
  int64_t n = -1;
  int st = guarded([&]() {
    Plan pl = make_plan(desc, params);
    n = pl.nT;
    return 0;
  });
  return st == 0 ? n : st;
}

int jolt_rotation(int32_t d_head, uint64_t seed, double *h_Q) {
  return guarded([&]() {
    JOLT_REQUIRE(d_head >= 1 && d_head <= 1024 && h_Q, JOLT_EINVAL, "bad rotation request");
    const std::vector<double> &Q = rotation(d_head, seed);
    memcpy(h_Q, Q.data(), Q.size() * sizeof(double));
    return 0;
  });
}

int jolt_eps2(int32_t d_head, double *h_eps2) {
  return guarded([&]() {
    JOLT_REQUIRE(d_head >= 8 && d_head <= 1024 && d_head % 8 == 0 && h_eps2, JOLT_EINVAL, "bad eps2 request");
    const std::vector<double> &t = eps2_table(d_head);
    memcpy(h_eps2, t.data(), 9 * sizeof(double));
    return 0;
  });
}

int jolt_test_wait_policy(uint32_t spin_limit, int32_t unreachable) {
  return guarded([&]() {
    g_spin_limit.store(spin_limit == 0 ? (1u << 21) : spin_limit);
    g_target_extra.store(unreachable ? 1u : 0u);
    return 0;
  });
}

int jolt_sketch_matrix(int32_t M, int32_t ell, int32_t dtype, uint64_t sketch_seed, void *d_omegaT, void *stream) {
  return guarded([&]() {
    JOLT_REQUIRE(M >= 1 && ell >= 1 && (long long)M * ell <= (1LL << 31), JOLT_EINVAL, "bad sketch shape");
    JOLT_REQUIRE(dtype == JOLT_F16 || dtype == JOLT_BF16 || dtype == JOLT_F32, JOLT_EINVAL, "bad dtype");
    JOLT_REQUIRE(d_omegaT != nullptr, JOLT_EINVAL, "null output");
    gen_omega(d_omegaT, dtype, M, ell, stream_key(sketch_seed, 2), S(stream));
    return 0;
  });
}

size_t jolt_layer_groups_workspace_bytes(const jolt_cache_desc *desc) {
  size_t out = 0;
  int st = guarded([&]() {
    LayerSetup ls;
    layer_setup(desc, 0, ls);
    Plan pl = make_plan(&ls.d1, &ls.p1);
    Arena ar;
    carve(ar, pl, sizes_for(pl, kGroupVecs, kGroupVecs));
    ar.take<double>((long long)pl.n_seq * std::max(pl.L - 1, 1) * kGroupVecs * kGroupVecs);
    out = ar.off + 4096;
    return 0;
  });
  return st == 0 ? out : 0;
}

int jolt_layer_groups(const void *d_K, const jolt_cache_desc *desc, uint64_t sketch_seed, int32_t *h_group_start,
                      int32_t *h_n_groups, double *h_scores, void *d_ws, size_t ws_bytes, void *stream) {
  return guarded([&]() {
    JOLT_REQUIRE(d_K && h_group_start && h_n_groups, JOLT_EINVAL, "null argument");
    JOLT_REQUIRE(d_ws != nullptr, JOLT_EWORKSPACE, "null workspace");
    LayerSetup ls;
    layer_setup(desc, sketch_seed, ls);
    Plan pl = make_plan(&ls.d1, &ls.p1);
    hipStream_t st = S(stream);
    Arena ar;
    ar.dry = false;
    ar.base = (char *)d_ws;
    ar.cap = ws_bytes;
    const int k = kGroupVecs, L = pl.L, nb = pl.n_cells;
    Sizes sz = sizes_for(pl, k, k);
    Bufs b = carve(ar, pl, sz);
    double *S = ar.take<double>((long long)pl.n_seq * std::max(L - 1, 1) * k * k);
    spectra_all(pl, b, sz, d_K, d_K, st);
    std::vector<int> kv(nb, k);
    Upload u;
    const size_t ok = u.add(kv.data(), nb * 4);
    upload(b, u, st);
    const long long ell = pl.ell, ld = pl.ell_ld;
    fill_f32(b.Wrows, (long long)nb * sz.kmax * ld, 0.f, st);
    sym_eigvecs(b.dT, b.eT, b.G64, b.betaT, ell, b.evT, ell, (int)ell, (const int *)(b.params + ok), sz.kmax, nb, b.Zw,
                (long long)sz.kmax * ell, b.work, (long long)invit_work_doubles((int)ell, sz.kmax), nullptr, b.Wrows,
                (long long)sz.kmax * ld, (int)ld, st);
    flash_factor_rows(pl, b, sz.kmax, k, b.bufB, st);
    std::vector<double> hS((size_t)pl.n_seq * std::max(L - 1, 1) * k * k, 0.0);
    if (L >= 2) {
      pair_cross(b.bufB, (long long)sz.kmax * pl.T_ld, pl.T_ld, pl.T, k, L, pl.n_seq, S, st);
      HIP_TRY(hipMemcpyAsync(hS.data(), S, hS.size() * sizeof(double), hipMemcpyDeviceToHost, st));
    }
    HIP_TRY(hipStreamSynchronize(st));
    std::vector<double> sc(std::max(L - 1, 0), 0.0);
    for (int l = 0; l + 1 < L; ++l) {
      double acc = 0.0;
      for (int q = 0; q < pl.n_seq; ++q) {
        const double *m = hS.data() + ((size_t)q * (L - 1) + l) * k * k;
        double f = 0.0;
        for (int i = 0; i < k * k; ++i) f += m[i] * m[i];
        acc += f / k;
      }
      sc[l] = acc / pl.n_seq;
      JOLT_REQUIRE(isfinite(sc[l]), JOLT_ENONFINITE, "layer grouping: non-finite alignment score");
    }
    const std::vector<int32_t> g = groups_from_scores(sc, L);
    *h_n_groups = (int32_t)g.size() - 1;
    memcpy(h_group_start, g.data(), g.size() * sizeof(int32_t));
    if (h_scores) memcpy(h_scores, sc.data(), sc.size() * sizeof(double));
    return 0;
  });
}

int jolt_spectra(const void *d_K, const void *d_V, const jolt_cache_desc *desc, const jolt_params *params,
                 double *d_specT, double *d_specD, double *d_norm2, float *d_UT, int32_t n_vec, void *d_ws,
                 size_t ws_bytes, void *stream) {
  return guarded([&]() {
    Plan pl = make_plan(desc, params);
    hipStream_t st = S(stream);
    Arena ar;
    ar.dry = false;
    ar.base = (char *)d_ws;
    ar.cap = ws_bytes;
    JOLT_REQUIRE(d_ws != nullptr, JOLT_EWORKSPACE, "null workspace");
    JOLT_REQUIRE(d_UT == nullptr || (n_vec >= 1 && n_vec <= pl.q), JOLT_EINVAL, "n_vec out of range");
    Sizes sz = sizes_worst(pl);
    if (d_UT) sz = sizes_for(pl, std::max(pl.rT.back(), (int)rup(n_vec, 8)), pl.rd.back());
    Bufs b = carve(ar, pl, sz);
    spectra_all(pl, b, sz, d_K, d_V, st);
    const int nb = pl.n_cells;
    HIP_TRY(hipMemcpyAsync(d_specT, b.specT, (size_t)nb * pl.nT * 8, hipMemcpyDeviceToDevice, st));
    HIP_TRY(hipMemcpyAsync(d_specD, b.specD, (size_t)nb * pl.D * 8, hipMemcpyDeviceToDevice, st));
    HIP_TRY(hipMemcpyAsync(d_norm2, b.norm2, (size_t)nb * 8, hipMemcpyDeviceToDevice, st));
    if (d_UT) {
      std::vector<int> kv(nb, n_vec);
      Upload u;
      size_t ok = u.add(kv.data(), nb * 4);
      upload(b, u, st);
      int *dk = (int *)(b.params + ok);
      const long long kmax = sz.kmax, Tld = pl.T_ld;
      if (pl.mode == JOLT_FLASH) {
        const long long ell = pl.ell, ld = pl.ell_ld;
        fill_f32(b.Wrows, (long long)nb * kmax * ld, 0.f, st);
        sym_eigvecs(b.dT, b.eT, b.G64, b.betaT, ell, b.evT, ell, (int)ell, dk, (int)kmax, nb, b.Zw, kmax * ell, b.work,
                    (long long)invit_work_doubles((int)ell, (int)kmax), nullptr, b.Wrows, kmax * ld, (int)ld, st);
        flash_factor_rows(pl, b, kmax, n_vec, b.bufB, st);
      } else {
        sym_eigvecs(b.dT, b.eT, b.G64, b.betaT, pl.T, b.specT, pl.nT, pl.T, dk, (int)kmax, nb, b.Zw, kmax * pl.T,
                    b.work, (long long)invit_work_doubles(pl.T, (int)kmax), nullptr, b.bufB, kmax * Tld, (int)Tld, st);
      }
      for (int c = 0; c < nb; ++c)
        HIP_TRY(hipMemcpy2DAsync(d_UT + (size_t)c * n_vec * pl.T, (size_t)pl.T * 4, b.bufB + (size_t)c * kmax * Tld,
                                 (size_t)Tld * 4, (size_t)pl.T * 4, (size_t)n_vec, hipMemcpyDeviceToDevice, st));
    }
    return 0;
  });
}

int jolt_allocate(int32_t n_cells, const int32_t *h_cell_shape, int32_t elem_bytes, const double *d_specT,
                  const int64_t *h_specT_off, const double *d_specD, const int64_t *h_specD_off,
                  const double *d_norm2, const jolt_params *params, double budget_bytes, jolt_pick *h_picks,
                  double *h_lambda, void *d_ws, size_t ws_bytes, void *stream) {
  return guarded([&]() {
    return allocate_on(n_cells, h_cell_shape, elem_bytes, d_specT, h_specT_off, d_specD, h_specD_off, d_norm2, params,
                       budget_bytes, h_picks, h_lambda, d_ws, ws_bytes, "workspace", stream);
  });
}

int jolt_allocate_static(int32_t n_cells, const int32_t *h_cell_shape, int32_t elem_bytes, const double *d_specT,
                         const int64_t *h_specT_off, const double *d_specD, const int64_t *h_specD_off,
                         const double *d_norm2, const jolt_params *params, double budget_bytes, jolt_pick *h_picks,
                         double *h_lambda, void *stream) {
  return guarded([&]() {
    char *ws = static_scratch();
    return allocate_on(n_cells, h_cell_shape, elem_bytes, d_specT, h_specT_off, d_specD, h_specD_off, d_norm2, params,
                       budget_bytes, h_picks, h_lambda, ws, kStaticScratchBytes, "static scratch (16 MiB)", stream);
  });
}

int jolt_compress(const void *d_K, const void *d_V, const jolt_cache_desc *desc, const jolt_params *params,
                  void *d_out, size_t out_bytes, void *d_ws, size_t ws_bytes, jolt_pick *h_picks, double *h_lambda,
                  void *stream) {
  return guarded([&]() {
    hipStream_t st = S(stream);
    JOLT_REQUIRE(d_out && h_picks, JOLT_EINVAL, "null output");
    JOLT_REQUIRE(d_ws != nullptr, JOLT_EWORKSPACE, "null workspace");
    JOLT_REQUIRE(d_K && d_V, JOLT_EINVAL, "null cache pointer");
    if (!equal_groups(desc))
      return compress_parts(d_K, d_V, desc, params, d_out, out_bytes, d_ws, ws_bytes, h_picks, h_lambda, st);
    Plan pl = make_plan(desc, params);
    Arena ar;
    ar.dry = false;
    ar.base = (char *)d_ws;
    ar.cap = ws_bytes;
    Sizes sz = sizes_worst(pl);
    Bufs b = carve(ar, pl, sz);
    const int nb = pl.n_cells;
    spectra_all(pl, b, sz, d_K, d_V, st);
    // ---- allocation
    std::vector<int> shape(4 * nb);
    std::vector<long long> offT(nb + 1), offD(nb + 1);
    for (int c = 0; c < nb; ++c) {
      shape[4 * c] = pl.G; shape[4 * c + 1] = pl.H; shape[4 * c + 2] = pl.T; shape[4 * c + 3] = pl.D;
      offT[c] = (long long)c * pl.nT;
      offD[c] = (long long)c * pl.D;
    }
    offT[nb] = (long long)nb * pl.nT;
    offD[nb] = (long long)nb * pl.D;
    Upload u;
    std::vector<size_t> o;
    upload_alloc_tables(u, pl, shape, offT, offD, o);
    upload(b, u, st);
    AllocDev ad = bind_alloc(b.params, o);
    const long long dense = (long long)nb * pl.cell_elems() * pl.c;
    const double budget = (double)dense / pl.C;
    AllocHost r;
    {
      Stage prof("allocate", st);
      r = allocate_cells(params->alloc_variant, nb, ad, shape, (int)pl.rT.size(), (int)pl.rd.size(),
                         (int)pl.bits.size(), pl.c, b.specT, b.specD, b.norm2, budget, b, st);
    }
    const std::vector<int> &pick = r.pick;
    std::vector<double> n2(nb);
    HIP_TRY(hipMemcpyAsync(n2.data(), b.norm2, nb * 8, hipMemcpyDeviceToHost, st));
    HIP_TRY(hipStreamSynchronize(st));
    for (int c = 0; c < nb; ++c) JOLT_REQUIRE(isfinite(n2[c]), JOLT_ENONFINITE, "non-finite ||X||^2 in a cell");
    for (int c = 0; c < nb; ++c) JOLT_REQUIRE(isfinite(r.perr[c]), JOLT_ENONFINITE, "non-finite spectrum in a cell");
    put_lambda(h_lambda, params->alloc_variant, r);
    JOLT_REQUIRE(r.status == 0, JOLT_EINFEASIBLE, "allocation infeasible: the smallest picks exceed the budget");
    const int nT = (int)pl.rT.size(), nD = (int)pl.rd.size();
    std::vector<CellPick> cp(nb);
    long long off = 0;
    int kmax = 8, kmax_d = 8;
    for (int c = 0; c < nb; ++c) {
      const int i = pick[c];
      CellPick &p = cp[c];
      p.bits = pl.bits[i / (nT * nD)];
      p.rT = pl.rT[(i / nD) % nT];
      p.rd = pl.rd[i % nD];
      p.sec = layout(pl.G, pl.H, pl.T, pl.D, pl.c, p.rT, p.rd, p.bits);
      p.off = off;
      off += p.sec.end;
      kmax = std::max(kmax, p.rT);
      kmax_d = std::max(kmax_d, p.rd);
      jolt_pick &h = h_picks[c];
      h.rT = p.rT; h.rd = p.rd; h.bits = p.bits; h.pad = 0;
      h.bytes = eq1_bytes(pl.G, pl.H, pl.T, pl.D, pl.c, p.rT, p.rd, p.bits);
      h.err_pred = r.perr[c];
      h.offset = p.off;
      h.section_bytes = p.sec.end;
    }
    JOLT_REQUIRE((size_t)off <= out_bytes, JOLT_EBUFFER, "output buffer too small for the blob");
    Sizes fsz = sizes_for(pl, kmax, kmax_d);
    // the fit reuses the worst-case carving (sizes only shrink)
    Sizes use = sz;
    use.kmax = fsz.kmax;
    use.kmax_d = fsz.kmax_d;
    use.Kb = fsz.Kb;
    stage_fit(pl, b, use, d_K, d_V, (char *)d_out, cp, st);
    return 0;
  });
}

int jolt_reconstruct(const void *d_blob, const jolt_cache_desc *desc, const jolt_params *params,
                     const jolt_pick *h_picks, void *d_K_out, void *d_V_out, void *d_ws, size_t ws_bytes,
                     void *stream) {
  return guarded([&]() {
    JOLT_REQUIRE(d_blob && h_picks && d_K_out && d_V_out && desc, JOLT_EINVAL, "null argument");
    JOLT_REQUIRE(((uintptr_t)d_K_out % 16) == 0 && ((uintptr_t)d_V_out % 16) == 0, JOLT_EINVAL,
                 "reconstruct: outputs must be 16-byte aligned");
    JOLT_REQUIRE(d_ws != nullptr, JOLT_EWORKSPACE, "null workspace");
    hipStream_t st = S(stream);
    const std::vector<Part> parts = split_parts(desc);
    for (const Part &pt : parts) {
      Plan pl = make_plan(&pt.d, params);
      const int c_bytes = pl.c;
      std::vector<RecCell> cells;
      for (int s = 0; s < desc->n_seq; ++s)
        for (int g : pt.groups)
          for (int t = 0; t < 2; ++t) {
            const int c = 2 * (s * desc->n_groups + g) + t;
            char *ob = (char *)(t == 0 ? d_K_out : d_V_out);
            const long long lay = (long long)s * desc->n_layers + desc->group_start[g];
            cells.push_back(RecCell{&h_picks[c], ob + lay * (long long)pl.H * pl.T * pl.D * c_bytes});
          }
      Arena ar;
      ar.dry = false;
      ar.base = (char *)d_ws;
      ar.cap = ws_bytes;
      reconstruct_cells(pl, cells, (const char *)d_blob, ar, st);  // parts run in stream order: scratch reused
    }
    return 0;
  });
}

// ----------------------------------------------------------------------------- fused decode
namespace {
// One decode step of one layer: its group, the two cells' picks and the launch shape of the chunked
// attention (about two blocks per CU over the KV heads, chunks of whole 128-token tiles).
struct AttnPlan {
  int g, lg, Gg, H, T, D, c, dtype, G, n_chunks, chunk, rtv_ld, PS, kmax, kmd, Kd;
  const jolt_pick *pk, *pv;
};

AttnPlan attn_plan(const jolt_cache_desc *d, const jolt_pick *picks, int seq, int layer, int n_q) {
  JOLT_REQUIRE(d && picks && d->group_start, JOLT_EINVAL, "null argument");
  JOLT_REQUIRE(d->n_seq >= 1 && d->n_layers >= 1 && d->n_heads >= 1 && d->n_tokens >= 1 && d->n_groups >= 1,
               JOLT_EINVAL, "cache shape must be positive");
  JOLT_REQUIRE(d->d_head == 64 || d->d_head == 128, JOLT_EINVAL, "d_head must be 64 or 128");
  JOLT_REQUIRE(d->dtype == JOLT_F16 || d->dtype == JOLT_BF16 || d->dtype == JOLT_F32, JOLT_EINVAL, "bad dtype");
  JOLT_REQUIRE(seq >= 0 && seq < d->n_seq && layer >= 0 && layer < d->n_layers, JOLT_EINVAL, "seq or layer out of range");
  JOLT_REQUIRE(d->group_start[0] == 0 && d->group_start[d->n_groups] == d->n_layers, JOLT_EINVAL,
               "group_start must run from 0 to n_layers");
  AttnPlan a;
  a.g = -1;
  for (int g = 0; g < d->n_groups; ++g) {
    JOLT_REQUIRE(d->group_start[g + 1] > d->group_start[g], JOLT_EINVAL, "group_start must be increasing");
    if (layer >= d->group_start[g] && layer < d->group_start[g + 1]) a.g = g;
  }
  a.lg = layer - d->group_start[a.g];
  a.Gg = d->group_start[a.g + 1] - d->group_start[a.g];
  a.H = d->n_heads; a.T = d->n_tokens; a.D = d->d_head; a.dtype = d->dtype; a.c = dtype_bytes(d->dtype);
  JOLT_REQUIRE(n_q >= a.H && n_q % a.H == 0 && n_q / a.H <= kAttnMaxG, JOLT_EINVAL,
               "n_q_heads must be a multiple of n_heads, at most 8 query heads per KV head");
  a.G = n_q / a.H;
  const int cell = 2 * (seq * d->n_groups + a.g);
  a.pk = &picks[cell];
  a.pv = &picks[cell + 1];
  for (const jolt_pick *p : {a.pk, a.pv})
    JOLT_REQUIRE(p->rT >= 8 && p->rT % 8 == 0 && p->rT <= a.T && p->rd >= 8 && p->rd % 8 == 0 && p->rd <= a.D &&
                     p->bits >= 0 && p->bits <= 8 && p->offset >= 0 && p->offset % 256 == 0,
                 JOLT_EINVAL, "bad pick");
  JOLT_REQUIRE(a.pv->rT <= kAttnMaxRank, JOLT_EINVAL, "value token rank above 512");
  const int tiles = (a.T + 127) / 128;
  const int want = std::max(1, std::min(kAttnMaxChunks, 512 / a.H));
  const int per = (tiles + std::min(want, tiles) - 1) / std::min(want, tiles);
  a.chunk = per * 128;
  a.n_chunks = (a.T + a.chunk - 1) / a.chunk;
  a.rtv_ld = (int)rup(a.pv->rT, 4);
  a.PS = 2 + a.rtv_ld + a.D;
  a.kmax = std::max(a.pk->rT, a.pv->rT);
  a.kmd = std::max(a.pk->rd, a.pv->rd);
  a.Kd = (int)rup(a.kmax, 32);  // whole 32-deep stages of D_h's rows (zero past each cell's r_T)
  return a;
}

struct AttnBufs {
  float *Udr, *Cr, *Dm, *am, *part;
  uint16_t *Dpl, *Qpl;
  char *params;
};
AttnBufs carve_attn(Arena &ar, const AttnPlan &a) {
  AttnBufs b;
  b.Udr = ar.take<float>(2LL * a.kmd * a.D);
  b.Cr = ar.take<float>(2LL * a.H * a.kmax * a.kmd);
  b.Dm = ar.take<float>(2LL * a.H * a.D * a.Kd);
  b.Dpl = ar.take<uint16_t>(3LL * 2 * a.H * a.D * a.Kd);
  b.Qpl = ar.take<uint16_t>(3LL * a.D * a.D);
  b.am = ar.take<float>(4);
  b.part = ar.take<float>((long long)a.n_chunks * a.H * a.G * a.PS);
  b.params = ar.take<char>(64 * 1024 + 2LL * a.D * a.D * 4);
  return b;
}
}  // namespace

size_t jolt_decode_attention_workspace_bytes(const jolt_cache_desc *desc, const jolt_pick *h_picks, int32_t seq,
                                             int32_t layer, int32_t n_q_heads) {
  try {
    AttnPlan a = attn_plan(desc, h_picks, seq, layer, n_q_heads);
    Arena dry;
    carve_attn(dry, a);
    return dry.off;
  } catch (...) {
    return 0;
  }
}

int jolt_rope_table(int32_t d_head, double base, int32_t n_pos, float *d_table, void *stream) {
  return guarded([&]() {
    JOLT_REQUIRE(d_table != nullptr, JOLT_EINVAL, "null table");
    JOLT_REQUIRE(d_head >= 2 && d_head <= 128 && d_head % 2 == 0, JOLT_EINVAL, "d_head must be even, at most 128");
    JOLT_REQUIRE(base > 1.0 && isfinite(base) && n_pos >= 0, JOLT_EINVAL, "bad base or position count");
    std::vector<float> inv(d_head / 2);
    for (int i = 0; i < d_head / 2; ++i) inv[i] = (float)std::pow(base, -2.0 * i / d_head);
    rope_table(inv.data(), d_head / 2, n_pos, d_table, S(stream));
    return 0;
  });
}

int jolt_decode_attention(const void *d_blob, const jolt_cache_desc *desc, const jolt_params *params,
                          const jolt_pick *h_picks, int32_t seq, int32_t layer, const float *d_q, int32_t n_q_heads,
                          const void *d_k_tail, const void *d_v_tail, int32_t n_tail, const float *d_rope,
                          int32_t n_rope_pos, float *d_out, void *d_ws, size_t ws_bytes, int32_t reuse_prepared,
                          void *stream) {
  return guarded([&]() {
    JOLT_REQUIRE(d_blob && params && d_q && d_rope && d_out, JOLT_EINVAL, "null argument");
    const AttnPlan a = attn_plan(desc, h_picks, seq, layer, n_q_heads);
    JOLT_REQUIRE(n_tail >= 0 && n_tail <= kAttnMaxTail && (n_tail == 0 || (d_k_tail && d_v_tail)), JOLT_EINVAL,
                 "tail: 0 .. 1024 tokens, both arrays given");
    JOLT_REQUIRE(n_rope_pos >= a.T + n_tail, JOLT_EINVAL, "the RoPE table must cover positions 0 .. T + n_tail - 1");
    JOLT_REQUIRE(d_ws != nullptr, JOLT_EWORKSPACE, "null workspace");
    hipStream_t st = S(stream);
    Arena ar;
    ar.dry = false;
    ar.base = (char *)d_ws;
    ar.cap = ws_bytes;
    AttnBufs b = carve_attn(ar, a);
    const int H = a.H, D = a.D;
    const int dmf = dec_mf(a.dtype), np = dmf == MF_F16 ? 2 : 3;  // the tile rebuild's type and planes
    const char *blob = (const char *)d_blob;
    Upload u;
    FactorCell fc[2];
    DecCell dc[2];
    {
      const std::vector<double> &Q = rotation(D, params->rot_seed);
      std::vector<float> qf(Q.size());
      for (size_t i = 0; i < Q.size(); ++i) qf[i] = (float)Q[i];
      u.add(qf.data(), qf.size() * 4);  // at offset 0
    }
    const float *Qdev = (const float *)b.params;
    for (int t = 0; t < 2; ++t) {
      const jolt_pick &p = t == 0 ? *a.pk : *a.pv;
      const Section sec = layout(a.Gg, H, a.T, D, a.c, p.rT, p.rd, p.bits);
      const char *base = blob + p.offset;
      const long long rows0 = (long long)a.lg * H * a.T;  // first residual row of the layer
      FactorCell &f = fc[t];
      memset(&f, 0, sizeof(f));
      f.UT = (void *)(base + sec.off_UT);
      f.Ud = (void *)(base + sec.off_Ud);
      f.core = (void *)(base + sec.off_core + (long long)a.lg * H * p.rT * p.rd * a.c);
      f.rT = p.rT; f.rd = p.rd; f.bits = p.bits;
      DecCell &d = dc[t];
      d.UT = f.UT;
      d.Dm = b.Dm + (long long)t * H * D * a.Kd;
      d.Dpl = b.Dpl + (long long)t * np * H * D * a.Kd;
      d.dpl_ps = (long long)H * D * a.Kd;
      d.Qpl = b.Qpl;
      d.qpl_ps = (long long)D * D;
      d.Q = Qdev;
      d.d_amax = b.am + t;
      d.scales = (const float *)(base + sec.off_scales) + rows0;
      d.codes = (const uint8_t *)(base + sec.off_codes) + rows0 * (D * p.bits / 8);
      d.out = nullptr;
      d.GH = H; d.rT = p.rT; d.bits = p.bits; d.Kd = a.Kd;
    }
    const size_t o_fc = u.add(fc, sizeof(fc));
    JOLT_REQUIRE(u.host.size() <= (size_t)(64 * 1024 + 2LL * D * D * 4), JOLT_EWORKSPACE, "parameter area too small");
    if (!reuse_prepared) {
      HIP_TRY(hipMemcpyAsync(b.params, u.host.data(), u.host.size(), hipMemcpyHostToDevice, st));
      // D_h = C_h U_d^T of the layer's heads for both cells (Dm[cell][h][n][r]), and their |max|
      fill_f32(b.Udr, 2LL * a.kmd * D, 0.f, st);
      fill_f32(b.Cr, 2LL * H * a.kmax * a.kmd, 0.f, st);
      get_small(a.dtype, (const FactorCell *)(b.params + o_fc), 2, a.kmax, a.kmd, D, H, b.Udr, b.Cr, st);
      amax_cells(b.Cr, (long long)H * a.kmax * a.kmd, (long long)H * a.kmax * a.kmd, 2, b.am + 2, st);
      fill_f32(b.Dm, 2LL * H * D * a.Kd, 0.f, st);  // the product writes columns < kmax
      GemmArgs g = ga();
      g.A = b.Udr; g.a_ld = D; g.a_bs = (long long)a.kmd * D; g.a_bs2 = 0; g.a_amax_c = 1.f;
      g.B = b.Cr; g.b_ld = a.kmd; g.b_bs = (long long)H * a.kmax * a.kmd; g.b_bs2 = (long long)a.kmax * a.kmd;
      g.b_amax = b.am + 2; g.ab_amax_bs = 1;
      g.inner = H;
      g.M = D; g.N = a.kmax; g.K = a.kmd;
      g.C = b.Dm; g.c_ld = a.Kd; g.c_bs = (long long)H * D * a.Kd; g.c_bs2 = (long long)D * a.Kd;
      gemm(MF_F16, SRC_F32, false, SRC_F32, true, g, 2 * H, 1, st);
      amax_cells(b.Dm, (long long)H * D * a.Kd, (long long)H * D * a.Kd, 2, b.am, st);
      split_planes(dmf, b.Dm, (long long)H * D * a.Kd, a.Kd, H * D, a.Kd, a.Kd, b.Dpl, (long long)np * H * D * a.Kd,
                   (long long)H * D * a.Kd, a.Kd, b.am, 1, 2, st);
      split_planes(dmf, Qdev, 0, D, D, D, D, b.Qpl, 0, (long long)D * D, D, nullptr, 0, 1, st);
    }
    AttnArgs at;
    at.k = dc[0];
    at.v = dc[1];
    at.q = d_q;
    at.rope = d_rope;
    at.part = b.part;
    at.T = a.T; at.D = D; at.H = H; at.G = a.G;
    at.chunk = a.chunk; at.n_chunks = a.n_chunks; at.rtv_ld = a.rtv_ld; at.PS = a.PS;
    at.scale = (float)(1.0 / std::sqrt((double)D));
    {
      Stage prof("attend_chunks", st);
      attend_cells(a.dtype, at, st);
    }
    AttnMergeArgs m;
    m.part = b.part;
    m.n_chunks = a.n_chunks; m.H = H; m.G = a.G; m.D = D; m.T = a.T;
    m.rTv = a.pv->rT; m.rtv_ld = a.rtv_ld; m.PS = a.PS; m.bits_v = a.pv->bits; m.Kd = a.Kd;
    m.DmV = b.Dm + (long long)H * D * a.Kd;
    m.Q = Qdev;
    m.k_tail = d_k_tail; m.v_tail = d_v_tail; m.n_tail = n_tail;
    m.q = d_q; m.rope = d_rope;
    m.scale = at.scale;
    m.out = d_out;
    {
      Stage prof("attend_merge", st);
      attend_merge(a.dtype, m, st);
    }
    return 0;
  });
}

size_t jolt_encode_residual_workspace_bytes(int32_t G, int32_t H, int32_t T, int32_t D, int32_t rT, int32_t rd) {
  if (G <= 0 || H <= 0 || T <= 0 || (D != 64 && D != 128) || rT < 8 || rd < 8) return 0;
  const long long GH = (long long)G * H, Kb = rup(D + rT, 32);
  long long bytes = 0;
  auto add = [&](long long n) { bytes += rup(std::max<long long>(n, 1), 256); };
  add(rd * D * 4LL); add(GH * rT * rd * 4LL); add(D * rd * 4LL); add(GH * D * Kb * 4LL); add(3 * GH * D * Kb * 2LL);
  add(16);
  add(64 * 1024 + 2LL * D * D * 4);
  return (size_t)bytes + 4096;
}

int jolt_encode_residual(const void *d_X, int32_t G, int32_t H, int32_t T, int32_t D, int32_t dtype, const void *d_UT,
                         const void *d_core, const void *d_Ud, int32_t rT, int32_t rd, int32_t bits, uint64_t rot_seed,
                         float *d_scales, uint8_t *d_codes, void *d_ws, size_t ws_bytes, void *stream) {
  return guarded([&]() {
    JOLT_REQUIRE(d_X && d_UT && d_core && d_Ud && d_scales && d_codes, JOLT_EINVAL, "null argument");
    JOLT_REQUIRE(G > 0 && H > 0 && T > 0 && (D == 64 || D == 128), JOLT_EINVAL, "bad shape");
    JOLT_REQUIRE(dtype == JOLT_F16 || dtype == JOLT_BF16 || dtype == JOLT_F32, JOLT_EINVAL, "bad dtype");
    JOLT_REQUIRE(rT >= 8 && rT % 8 == 0 && rT <= T && rd >= 8 && rd % 8 == 0 && rd <= D, JOLT_EINVAL, "bad ranks");
    JOLT_REQUIRE(bits >= 1 && bits <= 8, JOLT_EINVAL, "bits must lie in 1..8");
    JOLT_REQUIRE(((uintptr_t)d_X % 16) == 0 && ((uintptr_t)d_UT % 16) == 0 && ((uintptr_t)d_scales % 4) == 0 &&
                     ((uintptr_t)d_codes % 4) == 0,
                 JOLT_EINVAL, "X and U_T must be 16-byte aligned, scales and codes 4-byte aligned");
    JOLT_REQUIRE(d_ws != nullptr && ws_bytes >= jolt_encode_residual_workspace_bytes(G, H, T, D, rT, rd),
                 JOLT_EWORKSPACE, "workspace too small");
    hipStream_t st = S(stream);
    const int GH = G * H, Kb = (int)rup(D + rT, 32);
    Arena ar;
    ar.dry = false;
    ar.base = (char *)d_ws;
    ar.cap = ws_bytes;
    float *Udr = ar.take<float>((long long)rd * D);
    float *Cr = ar.take<float>((long long)GH * rT * rd);
    float *Vt = ar.take<float>((long long)D * rd);
    float *Bcat = ar.take<float>((long long)GH * D * Kb);
    const int P = dtype == JOLT_F16 ? 2 : 3;  // 16-bit planes of Bcat
    uint16_t *Bpl = ar.take<uint16_t>((long long)P * GH * D * Kb);
    float *am = ar.take<float>(4);
    char *pa = ar.take<char>(64 * 1024 + 2LL * D * D * 4);
    Upload u;
    FactorCell f;
    memset(&f, 0, sizeof(f));
    f.UT = (void *)d_UT; f.Ud = (void *)d_Ud; f.core = (void *)d_core; f.rT = rT; f.rd = rd; f.bits = bits;
    size_t o_fc = u.add(&f, sizeof(f));
    const std::vector<double> &Q = rotation(D, rot_seed);
    std::vector<float> qt(Q.size());
    for (int i = 0; i < D; ++i)
      for (int j = 0; j < D; ++j) qt[(size_t)j * D + i] = (float)Q[(size_t)i * D + j];
    size_t o_qt = u.add(qt.data(), qt.size() * 4);
    EncCell e;
    memset(&e, 0, sizeof(e));
    e.GH = GH; e.rT = rT; e.bits = bits; e.Kb = Kb;
    size_t o_ec = u.add(&e, sizeof(e));
    HIP_TRY(hipMemcpyAsync(pa, u.host.data(), u.host.size(), hipMemcpyHostToDevice, st));
    const float *Qtf = (const float *)(pa + o_qt);
    get_small(dtype, (const FactorCell *)(pa + o_fc), 1, rT, rd, D, GH, Udr, Cr, st);
    GemmArgs g = ga();
    g.A = Qtf; g.a_ld = D; g.a_amax_c = 1.f;
    g.B = Udr; g.b_ld = D; g.b_amax_c = 1.f;
    g.M = D; g.N = rd; g.K = D;
    g.C = Vt; g.c_ld = rd;
    gemm(MF_F16, SRC_F32, true, SRC_F32, true, g, 1, 1, st);
    amax_cells(Cr, (long long)GH * rT * rd, 0, 1, am + 1, st);
    fill_f32(Bcat, (long long)GH * D * Kb, 0.f, st);  // columns past D + r_T stay zero
    bcat_q(Bcat, 1, GH, D, Kb, Qtf, st);
    GemmArgs h = ga();
    h.A = Vt; h.a_ld = rd; h.a_amax_c = 1.f;
    h.B = Cr; h.b_ld = rd; h.b_bs2 = (long long)rT * rd; h.b_amax = am + 1; h.ab_amax_bs = 1;
    h.inner = GH;
    h.M = D; h.N = rT; h.K = rd;
    h.C = Bcat + D; h.c_ld = Kb; h.c_bs2 = (long long)D * Kb;
    h.alpha = -1.f;
    gemm(MF_F16, SRC_F32, true, SRC_F32, true, h, GH, 1, st);
    amax_cells(Bcat, (long long)GH * D * Kb, 0, 1, am, st);
    split_planes(dtype == JOLT_F16 ? MF_F16 : MF_BF16, Bcat, 0, Kb, GH * D, Kb, Kb, Bpl, 0, (long long)GH * D * Kb,
                 Kb, am, 0, 1, st);
    EncArgs ea;
    ea.xk = ea.xv = (const char *)d_X; ea.utb = (const char *)d_UT; ea.scb = (char *)d_scales;
    ea.cdb = (char *)d_codes; ea.bcat = (const char *)Bpl; ea.b_ps = (long long)GH * D * Kb;
    ea.bamax = am; ea.cells = (const EncCell *)(pa + o_ec);
    encode_cells(dtype, ea, 1, T, D, GH, st);
    return 0;
  });
}

}  // extern "C"
