// Joint Lagrangian rank/bit allocation (Sec. 3, Eqs. (1)-(4), "Solving the allocation").
//
// One workgroup: (1) suffix sums of every cell's token and feature spectra (sequential from
// the last entry, fp64), (2) the distortion/byte table over the (b, r_T, r_d) grid of every cell,
// e = eps^2(b) * ((tailT[r_T] + tailD[r_d]) / ||X||^2) and s = Eq. (1) bytes (exact integers),
// (3) geometric bisection on lambda with an exact per-cell argmin of e + lambda s (ties: smaller
// s, then b, r_T, r_d).  Every floating-point operation is explicitly rounded (no contraction) so
// the result is reproducible and independent of the launch shape.
#include <math.h>

#include "common.hpp"
#include "alloc.hpp"

namespace jolt {

namespace {

constexpr int AT = 1024;

// The grids are strictly ascending (bits, r_T and r_d are validated so on entry), so the
// tie-break order (b, r_T, r_d) is the order of the table index (b slowest, r_d fastest).
struct Best {
  double cost;
  long long s;
  int idx;
};

// index, in the caller's arrays, of cell k of this run
__device__ __forceinline__ int gcell(const AllocArgs &a, int k) { return a.cell_first + k * a.cell_step; }

__device__ __forceinline__ bool less_than(const Best &x, const Best &y) {
  if (x.cost != y.cost) return x.cost < y.cost;
  if (x.s != y.s) return x.s < y.s;
  return x.idx < y.idx;
}

__device__ Best shfl_best(const Best &v, int o) {
  Best r;
  r.cost = __shfl_xor(v.cost, o, 64);
  r.s = __shfl_xor(v.s, o, 64);
  r.idx = __shfl_xor(v.idx, o, 64);
  return r;
}

// The greedy per-cell search for bit-width index bi (Sec. 3, "Solving the allocation"): from the
// smallest grid ranks, step the mode whose next grid step removes the most error per added byte while
// that step lowers e + lambda s, until neither can; equal rates step the token mode.  Same fp64
// operations and roundings as the exact search.
__device__ Best greedy_walk(const double *ec, const long long *sc, int bi, int nT, int nD, double lam) {
  int iT = 0, iD = 0;
  for (int step = 0; step < nT + nD; ++step) {
    const int here = (bi * nT + iT) * nD + iD;
    const double eh = ec[here], sh = (double)sc[here];
    bool okT = false, okD = false;
    double rt = 0.0, rd = 0.0;
    if (iT + 1 < nT) {
      const int nx = here + nD;
      const double de = __dsub_rn(eh, ec[nx]), ds = __dsub_rn((double)sc[nx], sh);
      if (de > __dmul_rn(lam, ds)) {
        okT = true;
        rt = __ddiv_rn(de, ds);
      }
    }
    if (iD + 1 < nD) {
      const int nx = here + 1;
      const double de = __dsub_rn(eh, ec[nx]), ds = __dsub_rn((double)sc[nx], sh);
      if (de > __dmul_rn(lam, ds)) {
        okD = true;
        rd = __ddiv_rn(de, ds);
      }
    }
    if (!okT && !okD) break;
    if (okT && (!okD || rt >= rd)) ++iT;
    else ++iD;
  }
  const int i = (bi * nT + iT) * nD + iD;
  Best b;
  b.cost = __dadd_rn(ec[i], __dmul_rn(lam, (double)sc[i]));
  b.s = sc[i];
  b.idx = i;
  return b;
}

__global__ void __launch_bounds__(AT) alloc_kernel(AllocArgs a) {
  __shared__ int pick[AllocArgs::kMaxCells];
  __shared__ long long pick_s[AllocArgs::kMaxCells];  // bytes and distortion of each cell's pick
  __shared__ double pick_e[AllocArgs::kMaxCells];
  __shared__ double lam_s;
  __shared__ int done_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = AT / 64;
  const int nc = a.n_cells, nb = a.n_bits, nT = a.n_rT, nD = a.n_rd;
  const int per = nb * nT * nD;

  // (1) suffix sums at the grid ranks (one thread per cell and mode; sequential order)
  for (int w = tid; w < 2 * nc; w += AT) {
    const int c = w >> 1, mode = w & 1, g = gcell(a, c);
    const double *sp = mode == 0 ? a.specT + a.specT_off[g] : a.specD + a.specD_off[g];
    const int len = mode == 0 ? (int)(a.specT_off[g + 1] - a.specT_off[g]) : (int)(a.specD_off[g + 1] - a.specD_off[g]);
    const int *grid = mode == 0 ? a.rT_grid : a.rd_grid;
    const int ng = mode == 0 ? nT : nD;
    double *outp = mode == 0 ? a.tailT + (long long)c * nT : a.tailD + (long long)c * nD;
    double acc = 0.0;
    int gi = ng - 1;
    // ranks beyond the spectrum length discard nothing
    while (gi >= 0 && grid[gi] >= len) outp[gi--] = 0.0;
    int gv = gi >= 0 ? grid[gi] : -1;  // the next grid rank to emit
    // the spectrum is read 8 entries at a time (independent loads in flight), summed one by one
    for (int i0 = len - 1; i0 >= 0 && gi >= 0; i0 -= 8) {
      double x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = (i0 - u >= 0) ? sp[i0 - u] : 0.0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 - u;
        if (i >= 0 && gi >= 0) {
          acc = __dadd_rn(acc, x[u]);
          while (gi >= 0 && gv == i) {
            outp[gi--] = acc;
            gv = gi >= 0 ? grid[gi] : -1;
          }
        }
      }
    }
    while (gi >= 0) outp[gi--] = acc;
  }
  __syncthreads();
  // (2) table, cell by cell (per-cell values hoisted; 32-bit index arithmetic within a cell)
  for (int c = 0; c < nc; ++c) {
    const int g = gcell(a, c);
    const double n2 = a.norm2[g];
    const long long G = a.shape[4 * g], H = a.shape[4 * g + 1], T = a.shape[4 * g + 2], D = a.shape[4 * g + 3];
    const double *tT = a.tailT + (long long)c * nT, *tD = a.tailD + (long long)c * nD;
    double *ec = a.e + (long long)c * per;
    long long *sc = a.s + (long long)c * per;
    for (int rem = tid; rem < per; rem += AT) {
      const int bi = rem / (nT * nD), ti = (rem / nD) % nT, di = rem % nD;
      const double tsum = __dadd_rn(tT[ti], tD[di]);
      const double tau = (n2 > 0.0) ? __ddiv_rn(tsum, n2) : 0.0;
      ec[rem] = __dmul_rn(a.eps2[a.bits[bi]], tau);
      const long long rT = a.rT_grid[ti], rd = a.rd_grid[di], b = a.bits[bi];
      long long s = (G * H * rT * rd + T * rT + D * rd) * a.elem_bytes;
      if (b > 0) s += G * H * T * (b * D / 8 + 4);
      sc[rem] = s;
    }
  }
  __syncthreads();

  // (3) evaluation of the per-cell minimisers at lambda: one wave per cell; a lane visits its
  // candidates in ascending index order (so an equal cost and size never replaces its best) and
  // reads them in batches of 16 so that their loads are in flight together
  constexpr int EB = 16;
  auto evaluate = [&](double lam) {
    for (int c = wave; c < nc; c += nw) {
      Best best;
      best.cost = INFINITY;
      best.s = LLONG_MAX;
      best.idx = 0;  // any finite candidate replaces it; keeps the index valid for non-finite tables
      const double *ec = a.e + (long long)c * per;
      const long long *sc = a.s + (long long)c * per;
      if (a.greedy) {  // lane b walks bit-width b
        if (lane < nb) best = greedy_walk(ec, sc, lane, nT, nD, lam);
      } else
      for (int i0 = lane; i0 < per; i0 += 64 * EB) {
        double ev[EB];
        long long sv[EB];
#pragma unroll
        for (int u = 0; u < EB; ++u) {
          const int i = min(i0 + 64 * u, per - 1);
          ev[u] = ec[i];
          sv[u] = sc[i];
        }
#pragma unroll
        for (int u = 0; u < EB; ++u) {
          const int i = i0 + 64 * u;
          const double cost = __dadd_rn(ev[u], __dmul_rn(lam, (double)sv[u]));
          if (i < per && (cost < best.cost || (cost == best.cost && sv[u] < best.s))) {
            best.cost = cost;
            best.s = sv[u];
            best.idx = i;
          }
        }
      }
      for (int o = 32; o > 0; o >>= 1) {
        Best oth = shfl_best(best, o);
        if (less_than(oth, best)) best = oth;
      }
      if (lane == 0) {
        pick[c] = best.idx;
        pick_s[c] = sc[best.idx];
        pick_e[c] = ec[best.idx];
      }
    }
    __syncthreads();
  };
  // totals of the current picks, summed over the cells in order (read from LDS: one global
  // round trip per cell in this sequential loop would dominate the bisection)
  auto totals = [&](long long &S, double &E) {
    S = 0;
    E = 0.0;
    for (int c = 0; c < nc; ++c) {
      S += pick_s[c];
      E = __dadd_rn(E, pick_e[c]);
    }
  };
  auto store = [&](int status, double lam, int iters) {
    if (tid == 0) {
      long long S;
      double E;
      totals(S, E);
      a.out->status = status;
      a.out->lambda = lam;
      a.out->S = S;
      a.out->E = E;
      a.out->iters = iters;
    }
    for (int c = tid; c < nc; c += AT) {
      a.out_pick[gcell(a, c)] = pick[c];
      if (a.out_err) a.out_err[gcell(a, c)] = pick_e[c];
    }
    __syncthreads();
  };

  const double B = a.budget;
  double lo = 1e-30, hi = 1e10;
  evaluate(lo);
  long long S;
  double E;
  if (tid == 0) {
    totals(S, E);
    done_s = ((double)S <= B) ? 1 : 0;
  }
  __syncthreads();
  if (done_s) {
    store(0, lo, 0);
    return;
  }
  evaluate(hi);
  if (tid == 0) {
    totals(S, E);
    done_s = ((double)S > B) ? 1 : 0;
  }
  __syncthreads();
  if (done_s) {
    store(JOLT_EINFEASIBLE, hi, 0);
    return;
  }
  // keep the feasible end's picks in out_pick while bisecting
  for (int c = tid; c < nc; c += AT) a.out_pick[gcell(a, c)] = pick[c];
  __syncthreads();
  double hi_lam = hi;
  for (int it = 0; it < 50; ++it) {
    const double mid = __dsqrt_rn(__dmul_rn(lo, hi));
    evaluate(mid);
    if (tid == 0) {
      totals(S, E);
      const double Sd = (double)S;
      if (__dmul_rn(0.995, B) <= Sd && Sd <= B) done_s = 2;
      else if (Sd > B) { done_s = 0; lam_s = mid; }
      else { done_s = 1; lam_s = mid; }
    }
    __syncthreads();
    if (done_s == 2) {
      store(0, mid, it + 1);
      return;
    }
    if (done_s == 0) lo = lam_s;
    else {
      hi = lam_s;
      hi_lam = hi;
      for (int c = tid; c < nc; c += AT) a.out_pick[gcell(a, c)] = pick[c];
    }
    __syncthreads();
  }
  // no accept: the feasible end
  for (int c = tid; c < nc; c += AT) {
    const int i = a.out_pick[gcell(a, c)];
    pick[c] = i;
    pick_s[c] = a.s[(long long)c * per + i];
    pick_e[c] = a.e[(long long)c * per + i];
  }
  __syncthreads();
  store(0, hi_lam, 50);
}

// The same allocation with one workgroup per cell: the cell's suffix sums, table and argmin at
// each lambda are its workgroup's; after each evaluation every workgroup publishes its pick (index,
// bytes, distortion) with agent-coherent stores, bumps a step counter once they have completed,
// waits for all cells (bounded), reads every cell's pick and forms the totals in cell order, so all
// workgroups take the same bisection decisions and the result equals the one-workgroup kernel's.
// Exchange slots: two per cell (alternating by step), three 8-byte words each, in the cell's own
// token tail-sum area (free once its table is built).
__device__ __forceinline__ void x64store(void *p, unsigned long long v) {
  __hip_atomic_store((unsigned long long *)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long x64load(const void *p) {
  return __hip_atomic_load((unsigned long long *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void __launch_bounds__(AT) alloc_mwg_kernel(AllocArgs a, unsigned spin_limit, unsigned target_extra) {
  constexpr int kSpec = 4096;  // spectrum entries staged in LDS for the sequential suffix sums
  __shared__ double wcost[AT / 64];
  __shared__ long long ws[AT / 64];
  __shared__ int widx[AT / 64];
  __shared__ long long cs[AllocArgs::kMaxCells / 16];  // every cell's pick bytes at this step
  __shared__ double ce[AllocArgs::kMaxCells / 16];     // and distortion
  __shared__ double spec_l[kSpec];
  __shared__ int own_pick, fail_s;
  const int c = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = AT / 64;
  const int nc = a.n_cells, nb = a.n_bits, nT = a.n_rT, nD = a.n_rd;
  const int per = nb * nT * nD;
  unsigned *cnt = &a.out->sync;
  double *ec = a.e + (long long)c * per;
  long long *sc = a.s + (long long)c * per;

  // (1) suffix sums of this cell (thread 0: token mode, thread 1: feature mode; sequential order),
  // from LDS copies of the two spectra when they fit
  const int g = gcell(a, c);
  const int lenT = (int)(a.specT_off[g + 1] - a.specT_off[g]), lenD = (int)(a.specD_off[g + 1] - a.specD_off[g]);
  const bool staged = lenT + lenD <= kSpec;
  if (staged) {
    for (int i = tid; i < lenT; i += AT) spec_l[i] = a.specT[a.specT_off[g] + i];
    for (int i = tid; i < lenD; i += AT) spec_l[lenT + i] = a.specD[a.specD_off[g] + i];
  }
  __syncthreads();
  if (tid < 2) {
    const int mode = tid;
    const double *sp = staged ? (mode == 0 ? spec_l : spec_l + lenT)
                              : (mode == 0 ? a.specT + a.specT_off[g] : a.specD + a.specD_off[g]);
    const int len = mode == 0 ? lenT : lenD;
    const int *grid = mode == 0 ? a.rT_grid : a.rd_grid;
    const int ng = mode == 0 ? nT : nD;
    double *outp = mode == 0 ? a.tailT + (long long)c * nT : a.tailD + (long long)c * nD;
    double acc = 0.0;
    int gi = ng - 1;
    while (gi >= 0 && grid[gi] >= len) outp[gi--] = 0.0;
    int gv = gi >= 0 ? grid[gi] : -1;
    for (int i0 = len - 1; i0 >= 0 && gi >= 0; i0 -= 8) {
      double x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = (i0 - u >= 0) ? sp[i0 - u] : 0.0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 - u;
        if (i >= 0 && gi >= 0) {
          acc = __dadd_rn(acc, x[u]);
          while (gi >= 0 && gv == i) {
            outp[gi--] = acc;
            gv = gi >= 0 ? grid[gi] : -1;
          }
        }
      }
    }
    while (gi >= 0) outp[gi--] = acc;
  }
  if (tid == 0) fail_s = 0;
  __syncthreads();
  // (2) this cell's table
  {
    const double n2 = a.norm2[g];
    const long long G = a.shape[4 * g], H = a.shape[4 * g + 1], T = a.shape[4 * g + 2], D = a.shape[4 * g + 3];
    const double *tT = a.tailT + (long long)c * nT, *tD = a.tailD + (long long)c * nD;
    for (int rem = tid; rem < per; rem += AT) {
      const int bi = rem / (nT * nD), ti = (rem / nD) % nT, di = rem % nD;
      const double tsum = __dadd_rn(tT[ti], tD[di]);
      const double tau = (n2 > 0.0) ? __ddiv_rn(tsum, n2) : 0.0;
      ec[rem] = __dmul_rn(a.eps2[a.bits[bi]], tau);
      const long long rT = a.rT_grid[ti], rd = a.rd_grid[di], b = a.bits[bi];
      long long s = (G * H * rT * rd + T * rT + D * rd) * a.elem_bytes;
      if (b > 0) s += G * H * T * (b * D / 8 + 4);
      sc[rem] = s;
    }
  }
  __syncthreads();  // the tail sums of this cell are not read again: its exchange slots go there
  unsigned long long *xslot = (unsigned long long *)(a.tailT + (long long)c * nT);

  // argmin of this cell at lambda (thread order ascending in i, then the block in wave order; the
  // same total order (cost, bytes, index) as the one-workgroup kernel), published, then the totals
  int step = 0;
  long long S = 0;
  double E = 0.0;
  auto evaluate = [&](double lam) {
    Best best;
    best.cost = INFINITY;
    best.s = LLONG_MAX;
    best.idx = 0;
    if (a.greedy) {  // thread b walks bit-width b
      if (tid < nb) best = greedy_walk(ec, sc, tid, nT, nD, lam);
    } else {
      for (int i = tid; i < per; i += AT) {
        const long long sv = sc[i];
        const double cost = __dadd_rn(ec[i], __dmul_rn(lam, (double)sv));
        if (cost < best.cost || (cost == best.cost && sv < best.s)) {
          best.cost = cost;
          best.s = sv;
          best.idx = i;
        }
      }
    }
    for (int o = 32; o > 0; o >>= 1) {
      Best oth = shfl_best(best, o);
      if (less_than(oth, best)) best = oth;
    }
    if (lane == 0) {
      wcost[wave] = best.cost;
      ws[wave] = best.s;
      widx[wave] = best.idx;
    }
    __syncthreads();
    if (tid == 0) {
      Best b = best;
      for (int w = 1; w < nw; ++w) {
        Best o;
        o.cost = wcost[w];
        o.s = ws[w];
        o.idx = widx[w];
        if (less_than(o, b)) b = o;
      }
      own_pick = b.idx;
      unsigned long long *sl = xslot + 3 * (step & 1);
      x64store(sl, (unsigned long long)b.idx);
      x64store(sl + 1, (unsigned long long)sc[b.idx]);
      x64store(sl + 2, (unsigned long long)__double_as_longlong(ec[b.idx]));
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(0);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (!fail_s) {
        const unsigned target = (unsigned)nc * (unsigned)(step + 1) + target_extra;
        unsigned it = 0;
        while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
          if (++it > spin_limit) {
            fail_s = 1;
            __hip_atomic_fetch_or(&a.out->err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      }
    }
    __syncthreads();
    for (int q = tid; q < nc; q += AT) {
      const unsigned long long *sl = (const unsigned long long *)(a.tailT + (long long)q * nT) + 3 * (step & 1);
      cs[q] = (long long)x64load(sl + 1);
      ce[q] = __longlong_as_double((long long)x64load(sl + 2));
    }
    __syncthreads();
    if (tid == 0) {
      long long St = 0;
      double Et = 0.0;
      for (int q = 0; q < nc; ++q) {
        St += cs[q];
        Et = __dadd_rn(Et, ce[q]);
      }
      cs[nc] = St;  // broadcast slot (cs has room: nc < kMaxCells / 16)
      ce[nc] = Et;
    }
    __syncthreads();
    S = cs[nc];
    E = ce[nc];
    ++step;
    __syncthreads();  // cs / ce are rewritten by the next evaluation
  };
  auto finish = [&](int status, double lam, int iters, int pick) {
    if (tid == 0) {
      a.out_pick[g] = pick;
      if (a.out_err) a.out_err[g] = ec[pick];
      if (c == 0) {
        a.out->status = fail_s ? kAllocEsync : status;
        a.out->lambda = lam;
        a.out->iters = iters;
      }
    }
  };
  // totals of the final picks (the same cell-order sums) are written by workgroup 0
  auto finish_totals = [&](long long St, double Et) {
    if (tid == 0 && c == 0) {
      a.out->S = St;
      a.out->E = Et;
    }
  };

  const double B = a.budget;
  double lo = 1e-30, hi = 1e10;
  evaluate(lo);
  if ((double)S <= B) {
    finish(0, lo, 0, own_pick);
    finish_totals(S, E);
    return;
  }
  evaluate(hi);
  if ((double)S > B) {
    finish(JOLT_EINFEASIBLE, hi, 0, own_pick);
    finish_totals(S, E);
    return;
  }
  int feas = own_pick;  // this cell's pick at the feasible end
  long long Sf = S;
  double Ef = E;
  double hi_lam = hi;
  for (int it = 0; it < 50; ++it) {
    const double mid = __dsqrt_rn(__dmul_rn(lo, hi));
    evaluate(mid);
    const double Sd = (double)S;
    if (__dmul_rn(0.995, B) <= Sd && Sd <= B) {
      finish(0, mid, it + 1, own_pick);
      finish_totals(S, E);
      return;
    }
    if (Sd > B) lo = mid;
    else {
      hi = mid;
      hi_lam = hi;
      feas = own_pick;
      Sf = S;
      Ef = E;
    }
  }
  // no accept: the feasible end
  finish(0, hi_lam, 50, feas);
  finish_totals(Sf, Ef);
}

}  // namespace

namespace {
__global__ void alloc_sync_reset_kernel(AllocOut *o) {
  o->sync = 0u;
  o->err = 0u;
  o->status = 0;
}
}  // namespace

void run_alloc(const AllocArgs &a, hipStream_t st) {
  JOLT_REQUIRE(a.n_cells > 0 && a.n_cells <= AllocArgs::kMaxCells, JOLT_EINVAL, "allocate: too many cells");
  // one workgroup per cell when all of them can be resident at once and the exchange slots fit
  int dev = 0, cus = 0, occ = 0;
  bool multi = a.n_cells >= 2 && a.n_cells < AllocArgs::kMaxCells / 16 && a.n_rT >= 6;
  if (multi) {
    multi = hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, (const void *)alloc_mwg_kernel, AT, 0) == hipSuccess &&
            (long long)cus * occ >= a.n_cells;
    (void)hipGetLastError();
  }
  // the step counter and the lapse word start at zero for either kernel (the host reads err after both)
  hipLaunchKernelGGL(alloc_sync_reset_kernel, dim3(1), dim3(1), 0, st, a.out);
  HIP_LAUNCH_CHECK();
  if (multi) {
    // cooperative launch: the runtime starts it only if all of its workgroups can be resident at once
    // (each waits for the others' picks after every evaluation); if it refuses, one workgroup runs
    // the whole allocation (identical decisions and results)
    const WaitPolicy wp = wait_policy();
    AllocArgs a_ = a;
    unsigned sl_ = wp.spin_limit, te_ = wp.target_extra;
    void *args[] = {&a_, &sl_, &te_};
    if (hipLaunchCooperativeKernel((const void *)alloc_mwg_kernel, dim3(a.n_cells), dim3(AT), args, 0, st) ==
        hipSuccess)
      return;
    (void)hipGetLastError();
  }
  hipLaunchKernelGGL(alloc_kernel, dim3(1), dim3(AT), 0, st, a);
  HIP_LAUNCH_CHECK();
}

}  // namespace jolt
