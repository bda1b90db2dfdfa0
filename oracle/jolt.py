"""JoLT / FlashJoLT compression, plain and slow, in numpy float64 (oracle).

TEST INFRASTRUCTURE ONLY (see the package header): the product path never
imports this module.

Source: Krishnan & Schulz, "A JoLT for the KV Cache" (arXiv 2607.12550v2).
  Sec. 3 "Method": cells (g, t) as 4th-order tensors |g| x n_h x T x d_h;
      "Partial Tucker backbone" (ST-HOSVD, token mode first);
      "Rotated low-bit residual" (seeded Gaussian QR rotation, per-row b-bit,
      one fp32 scale per row);
      "Joint Lagrangian allocation", Eq. (1) bytes and Eq. (2) error surrogate;
      "Solving the allocation", Eqs. (3)-(4), geometric bisection on lambda.
  Sec. 3.1 "FlashJoLT": randomized token SVD, synthetic tail entry, Eq. (5).

Readings of points the pages leave open (each is listed in the design notes):
  * quantizer: symmetric mid-tread, q_max = 2^(b-1)-1, s = absmax/q_max in
    fp32, code = clip(rint(x/s)); the decision is taken in fp32 because the
    pages fix the scale at fp32.  b = 1 is a sign code with s = absmax.
  * codes are stored offset-binary (code + q_max), b bits each, LSB-first
    within a row's bit stream.
  * c (bytes per stored scalar) is the element size of the cache dtype; the
    factors and core are stored in that dtype (round-to-nearest-even) and the
    residual is taken against the backbone rebuilt from the rounded factors.
  * the per-cell minimisation is an exhaustive argmin over the rank/bit grid
    (the exact minimisation that the Everett argument needs), ties broken by
    smaller bytes, then smaller b, r_T, r_d.
  * bisection bracket lambda in [1e-30, 1e10] per byte, midpoint sqrt(lo*hi),
    accept 0.995 B <= S <= B, else after 50 steps the feasible end.
"""
import math

import numpy as np

from . import rng

__all__ = [
    "DTYPE_BYTES", "to_f64", "round_to_dtype", "qmax", "quantize_rows", "dequantize_rows",
    "pack_rows", "unpack_rows", "rotation", "sketch_matrix", "eps2_calibrate", "qcap_eq5",
    "cell_bytes", "token_unfolding", "feature_spectrum", "token_factors_exact",
    "token_factors_flash", "layer_token_basis", "alignment_scores", "group_layers", "suffix_sums", "cell_table", "argmin_cell", "allocate",
    "argmin_cell_greedy", "allocate_with", "allocate_greedy", "allocate_kv_decoupled", "allocate_uniform_ranks",
    "fit_cell", "rotated_residual", "encode_cell", "decode_cell", "cells_of_cache", "section_layout",
    "write_blob", "read_blob_cell", "compress", "reconstruct", "CellShape",
]

DTYPE_BYTES = {"f16": 2, "bf16": 2, "f32": 4}
DTYPE_CODE = {"f16": 0, "bf16": 1, "f32": 2}
BLOB_MAGIC = 0x544C4F4A  # "JOLT" little-endian
BLOB_VERSION = 1
HEADER_BYTES = 256
ALIGN = 256


# ----------------------------------------------------------------------------
# storage dtypes
# ----------------------------------------------------------------------------
def to_f64(a, dtype):
    """Upcast a stored cache/factor array to float64.  bf16 arrays are raw uint16 bits."""
    if dtype == "bf16":
        a = np.asarray(a, dtype=np.uint16)
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(a).astype(np.float64)


def _round_mantissa(x, mant_bits, min_exp):
    """Round float64 to a binary format with ``mant_bits`` fraction bits, round-half-even.

    min_exp is the exponent of the smallest normal number; below it the spacing
    stays fixed (gradual underflow).  Overflow is not handled (factors are O(1)).
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    _, ex = np.frexp(np.where(ax > 0, ax, 1.0))  # ax = m 2^ex, m in [0.5, 1)
    e = (ex - 1).astype(np.float64)
    e = np.maximum(e, min_exp)
    q = np.ldexp(1.0, (e - mant_bits).astype(np.int64))
    return np.rint(x / q) * q


def round_to_dtype(x, dtype):
    """fp64 -> storage dtype value (returned as float64 holding the rounded value)."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "f16":
        return _round_mantissa(x, 10, -14)
    if dtype == "bf16":
        return _round_mantissa(x, 7, -126)
    raise ValueError(dtype)


def encode_dtype(x64, dtype):
    """Rounded float64 values -> the bytes of the storage dtype."""
    if dtype == "f32":
        return np.asarray(x64, dtype=np.float32)
    if dtype == "f16":
        return np.asarray(x64).astype(np.float16)  # exact: already representable
    if dtype == "bf16":
        f = np.asarray(x64).astype(np.float32)  # exact: already representable
        return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# quantizer (Sec. 3, "Rotated low-bit residual")
# ----------------------------------------------------------------------------
def qmax(b):
    return (1 << (b - 1)) - 1 if b >= 2 else 1


def quantize_rows(x_rot, b):
    """Per-row uniform b-bit quantisation with one fp32 scale per row.

    Returns (u, s): u is the stored unsigned code (offset binary), s the fp32
    scale.  The rounding decision is taken in fp32.
    """
    x = np.asarray(x_rot, dtype=np.float64).astype(np.float32)
    a = np.max(np.abs(x), axis=1)  # exact in fp32
    if b == 1:
        s = a.astype(np.float32)
        u = (x >= 0).astype(np.uint8)
        return u, s
    qm = np.float32(qmax(b))
    s = (a / qm).astype(np.float32)  # IEEE fp32 division
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    q = np.rint((x / safe[:, None]).astype(np.float32))
    q = np.clip(q, -qm, qm)
    q = np.where(s[:, None] > 0, q, np.float32(0.0))
    u = (q.astype(np.int32) + int(qm)).astype(np.uint8)
    return u, s


def dequantize_rows(u, s, b):
    """Stored codes + fp32 scales -> fp32 values (fp32 product code*s)."""
    s = np.asarray(s, dtype=np.float32)
    if b == 1:
        c = np.where(np.asarray(u) > 0, np.float32(1.0), np.float32(-1.0)).astype(np.float32)
    else:
        c = (np.asarray(u).astype(np.int32) - qmax(b)).astype(np.float32)
    return (c * s[:, None]).astype(np.float32)


def pack_rows(u, b):
    """LSB-first bit stream per row: element i occupies stream bits [i*b, (i+1)*b)."""
    u = np.asarray(u, dtype=np.uint8)
    rows, D = u.shape
    bits = (u[:, :, None] >> np.arange(b, dtype=np.uint8)[None, None, :]) & 1
    bits = bits.reshape(rows, D * b)
    return np.packbits(bits, axis=1, bitorder="little")


def unpack_rows(packed, b, D):
    packed = np.asarray(packed, dtype=np.uint8)
    rows = packed.shape[0]
    bits = np.unpackbits(packed, axis=1, bitorder="little")[:, : D * b].reshape(rows, D, b)
    w = (1 << np.arange(b)).astype(np.uint16)
    return (bits.astype(np.uint16) * w[None, None, :]).sum(axis=2).astype(np.uint8)


# ----------------------------------------------------------------------------
# seeded rotation and sketch
# ----------------------------------------------------------------------------
def rotation(D, seed):
    """d_h x d_h Q factor of a seeded Gaussian, signs fixed so diag(R) > 0 (Sec. 3)."""
    G = rng.gaussians(seed, rng.STREAM_ROTATION, D * D).reshape(D, D)
    Q, R = np.linalg.qr(G)
    sgn = np.sign(np.diag(R))
    sgn[sgn == 0] = 1.0
    return Q * sgn[None, :]


def sketch_matrix(M, ell, seed, dtype):
    """Gaussian test matrix Omega (M x ell), element (m, c) = stream index m*ell + c,
    rounded to the cache dtype (Sec. 3.1 randomized SVD; Halko et al.)."""
    g = rng.gaussians(seed, rng.STREAM_SKETCH, M * ell).reshape(M, ell)
    return round_to_dtype(g, dtype)


def eps2_calibrate(D, bits, rows=1 << 18, seed=0):
    """eps^2(b): fraction of Gaussian energy the b-bit row quantiser fails to recover
    (Sec. 3, Eq. (2); eps^2(0) = 1).  Gaussian rows are rotation invariant, so the
    round trip quantises the rows directly."""
    num = {b: 0.0 for b in bits if b > 0}
    den = 0.0
    chunk = 1 << 14
    for r0 in range(0, rows, chunk):
        n = min(chunk, rows - r0)
        x = rng.gaussians(seed, rng.STREAM_CALIBRATION, n * D, start=r0 * D).reshape(n, D)
        den += float(np.sum(x ** 2))
        for b in num:
            u, s = quantize_rows(x, b)
            xh = dequantize_rows(u, s, b).astype(np.float64)
            num[b] += float(np.sum((x - xh) ** 2))
    out = {0: 1.0} if 0 in bits else {}
    for b in num:
        out[b] = num[b] / den
    return out


def qcap_eq5(T, C):
    """Eq. (5): q_cap = min(max(q_min(C), ceil(T/32)), 512), q_min = 32 if C <= 4 else 64."""
    qmin = 32 if C <= 4 else 64
    return min(max(qmin, -(-T // 32)), 512)


# ----------------------------------------------------------------------------
# Eq. (1) bytes and the cell shape
# ----------------------------------------------------------------------------
class CellShape:
    def __init__(self, G, H, T, D):
        self.G, self.H, self.T, self.D = int(G), int(H), int(T), int(D)

    @property
    def M(self):
        return self.G * self.H * self.D

    @property
    def R(self):
        return self.G * self.H * self.T

    def __repr__(self):
        return f"CellShape({self.G},{self.H},{self.T},{self.D})"


def cell_bytes(sh, c, rT, rd, b):
    """Eq. (1) in exact integer bytes: (|g| n_h r_T r_d + T r_T + d_h r_d) c
    + [b>0] (b + 32/d_h)/8 |g| n_h T d_h  ==  ... + [b>0] R (b d_h/8 + 4)."""
    core = (sh.G * sh.H * rT * rd + sh.T * rT + sh.D * rd) * c
    resid = sh.R * (b * sh.D // 8 + 4) if b > 0 else 0
    return core + resid


# ----------------------------------------------------------------------------
# spectra and token factors
# ----------------------------------------------------------------------------
def token_unfolding(X):
    """X (G,H,T,D) -> X_(T) (T x G*H*D), column index (g, h, d) with d fastest."""
    G, H, T, D = X.shape
    return np.ascontiguousarray(X.transpose(2, 0, 1, 3).reshape(T, G * H * D))


def feature_spectrum(X):
    """Unprojected feature-mode spectrum: squared singular values of the (rows x d_h)
    unfolding, descending (Sec. 3, Eq. (2) uses the unprojected spectra)."""
    D = X.shape[-1]
    s = np.linalg.svd(X.reshape(-1, D), compute_uv=False)
    return s ** 2


def token_factors_exact(Xt):
    """Exact economy SVD of the token unfolding: (U, sigma^2)."""
    U, s, _ = np.linalg.svd(Xt, full_matrices=False)
    return U, s ** 2


def token_factors_flash(Xt, Omega, q, power_iters, norm2):
    """FlashJoLT token factors (Sec. 3.1) by randomized subspace iteration
    (Halko, Martinsson & Tropp 2011, Alg. 4.4) with the given test matrix.

    Returns (U (T x q), spectrum of length q+1 whose last entry is the synthetic
    tail ||X||^2 - sum of the q computed sigma^2, floored at zero)."""
    Q, _ = np.linalg.qr(Xt @ Omega)
    for _ in range(power_iters):
        Z, _ = np.linalg.qr(Xt.T @ Q)
        Q, _ = np.linalg.qr(Xt @ Z)
    Bm = Q.T @ Xt
    Ub, s, _ = np.linalg.svd(Bm, full_matrices=False)
    U = Q @ Ub[:, :q]
    sig2 = s[:q] ** 2
    tail = max(0.0, norm2 - float(np.sum(sig2)))
    return U, np.concatenate([sig2, [tail]])


# ----------------------------------------------------------------------------
# the distortion / byte table and the Lagrangian allocation (Eqs. (1)-(4))
# ----------------------------------------------------------------------------
def suffix_sums(spec):
    """t[r] = sum_{i >= r} spec[i], accumulated sequentially from the last entry;
    t has len(spec)+1 entries with t[n] = 0."""
    spec = np.asarray(spec, dtype=np.float64)
    t = np.zeros(len(spec) + 1)
    acc = 0.0
    for i in range(len(spec) - 1, -1, -1):
        acc = acc + float(spec[i])
        t[i] = acc
    return t


def cell_table(sh, c, specT, specD, norm2, rT_grid, rd_grid, bits, eps2):
    """Rows (b, r_T, r_d, e, s) for every grid point of one cell.
    tau = (discarded token mass + discarded feature mass) / ||X||^2; e = eps2(b) tau."""
    tT = suffix_sums(specT)
    tD = suffix_sums(specD)
    rows = []
    for b in bits:
        for rT in rT_grid:
            for rd in rd_grid:
                tau = (tT[rT] + tD[rd]) / norm2 if norm2 > 0 else 0.0
                e = eps2[b] * tau
                rows.append((b, rT, rd, e, cell_bytes(sh, c, rT, rd, b)))
    b_, rT_, rd_, e_, s_ = map(np.array, zip(*rows))
    return {"b": b_.astype(np.int64), "rT": rT_.astype(np.int64), "rd": rd_.astype(np.int64),
            "e": e_.astype(np.float64), "s": s_.astype(np.int64)}


def argmin_cell(tab, lam):
    """Exact per-cell minimiser of e + lambda s; ties: smaller s, b, r_T, r_d."""
    cost = tab["e"] + lam * tab["s"].astype(np.float64)
    order = np.lexsort((tab["rd"], tab["rT"], tab["b"], tab["s"], cost))
    return int(order[0])


LAMBDA_LO = 1e-30
LAMBDA_HI = 1e10
MAX_BISECT = 50


def allocate(tables, budget):
    """Geometric bisection on lambda (Sec. 3, "Solving the allocation").

    Returns dict(status, lam, picks=[index per cell], S, E, iters)."""
    def evaluate(lam):
        idx = [argmin_cell(t, lam) for t in tables]
        S = int(sum(int(t["s"][i]) for t, i in zip(tables, idx)))
        E = float(sum(float(t["e"][i]) for t, i in zip(tables, idx)))
        return idx, S, E

    lo, hi = LAMBDA_LO, LAMBDA_HI
    idx, S, E = evaluate(lo)
    if S <= budget:
        return {"status": 0, "lam": lo, "picks": idx, "S": S, "E": E, "iters": 0}
    idx_hi, S_hi, E_hi = evaluate(hi)
    if S_hi > budget:
        return {"status": -2, "lam": hi, "picks": idx_hi, "S": S_hi, "E": E_hi, "iters": 0}
    for it in range(MAX_BISECT):
        mid = math.sqrt(lo * hi)
        idx, S, E = evaluate(mid)
        if 0.995 * budget <= S <= budget:
            return {"status": 0, "lam": mid, "picks": idx, "S": S, "E": E, "iters": it + 1}
        if S > budget:
            lo = mid
        else:
            hi, idx_hi, S_hi, E_hi = mid, idx, S, E
    return {"status": 0, "lam": hi, "picks": idx_hi, "S": S_hi, "E": E_hi, "iters": MAX_BISECT}


# ----------------------------------------------------------------------------
# allocator variants (Sec. 3 "Solving the allocation" greedy search; Sec. 4.4 ablations)
# ----------------------------------------------------------------------------
def argmin_cell_greedy(tab, lam, n_rT, n_rd):
    """The pages' per-cell search at fixed lambda: for each bit-width, start at the smallest token and
    feature grid ranks and take one rank step at a time, in the mode whose next grid step removes the
    most error per added byte, as long as that step lowers e + lambda s (its error reduction exceeds
    lambda times its byte increment); stop when neither mode can step.  The cell keeps the bit-width
    with the smallest e + lambda s (ties: smaller bytes, then smaller b).  On equal descent rates the
    token mode steps first.  Table index: b-major, then r_T, then r_d."""
    e, sz = tab["e"], tab["s"].astype(np.float64)
    n_b = len(e) // (n_rT * n_rd)
    best = None
    for bi in range(n_b):
        iT, iD = 0, 0
        while True:
            here = (bi * n_rT + iT) * n_rd + iD
            moves = []
            if iT + 1 < n_rT:
                nxt = (bi * n_rT + iT + 1) * n_rd + iD
                de, ds = e[here] - e[nxt], sz[nxt] - sz[here]
                if de > lam * ds:
                    moves.append((de / ds, 0, nxt))
            if iD + 1 < n_rd:
                nxt = (bi * n_rT + iT) * n_rd + iD + 1
                de, ds = e[here] - e[nxt], sz[nxt] - sz[here]
                if de > lam * ds:
                    moves.append((de / ds, 1, nxt))
            if not moves:
                break
            rate, mode, nxt = max(moves, key=lambda m: (m[0], -m[1]))
            if mode == 0:
                iT += 1
            else:
                iD += 1
        i = (bi * n_rT + iT) * n_rd + iD
        key = (e[i] + lam * sz[i], sz[i], bi)
        if best is None or key < best[0]:
            best = (key, i)
    return int(best[1])


def allocate_with(tables, budget, argmin):
    """Geometric bisection on lambda (as allocate) with a given per-cell minimiser argmin(table, lam)."""
    def evaluate(lam):
        idx = [argmin(t, lam) for t in tables]
        return idx, int(sum(int(t["s"][i]) for t, i in zip(tables, idx))), \
            float(sum(float(t["e"][i]) for t, i in zip(tables, idx)))

    lo, hi = LAMBDA_LO, LAMBDA_HI
    idx, S, E = evaluate(lo)
    if S <= budget:
        return {"status": 0, "lam": lo, "picks": idx, "S": S, "E": E, "iters": 0}
    idx_hi, S_hi, E_hi = evaluate(hi)
    if S_hi > budget:
        return {"status": -2, "lam": hi, "picks": idx_hi, "S": S_hi, "E": E_hi, "iters": 0}
    for it in range(MAX_BISECT):
        mid = math.sqrt(lo * hi)
        idx, S, E = evaluate(mid)
        if 0.995 * budget <= S <= budget:
            return {"status": 0, "lam": mid, "picks": idx, "S": S, "E": E, "iters": it + 1}
        if S > budget:
            lo = mid
        else:
            hi, idx_hi, S_hi, E_hi = mid, idx, S, E
    return {"status": 0, "lam": hi, "picks": idx_hi, "S": S_hi, "E": E_hi, "iters": MAX_BISECT}


def allocate_greedy(tables, budget, n_rT, n_rd):
    """The Lagrangian allocation with the pages' greedy per-cell search instead of the exact argmin."""
    return allocate_with(tables, budget, lambda t, lam: argmin_cell_greedy(t, lam, n_rT, n_rd))


def allocate_kv_decoupled(tables, budget, dense_bytes):
    """Keys and values under budgets of their own (Sec. 4.4 "Allocation strategy"): cells alternate K, V
    (cell order (sequence, group, K|V)); each kind gets the budget in proportion to its dense bytes.
    Returns the two allocations' picks merged in cell order, both lambdas and the worse status."""
    out = {"picks": [0] * len(tables), "lam": [], "status": 0, "S": 0, "E": 0.0}
    for kind in (0, 1):
        cells = [c for c in range(len(tables)) if c % 2 == kind]
        share = sum(dense_bytes[c] for c in cells) / float(sum(dense_bytes))
        r = allocate([tables[c] for c in cells], budget * share)
        out["lam"].append(r["lam"])
        out["status"] = min(out["status"], r["status"])
        out["S"] += r["S"]
        out["E"] += r["E"]
        for c, i in zip(cells, r["picks"]):
            out["picks"][c] = i
    return out


def allocate_uniform_ranks(tables, budget, n_rT, n_rd):
    """One (r_T, r_d) for every cell, bit-widths still allocated per cell by the Lagrangian (Sec. 4.4
    "Per-group ranks"): for every grid pair, the bisection over the cells' bit-widths at that pair; the
    pair whose feasible allocation has the smallest total error wins (ties: smaller total bytes, then
    the earlier pair).  Returns the allocation with picks as full-table indices and the pair."""
    best = None
    for iT in range(n_rT):
        for iD in range(n_rd):
            sub = []
            for t in tables:
                n_b = len(t["e"]) // (n_rT * n_rd)
                ix = np.array([(bi * n_rT + iT) * n_rd + iD for bi in range(n_b)])
                sub.append({k: v[ix] for k, v in t.items()} | {"_ix": ix})
            r = allocate(sub, budget)
            if r["status"] != 0:
                continue
            key = (r["E"], r["S"], iT, iD)
            if best is None or key < best[0]:
                picks = [int(t["_ix"][i]) for t, i in zip(sub, r["picks"])]
                best = (key, dict(r, picks=picks, pair=(iT, iD)))
    if best is None:
        return {"status": -2, "picks": None}
    return best[1]


# ----------------------------------------------------------------------------
# fit, residual, decode (Sec. 3, "Partial Tucker backbone", "Rotated low-bit residual")
# ----------------------------------------------------------------------------
def _sign_normalise(U):
    idx = np.argmax(np.abs(U), axis=0)
    sgn = np.sign(U[idx, np.arange(U.shape[1])])
    sgn[sgn == 0] = 1.0
    return U * sgn[None, :]


def fit_cell(X, UT_r, rd):
    """ST-HOSVD with the token factor given: project, then the feature factor of the
    projected tensor, then the core.  Returns (U_T, U_d, core, projected spectrum)."""
    G, H, T, D = X.shape
    UT = _sign_normalise(np.asarray(UT_r, dtype=np.float64))
    Y = np.einsum("tr,ghtd->ghrd", UT, X, optimize=True)               # token-projected tensor
    Yr = Y.reshape(-1, D)
    w, V = np.linalg.eigh(Yr.T @ Yr)
    order = np.argsort(w)[::-1]
    w, V = w[order], V[:, order]
    Ud = _sign_normalise(V[:, :rd])
    core = np.einsum("ghrd,dk->ghrk", Y, Ud, optimize=True)
    return UT, Ud, core, np.maximum(w, 0.0)


def rotated_residual(X, UTr, Udr, Cr, Qrot):
    """Backbone U_T core U_d^T from the stored (rounded) factors, and the residual rows
    (X - backbone) rotated along features, E Q (rows in (layer, head, token) order)."""
    Xt = np.einsum("tr,ghrk,dk->ghtd", UTr, Cr, Udr, optimize=True)
    D = X.shape[-1]
    return Xt, (X - Xt).reshape(-1, D) @ Qrot


def encode_cell(X, UT, Ud, core, b, Qrot, dtype):
    """Round factors to the storage dtype, rebuild the backbone from the rounded
    factors, take the residual, rotate it along features and quantise it per row."""
    UTr = round_to_dtype(UT, dtype)
    Udr = round_to_dtype(Ud, dtype)
    Cr = round_to_dtype(core, dtype)
    Xt, Erot = rotated_residual(X, UTr, Udr, Cr, Qrot)
    out = {"UT": UTr, "Ud": Udr, "core": Cr, "backbone": Xt, "b": b}
    if b > 0:
        u, s = quantize_rows(Erot, b)
        out["u"], out["scales"] = u, s
    return out


def decode_cell(UT, Ud, core, b, u, scales, Qrot, shape):
    """Backbone plus the de-rotated, dequantised residual (float64)."""
    Xt = np.einsum("tr,ghrk,dk->ghtd", UT, core, Ud, optimize=True)
    if b > 0:
        D = shape[-1]
        Erot = dequantize_rows(u, scales, b).astype(np.float64)
        Xt = Xt + (Erot @ Qrot.T).reshape(shape)
    return Xt


# ----------------------------------------------------------------------------
# layer grouping by token-subspace alignment (Sec. 3, "Method", and its footnote on size bounds)
# ----------------------------------------------------------------------------
def layer_token_basis(Xl, k=8):
    """Top-k token-mode left singular vectors of one layer's key cache (n_h x T x d_h): the columns of
    U of the SVD of the T x (n_h d_h) unfolding, as a T x k array with orthonormal columns."""
    H, T, D = Xl.shape
    A = Xl.transpose(1, 0, 2).reshape(T, H * D)
    U, _, _ = np.linalg.svd(A, full_matrices=False)
    return U[:, :k]


def alignment_scores(K, k=8):
    """Score of each pair of consecutive layers (l, l+1) of a key cache (L x n_h x T x d_h): the mean
    squared cosine between their token bases, read as the mean of the squared cosines of the k
    principal angles between the two k-dimensional subspaces, ||U_l^T U_{l+1}||_F^2 / k (independent
    of the choice of basis inside each subspace).  Returns L-1 scores."""
    K = np.asarray(K, dtype=np.float64)
    U = [layer_token_basis(K[l], k) for l in range(K.shape[0])]
    return np.array([float(np.sum((U[l].T @ U[l + 1]) ** 2)) / k for l in range(len(U) - 1)])


def group_layers(scores, min_size=2, max_size=8):
    """Contiguous layer groups from the L-1 consecutive-layer scores: a new group starts where the
    score falls below the median of all scores, but only once the current group holds min_size
    layers; a group is closed at max_size layers whatever the score; a trailing group of one layer
    joins its predecessor.  Returns the start offsets (n_groups + 1 entries, last = L)."""
    scores = np.asarray(scores, dtype=np.float64)
    L = len(scores) + 1
    med = float(np.median(scores)) if len(scores) else 0.0
    sizes = [1]
    for l in range(1, L):
        if sizes[-1] >= max_size or (scores[l - 1] < med and sizes[-1] >= min_size):
            sizes.append(1)
        else:
            sizes[-1] += 1
    if len(sizes) > 1 and sizes[-1] == 1:
        last = sizes.pop()
        sizes[-1] += last
    return [int(v) for v in np.concatenate([[0], np.cumsum(sizes)])]


# ----------------------------------------------------------------------------
# cache -> cells, blob layout
# ----------------------------------------------------------------------------
def cells_of_cache(K, V, group_start):
    """Cells in order (sequence, group, K|V); each (G,H,T,D) float64 view source."""
    n_seq = K.shape[0]
    out = []
    for s in range(n_seq):
        for g in range(len(group_start) - 1):
            l0, l1 = group_start[g], group_start[g + 1]
            out.append((s, g, 0, K[s, l0:l1]))
            out.append((s, g, 1, V[s, l0:l1]))
    return out


def _al(n):
    return (n + ALIGN - 1) // ALIGN * ALIGN


def section_layout(sh, c, rT, rd, b):
    """Byte offsets inside one cell section (all 256-byte aligned)."""
    off = {"header": 0, "UT": HEADER_BYTES}
    off["Ud"] = off["UT"] + _al(sh.T * rT * c)
    off["core"] = off["Ud"] + _al(sh.D * rd * c)
    off["scales"] = off["core"] + _al(sh.G * sh.H * rT * rd * c)
    if b > 0:
        off["codes"] = off["scales"] + _al(sh.R * 4)
        off["end"] = off["codes"] + _al(sh.R * sh.D * b // 8)
    else:
        off["codes"] = off["scales"]
        off["end"] = off["scales"]
    return off


def write_blob(cells_enc, shapes, dtype):
    """Concatenate cell sections; returns (bytes, offsets)."""
    c = DTYPE_BYTES[dtype]
    parts, offsets, pos = [], [], 0
    for enc, sh in zip(cells_enc, shapes):
        rT, rd, b = enc["UT"].shape[1], enc["Ud"].shape[1], enc["b"]
        lay = section_layout(sh, c, rT, rd, b)
        buf = bytearray(lay["end"])
        hdr = np.array([BLOB_MAGIC, BLOB_VERSION, sh.G, sh.H, sh.T, sh.D, rT, rd, b,
                        DTYPE_CODE[dtype]], dtype=np.uint32)
        buf[0:hdr.nbytes] = hdr.tobytes()

        def put(key, arr):
            bts = np.ascontiguousarray(arr).tobytes()
            buf[lay[key]:lay[key] + len(bts)] = bts

        put("UT", encode_dtype(enc["UT"], dtype))
        put("Ud", encode_dtype(enc["Ud"], dtype))
        put("core", encode_dtype(enc["core"], dtype))
        if b > 0:
            put("scales", np.asarray(enc["scales"], dtype=np.float32))
            put("codes", pack_rows(enc["u"], b))
        offsets.append(pos)
        parts.append(bytes(buf))
        pos += len(buf)
    return b"".join(parts), offsets


def read_blob_cell(blob, offset, dtype):
    """Parse one cell section written by any producer of the documented layout."""
    hdr = np.frombuffer(blob, dtype=np.uint32, count=10, offset=offset)
    if int(hdr[0]) != BLOB_MAGIC:
        raise ValueError("bad magic")
    G, H, T, D, rT, rd, b = (int(v) for v in hdr[2:9])
    sh = CellShape(G, H, T, D)
    c = DTYPE_BYTES[dtype]
    lay = section_layout(sh, c, rT, rd, b)
    npdt = {"f16": np.float16, "bf16": np.uint16, "f32": np.float32}[dtype]

    def get(key, count):
        return np.frombuffer(blob, dtype=npdt, count=count, offset=offset + lay[key])

    UT = to_f64(get("UT", T * rT), dtype).reshape(T, rT)
    Ud = to_f64(get("Ud", D * rd), dtype).reshape(D, rd)
    core = to_f64(get("core", G * H * rT * rd), dtype).reshape(G, H, rT, rd)
    u = s = None
    if b > 0:
        s = np.frombuffer(blob, dtype=np.float32, count=sh.R, offset=offset + lay["scales"])
        packed = np.frombuffer(blob, dtype=np.uint8, count=sh.R * D * b // 8,
                               offset=offset + lay["codes"]).reshape(sh.R, D * b // 8)
        u = unpack_rows(packed, b, D)
    return {"shape": sh, "rT": rT, "rd": rd, "b": b, "UT": UT, "Ud": Ud, "core": core,
            "u": u, "scales": s}


# ----------------------------------------------------------------------------
# whole-cache compress / reconstruct
# ----------------------------------------------------------------------------
def compress(K, V, group_start, dtype, params, keep=False):
    """Full JoLT / FlashJoLT compression of a cache (Sec. 3, Sec. 3.1).

    K, V: arrays (n_seq, L, H, T, D) in the storage dtype (bf16 as raw uint16).
    params: dict(mode 'exact'|'flash', oversample, power_iters, qcap (None -> Eq. 5),
            rT_grid, rd_grid, bits, eps2 {b: value}, target_ratio, rot_seed, sketch_seed,
            alloc 'joint' (default) | 'greedy' | 'kv_decoupled' | 'uniform').
    """
    c = DTYPE_BYTES[dtype]
    n_seq, L, H, T, D = K.shape
    bits = sorted(set(params["bits"]) | {0})
    eps2 = params["eps2"]
    Qrot = rotation(D, params.get("rot_seed", 0))
    cells = cells_of_cache(K, V, group_start)
    shapes, tables, infos = [], [], []
    flash = params["mode"] == "flash"
    C = float(params["target_ratio"])
    omega_cache = {}
    for (s, g, t, Xs) in cells:
        X = to_f64(Xs, dtype)
        G = X.shape[0]
        sh = CellShape(G, H, T, D)
        Xt = token_unfolding(X)
        norm2 = float(np.sum(X * X))
        specD = feature_spectrum(X)
        if flash:
            q = params.get("qcap") or qcap_eq5(T, C)
            ell = min(q + params["oversample"], T, sh.M)
            q = min(q, ell)
            if (sh.M, ell) not in omega_cache:
                omega_cache[(sh.M, ell)] = sketch_matrix(sh.M, ell, params.get("sketch_seed", 0), dtype)
            U, specT = token_factors_flash(Xt, omega_cache[(sh.M, ell)], q,
                                           params["power_iters"], norm2)
        else:
            U, specT = token_factors_exact(Xt)
        tab = cell_table(sh, c, specT, specD, norm2, params["rT_grid"], params["rd_grid"], bits, eps2)
        shapes.append(sh)
        tables.append(tab)
        infos.append({"seq": s, "group": g, "kv": t, "norm2": norm2, "specT": specT,
                      "specD": specD, "U": U, "X": X if keep else None})
    dense = sum(sh.R * sh.D * c for sh in shapes)
    budget = dense / C
    variant = params.get("alloc", "joint")
    nR, nD = len(params["rT_grid"]), len(params["rd_grid"])
    if variant == "greedy":
        al = allocate_greedy(tables, budget, nR, nD)
    elif variant == "kv_decoupled":
        al = allocate_kv_decoupled(tables, budget, [sh.R * sh.D * c for sh in shapes])
    elif variant == "uniform":
        al = allocate_uniform_ranks(tables, budget, nR, nD)
    else:
        al = allocate(tables, budget)
    result = {"status": al["status"], "lam": al.get("lam"), "budget": budget, "dense_bytes": dense,
              "S": al.get("S"), "E_pred": al.get("E"), "iters": al.get("iters"), "cells": []}
    if al["status"] != 0:
        return result
    encs = []
    for k, (info, sh, tab) in enumerate(zip(infos, shapes, tables)):
        i = al["picks"][k]
        b, rT, rd = int(tab["b"][i]), int(tab["rT"][i]), int(tab["rd"][i])
        X = info["X"] if keep else to_f64(cells[k][3], dtype)
        UT, Ud, core, wproj = fit_cell(X, info["U"][:, :rT], rd)
        enc = encode_cell(X, UT, Ud, core, b, Qrot, dtype)
        Xhat = decode_cell(enc["UT"], enc["Ud"], enc["core"], b, enc.get("u"), enc.get("scales"),
                           Qrot, X.shape)
        err2 = float(np.sum((X - Xhat) ** 2))
        encs.append(enc)
        cell = dict(info)
        cell.update({"rT": rT, "rd": rd, "b": b, "bytes": int(tab["s"][i]), "e_pred": float(tab["e"][i]),
                     "err2": err2, "rel_err": math.sqrt(err2 / info["norm2"]) if info["norm2"] > 0 else 0.0,
                     "specD_proj": wproj, "UT_fit": UT, "Ud_fit": Ud})
        if keep:
            cell["enc"] = enc
            cell["Xhat"] = Xhat
        else:
            cell["X"] = None
        result["cells"].append(cell)
    blob, offsets = write_blob(encs, shapes, dtype)
    result["blob"] = blob
    result["offsets"] = offsets
    for cell, off in zip(result["cells"], offsets):
        cell["offset"] = off
    return result


def reconstruct(blob, offsets, dtype, rot_seed, D):
    """Dense float64 reconstruction of every cell section in ``blob``."""
    Qrot = rotation(D, rot_seed)
    out = []
    for off in offsets:
        c = read_blob_cell(blob, off, dtype)
        sh = c["shape"]
        out.append(decode_cell(c["UT"], c["Ud"], c["core"], c["b"], c["u"], c["scales"], Qrot,
                               (sh.G, sh.H, sh.T, sh.D)))
    return out
