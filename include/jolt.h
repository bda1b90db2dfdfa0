/*
 * jolt.h -- C ABI of libjolt, a JoLT / FlashJoLT KV-cache compressor for AMD
 * Instinct MI355X (gfx950).
 *
 * Method: Krishnan & Schulz, "A JoLT for the KV Cache: Near-Lossless KV Cache
 * Compression via Joint Rank-bit Allocation" (arXiv 2607.12550v2).
 *   Sec. 3 "Method": each layer group g of the prefill cache and each of K, V
 *     is a cell X in R^{|g| x n_h x T x d_h}.  The cell is stored as a partial
 *     Tucker backbone (token factor U_T, feature factor U_d, core) plus the
 *     truncation residual, rotated along features by the Q factor of a seeded
 *     Gaussian and quantised per row at b bits with one fp32 scale per row.
 *   Sec. 3, Eq. (1): bytes of a cell; Eq. (2): error surrogate
 *     e = eps^2(b) tau(r_T, r_d); Eqs. (3)-(4): one Lagrangian over all cells,
 *     lambda found by geometric bisection (0.5% of the budget or 50 steps).
 *   Sec. 3.1 "FlashJoLT": randomized token SVD with q_cap vectors (Eq. (5))
 *     and one synthetic tail entry carrying the energy not computed.
 *
 * Conventions for every entry point
 *   - Pointers prefixed d_ are device pointers, h_ host pointers.  The caller
 *     owns every buffer; the library never allocates or frees device memory
 *     and keeps no pointer after returning.  Work is enqueued on the given
 *     HIP stream (passed as void*, NULL = default stream).
 *   - A cache tensor (K or V) is contiguous [n_seq][n_layers][n_heads][n_tokens][d_head]
 *     in the element type given by jolt_cache_desc.dtype.
 *   - Cells are ordered (sequence, group, K|V): cell 2*(s*n_groups + g) + t.
 *   - Every entry point returns a jolt_status; on failure jolt_last_error()
 *     returns a thread-local message.  Nothing is thrown across the ABI.
 *   - Calls that share one workspace must not overlap; distinct workspaces
 *     may be used concurrently.  Concurrent calls on one device contend for its
 *     compute units: the FlashJoLT eigensolver (jolt_compress, jolt_spectra)
 *     reduces each B B^T matrix with several workgroups that wait for one
 *     another, and the allocation (jolt_compress, jolt_allocate) runs one
 *     workgroup per cell that exchange their picks, so each must have all its
 *     workgroups resident at once.  Both are cooperative launches: the runtime
 *     starts one only if all its workgroups can be resident together, and when
 *     it refuses, the library runs the one-workgroup form of the same step
 *     instead (same results, slower).  The waits are also bounded: if the
 *     workgroups still cannot all be scheduled in time, the affected cells get
 *     NaN spectra (jolt_compress then fails with JOLT_ENONFINITE) or the
 *     allocation fails with JOLT_EHIP, rather than the call hanging.
 */
#ifndef JOLT_H
#define JOLT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  JOLT_OK = 0,
  JOLT_EINVAL = -1,      /* bad shape, grid, dtype or argument */
  JOLT_EINFEASIBLE = -2, /* budget below the smallest attainable total bytes */
  JOLT_EWORKSPACE = -3,  /* workspace smaller than jolt_workspace_bytes() */
  JOLT_EHIP = -4,        /* HIP runtime error (message in jolt_last_error) */
  JOLT_ENONFINITE = -5,  /* ||X||_F^2 of a cell is not finite */
  JOLT_EBUFFER = -6      /* output buffer smaller than needed */
} jolt_status;

typedef enum { JOLT_F16 = 0, JOLT_BF16 = 1, JOLT_F32 = 2 } jolt_dtype;
typedef enum { JOLT_EXACT = 0, JOLT_FLASH = 1 } jolt_mode;

/* One or more independent prefill caches with identical shapes. */
typedef struct {
  int32_t n_seq, n_layers, n_heads, n_tokens, d_head; /* d_head in {64, 128} */
  int32_t dtype;                                      /* jolt_dtype */
  int32_t n_groups;
  const int32_t *group_start; /* host, n_groups+1 entries, 0 = s_0 < ... < s_G = n_layers */
} jolt_cache_desc;

/* Compression parameters. */
typedef struct {
  int32_t mode;        /* jolt_mode */
  int32_t oversample;  /* FlashJoLT: ell = q_cap + oversample (clamped to min(T, M)) */
  int32_t power_iters; /* FlashJoLT: subspace iterations (Halko et al.) */
  int32_t qcap;        /* FlashJoLT: token vectors computed; <= 0 selects Eq. (5) */
  const int32_t *rT_grid; int32_t n_rT; /* host, strictly ascending token ranks */
  const int32_t *rd_grid; int32_t n_rd; /* host, strictly ascending feature ranks <= d_head */
  const int32_t *bits; int32_t n_bits;  /* host, residual bit-widths in 0..8; 0 is always added */
  const double *eps2;   /* host, 9 entries indexed by b (eps2[0] must be 1), or NULL: the
                           library calibrates eps^2(b) on 2^18 Gaussian rows (seed 0) */
  double target_ratio;  /* C > 1: budget B = (dense bytes of all cells) / C */
  uint64_t rot_seed;    /* seed of the feature rotation */
  uint64_t sketch_seed; /* seed of the FlashJoLT Gaussian test matrix */
  int32_t alloc_variant; /* jolt_alloc_variant flags; 0 = joint allocation, exact per-cell argmin */
} jolt_params;

/* Allocator variants (jolt_params.alloc_variant), all on the same distortion/byte table:
 *   JOLT_ALLOC_GREEDY        the per-cell minimiser is the pages' greedy rank search (Sec. 3, "Solving
 *                            the allocation"): per bit-width, start at the smallest grid ranks and step
 *                            the mode whose next grid step removes the most error per added byte while
 *                            that step lowers e + lambda s; keep the bit-width of smallest e + lambda s
 *                            (equal rates: the token mode steps first).
 *   JOLT_ALLOC_KV_DECOUPLED  keys and values are allocated separately (Sec. 4.4, "Allocation strategy"):
 *                            the K cells (even cell indices) and the V cells (odd) each run their own
 *                            bisection, under the budget's share of their dense bytes |g| n_h T d_h c;
 *                            combinable with JOLT_ALLOC_GREEDY; needs at least two cells.
 *   JOLT_ALLOC_UNIFORM_RANKS every cell takes the same (r_T, r_d) (Sec. 4.4, "Per-group ranks"); the
 *                            bit-widths are still allocated per cell: for every grid pair a bisection over
 *                            the cells' bit-widths; the feasible pair of smallest total error wins (ties:
 *                            fewer bytes, then the earlier pair).  Not combinable with the others.
 * Unknown flags, or uniform ranks with another flag: JOLT_EINVAL.  The multiplier of a uniform-rank
 * allocation is that of the winning pair's bisection.
 * Rank-only compression (bits = {0}) and a token-rank cap (the token grid cut at the cap, Appendix A)
 * are restrictions of the grids. */
typedef enum {
  JOLT_ALLOC_JOINT = 0,
  JOLT_ALLOC_GREEDY = 1,
  JOLT_ALLOC_KV_DECOUPLED = 2,
  JOLT_ALLOC_UNIFORM_RANKS = 4
} jolt_alloc_variant;

/* Allocation of one cell, and where its section sits in the blob. */
typedef struct {
  int32_t rT, rd, bits, pad;
  int64_t bytes;         /* Eq. (1) bytes of the pick */
  double err_pred;       /* Eq. (2) surrogate e = eps^2(b) tau(r_T, r_d) */
  int64_t offset;        /* byte offset of the cell section in the blob (256-aligned) */
  int64_t section_bytes; /* padded bytes of the section (header + 256-aligned parts) */
} jolt_pick;

/* Workspace (device bytes) needed by jolt_compress / jolt_reconstruct for this cache and
 * these parameters; 0 on invalid arguments. */
size_t jolt_workspace_bytes(const jolt_cache_desc *desc, const jolt_params *params);

/* Upper bound of the blob size written by jolt_compress: B + per-section padding. */
size_t jolt_output_bytes(const jolt_cache_desc *desc, const jolt_params *params);

/* Lagrangian allocation alone (Sec. 3, Eqs. (1)-(4), "Solving the allocation").
 *   n_cells        number of cells.
 *   h_cell_shape   host int32[n_cells][4] = {|g|, n_h, T, d_h}.
 *   elem_bytes     c of Eq. (1): bytes per stored scalar.
 *   d_specT        device double: cell i's token spectrum (sigma^2, descending; FlashJoLT
 *                  spectra end with the tail entry) at d_specT[h_specT_off[i] ..
 *                  h_specT_off[i+1]).
 *   d_specD        device double: unprojected feature spectrum, same convention with h_specD_off.
 *   d_norm2        device double[n_cells]: ||X||_F^2.
 *   params         grids, bits, eps2 (target_ratio, mode and seeds are ignored).
 *   budget_bytes   B.
 *   h_picks        host jolt_pick[n_cells] (offset/section_bytes are set as if the cells were
 *                  written back to back in order).
 *   h_lambda       host double: the multiplier returned (may be NULL); with JOLT_ALLOC_KV_DECOUPLED
 *                  host double[2]: the keys' multiplier, then the values'.
 * Every grid rank must satisfy r_T <= (length of the cell's token spectrum) and r_d <= d_h,
 * else JOLT_EINVAL (for a FlashJoLT spectrum, whose last entry is the tail, the caller keeps
 * r_T <= q_cap).  JOLT_EINFEASIBLE if even the smallest picks exceed B.
 * Synchronises the stream once (to read the picks). */
int jolt_allocate(int32_t n_cells, const int32_t *h_cell_shape, int32_t elem_bytes,
                  const double *d_specT, const int64_t *h_specT_off,
                  const double *d_specD, const int64_t *h_specD_off,
                  const double *d_norm2, const jolt_params *params, double budget_bytes,
                  jolt_pick *h_picks, double *h_lambda, void *d_ws, size_t ws_bytes,
                  void *stream);

/* jolt_allocate without a workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same arguments,
 * results and errors as jolt_allocate, minus d_ws / ws_bytes: the tables, exchange slots and parameter
 * area live in a 16 MiB scratch array of the library, one per device, held until the process ends.
 * Calls whose tables need more (about n_cells * n_bits * n_rT * n_rd * 16 bytes plus a few KB) fail
 * with JOLT_EWORKSPACE before any work is enqueued.  The call allocates nothing; every call on a
 * device shares that device's scratch, so calls that overlap on one device race (the caller
 * serialises them; one call ends with its stream synchronisation). */
int jolt_allocate_static(int32_t n_cells, const int32_t *h_cell_shape, int32_t elem_bytes,
                         const double *d_specT, const int64_t *h_specT_off,
                         const double *d_specD, const int64_t *h_specD_off,
                         const double *d_norm2, const jolt_params *params, double budget_bytes,
                         jolt_pick *h_picks, double *h_lambda, void *stream);

/* Whole compression of K and V (Sec. 3 and Sec. 3.1): spectra, allocation under one budget,
 * ST-HOSVD fit, rotated b-bit residual.  Writes the blob (layout below) to d_out.
 *   h_picks   host jolt_pick[n_seq*n_groups*2]; h_lambda host double (may be NULL; two doubles, keys'
 *             then values', with JOLT_ALLOC_KV_DECOUPLED).
 * Synchronises the stream once (to read the picks); the blob is complete when the stream
 * reaches the end of the enqueued work.
 *
 * Blob layout: cell sections back to back in cell order, each 256-aligned:
 *   +0    header: uint32 {0x544C4F4A, 1, |g|, n_h, T, d_h, r_T, r_d, b, dtype}, padded to 256
 *   +256  U_T   [T][r_T]            storage dtype (= cache dtype)
 *         U_d   [d_h][r_d]          storage dtype              (256-aligned)
 *         core  [|g|][n_h][r_T][r_d] storage dtype             (256-aligned)
 *         scales[|g| n_h T] fp32 (only if b > 0)                (256-aligned)
 *         codes [|g| n_h T][d_h b / 8] bytes (only if b > 0)    (256-aligned)
 * Row r = (l*n_h + h)*T + t of the residual holds the rotated coordinates of
 * (X - backbone)[l,h,t,:] Q; code u = q + q_max (b >= 2, q_max = 2^(b-1)-1,
 * value q*scale) or u = 1 for +scale / 0 for -scale (b = 1); element i occupies
 * bits [i*b, (i+1)*b) of the row's little-endian bit stream. */
int jolt_compress(const void *d_K, const void *d_V, const jolt_cache_desc *desc,
                  const jolt_params *params, void *d_out, size_t out_bytes, void *d_ws,
                  size_t ws_bytes, jolt_pick *h_picks, double *h_lambda, void *stream);

/* Dense reconstruction from a blob (Sec. 3: decoding undoes the rotation and adds the
 * dequantised residual to the low-rank backbone).  d_K_out / d_V_out have the cache layout and
 * dtype of desc, 16-byte aligned (else JOLT_EINVAL).  h_picks are the picks jolt_compress
 * returned: rT, rd, bits and offset of every cell section are read from them (the section headers
 * repeat them for self-description).  Only params->rot_seed is used from params.  Fully
 * asynchronous. */
int jolt_reconstruct(const void *d_blob, const jolt_cache_desc *desc, const jolt_params *params,
                     const jolt_pick *h_picks, void *d_K_out, void *d_V_out, void *d_ws,
                     size_t ws_bytes, void *stream);

/* RoPE cosine / sine table for jolt_decode_attention (rotate-half pairs: dimension i turns with
 * i + d_h/2).  d_table: device float[n_pos][d_head/2][2] = {cos a, sin a} with a the fp32 product of
 * fp32(p) and fp32(base^(-2i/d_head)) (the product rounded to fp32, as the usual fp32 RoPE does),
 * p < n_pos, i < d_head/2.  The table depends on positions only: one table serves every layer and
 * head.  d_head even, at most 128; base > 1.  Asynchronous on the stream. */
int jolt_rope_table(int32_t d_head, double base, int32_t n_pos, float *d_table, void *stream);

/* Workspace bytes of jolt_decode_attention for this layer (0 on invalid arguments). */
size_t jolt_decode_attention_workspace_bytes(const jolt_cache_desc *desc, const jolt_pick *h_picks,
                                             int32_t seq, int32_t layer, int32_t n_q_heads);

/* One decode step of one layer, evaluated over the compressed cells (Sec. 4.5, "Fused decode
 * kernel"): no dense K or V of the layer is written to memory.  Keys are rebuilt per 128-token tile
 * on chip from U_T, the core and U_d plus the de-rotated residual, rotated by RoPE at their
 * positions and scored; values are accumulated in rank space against the value token factor and
 * in the rotated frame against the value codes, and expanded once per head.  Equal, up to rounding,
 * to softmax attention over the reconstruction jolt_reconstruct gives, with keys rotated by RoPE.
 *   d_blob, desc, params, h_picks   as written by jolt_compress (params: rot_seed is used).
 *   seq, layer     the sequence and the layer (any layer group size).
 *   d_q            device float[n_q_heads][d_h]: the step's queries, already rotated at their own
 *                  position; query head j reads KV head j / (n_q_heads / n_h) (grouped-query
 *                  attention; 1 to 8 query heads per KV head).
 *   d_k_tail, d_v_tail  device, cache dtype, [n_h][n_tail][d_h]: tokens newer than the compressed
 *                  ones (keys before RoPE, positions T .. T + n_tail - 1); NULL when n_tail == 0;
 *                  n_tail <= 1024.
 *   d_rope, n_rope_pos  a table from jolt_rope_table covering positions 0 .. T + n_tail - 1.
 *   d_out          device float[n_q_heads][d_h].
 *   d_ws, ws_bytes at least jolt_decode_attention_workspace_bytes: the layer's prepared state (its
 *                  backbone slices D_h = C_h U_d^T of both cells, the rotation) and the chunk states
 *                  of the split over tokens.
 *   reuse_prepared 0: the call prepares the state into d_ws first.  1: d_ws already holds the state a
 *                  previous call prepared for the same blob, picks, seq and layer (a decode loop
 *                  prepares each layer once and passes 1 on later steps); nothing is checked.
 * Scores are scaled by 1/sqrt(d_h); no mask.  Value token ranks up to 512.  Asynchronous on the
 * stream (the argument checks run on the host first; errors as elsewhere). */
int jolt_decode_attention(const void *d_blob, const jolt_cache_desc *desc, const jolt_params *params,
                          const jolt_pick *h_picks, int32_t seq, int32_t layer, const float *d_q,
                          int32_t n_q_heads, const void *d_k_tail, const void *d_v_tail,
                          int32_t n_tail, const float *d_rope, int32_t n_rope_pos, float *d_out,
                          void *d_ws, size_t ws_bytes, int32_t reuse_prepared, void *stream);

/* Spectra and token factors only (Sec. 3 ST-HOSVD inputs; Sec. 3.1 randomized token SVD).
 *   d_specT   device double[n_cells][nT]  token spectrum, nT = q_cap+1 (FlashJoLT, last entry
 *             is the tail) or min(T, |g| n_h d_h) (exact).
 *   d_specD   device double[n_cells][d_h] unprojected feature spectrum.
 *   d_norm2   device double[n_cells].
 *   d_UT      device float[n_cells][n_vec][T]: row r of cell c is token factor column r, or NULL.
 *   n_vec     number of token factor columns wanted (<= q_cap, resp. <= min(T, M)).
 * Fully asynchronous. */
int jolt_spectra(const void *d_K, const void *d_V, const jolt_cache_desc *desc,
                 const jolt_params *params, double *d_specT, double *d_specD, double *d_norm2,
                 float *d_UT, int32_t n_vec, void *d_ws, size_t ws_bytes, void *stream);

/* Spectrum-vector length per cell used by jolt_spectra (q_cap+1 or min(T, M)); <= 0 on error. */
int64_t jolt_token_spectrum_len(const jolt_cache_desc *desc, const jolt_params *params);

/* Residual stage of one cell with the factors given (Sec. 3, "Rotated low-bit residual"):
 * rebuild the backbone U_T core U_d^T, subtract it from X, rotate along features and quantise
 * each row at b bits.  X is [G][H][T][D] and the factors are in the storage dtype `dtype`
 * (U_T [T][rT], core [G][H][rT][rd], U_d [D][rd]).  Writes d_scales (fp32[G*H*T]) and
 * d_codes ([G*H*T][D*b/8] bytes).  1 <= b <= 8.  Fully asynchronous. */
int jolt_encode_residual(const void *d_X, int32_t G, int32_t H, int32_t T, int32_t D,
                         int32_t dtype, const void *d_UT, const void *d_core, const void *d_Ud,
                         int32_t rT, int32_t rd, int32_t bits, uint64_t rot_seed,
                         float *d_scales, uint8_t *d_codes, void *d_ws, size_t ws_bytes,
                         void *stream);

/* Workspace (device bytes) needed by jolt_encode_residual; 0 on invalid arguments. */
size_t jolt_encode_residual_workspace_bytes(int32_t G, int32_t H, int32_t T, int32_t D, int32_t rT, int32_t rd);

/* Layer grouping by token-subspace alignment (Sec. 3 "Method", with its footnote on group sizes).
 * For every layer, the top 8 token-mode singular vectors of its key cache (the T x n_h d_h unfolding;
 * randomized subspace iteration with 24 extra vectors and 3 power iterations, Gaussian test matrix
 * drawn from sketch_seed); each pair of consecutive layers is scored by the mean squared cosine of
 * the principal angles between their bases, ||U_l^T U_{l+1}||_F^2 / 8 (averaged over the n_seq
 * sequences); a new group starts where a score falls below the median of all scores, once the current
 * group holds two layers; a group closes at eight layers; a trailing single layer joins its predecessor.
 *   d_K             device key cache [n_seq][n_layers][n_heads][n_tokens][d_head] (desc->n_groups and
 *                   desc->group_start are ignored).
 *   h_group_start   host int32[n_layers + 1]: the group start offsets (first 0, last n_layers).
 *   h_n_groups      host int32: number of groups.
 *   h_scores        host double[n_layers - 1], or NULL: the scores.
 * Workspace: jolt_layer_groups_workspace_bytes(desc).  Synchronises the stream once.  The result can
 * be passed to jolt_compress as desc->group_start (groups of unequal size). */
size_t jolt_layer_groups_workspace_bytes(const jolt_cache_desc *desc);
int jolt_layer_groups(const void *d_K, const jolt_cache_desc *desc, uint64_t sketch_seed, int32_t *h_group_start,
                      int32_t *h_n_groups, double *h_scores, void *d_ws, size_t ws_bytes, void *stream);

/* FlashJoLT Gaussian test matrix (Sec. 3.1, randomized range finder), as jolt_compress draws it:
 * element (m, c) of Omega (M x ell) is Gaussian number m*ell + c of the sketch stream of
 * sketch_seed (SplitMix64 + Box-Muller), rounded once to dtype.  Written transposed, as
 * d_omegaT[c][m] (device, ell*M elements of dtype; caller-owned).  JOLT_EINVAL on bad sizes or
 * dtype.  Fully asynchronous.  Stage entry point for checking the sketch. */
int jolt_sketch_matrix(int32_t M, int32_t ell, int32_t dtype, uint64_t sketch_seed, void *d_omegaT,
                       void *stream);

/* Testing hook for the bounded cross-workgroup waits (per-cell allocation, multi-workgroup
 * tridiagonalisation).  spin_limit sets the polls each wait may take (0 restores the default);
 * unreachable != 0 raises every wait's target so that it is never met, so each wait lapses after
 * spin_limit polls while every kernel still runs to its end: the calls that follow must then fail
 * with JOLT_EHIP (allocation) or JOLT_ENONFINITE (spectra).  Process-wide; not for production
 * use.  Always JOLT_OK. */
int jolt_test_wait_policy(uint32_t spin_limit, int32_t unreachable);

/* Host set-up values (computed once per process and cached; Sec. 3). */
int jolt_rotation(int32_t d_head, uint64_t seed, double *h_Q /* [d_head][d_head] */);
int jolt_eps2(int32_t d_head, double *h_eps2 /* [9], indexed by b */);

/* Stage timing for measurement: when enabled, every stage of the calls that follow records a
 * pair of HIP events on the caller's stream.  jolt_profile_read() waits for the recorded
 * events, writes the stage names ('\n'-separated) to h_names, the summed milliseconds to
 * h_ms and the number of occurrences to h_count, clears the records and returns the number
 * of distinct stages (or a negative status). */
int jolt_profile(int32_t enable);
int32_t jolt_profile_read(char *h_names, int32_t names_bytes, double *h_ms, int32_t *h_count, int32_t max_stages);

/* Thread-local message of the last failing call ("" if none). */
const char *jolt_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* JOLT_H */
