/*
 * gpex.h -- C ABI of the MI355X (gfx950) excursion-set simulation library.
 *
 * The library computes, on one GPU, the hot path of the workflow described in
 * "Mixed-Precision GPU Acceleration for Confidence Regions of Spatial Excursion Sets"
 * (Zhang, Abdulah, Cao, French, Alomairy, Genton, Keyes):
 *   covariance tile generation and per-tile statistics         (Sec. V, Eq. 4; Sec. V-D)
 *   precision plan: tile map, Eq. 10/11 checks, scale s        (Sec. IV-B, V-D, V-E, Eq. 12)
 *   adaptive mixed-precision tile Cholesky of s^2 V            (Sec. IV-B; Algorithm 2, step 12)
 *   standard normals, compensation B = Z/s, TRMM M = L_s B     (Sec. IV-C, Eq. 3; Algorithm 1)
 *   universal kriging weights, predictor and MSPE              (Sec. V-A, Eq. 5, Eq. 6)
 *   conditioning, exceedance/extrema scan, calibration         (Sec. V-B, Eq. 7; V-C, Eq. 8, 9)
 *
 * Conventions (all entry points):
 *   - Pointers named d_* are device pointers owned by the caller (for example torch tensors
 *     on the context's device); pointers named h_* are host pointers owned by the caller.
 *     The library never frees caller memory.
 *   - Device memory the library needs (tile storage and the factor's FP16 copy, owned by a tiled
 *     handle; grow-only workspaces and flags, owned by the context) comes from the allocator given
 *     at context creation, or from hipMalloc / hipFree when none is given.  A context keeps its
 *     workspaces between calls, so repeated calls of the same sizes allocate nothing.
 *   - Matrices are column-major with an explicit leading dimension; vectors are contiguous.
 *   - All device work is enqueued on the stream given at context creation.  Entry points that
 *     return host values (info, diagnostics, psi/phi, region statistics) synchronise that
 *     stream before returning; gpex_cov_gen also synchronises (the precision plan needs the
 *     tile statistics on the host).
 *   - Return value: GPEX_OK (0); a negative code for misuse or a HIP failure (message via
 *     gpex_last_error); a positive code for a numerical condition the method names.
 *   - The library does not reorder locations: callers pass them in the order they want the
 *     tiles to follow (a space-filling order keeps near-diagonal tiles strongly correlated).
 *   - A context and the objects created through it are not thread-safe.
 *
 * Precision codes used in maps: 0 = FP64, 1 = FP32, 2 = FP16 (255 above the diagonal).
 */
#ifndef GPEX_H
#define GPEX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct gpex_ctx_s* gpex_ctx_t;
typedef struct gpex_tiled_s* gpex_tiled_t;

typedef enum {
    GPEX_OK = 0,
    GPEX_ERR_ARG = -1,           /* invalid argument (message names it) */
    GPEX_ERR_HIP = -2,           /* a HIP runtime call failed */
    GPEX_ERR_NOMEM = -3,         /* device allocation failed */
    GPEX_ERR_STATE = -4,         /* object in the wrong state (e.g. TRMM of an unfactored matrix) */
    GPEX_ERR_NOT_SPD = 1,        /* Cholesky met a non-positive pivot; info holds the column */
    GPEX_ERR_MSPE_NONPOS = 2,    /* some v_i <= 0: Sec. V-C requires positive MSPEs */
    GPEX_ERR_EMPTY_SAMPLE = 3,   /* psi or phi sample empty: Sec. V-C needs both non-empty */
    GPEX_WARN_CHECKS_FAILED = 4, /* Eq. 10 or Eq. 11 failed under a user tolerance (reported only) */
    GPEX_WARN_FP16_OVERFLOW = 5  /* a value stored in FP16 rounded to +-inf */
} gpex_status;

/* Covariance model.  kind 0: Matern sigma2 2^(1-nu) / Gamma(nu) r^nu K_nu(r) with the distance
 * scaled by the range (r = d / range): nu in {0.5, 1.5, 2.5} in closed form, sigma2 e^-r,
 * sigma2 (1 + r) e^-r, sigma2 (1 + r + r^2/3) e^-r; any other nu in [0.05, 8] through a quadrature
 * of K_nu (relative error about 1e-14; some 60 times the closed forms' time per entry; r below
 * 1e-30 is evaluated at 1e-30).  kind 1: Gaussian sigma2 exp(-d^2 / range) ("Massively parallel
 * approximate Gaussian process regression", isotropic Gaussian correlation).  d is the Euclidean
 * distance in the plane.  nugget is added to every diagonal entry unless a per-location diagonal
 * is given.  Other kinds or orders: GPEX_ERR_ARG. */
typedef struct {
    int kind;
    double sigma2, range, nu, nugget;
} gpex_cov_params;

/* Precision options.  amp = 0: every tile FP64 and s = 1 (Algorithm 1, AMP = 0 branch).
 * amp = 1: with r = ||V_ij||_F / ||V||_F and NT tile rows, off-diagonal tile (i, j) goes to FP16
 * when allow_fp16 and r * NT * 2^-10 <= tol, else to FP32 when r * NT * 2^-23 <= tol, else stays
 * FP64; unscaled_rule != 0 drops the NT factor (r * eps <= tol).  tol is the pages' fixedacc.
 * auto_tol != 0 (automatic mode, Sec. V-D): tol starts at 1e-4 (the given tol is ignored) and is
 * multiplied by 0.9 while Eq. 10 or Eq. 11 fails and FP16 tiles remain (at most 2000 rounds);
 * the final tol and the number of reductions are reported in gpex_diag.
 * fp16_dest_emulation != 0 (amp = 1 only; the tile size must be a multiple of 128): the
 * simulation product keeps its destination in FP16 between k-tasks as Algorithm 1 does (the
 * diagonal product is rounded to FP16, then after each off-diagonal tile k the running sum is
 * rounded to FP16), each task accumulating in FP32.  Default 0: one FP32 sum over the whole row
 * added to the FP64 result (more accurate, Sec. V-F leaves the accumulation to the platform). */
typedef struct {
    int amp;
    double tol;
    int allow_fp16;
    int unscaled_rule;
    int auto_tol;
    int fp16_dest_emulation;
} gpex_prec_opts;

/* Diagnostics of the plan (Sec. V-D, V-E) and of the simulation input (Algorithm 1). */
typedef struct {
    double s;             /* applied covariance scale, Eq. 12 (1 when unscaled) */
    double frob;          /* ||V||_F of the unscaled matrix */
    double l_bound;       /* l = max_f l_f (normal-range lower bound) */
    double u_bound;       /* u_s = min(65504, min_f u_f, u_factor) */
    double l_bound_sub;   /* lower bound with the subnormal limits (reported when l > u_s) */
    double r_hp;          /* Eq. 10 ratio v_max^HP / v_min^HP (NaN without FP16 tiles) */
    double rho1, rho2;    /* Eq. 11 ratios */
    double norm_B;        /* ||Z / s||_F of the simulation input (gpex_trmm_sim) */
    int eq10_pass, eq11_pass, lower_exceeds_upper, fp16_overflow;
    int64_t tiles[3];     /* lower tiles per precision: FP64, FP32, FP16 */
    double tol;           /* tolerance the map was built with (the final one in automatic mode) */
    int64_t tol_reductions; /* automatic mode: number of 0.9 reductions applied */
    double u_factor;      /* 65504 / sqrt(max_i V_ii): u_s also stays below it, so that the FP16
                             cast of L_s (Algorithm 1) stays finite (|(L_s)_ij| <= s sqrt(V_ii)) */
} gpex_diag;

typedef struct {
    double q_in, q_out;   /* critical values q_in = Q_{1-alpha}(phi), q_out = Q_alpha(psi) */
    int64_t n_psi, n_phi; /* sample sizes after dropping empty-set sentinels */
} gpex_region_stats;

/* ---- context ------------------------------------------------------------------------------ */
/* Binds HIP device `device` and the stream `hip_stream` (a hipStream_t; NULL = null stream).
 * alloc / dealloc (both given or both NULL) supply device memory: alloc(bytes, user) returns a
 * device pointer (NULL when out of memory: the entry point then returns GPEX_ERR_NOMEM) and
 * dealloc(ptr, user) releases it.  The allocator must be ordered on hip_stream (memory released
 * after queued work may be handed out again only to work queued after it, as torch's caching
 * allocator does for its stream); without one the library uses hipMalloc / hipFree.
 * *out receives the context.  Every entry point queues its work on that stream and, where it
 * forks work onto streams of its own (the factorization's look-ahead stream, the context's side
 * stream for the ragged edges of large GEMM launches; both created on first use, default
 * priority), joins them back to it with events before returning.  Errors: GPEX_ERR_ARG,
 * GPEX_ERR_HIP, GPEX_ERR_NOMEM. */
int gpex_ctx_create(int device, void* hip_stream, void* (*alloc)(size_t, void*),
                    void (*dealloc)(void*, void*), void* user, gpex_ctx_t* out);
/* Synchronises the context's streams and releases everything the context owns (flags, the
 * workspaces, the extra streams and their events).  Tiled handles keep working after their
 * context is destroyed only for gpex_tiled_info / gpex_tiled_stats / gpex_tiled_destroy.
 * Errors: GPEX_ERR_ARG. */
int gpex_ctx_destroy(gpex_ctx_t ctx);
/* Synchronises the context stream and releases the context's workspaces (they are taken again,
 * at the size the next call needs, by the next call).  Errors: GPEX_ERR_ARG, GPEX_ERR_HIP. */
int gpex_ctx_release_workspace(gpex_ctx_t ctx);
/* on != 0: serial schedule.  Every launch runs on the context stream in program order: the
 * factorization's look-ahead stream and the side stream of split GEMM launches are not used.
 * Each tile receives the same operations in the same order and from the same kernels as in
 * the concurrent schedule, so results are bitwise identical; the switch exists to check that.
 * Errors: GPEX_ERR_ARG. */
int gpex_ctx_set_serial(gpex_ctx_t ctx, int on);
/* Text of the last non-OK status on this context (valid until the next call on it). */
const char* gpex_last_error(gpex_ctx_t ctx);
/* Library version string. */
const char* gpex_version(void);

/* ---- covariance generation + precision plan -------------------------------------------- */
/* Generates the n x n covariance of the locations d_loc (SoA: x in d_loc[0..n), y in
 * d_loc[n..2n)), Eq. 4 of the mixed-precision page (joint covariance, prediction rows first
 * when the caller orders them so).  The diagonal gets d_diag_add[i] when d_diag_add is not
 * NULL (this is how tau^2 enters only the observation rows), else params->nugget.
 * The matrix is cut into nb x nb tiles (NT = ceil(n / nb), last tile padded with an identity
 * diagonal and zeros).  One pass evaluates every entry, writes V in FP64 and computes per-tile
 * sum of squares, minimum and maximum; the host plans the precision map and s (Sec. V-D, V-E);
 * each reduced-precision tile is then converted in place to s^2 V_ij in its precision (round to
 * nearest even).  FP64 tiles keep V until gpex_potrf_mp applies s^2 in its first step.  Every
 * lower tile has an FP64-sized slot (8 nb^2 bytes), whatever its precision.
 * *out receives a library-owned tiled matrix (release with gpex_tiled_destroy).
 * diag may be NULL.  Synchronises.  Returns GPEX_OK, GPEX_WARN_CHECKS_FAILED (Eq. 10/11 failed:
 * results still produced), GPEX_WARN_FP16_OVERFLOW, or an error.
 * Constraints: n >= 1, 16 <= nb <= 2048 and nb % 16 == 0. */
int gpex_cov_gen(gpex_ctx_t ctx, const double* d_loc, int64_t n, const double* d_diag_add,
                 const gpex_cov_params* params, int nb, const gpex_prec_opts* opts,
                 gpex_tiled_t* out, gpex_diag* diag);

/* Host-only planning from tile statistics (no device work): h_stats holds 3*nt*(nt+1)/2 doubles
 * (sum of squares, min, max per lower tile, row-packed), h_map receives nt*nt bytes (row-major,
 * 255 above the diagonal), diag the Eq. 10/11 values and the Eq. 12 scale.  This is the plan
 * gpex_cov_gen applies; it lets a caller re-plan cached statistics under another tolerance (or
 * run the automatic refinement) without regenerating the matrix, and reuse a final tolerance
 * from an earlier automatic run.  Returns GPEX_OK or GPEX_ERR_ARG. */
int gpex_plan(const double* h_stats, int64_t nt, const gpex_prec_opts* opts, uint8_t* h_map,
              gpex_diag* diag);

/* Sizes, map and scale of a tiled matrix.  h_map (NT*NT bytes, row-major, may be NULL). */
int gpex_tiled_info(gpex_tiled_t t, int64_t* n, int* nb, int64_t* nt, uint8_t* h_map, double* s);
/* Per-tile statistics of the unscaled matrix, 3 doubles per lower tile (sum of squares, min,
 * max) in row-packed order t = i(i+1)/2 + j.  h_stats holds 3*NT*(NT+1)/2 doubles. */
int gpex_tiled_stats(gpex_tiled_t t, double* h_stats);
/* Copies the stored lower tiles, converted to FP64 and unscaled (reduced-precision tiles divided
 * by s^2 before the factorisation, every tile by s after it, so a matrix reads as V and a factor
 * as chol(V)), into the
 * dense n x n column-major d_out (leading dimension ld >= n); entries above the diagonal tiles
 * are set to 0.  Enqueued on ctx. */
int gpex_tiled_to_dense(gpex_ctx_t ctx, gpex_tiled_t t, double* d_out, int64_t ld);
/* Same conversion for the sub-block rows [r0, r0 + rows) x columns [c0, c0 + cols) of the n x n
 * matrix (0 <= r0, c0; r0 + rows <= n; c0 + cols <= n) into d_out (rows x cols, leading
 * dimension ld >= rows); parts above the diagonal tiles read as 0 (for a diagonal tile the
 * stored upper triangle is copied: symmetric values before factorisation, zeros after).
 * Used to check leading blocks and sampled rows of large factors.  Enqueued on ctx. */
int gpex_tiled_block(gpex_ctx_t ctx, gpex_tiled_t t, int64_t r0, int64_t c0, int64_t rows,
                     int64_t cols, double* d_out, int64_t ld);
/* Raw values of a block, converted exactly to FP64 with no unscaling: which = 0 reads the stored
 * tiles (before the factorisation s^2 V in reduced-precision tiles and V in FP64 tiles; L_s after
 * it; entries above the diagonal tiles read 0),
 * which = 1 the FP16 copy of the off-diagonal factor tiles that the simulation product multiplies
 * with (Algorithm 1, cast16 of L_s; entries in diagonal tiles and above read 0), which = 2 the
 * diagonal tiles as the simulation product's two FP16 parts hi + lo (hi = cast16(L_s), lo =
 * cast16(L_s - hi); entries outside diagonal tiles read 0); which = 1 and 2 need a factor of more
 * than one tile row computed with amp = 1, else GPEX_ERR_STATE.  Lets a caller check that every
 * stored value is a value of its tile's precision and that the FP16 copy is cast16 of the stored
 * factor.  Block bounds and ld as in gpex_tiled_block.  Enqueued on ctx. */
int gpex_tiled_block_raw(gpex_ctx_t ctx, gpex_tiled_t t, int which, int64_t r0, int64_t c0, int64_t rows,
                         int64_t cols, double* d_out, int64_t ld);
int gpex_tiled_destroy(gpex_tiled_t t);

/* ---- mixed-precision tile Cholesky ------------------------------------------------------- */
/* Factors the tiled matrix in place, s^2 V = L_s L_s^T (Sec. IV-B; Algorithm 2, step 12), keeping
 * the precision map.  Step k: the diagonal tile is factored in FP64 together with its explicit
 * inverse T_k; every panel tile (i, k) is solved as A_ik T_k^T on FP64 matrix cores and rounded
 * once to its own precision (a reduced-precision solve through T_k loses definiteness on strongly
 * correlated covariances); every trailing tile is updated in its own precision with the operands
 * converted to it (FP16 tiles on FP16 matrix cores with FP32 accumulation and one FP16 rounding per
 * update), diagonal tiles in FP64.  With amp = 1 the panel solves also write the FP16 copy of
 * each off-diagonal factor tile that gpex_trmm_sim multiplies with (Algorithm 1, cast16; the
 * FP16 updates read their operands from it too), once the factor is complete each diagonal tile
 * as two FP16 parts beside it (hi = cast16(L_kk), lo = cast16(L_kk - hi)), and FP32 / FP64
 * copies of the panel tiles that feed updates of another precision (workspace: up to
 * 24 nb^2 (NT - 1) bytes).
 * *info = 0, or the 1-based column of the first non-positive pivot: then GPEX_ERR_NOT_SPD and the
 * handle is marked failed (its tiles were overwritten in place): gpex_potrf_mp, gpex_trmm_sim,
 * gpex_tiled_block and gpex_tiled_to_dense then return GPEX_ERR_STATE.  GPEX_WARN_FP16_OVERFLOW
 * (the factor is usable, diag.fp16_overflow set) when a value stored in FP16 became +-inf.
 * Synchronises. */
int gpex_potrf_mp(gpex_ctx_t ctx, gpex_tiled_t a, int64_t* info);

/* ---- simulation --------------------------------------------------------------------------- */
/* Standard normals of the seeded counter-based generator into d_Z (n x nsim, leading dim ld):
 * element (i, j) has linear index l = j n + i, pair p = l / 2, Philox4x32-10 counter
 * (p mod 2^32, p / 2^32, stream, 0) and key (seed mod 2^32, seed / 2^32); u1 from output words
 * 0-1, u2 from words 2-3 as ((w >> 11) + 1/2) 2^-53; Z_2p = sqrt(-2 ln u1) cos(2 pi u2),
 * Z_2p+1 = sqrt(-2 ln u1) sin(2 pi u2).  Enqueued on ctx. */
int gpex_normals(gpex_ctx_t ctx, uint64_t seed, uint32_t stream, int64_t n, int64_t nsim,
                 double* d_Z, int64_t ld);

/* M = L_s B with B = Z / s (Algorithm 1 and Eq. 3 of the mixed-precision page).  Z is either
 * the explicit d_Z (n x nsim, leading dimension n) or, when d_Z is NULL, the seeded normals of
 * gpex_normals(seed, stream 0).  With amp = 1, B is rounded to FP16, each off-diagonal L tile
 * is converted to FP16 and multiplied on FP16 matrix cores, the diagonal tile is applied at
 * about FP32 accuracy (where the 256 x 256 row-panel kernel takes the product: its two FP16
 * parts hi + lo on FP16 matrix cores, summed with the row; otherwise an FP32 copy on FP32
 * matrix cores), all with FP32 accumulation, and M is written in FP64 (with
 * fp16_dest_emulation the running sum is kept in FP16 between k-tasks, see gpex_prec_opts);
 * with amp = 0 everything is FP64.  d_M: n x nsim, leading dimension ldm >= n; exactly rows [0, n) and columns [0, nsim)
 * are written (the products compute the tile padding but do not store it).  diag (may be NULL)
 * receives the plan's diagnostics with norm_B.  Requires a factored matrix (GPEX_ERR_STATE
 * otherwise).  Returns GPEX_WARN_FP16_OVERFLOW (M is written) when an entry of Z / s overflowed
 * in FP16.  Synchronises before returning.  The context keeps the workspace of its largest call
 * (the FP16 or FP64 input B padded to NT nb rows and a multiple of 128 columns: 2 or 8 bytes per
 * element) until it is destroyed or its workspace released. */
int gpex_trmm_sim(gpex_ctx_t ctx, gpex_tiled_t l, int64_t nsim, uint64_t seed, const double* d_Z,
                  double* d_M, int64_t ldm, gpex_diag* diag);

/* ---- universal kriging -------------------------------------------------------------------- */
/* Universal kriging (Sec. V-A, Eq. 5, Eq. 6) with trend design rows (1, x, y) when k_trend = 3
 * (k_trend = 0: no trend).  Sigma_y = V_o + tau2 I is factored in FP64 tiles of size nb;
 * W = Sigma_y^-1 [V_op - X_o H] via the retained factor, zhat = W^T y_o and
 * v_i = sigma2 + w_i^T Sigma_y w_i - 2 w_i^T c_i, evaluated with Sigma_y W = V_op - X_o H.
 * d_loc_o (2*n_o, SoA), d_loc_p (2*n_p, SoA), d_y_o (n_o).  Outputs: d_W (n_o x n_p,
 * leading dimension n_o), d_zhat (n_p), d_v (n_p).  params->nugget is ignored (tau2 is the
 * observation-block diagonal).  *info as in gpex_potrf_mp (-1: trend system not SPD).
 * Synchronises. */
int gpex_krige(gpex_ctx_t ctx, const double* d_loc_o, int64_t n_o, const double* d_loc_p,
               int64_t n_p, const double* d_y_o, int k_trend, const gpex_cov_params* params,
               double tau2, int nb, double* d_W, double* d_zhat, double* d_v, int64_t* info);

/* ---- conditioning, exceedances and confidence regions ----------------------------------- */
/* S = M_p + W^T (y_o 1^T - M_o) (Eq. 7; with n_o = 0, S = M), then the fused scan of Eq. 8:
 *   d_counts[i] = #{j : S_ij >= u} (int64, n_p), d_sizes[j] = #{i : S_ij >= u} (int32, nsim).
 * When d_zhat and d_v are given: t = (zhat - u) / sqrt(v) (Eq. 1), psi_j = min of t over
 * {S_ij >= u} (+inf if empty), phi_j = max of t over {S_ij <= u} (-inf if empty) into h_psi,
 * h_phi (host, nsim); samples without sentinels, q_out = Q_{1-c}(psi), q_in = Q_c(phi) with
 * Eq. 9 (p read as a six-place decimal, exact integer ceiling); d_cout[i] = t_i >= q_out,
 * d_cin[i] = t_i > q_in (uint8, n_p); st receives q_in, q_out, n_psi, n_phi.
 * d_M: (n_p + n_o) x nsim, leading dimension ldm, prediction rows first.  d_W (n_o x n_p, ld
 * n_o) and d_y_o are needed when n_o > 0.  d_S (may be NULL) receives S (n_p x nsim, ld n_p).
 * Returns GPEX_ERR_MSPE_NONPOS when some v_i <= 0 and GPEX_ERR_EMPTY_SAMPLE when a sample is
 * empty (counts and psi/phi are still written).  Synchronises when d_zhat is given; otherwise
 * the counts and sizes are queued on the context stream and the call returns at once.
 * Temporaries (S when d_S is NULL and n_o > 0, the residual, t, per-group partials) live in a
 * context workspace. */
int gpex_excursion_regions(gpex_ctx_t ctx, const double* d_M, int64_t ldm, int64_t n_p,
                           int64_t n_o, int64_t nsim, const double* d_W, const double* d_y_o,
                           const double* d_zhat, const double* d_v, double u, double level_c,
                           int64_t* d_counts, int32_t* d_sizes, double* h_psi, double* h_phi,
                           uint8_t* d_cin, uint8_t* d_cout, double* d_S, gpex_region_stats* st);

/* The negative excursion set A-_u(Z) = {s : Z(s) <= u} ("Mixed-Precision GPU Acceleration for
 * Confidence Regions of Spatial Excursion Sets", Sec. III: negative excursions by reversing the
 * sign of the process and the threshold): the same arguments, conditioning and outputs as
 * gpex_excursion_regions, computed for -S, -u and -zhat, i.e. d_counts[i] = #{j : S_ij <= u},
 * d_sizes[j] = #{i : S_ij <= u}, t = (u - zhat) / sqrt(v), psi_j = min of t over {S_ij <= u},
 * phi_j = max of t over {S_ij >= u}, and q_out, q_in, d_cout, d_cin from them as above (they bound
 * the negative excursion set).  d_S (when given) receives S itself, not -S.  Same return codes. */
int gpex_excursion_regions_below(gpex_ctx_t ctx, const double* d_M, int64_t ldm, int64_t n_p,
                                 int64_t n_o, int64_t nsim, const double* d_W, const double* d_y_o,
                                 const double* d_zhat, const double* d_v, double u, double level_c,
                                 int64_t* d_counts, int32_t* d_sizes, double* h_psi, double* h_phi,
                                 uint8_t* d_cin, uint8_t* d_cout, double* d_S, gpex_region_stats* st);

/* Allocation-free variant of gpex_excursion_regions, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, results and return codes, with these differences:
 *   - the temporaries (t, per-group partials, psi/phi, and W^T y_o when n_o > 0) live in one fixed
 *     32 MiB device array per GPU that the library holds from its load until the process ends;
 *     a call whose temporaries need more returns GPEX_ERR_ARG (about 8 n_p + 20 G nsim + 16 nsim
 *     bytes, with G <= 256 row groups: n_p = 10^6 with nsim = 2,000 fits);
 *   - d_S is required when n_o > 0, and Eq. 7 is evaluated without the n_o x nsim residual:
 *     S = M_p - W^T M_o, then S += (W^T y_o) 1^T (the same S up to rounding order);
 *   - the conditioning product runs on the context stream only (no side stream is created).
 * It calls no hipMalloc / hipFree and no allocating library routine.  Every call on one GPU
 * shares that GPU's array, and the array keeps the last call's contents: calls that overlap on
 * one GPU (several contexts or threads) race, so callers serialise them. */
int gpex_excursion_regions_noalloc(gpex_ctx_t ctx, const double* d_M, int64_t ldm, int64_t n_p,
                                   int64_t n_o, int64_t nsim, const double* d_W, const double* d_y_o,
                                   const double* d_zhat, const double* d_v, double u, double level_c,
                                   int64_t* d_counts, int32_t* d_sizes, double* h_psi, double* h_phi,
                                   uint8_t* d_cin, uint8_t* d_cout, double* d_S, gpex_region_stats* st);

/* ---- timing support ------------------------------------------------------------------------ */
/* Per-phase device time of the last gpex_potrf_mp / gpex_trmm_sim on ctx, measured with HIP
 * events recorded around the launches on the streams they run on (enable with
 * gpex_ctx_set_timing(ctx, 1); it adds event records and no synchronisation).  out[32]:
 *   [0] potrf total ms;
 *   [1..3] trailing-update launches computing in FP64: summed launch ms, launch count, flops on
 *          whole tiles (2 nb^3 per off-diagonal tile, nb^3 per diagonal tile);
 *   [4..6] the same for FP32 launches, [7..9] for FP16 launches;
 *   [10] trmm total ms, [11] trmm matrix-core launches ms;
 *   [12..14] trailing-update flops per precision (FP64, FP32, FP16) on the tiles' true sizes
 *          (the last tile row and column hold n - (NT - 1) nb rows);
 *   [15..17] busy ms of the trailing-update launches per precision: the union of their launch
 *          intervals (launches of the two streams overlap, so [1], [4], [7] may exceed it);
 *   [18] trmm: ms of the row-panel launch of the simulation product (off-diagonal tiles, with
 *          the diagonal tiles where the 256 x 256 kernel takes them);
 *   [19] trmm: 1 when that launch applied the diagonal tiles too, else 0;
 *   [20..31] reserved (0). */
int gpex_ctx_set_timing(gpex_ctx_t ctx, int on);
int gpex_ctx_timings(gpex_ctx_t ctx, double* out32);

#ifdef __cplusplus
}
#endif
#endif /* GPEX_H */
