/*
 * shampoo.h -- C ABI of the batched block preconditioner step of
 * block-diagonal Shampoo, for AMD Instinct MI355X (gfx950).
 *
 * Sources cited below (titles of the pages; sections as named there):
 *   [DASH]  "DASH: Faster Shampoo via Batched Block Preconditioning and
 *           Efficient Inverse-Root Solvers", source-linked AI summary.
 *   [3DS]   "3D-Shampoo optimizer" README.
 *   [NOTES] "Shampoo" notes (regret, Kronecker bound, scale, grafting).
 *   [DIST]  "A Distributed Data-Parallel PyTorch Implementation of the
 *           Distributed Shampoo Optimizer ..." (abstract).
 *
 * Conventions shared by every entry point:
 *   - Layout: row-major.  A "stack" is a contiguous [n, B, B] array; matrix b
 *     starts at element b*B*B.  Block tables are arrays of shampoo_block.
 *   - Ownership: the caller owns every buffer.  No entry point allocates or
 *     frees device memory; scratch comes in through an explicit workspace
 *     whose size the matching *_workspace call reports.  Pointers named *_dev
 *     and all stacks are device pointers; everything else is host memory.
 *   - Streams: all device work is enqueued, in order, on the given stream.
 *     No entry point synchronises the device except shampoo_check_flags.
 *   - Errors: arguments are validated before the first launch, so a call
 *     that returns an error has enqueued nothing.  No C++ exception crosses
 *     the ABI.  shampoo_last_error() returns a thread-local message for the
 *     last non-OK status of the calling thread.  A failed launch returns
 *     SHAMPOO_E_HIP; faults that surface later are reported by the next
 *     synchronising HIP call of the caller.
 *   - Numerical failures are not errors: they set per-matrix flag bits
 *     (SHAMPOO_FLAG_*) in a caller-provided int32 array, written with atomic
 *     OR (the caller clears it).
 */
#ifndef SHAMPOO_H
#define SHAMPOO_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum shampoo_status {
  SHAMPOO_OK = 0,
  SHAMPOO_E_INVALID = 1,     /* bad argument: null pointer, size, enum value */
  SHAMPOO_E_UNSUPPORTED = 2, /* valid but not implemented combination */
  SHAMPOO_E_WORKSPACE = 3,   /* workspace smaller than the *_workspace size */
  SHAMPOO_E_HIP = 4,         /* a HIP runtime call or kernel launch failed */
  SHAMPOO_E_NONFINITE = 5    /* shampoo_check_flags found a flagged matrix */
} shampoo_status;

typedef enum shampoo_dtype {
  SHAMPOO_F32 = 0,
  SHAMPOO_F16 = 1,
  SHAMPOO_BF16 = 2,
  SHAMPOO_F64 = 3
} shampoo_dtype;

/* Inverse-root solvers.  [NOTES] "Roots on idle CPUs, partial preconditioners
 * for large layers, and grafting" (coupled Newton of Guo-Higham / Iannazzo);
 * [DASH] "3. Inverse Root Methods" (Newton-DB); [DASH] "A.1/A.2 Chebyshev
 * polynomials" (Chebyshev series summed by Clenshaw's recurrence). */
typedef enum shampoo_method {
  SHAMPOO_CN = 0,
  SHAMPOO_NDB = 1,
  SHAMPOO_CHEBYSHEV = 2
} shampoo_method;

/* How a Chebyshev series is summed (shampoo_root_opts.cheb_eval).  Both give
 * the same polynomial up to rounding.
 * CLENSHAW: Clenshaw's recurrence, d - 1 products for degree d ([DASH]
 *   "A.2 Chebyshev polynomials for matrices").
 * PS: the baby-step/giant-step split of Paterson and Stockmeyer (SIAM J.
 *   Comput. 2(1), 1973) carried out in the Chebyshev basis.  With
 *   y = T_m(S), T_mj = T_j(y) and T_(mj+i) = 2 T_j(y) T_i - T_(mj-i) turn
 *   the series into sum_j T_j(y) a_j(S), deg a_j < m; the a_j are combined
 *   from T_0..T_(m-1) (m - 1 products) and the outer series in y is summed
 *   by Clenshaw's recurrence (about d/m products).  m minimises the count:
 *   6 products at d = 16, 8 at d = 25, against 15 and 24. */
typedef enum shampoo_cheb_eval {
  SHAMPOO_CHEB_CLENSHAW = 0,
  SHAMPOO_CHEB_PS = 1
} shampoo_cheb_eval;

/* [DASH] "3. Inverse Root Methods": Frobenius-norm scaling, or the largest
 * Rayleigh quotient of a half-precision multi-start power iteration. */
typedef enum shampoo_scaling {
  SHAMPOO_SCALE_FROBENIUS = 0,
  SHAMPOO_SCALE_POWER = 1
} shampoo_scaling;

/* Grafting.  [3DS] "Hyperparameters" (layer-wise onto SGD), "How to use"
 * (lr 0.1, momentum 0.9); [DASH] "2. Preliminaries on Shampoo" (Adam). */
typedef enum shampoo_graft {
  SHAMPOO_GRAFT_SGD = 0,
  SHAMPOO_GRAFT_MOMENTUM = 1,
  SHAMPOO_GRAFT_ADAM = 2,
  SHAMPOO_GRAFT_NONE = 3     /* W <- W - lr D, no rescaling */
} shampoo_graft;

/* Per-matrix flag bits. */
#define SHAMPOO_FLAG_NONFINITE 1  /* a NaN or Inf in the output root */
#define SHAMPOO_FLAG_ZERO_SCALE 2 /* scale s was 0 or not finite: output set to 0 */
#define SHAMPOO_FLAG_PI_FALLBACK 4 /* power iteration gave no positive finite
                                      quotient: Frobenius scale used instead */
#define SHAMPOO_FLAG_RECOMPUTED_F64 8 /* shampoo_step fallback: the root was
                                         recomputed with the float64 chain */
#define SHAMPOO_FLAG_KEPT_PREVIOUS 16 /* shampoo_step fallback: the factor's
                                         previous root was kept */
#define SHAMPOO_FLAG_RESIDUAL 32  /* the solver residual exceeded
                                     shampoo_root_opts.residual_bound (or was
                                     not finite) */

/* What shampoo_step does with a factor whose new root failed: not finite,
 * a zero scale, or (when root.residual_bound > 0) a solver residual above the
 * bound.  [NOTES] "Spreading the preconditioners across GPUs ...": a root
 * whose float32 eigendecomposition fails is computed again in float64. */
typedef enum shampoo_fallback {
  SHAMPOO_FALLBACK_NONE = 0,     /* write the root as computed and flag it */
  SHAMPOO_FALLBACK_KEEP = 1,     /* keep the factor's previous root */
  SHAMPOO_FALLBACK_F64 = 2       /* recompute the non-finite and residual-
                                    flagged factors with the float64 chain
                                    (same method and counts, no residual
                                    check), keeping the previous root where
                                    that is not finite (and for zero scales);
                                    synchronises the stream to count them; as
                                    KEEP when root.compute is already F64 */
} shampoo_fallback;

/* One row of a block table (32 bytes, plain old data).  [DASH] "4. Blocking
 * Strategy"; [3DS] "Hyperparameters" (block_size, 0 = never split).
 * param: parameter index; (brow, bcol): position in the parameter's block
 * grid; (row0, col0): offset of the block's first element in the
 * parameter's 2-D view; (rows, cols): valid extent (< B on ragged edges);
 * B: side of the zero-padded stacked block. */
typedef struct shampoo_block {
  int32_t param, brow, bcol, row0, col0, rows, cols, B;
} shampoo_block;

/* A 2-D device matrix: element (r, c) at data[r * ld + c]. */
typedef struct shampoo_matrix {
  void* data;
  int64_t rows, cols, ld;
} shampoo_matrix;

/* A parameter as seen by shampoo_step (device array of these).
 * w: float32 weights [rows, ld]; g: gradient [rows, ld] in the step's g_dt;
 * m: momentum buffer (MOMENTUM) or Adam first moment (ADAM), float32, else NULL;
 * v: Adam second moment (ADAM), float32, else NULL;
 * first_block: table index of the parameter's block (0, 0); its blocks are
 * the next ceil(rows/B) * ceil(cols/B) table rows in row-major grid order. */
typedef struct shampoo_param {
  float* w;
  const void* g;
  float* m;
  float* v;
  int64_t rows, cols, ld;
  int64_t first_block;
} shampoo_param;

/* Inverse-root options.
 * method/scaling: shampoo_method / shampoo_scaling.
 * compute: arithmetic of the solver chain.  SHAMPOO_F32: float32 MFMA;
 *   SHAMPOO_F16: half-precision products with float32 accumulation and
 *   float32 iterates ([DASH] "A.3 Numerical Precision"): each product's
 *   result is rounded to float32, and a value that only later products read
 *   is kept as its half rounding (what those products would read from the
 *   float32 iterate), so each iterate buffer of the workspace holds a float32
 *   and a half part (1.5x the float32 buffers); SHAMPOO_F64: float64 MFMA
 *   (iterates float64).
 * iters: coupled-Newton iterations, or Newton-DB iterations of the first
 *   call; iters2: Newton-DB iterations of the second call (p = 4 only).
 * pi_vectors (1..32), pi_iters (>= 1): power-iteration start vectors and
 *   products before the Rayleigh quotients; pi_start_dev: device float32
 *   [pi_vectors, B] start vectors (required for SHAMPOO_SCALE_POWER).
 * cheb_degree (>= 0), cheb_points (0 = 4 (degree + 1)): Chebyshev fit;
 *   cheb_eps: the fit interval is [cheb_eps, 1 + cheb_eps]; cheb_eval:
 *   shampoo_cheb_eval, how the series is summed.
 * eps: added to the diagonal of each matrix's valid region before scaling
 *   ([DASH] "2. Preliminaries on Shampoo"; added once, see [DASH] "B.1").
 * tol: the Newton iterations (CN, NDB), any compute type; 0 runs
 *   exactly `iters` (and `iters2`) iterations (the fixed count of [3DS]
 *   "Hyperparameters", fix_iter).  tol > 0 stops early once every matrix is
 *   within tol over its valid region: coupled Newton ||M - I||_F <= tol
 *   (every eigenvalue of M = X^p A_s within tol of 1), checked after each M
 *   update, X then taking its last update; Newton-DB ||ZY - I||_F <= tol in
 *   each call, checked after each T product, the call then ending with that
 *   iteration as its last (the chain is planned again with that count).
 *   Matrices that cannot converge are not waited for: an iterate turned
 *   NaN, or a scale that is zero or not finite (the final pass flags them).
 *   Rounding keeps ||M - I||_F near u sqrt(v) .. u v (u the unit roundoff,
 *   v the valid size), so tol must lie above that: 1e-4 suits float32 up
 *   to v = 1024.  F16 chains check the half copy of the iterate, the one
 *   the next products read; it settles near 2.6e-2 at v = 1024, where
 *   0.1 suits.  A check first reads the diagonals: |tr M - v| / sqrt(v), a
 *   lower bound of ||M - I||_F, above tol settles "not converged" without
 *   the Frobenius pass (the same decision).  Each check synchronises the
 *   stream with the host (one flag read, two when the diagonals pass), so
 *   work queued after it on other streams is not enqueued until the solve
 *   ends; `iters` stays the upper bound; the float64 recomputation of
 *   shampoo_step's fallback runs the full count.
 * residual_out_dev, residual_bound: the solver residual ||X^p A_s - I||_F /
 *   sqrt(v) of each matrix's chain result X (before unscaling; equal to
 *   ||out^p (in + eps I) - I||_F / sqrt(v)), v the valid size, from p - 1
 *   products or log2(p) squarings (symmetric products when X is exactly
 *   symmetric, every method but NDB) and a full product with the
 *   regenerated A_s, all in the
 *   chain's iterate precision (float32 for F32 and F16 chains, float64 for
 *   F64), and one Frobenius pass.  It is computed when residual_out_dev
 *   (device float32 [n]) is non-NULL or residual_bound > 0; residual_bound > 0
 *   sets SHAMPOO_FLAG_RESIDUAL on matrices whose residual exceeds it or is
 *   not finite (matrices with a zero scale are left to ZERO_SCALE).  The
 *   products need up to three iterate buffers beside the result, which the
 *   workspace query includes.  For Chebyshev the residual also measures the
 *   fit's own error (the polynomial approximates (A_s + cheb_eps I)^(-1/p)). */
typedef struct shampoo_root_opts {
  int32_t method;
  int32_t scaling;
  int32_t compute;
  int32_t iters;
  int32_t iters2;
  int32_t pi_vectors;
  int32_t pi_iters;
  int32_t cheb_degree;
  int32_t cheb_points;
  int32_t cheb_eval;
  double eps;
  double cheb_eps;
  const float* pi_start_dev;
  double tol;
  float* residual_out_dev;
  double residual_bound;
} shampoo_root_opts;

/* Arguments of one shampoo_step over one stack (one block size B). */
typedef struct shampoo_step_args {
  int32_t nparams;
  int32_t B;
  int64_t nblk;
  const shampoo_param* params_dev;  /* device [nparams] */
  const shampoo_block* table_dev;   /* device [nblk], as planned for B */
  shampoo_dtype g_dt;               /* SHAMPOO_F32 or SHAMPOO_BF16 */
  int32_t p;                        /* root order, 4 for Shampoo */
  shampoo_dtype stats_dt;           /* SHAMPOO_F32 or SHAMPOO_F64: element type of LR and roots */
  int32_t fallback;                 /* shampoo_fallback, for factors whose new root is not finite */
  void* LR;                         /* device [2 nblk, B, B] stats_dt: L stack then R stack (state) */
  void* roots;                      /* device [2 nblk, B, B] stats_dt: inverse roots (state) */
  double beta2;                     /* statistics EMA; 1 = plain sum */
  int32_t recompute_roots;          /* 0: reuse `roots` from an earlier step */
  shampoo_root_opts root;
  int32_t graft;                    /* shampoo_graft */
  int32_t graft_blockwise;          /* 0: norms per parameter (layer-wise); 1: per block */
  float lr;
  float momentum;                   /* MOMENTUM */
  float beta1, graft_beta2, graft_eps; /* ADAM */
  int32_t t;                        /* 1-based step count (Adam bias correction) */
  int32_t* flags_dev;               /* device int32 [2 nblk] or NULL */
  float* dstack;                    /* device f32 [nblk, B, B] or NULL: receives D (ungrafted) on each
                                       block's valid region (the padding too, unless table_host marks
                                       ragged blocks) */
  void* ws;
  size_t ws_bytes;
  const shampoo_block* table_host;  /* host copy of table_dev, or NULL.  When given, each factor's
                                       root is computed in a stack of side roundup64(valid size)
                                       (L: rows, R: cols) rather than B, grouped by that side, and
                                       written back zero-padded to B: the padded work of narrow
                                       blocks disappears ([DASH] "4. Blocking Strategy" groups
                                       blocks by shape).  The workspace then depends on it.
                                       The groups are planned on the host from this copy; the
                                       device orders the factors from table_dev, so the two
                                       must hold the same rows.  Ignored for B > 8192.  When some
                                       block is narrower than B, the statistics and preconditioning
                                       products also skip each block's padding ([DASH] "4. Blocking
                                       Strategy": no padded work): L and R are computed on the valid
                                       rows x rows and cols x cols regions (their padding stays as it
                                       was, zero from the caller's initialisation), and D on the valid
                                       rows x cols region, in 64 x 64 tiles. */
  shampoo_dtype precond_dt;         /* SHAMPOO_F32 (0, the default): D = Lr G Rr in the roots'
                                       precision.  SHAMPOO_BF16 (bfloat16 gradients and float32
                                       statistics only): both roots and E = G Rr are rounded to
                                       bfloat16 and the two products run on bfloat16 matrix cores
                                       with float32 accumulation; D stays float32.  The half-precision
                                       products of [DASH] "A.3 Numerical Precision" (float32
                                       accumulation) carried over to the preconditioning products:
                                       the search direction then carries bfloat16 rounding (about
                                       3e-3 relative on the decoder set after step 1). */
} shampoo_step_args;

/* Version string of the library. */
const char* shampoo_version(void);

/* Thread-local message of the calling thread's last non-OK status. */
const char* shampoo_last_error(void);

/* Block plan (host only, no device work).  [DASH] "4. Blocking Strategy";
 * [3DS] "Hyperparameters".  shapes2d: host int64 [nparams, 2] (rows, cols)
 * of the 2-D views; block_sizes: host int32 [nparams] (0 = one block of side
 * max(rows, cols)).  Blocks are listed parameter by parameter, row-major over
 * each block grid.  *nblk is the capacity of `out` on entry and the number of
 * blocks on return; with out == NULL only the count is returned.
 * Errors: E_INVALID for negative sizes or block sizes, or if the count
 * exceeds the capacity (then *nblk holds the count needed). */
shampoo_status shampoo_plan_blocks(const int64_t* shapes2d, const int32_t* block_sizes,
                                   int32_t nparams, shampoo_block* out, int64_t* nblk);

/* Pack parameter-layout matrices into a zero-padded block stack.  [DASH]
 * "4. Blocking Strategy" (stacking blocks into 3-D tensors).
 * mats_dev: device [nparams] shampoo_matrix indexed by table.param;
 * table_dev: device [nblk]; stack: device [nblk, B, B] in dtype dt;
 * stack_t: NULL, or device [nblk, B, B] receiving each block transposed.
 * dt: SHAMPOO_F32, SHAMPOO_BF16, SHAMPOO_F16 or SHAMPOO_F64.
 * Bit-exact copy; the padding is written as +0.  Errors: E_INVALID for null
 * pointers, nblk < 0 or B < 1. */
shampoo_status shampoo_pack_blocks(const shampoo_matrix* mats_dev, int32_t nparams,
                                   const shampoo_block* table_dev, int64_t nblk, int32_t B,
                                   shampoo_dtype dt, void* stack, void* stack_t,
                                   hipStream_t stream);

/* Inverse of shampoo_pack_blocks for float32 stacks: writes each block's
 * valid region into the parameter-layout matrices mats_dev (float32). */
shampoo_status shampoo_unpack_blocks(const float* stack, const shampoo_block* table_dev,
                                     int64_t nblk, int32_t B, const shampoo_matrix* mats_dev,
                                     int32_t nparams, hipStream_t stream);

/* Statistics.  [DASH] "2. Preliminaries on Shampoo"; [NOTES] "The geometric
 * mean of the two bounds is the Kronecker bound" (sums over steps):
 *   L_b <- beta2 L_b + (1 - beta2) G_b G_b^T,  R_b <- beta2 R_b + (1 - beta2) G_b^T G_b,
 * and L_b += G_b G_b^T, R_b += G_b^T G_b when beta2 == 1.
 * gstack, gstack_t: device [nblk, B, B] block stack and its per-block
 * transpose (as written by shampoo_pack_blocks) in g_dt (F32 or BF16);
 * LR: device [2 nblk, B, B] in stats_dt (F32: float32 matrix cores; F64:
 * float64 matrix cores, the gradient widened exactly), L_0..L_(nblk-1) then
 * R_0..R_(nblk-1), updated in place; kept exactly symmetric.  B must be a
 * multiple of 64. */
shampoo_status shampoo_update_stats(const void* gstack, const void* gstack_t, shampoo_dtype g_dt,
                                    int64_t nblk, int32_t B, void* LR, shampoo_dtype stats_dt,
                                    double beta2, hipStream_t stream);

/* Workspace bytes for shampoo_inverse_root with these arguments (0 for
 * n = 0); the call's limits apply (E_UNSUPPORTED for n > 65535). */
shampoo_status shampoo_inverse_root_workspace(int64_t n, int32_t B, int32_t p,
                                              const shampoo_root_opts* opts, size_t* bytes);

/* Batched inverse p-th roots of symmetric positive definite matrices.
 * in: device [n, B, B] in io_dt (F32 or F64), symmetric; out: device
 * [n, B, B] in io_dt, receives (A + eps I)^(-1/p) on each valid region and 0
 * elsewhere (in may equal out).  valid_dev: device int32 [n] valid sizes
 * (matrix b uses its leading valid[b] x valid[b] region; the rest is
 * treated as padding) or NULL for all B.  scale_out_dev: device f32 [n]
 * receiving the scale s of each matrix, or NULL.  flags_dev: device int32 [n]
 * flag bits (OR-ed), or NULL.  Steps ([DASH] "3. Inverse Root Methods",
 * "A.2"): A = in + eps I; s = ||A||_F, or (power) s = ||A||_F times the
 * largest Rayleigh quotient of A/||A||_F; A_s = A/s with the padding set to
 * the identity; X = solver(A_s); out = X s^(-1/p).
 * Supported: CN with p in {1, 2, 4, 8}; NDB with p in {2, 4}; Chebyshev with
 * p >= 1; compute F32, F16 or F64; power scaling with B <= 1024.  B must be a
 * multiple of 64; n at most 65535 (n = 0 returns at once).  Errors:
 * E_INVALID, E_UNSUPPORTED, E_WORKSPACE, E_HIP. */
shampoo_status shampoo_inverse_root(const void* in, void* out, shampoo_dtype io_dt, int64_t n,
                                    int32_t B, int32_t p, const shampoo_root_opts* opts,
                                    const int32_t* valid_dev, float* scale_out_dev,
                                    int32_t* flags_dev, void* ws, size_t ws_bytes,
                                    hipStream_t stream);

/* shampoo_inverse_root without a workspace argument, for callers that cannot
 * allocate device memory (code under stream capture into a graph, tight
 * serving loops, harnesses that forbid allocation).  Same arguments, steps,
 * kernels, results and errors as shampoo_inverse_root; the workspace is a
 * 64 MiB device array inside the library (one copy per device, allocated
 * when the library's device code is loaded on that device and held until
 * the process ends).  Calls needing more scratch than that (the
 * shampoo_inverse_root_workspace size) fail with E_WORKSPACE before any
 * launch; e.g. 64 matrices 128 x 128 by coupled Newton or Newton-DB need 20
 * MiB in float32 and 40 MiB in float64.  Nothing in the scratch needs to
 * start at zero.
 * Every call on one device shares that device's array, which keeps the last
 * call's contents: calls that overlap on one device (on different streams,
 * or from different threads, without ordering between them) race on it.
 * Calls no hipMalloc, hipFree or allocating library routine. */
shampoo_status shampoo_inverse_root_noalloc(const void* in, void* out, shampoo_dtype io_dt, int64_t n,
                                            int32_t B, int32_t p, const shampoo_root_opts* opts,
                                            const int32_t* valid_dev, float* scale_out_dev,
                                            int32_t* flags_dev, hipStream_t stream);

/* Workspace bytes for shampoo_precondition: nblk * B * B * sizeof(roots_dt);
 * E_UNSUPPORTED for a B that is not a multiple of 64 or a batch the call
 * refuses (more than 65535 blocks). */
shampoo_status shampoo_precondition_workspace(int64_t nblk, int32_t B, shampoo_dtype roots_dt,
                                              size_t* bytes);

/* Search direction per block.  [NOTES] "AdaGrad's regret argument goes
 * through with the Kronecker preconditioner": S^(-1) vec(G) with
 * S = L^(1/4) (x) R^(1/4), i.e. D_b = Lr_b G_b Rr_b.
 * roots: device [2 nblk, B, B] in roots_dt (F32 or F64; inverse roots of L
 * then of R, symmetric; the products run in that precision); gstack: device
 * [nblk, B, B] in g_dt (F32 or BF16); dstack: device f32 [nblk, B, B].
 * B must be a multiple of 64. */
shampoo_status shampoo_precondition(const void* roots, shampoo_dtype roots_dt, const void* gstack,
                                    shampoo_dtype g_dt, int64_t nblk, int32_t B, float* dstack,
                                    void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes for shampoo_step with these arguments (ws fields ignored). */
shampoo_status shampoo_step_workspace(const shampoo_step_args* args, size_t* bytes);

/* One full preconditioner step over one stack: pack, statistics, inverse
 * roots (unless recompute_roots == 0), preconditioning, grafting and the
 * weight update ([3DS] "Hyperparameters"; [DASH] "2. Preliminaries on
 * Shampoo"; [NOTES] "Grafting corrects Shampoo's eigenvalues").  Per
 * parameter (or per block with graft_blockwise): D_g = (||Delta||_F /
 * ||D||_F) D (0 when D = 0) with Delta = G (SGD, MOMENTUM) or the
 * bias-corrected Adam direction; SGD/ADAM: W -= lr D_g; MOMENTUM:
 * M = momentum M + D_g, W -= lr M; NONE: W -= lr D.  Norms are reduced in a
 * fixed order, so two identical calls give identical bits.
 * Roots that come out non-finite or with a zero scale are handled by
 * args->fallback (shampoo_fallback); the flags of the step's factors are
 * OR-ed into flags_dev (NONFINITE and ZERO_SCALE describe the first attempt,
 * RECOMPUTED_F64 and KEPT_PREVIOUS what the fallback did).  FALLBACK_F64
 * waits for the stream once (to count the flagged factors) and needs the
 * larger workspace that shampoo_step_workspace reports for it. */
shampoo_status shampoo_step(const shampoo_step_args* args, hipStream_t stream);

/* Synchronises `stream`, then returns E_NONFINITE if any of the n flags is
 * set, else OK. */
shampoo_status shampoo_check_flags(const int32_t* flags_dev, int64_t n, hipStream_t stream);

/* Optional timing of the batched products (for benchmarks).  While enabled
 * with capacity > 0, shampoo_inverse_root records a HIP event pair on its
 * stream around each of its batched-product launches, up to `capacity`
 * launches; capacity 0 disables and releases the events (host objects, no
 * device memory).  Process-wide state on the current device; not thread-safe.
 * shampoo_timing_read waits for the recorded events and writes the duration
 * in milliseconds of each recorded launch (at most `capacity` of them) to
 * `ms`, their number to *count, and restarts the recording. */
shampoo_status shampoo_timing_enable(int32_t capacity);
shampoo_status shampoo_timing_read(float* ms, int32_t capacity, int32_t* count);

/* Matrix-core throughput microbenchmark (for the roofline denominators).
 * Launches, on `stream`, a kernel whose waves (8 per SIMD on every CU) each
 * issue a long chain of independent 16x16 MFMAs from registers (no memory
 * traffic), times it with a HIP event pair and waits for it.
 *   dt    F32 (v_mfma_f32_16x16x4_f32), F64 (v_mfma_f64_16x16x4_f64),
 *         F16 (v_mfma_f32_16x16x32_f16) or BF16 (v_mfma_f32_16x16x32_bf16);
 *   sink_dev  device buffer of at least 64 bytes (written only under a
 *         condition that never holds; it keeps the results live);
 *   tflops    out: dense TFLOP/s achieved.
 * Errors: E_UNSUPPORTED for another dtype, E_INVALID for null pointers,
 * E_HIP for launch/event failures. */
shampoo_status shampoo_mfma_peak(shampoo_dtype dt, void* sink_dev, hipStream_t stream, double* tflops);

#ifdef __cplusplus
}
#endif

#endif /* SHAMPOO_H */
