/*
 * muon_adamw.h - C ABI of the MI355X (gfx950) hybrid Muon + AdamW optimizer step.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensor pointers are DEVICE pointers owned by the caller; descriptor arrays
 *   (items, params, coefficient tables, descs) are HOST pointers read during
 *   the call only.  The library never allocates tensor memory.  Scratch space
 *   is the caller's workspace (`ws`, `ws_bytes`, device, 256-byte aligned);
 *   each entry point that needs one has a *_workspace_bytes() query.
 * - Every computing call enqueues on `stream` (a hipStream_t; NULL = the
 *   default stream) and returns without synchronising.
 * - Everything is validated before anything is enqueued: a non-MO_OK status
 *   means no tensor was modified.  mo_last_error() then holds a message
 *   (thread-local).  No C++ exception crosses this boundary.
 * - Storage dtypes: MO_F32 (IEEE binary32) and MO_BF16 (upper half of a
 *   binary32; conversions round to nearest, ties to even).  Optimizer states
 *   (momentum, exp_avg, exp_avg_sq, NorMuon v) are always fp32.
 * - Matrices are row-major; `ld` is the row stride in elements.  Vector loads
 *   need 16-byte aligned base pointers (MO_EALIGN otherwise).
 * - Calls that share a workspace must be ordered on one stream.
 */
#ifndef MUON_ADAMW_H
#define MUON_ADAMW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mo_status {
  MO_OK = 0,
  MO_EINVAL = 1,      /* bad argument (NULL pointer, negative size, bad hyper-parameter) */
  MO_ESHAPE = 2,      /* view / split does not match the stored shape */
  MO_ECONFLICT = 3,   /* two different views registered for one parameter identity */
  MO_EEMPTY = 4,      /* no trainable parameter */
  MO_EDTYPE = 5,      /* unsupported dtype */
  MO_EWORKSPACE = 6,  /* workspace missing or too small */
  MO_EHIP = 7,        /* a HIP runtime call failed */
  MO_EALIGN = 8       /* pointer not 16-byte aligned */
} mo_status;

typedef enum mo_dtype { MO_F32 = 0, MO_BF16 = 1 } mo_dtype;

/* Arithmetic of the Newton-Schulz products: bf16 operands with fp32
 * accumulation (MFMA bf16), or fp32 operands with fp32 accumulation. */
typedef enum mo_ns_precision { MO_NS_BF16 = 0, MO_NS_F32 = 1 } mo_ns_precision;

typedef enum mo_role { MO_ROLE_MATRIX = 0, MO_ROLE_EMBEDDING = 1, MO_ROLE_HEAD = 2,
                       MO_ROLE_NORM = 3 } mo_role;

typedef enum mo_algorithm { MO_ALG_SKIP = -1, MO_ALG_ADAMW = 0, MO_ALG_MUON = 1 } mo_algorithm;

#define MO_MAX_NDIM 8
#define MO_MAX_SPLIT 8
#define MO_NS_MAX_STEPS 64
#define MO_MAX_GROUPS 256

const char* mo_status_str(mo_status s);
/* Message of the last failing call on this thread ("" if none). */
const char* mo_last_error(void);
/* Library version string. */
const char* mo_version(void);
/* sizeof() of the ABI structs, for binding self-checks: 0 mo_momentum_item,
 * 1 mo_ns_item, 2 mo_adamw_item, 3 mo_param_desc, 4 mo_route_out, 5 mo_param,
 * 6 mo_hparams, 7 mo_step_args, 8 mo_lr_schedule, 9 mo_ns_options,
 * 10 mo_plan_options, 11 mo_group, 12 mo_spectral_item; 0 for any other index. */
size_t mo_abi_struct_size(int32_t which);

/* ------------------------------------------------------------------------
 * muon_momentum - Muon momentum buffer and Nesterov direction.
 *
 * Per item, elementwise:  B <- mu * B + G;  D <- G + mu * B (nesterov != 0,
 * using the updated B) or D <- B (nesterov == 0).
 * Source: OMN "Dual-Manifold Optimization" page, Muon-path paragraph (buffer
 * accumulating gradients at 0.95, Nesterov-style direction adding the scaled
 * buffer back to the gradient, zeros-initialised buffer); NorMuon paper,
 * section 2.2, eq. (1).
 *   grad      device, `grad_dtype`, numel elements, read only.  NULL = no
 *             gradient this step: the item is skipped (buffer untouched).
 *   momentum  device fp32, numel elements, updated in place.
 *   dir       device, `dir_dtype`, numel elements, written.  May be NULL
 *             (only the buffer is updated).
 * Workspace: muon_momentum_workspace_bytes(n) bytes (descriptor table).
 * ------------------------------------------------------------------------ */
typedef struct mo_momentum_item {
  const void* grad;
  float* momentum;
  void* dir;
  int64_t numel;
  int32_t grad_dtype;
  int32_t dir_dtype;
} mo_momentum_item;

size_t muon_momentum_workspace_bytes(int32_t n);
mo_status muon_momentum(const mo_momentum_item* items, int32_t n, float mu, int32_t nesterov,
                        void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Newton-Schulz options (every field has a default; see mo_ns_options_default).
 *
 *   gram_space         1: run slices in Gram space where the library's rule
 *                      admits it (the default); 0: the plain iteration
 *                      everywhere.  Gram space: the iteration X <- a X + b A X
 *                      (+ c A^2 X), A = X X^T, keeps every iterate of the form
 *                      Q X0 with Q a polynomial in A0 = X0 X0^T, so the
 *                      iterations can run on s x s matrices (A_{k+1} =
 *                      P_k A_k P_k, Q_{k+1} = P_k Q_k) and X0 is multiplied
 *                      once, by Q_N.  Equal to the plain iteration up to
 *                      rounding.  Rule: bf16 path only, and the table's
 *                      small-singular-value gain prod_k a_k^2 at most 1024
 *                      (Gram space carries A, whose small eigenvalues are the
 *                      squares of X's, so its bf16 rounding grows with that
 *                      gain where the plain iteration's grows with its square
 *                      root: the cubic set qualifies up to 8 iterations, the
 *                      quintic up to 5); then slices with a short side of 64
 *                      to 128 (slice-resident kernel) and GEMM-path slices
 *                      whose long side is at least 1.25 times the short side
 *                      (on a square slice it saves no work).
 *   big_tile_min_work  GEMM-path slices with a short side of at least 512
 *                      use 256 x 256 tiles when the batch holds at least this
 *                      many such upper-triangle Gram tiles (-1: 512, two per
 *                      CU; 0: always); otherwise 128 x 128 tiles.
 *   few_tile_max       bf16 launches of fewer 128 x 128 tiles than this split
 *                      each tile over 8 waves (-1: 512; 0: never).
 * The choices change launch shapes and rounding order only; every choice
 * meets the same tolerances.
 * ------------------------------------------------------------------------ */
typedef struct mo_ns_options {
  int32_t gram_space;
  int32_t big_tile_min_work;
  int32_t few_tile_max;
  int32_t reserved;
} mo_ns_options;

/* Fills *o with the defaults (gram_space 1, big_tile_min_work -1,
 * few_tile_max -1).  No-op for NULL. */
void mo_ns_options_default(mo_ns_options* o);

/* ------------------------------------------------------------------------
 * ns_orthogonalize_batched - Newton-Schulz orthogonalisation of many
 * independent matrices.
 *
 * Per item (one independent matrix D of rows x cols, e.g. one slice of a
 * registered view):
 *   alpha = max(max|D|, 1e-7);  X = D / alpha;  X <- X / (||X||_F + 1e-7);
 *   if rows > cols: X <- X^T   (the Gram is formed on the short side);
 *   for k in 0..steps-1, (a, b, c) = coeffs[k]:
 *       A = X X^T;  X <- a X + (b A + c A A) X;
 *   orientation restored; out = X (in out_dtype).
 * Source: OMN page, Muon-path paragraphs (fp32 direction, max-abs rescale
 * clamped at 1e-7, Frobenius normalisation with epsilon, transpose when tall,
 * five polynomial iterations, orientation restored); NorMuon paper section
 * 2.2 eq. (5) for the (a, b, c) iteration; MuonClip page, "Newton-Schulz
 * Orthogonalization", for the cubic set (1.5, -0.5, 0).
 *   items[i].in   device, in_dtype, rows x cols with row stride ld_in.
 *   items[i].out  device, out_dtype, rows x cols with row stride ld_out; may
 *                 alias `in` (the input is fully consumed first).
 *   coeffs        host, [steps][3] floats (a, b, c) per iteration,
 *                 1 <= steps <= MO_NS_MAX_STEPS, all finite.
 *   precision     mo_ns_precision.
 *   opts          host, nullable (NULL = mo_ns_options_default).
 * Workspace: ns_workspace_bytes(items, n, coeffs, steps, precision, opts);
 * with coeffs == NULL the query returns the most any table can need.  All
 * sizes must be >= 1 and cols, rows <= 65536.
 * ------------------------------------------------------------------------ */
typedef struct mo_ns_item {
  const void* in;
  void* out;
  int64_t rows;
  int64_t cols;
  int64_t ld_in;
  int64_t ld_out;
  int32_t in_dtype;
  int32_t out_dtype;
} mo_ns_item;

size_t ns_workspace_bytes(const mo_ns_item* items, int32_t n, const float* coeffs, int32_t steps,
                          int32_t precision, const mo_ns_options* opts);
mo_status ns_orthogonalize_batched(const mo_ns_item* items, int32_t n, const float* coeffs,
                                   int32_t steps, int32_t precision, const mo_ns_options* opts,
                                   void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * muon_spectral_estimate - power-iteration estimate of each matrix's largest
 * singular value, as the spectral-cap guard on the Muon buffer computes it.
 *
 * OMN "Dual-Manifold Optimization" page, Muon-path paragraph: an optional
 * spectral-cap guard with power-iteration estimation, inactive by default in
 * the recipe.  The page prints no formula; this library's reading:
 *   v_0 = ones(cols) / sqrt(cols);
 *   v_{k+1} = B^T B v_k / ||B^T B v_k||   for k < iters (stops at 0 if it vanishes);
 *   sigma = ||B v_iters||.
 * In the grouped step (hparams spectral_cap > 0) each independent matrix of
 * the buffer, after B <- mu B + G, is rescaled to (cap / sigma) B when sigma
 * > cap, and the Nesterov direction is formed from the rescaled buffer.
 *   items[i].b      device fp32, rows x cols, row stride ld (>= cols).
 *   sigma_out       device fp64, n entries, written.
 *   iters           0..64.
 * Sums run in fp64.  Workspace: muon_spectral_workspace_bytes(items, n).
 * ------------------------------------------------------------------------ */
typedef struct mo_spectral_item {
  const float* b;
  int64_t rows;
  int64_t cols;
  int64_t ld;
} mo_spectral_item;

size_t muon_spectral_workspace_bytes(const mo_spectral_item* items, int32_t n);
mo_status muon_spectral_estimate(const mo_spectral_item* items, int32_t n, int32_t iters,
                                 double* sigma_out, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * normuon_rownorm - NorMuon per-row second-moment normalisation, in place.
 *
 * For each row i of O (rows x cols, stride ld):
 *   ms_i = (1/cols) sum_j O_ij^2;  v_i <- beta2 v_i + (1 - beta2) ms_i;
 *   O_ij <- O_ij / (sqrt(v_i) + eps).
 * Source: NorMuon paper, section 3.1 (per-neuron second moment v in R^m,
 * mean square of each row of O_t, EMA with decay beta2, row-wise
 * normalisation after orthogonalisation).  v_0 = 0 is the caller's zeroed
 * buffer; no bias correction.
 *   O  device, dtype, updated in place.   v  device fp32 [rows], in-out.
 * ------------------------------------------------------------------------ */
mo_status normuon_rownorm(void* O, int32_t dtype, int64_t rows, int64_t cols, int64_t ld,
                          float* v, float beta2, float eps, void* stream);

/* ------------------------------------------------------------------------
 * muon_update - scaled Muon weight update.
 *
 *   W <- W (1 - lr wd) - lr * scale * U      (rows x cols)
 * with scale normally sqrt(max(1, rows/cols)) of the independent matrix.
 * Source: NorMuon paper section 2.2 eq. (3); OMN page, rectangular-scaling
 * paragraph (sqrt(max(1, m/n)), m x n in out-by-in orientation); decoupled
 * weight decay is zero in the OMN recipe (weight-decay paragraph).
 *   W  device, w_dtype, stride ld_w, in place.   U  device, u_dtype, ld_u.
 * ------------------------------------------------------------------------ */
mo_status muon_update(void* W, int32_t w_dtype, const void* U, int32_t u_dtype, int64_t rows,
                      int64_t cols, int64_t ld_w, int64_t ld_u, float lr, float wd, float scale,
                      void* stream);

/* ------------------------------------------------------------------------
 * adamw_clip_step - AdamW over a set of parameters with one global-norm clip.
 *
 *   T = sqrt(sum over every item with a gradient of sum G^2)   (fp64)
 *   kappa = max_norm / T if max_norm > 0 and T > max_norm, else 1
 *   per element: g = kappa G;  m <- b1 m + (1-b1) g;  v <- b2 v + (1-b2) g^2;
 *   W <- W (1 - lr wd) - lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)
 * Source: OMN page, recipe paragraph (betas (0.90, 0.95), epsilon 1e-8,
 * clipping at 1.0 over AdamW parameters only, zero decay); Qwen3.8 optimizer
 * notes, Adam / AdamW background (bias-corrected moments, decoupled decay).
 *   items[i].param       device, dtype, numel, in place.
 *   items[i].grad        device, dtype, numel, read only; NULL = skipped
 *                        (not in T, param and moments untouched).
 *   items[i].exp_avg     device fp32 m;  items[i].exp_avg_sq  device fp32 v.
 *   items[i].step        t >= 1 of this update (caller increments).
 *   items[i].weight_decay  decoupled decay of the item's group.
 *   norm_out             device fp64 scalar receiving T (nullable).
 * Workspace: adamw_workspace_bytes(items, n).
 * ------------------------------------------------------------------------ */
typedef struct mo_adamw_item {
  void* param;
  const void* grad;
  float* exp_avg;
  float* exp_avg_sq;
  int64_t numel;
  int32_t dtype;
  int32_t step;
  float weight_decay;
  float reserved;
} mo_adamw_item;

size_t adamw_workspace_bytes(const mo_adamw_item* items, int32_t n);
mo_status adamw_clip_step(const mo_adamw_item* items, int32_t n, float lr, float beta1,
                          float beta2, float eps, float max_norm, double* norm_out, void* ws,
                          size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * adamw_clip_step_noalloc - adamw_clip_step without a workspace argument,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments (minus ws, ws_bytes), arithmetic, kernels and results as
 * adamw_clip_step.  The scratch the step needs (segment table, fp64 partial
 * sums, the norm and the clip factor) is a fixed 1 MiB array in device
 * memory that the library holds on every GPU it runs on until the process
 * ends; the call itself allocates nothing (no hipMalloc, no pinned staging,
 * no timing events) and writes everything it reads from that array, so no
 * clearing is needed between calls.  Limits: at most 64 items with a
 * gradient and about 1.07e9 elements in all (ceil(numel / 2048) blocks per
 * item, one partial per 4 blocks, 130,016 partials); beyond them MO_EWORKSPACE
 * with the numbers in mo_last_error(), before anything is enqueued.  Calls
 * that overlap on one GPU (different streams, unordered) share the array and
 * race; order them on one stream.
 * ------------------------------------------------------------------------ */
mo_status adamw_clip_step_noalloc(const mo_adamw_item* items, int32_t n, float lr, float beta1,
                                  float beta2, float eps, float max_norm, double* norm_out,
                                  void* stream);

/* ------------------------------------------------------------------------
 * Host-only: routing predicate and view expansion (no GPU needed).
 *
 * mo_route follows the kimi-k3 "build_parameter_groups" page ("Exclusion and
 * decay rules"; "Classification happens once per original parameter
 * identity"), with the OMN page's routing paragraph for the embedding:
 *   requires_grad == 0, or an identity already seen    -> MO_ALG_SKIP
 *   ndim < 2 or no_decay                               -> AdamW, decay 0
 *   ndim == 2 and role not embedding/head              -> Muon (view, split), decay 1
 *   otherwise                                          -> AdamW, decay 1
 * Groups are keyed by (algorithm, view, split, exclude_mask, decay) in order
 * of first appearance; out[i].group is the group index (-1 when skipped).
 * Views are validated ("Recording independent matrix geometry"): MO_ESHAPE
 * for a bad view or split, MO_ECONFLICT for two views on one identity,
 * MO_EEMPTY when nothing is trainable.
 *
 * exclude_mask follows the Qwen3.8 optimizer notes (section 4, fused
 * matrices): the gate/vector sub-blocks of a fused weight that do not suit
 * Muon are stepped by AdamW.  Bit j names split piece j, in every view matrix
 * alike (this library's encoding; the notes give none).  It needs split
 * sizes, bits below nsplit and at least one piece left to Muon, else
 * MO_ESHAPE; it is ignored when the weight does not route to Muon.
 * out[i].nslices counts the Muon slices only.
 * ------------------------------------------------------------------------ */
typedef struct mo_param_desc {
  const char* name;       /* informational, may be NULL */
  int64_t ident;          /* parameter identity: tied parameters share it */
  int32_t ndim;
  int32_t role;           /* mo_role */
  int64_t shape[MO_MAX_NDIM];
  int32_t no_decay;
  int32_t requires_grad;
  int32_t view_ndim;      /* 0 = no view */
  int32_t nsplit;         /* 0 = no split */
  int64_t view[MO_MAX_NDIM];
  int64_t split[MO_MAX_SPLIT];
  uint32_t exclude_mask;  /* bit j: split piece j of every view matrix goes to AdamW */
  int32_t reserved;
} mo_param_desc;

typedef struct mo_route_out {
  int32_t algorithm;      /* mo_algorithm */
  int32_t decay;          /* 0 / 1 */
  int32_t group;          /* group index or -1 */
  int32_t nslices;        /* independent matrices (Muon), 0 otherwise */
} mo_route_out;

mo_status mo_route(const mo_param_desc* descs, int32_t n, mo_route_out* out, int32_t* ngroups);

/* Independent sub-matrices of a stored (rows, cols) weight under a view
 * (view_ndim == 0: the whole weight).  Writes (row_offset, rows, cols)
 * triples to out_slices[3*k ...]; *nslices receives the count even when it
 * exceeds max_slices (then MO_EINVAL).  Source: kimi-k3 page, "The layout
 * declarations are literal" (leading view axes flatten row-major onto the
 * stored rows; split sizes cut each view matrix's rows). */
mo_status mo_expand_view(int64_t rows, int64_t cols, int32_t view_ndim, const int64_t* view,
                         int32_t nsplit, const int64_t* split, int64_t* out_slices,
                         int32_t max_slices, int32_t* nslices);

/* ------------------------------------------------------------------------
 * Host-only: token-clock learning-rate schedule.
 *
 * OMN "Dual-Manifold Optimization" page (opening summary; recipe paragraph on
 * separate peaks): warmup over the first 2B tokens, the peak held to 164B,
 * then a square-root cooldown to an absolute floor of 1e-5 at about 193B;
 * Muon and AdamW follow the same phases from their own peaks (0.01, 3e-4) on
 * one token clock.  The page prints no formula; this library's reading, with
 * tau the clock after the current accumulation window is counted:
 *   tau < W:           lr = peak * tau / W
 *   W <= tau < S:      lr = peak
 *   S <= tau < E:      lr = floor + (peak - floor) * (1 - sqrt((tau - S) / (E - S)))
 *   tau >= E:          lr = floor
 * mo_lr_at writes lr (fp64) for one peak.  MO_EINVAL for a NULL pointer,
 * tau < 0 or a NaN, unless 0 <= W <= S <= E and 0 <= floor <= peak.
 * ------------------------------------------------------------------------ */
typedef struct mo_lr_schedule {
  double peak;
  double warmup_tokens;      /* W, the page's value 2e9 */
  double stable_end_tokens;  /* S, 164e9 */
  double end_tokens;         /* E, about 193e9 */
  double floor;              /* 1e-5 */
} mo_lr_schedule;

mo_status mo_lr_at(const mo_lr_schedule* s, double tokens, double* lr);

/* ------------------------------------------------------------------------
 * Plan + grouped hybrid step over a parameter-group table.
 *
 * The group table follows the kimi-k3 "build_parameter_groups" page: each
 * group lists its params with their algorithm and weight decay (plus, for
 * Muon, the registered view and split sizes of each param).  A plan is made
 * either from such a table (mo_plan_create_groups: each group with its own
 * hyper-parameters) or from a flat parameter list that the library routes
 * itself (mo_plan_create: mo_route's groups, all on one hyper-parameter
 * block, decay where the routing key decays).  Plan creation is host-only;
 * the plan keeps the tensor pointers given here; its small device-side
 * descriptor tables are allocated and uploaded on the first mo_grouped_step
 * call and freed by mo_plan_destroy.
 *
 * mo_grouped_step runs one full hybrid step on `stream`:
 *   Muon params with a grad: momentum -> per-slice Newton-Schulz ->
 *     [NorMuon row normalisation] -> shape scale -> update, each with its
 *     group's lr, decay, momentum, coefficient table and NorMuon setting;
 *   AdamW params with a grad, over every AdamW group jointly: one global-norm
 *     clip (the OMN page's clip over the AdamW parameters), then AdamW with
 *     each group's lr, decay, betas and eps; the per-parameter step counter t
 *     is kept by the plan and incremented after each call.
 *   A call made under HIP stream capture (after one ordinary call on the same
 *     workspace, which uploads the tables) records the whole step; each
 *     replay of the graph runs it with the learning rates of the capture and
 *     AdamW's next step count (kept on the device); mo_plan_get_steps counts
 *     calls, not replays.
 *   Excluded pieces of a Muon param (exclude_mask) are AdamW parameters of
 *     their own: they join the clip norm and take the AdamW update (the
 *     group's adamw_lr, adamw_wd, betas, eps) with the param's step counter,
 *     reading and writing exp_avg / exp_avg_sq at the same element offsets as
 *     the param; Muon leaves their rows alone (momentum, direction and
 *     weight).  Such a param needs momentum, exp_avg and exp_avg_sq buffers of
 *     numel elements, and each excluded piece must start on a 16-byte
 *     boundary in all four (MO_EALIGN).
 * Sources: as for the individual entry points above; the ordering of NorMuon
 * before the shape scale is this library's reading (the pages do not order
 * them).
 * ------------------------------------------------------------------------ */
typedef struct mo_param {
  mo_param_desc desc;
  void* param;            /* device W (dtype) */
  const void* grad;       /* device G (dtype); NULL = no gradient (skipped) */
  int32_t dtype;          /* mo_dtype of W and G */
  int32_t reserved;
  float* momentum;        /* Muon: fp32, numel */
  float* normuon_v;       /* Muon with NorMuon: fp32, rows; else NULL */
  float* exp_avg;         /* AdamW: fp32, numel */
  float* exp_avg_sq;      /* AdamW: fp32, numel */
} mo_param;

typedef struct mo_hparams {
  float muon_lr;
  float muon_wd;
  float mu;
  int32_t nesterov;
  int32_t ns_steps;
  int32_t ns_precision;                       /* mo_ns_precision */
  float ns_coeffs[MO_NS_MAX_STEPS][3];        /* (a, b, c) per iteration */
  int32_t normuon;
  float normuon_beta2;
  float normuon_eps;
  float adamw_lr;
  float beta1;
  float beta2;
  float eps;
  float adamw_wd;
  float max_norm;
  float spectral_cap;     /* Muon: the spectral-cap guard's cap tau; 0 = off */
  int32_t spectral_iters; /* Muon: power iterations of the guard's estimate, 0..64 */
} mo_hparams;

/* One group of mo_plan_create_groups.  Muon groups read muon_lr, muon_wd,
 * mu, nesterov, ns_steps, ns_precision, ns_coeffs, the normuon fields and the
 * spectral-cap fields of `hp` (and the AdamW fields for excluded pieces);
 * AdamW groups read adamw_lr, adamw_wd, beta1, beta2, eps.  max_norm must be
 * the same in every group that has AdamW items (the clip norm is joint).  A
 * Muon group's params must be 2-D. */
typedef struct mo_group {
  int32_t algorithm;      /* MO_ALG_MUON or MO_ALG_ADAMW */
  int32_t nparams;
  const mo_param* params; /* host array of nparams */
  mo_hparams hp;
} mo_group;

/* Per-step arguments (NULL = none).  The learning rate of group g this step
 * is group_lr[g] when g < n_group_lr and group_lr[g] >= 0; else muon_lr
 * (Muon groups) or adamw_lr (AdamW groups, and the excluded pieces of Muon
 * groups) when >= 0; else the group's own hp value.  A scheduler drives the
 * rates through these fields (the OMN page steps both schedules from one
 * token clock; see mo_lr_at). */
typedef struct mo_step_args {
  float muon_lr;
  float adamw_lr;
  double* norm_out;       /* device fp64 scalar receiving the AdamW pre-clip norm T (nullable) */
  const float* group_lr;  /* host, n_group_lr entries (nullable) */
  int32_t n_group_lr;
  int32_t reserved;
} mo_step_args;

typedef struct mo_plan mo_plan;

/* Plan options: the Newton-Schulz options (mo_ns_options) of every Muon
 * slice of the plan, and keep_ns_output (0 / 1, as mo_plan_keep_ns_output).
 * NULL = mo_plan_options_default. */
typedef struct mo_plan_options {
  mo_ns_options ns;
  int32_t keep_ns_output;
  int32_t reserved;
} mo_plan_options;

void mo_plan_options_default(mo_plan_options* o);

/* Routes params (mo_route) and makes one group per routing key on `hp`.
 * Plan order of the params is the order given. */
mo_status mo_plan_create(const mo_param* params, int32_t n, const mo_hparams* hp,
                         const mo_plan_options* opts, mo_plan** out);
/* Plan over a caller's group table (at most MO_MAX_GROUPS groups).  Plan
 * order of the params is group by group, in table order; params with
 * requires_grad == 0 are skipped.  MO_ECONFLICT when a parameter identity
 * appears twice, MO_EEMPTY when nothing is trainable, MO_EINVAL for a bad
 * algorithm or hyper-parameter (or differing max_norm), MO_ESHAPE for a Muon
 * param that is not 2-D or a bad view. */
mo_status mo_plan_create_groups(const mo_group* groups, int32_t ngroups,
                                const mo_plan_options* opts, mo_plan** out);
void mo_plan_destroy(mo_plan* plan);
size_t mo_plan_workspace_bytes(const mo_plan* plan);
/* Number of params (plan order) and of groups (0 for NULL). */
int32_t mo_plan_num_params(const mo_plan* plan);
int32_t mo_plan_num_groups(const mo_plan* plan);
/* Host queries for tests: routing of each param and the slice table. */
mo_status mo_plan_route(const mo_plan* plan, mo_route_out* out, int32_t n);
int32_t mo_plan_num_slices(const mo_plan* plan);
/* (param index, row_offset, rows, cols) per slice. */
mo_status mo_plan_slices(const mo_plan* plan, int64_t* out4, int32_t max_slices);
/* AdamW step counters (per param, plan order; 0 for non-AdamW). */
mo_status mo_plan_get_steps(const mo_plan* plan, int32_t* steps, int32_t n);
mo_status mo_plan_set_steps(mo_plan* plan, const int32_t* steps, int32_t n);
mo_status mo_grouped_step(mo_plan* plan, const mo_step_args* args, void* ws, size_t ws_bytes,
                          void* stream);
/* Where the last grouped step left the Newton-Schulz output O of one slice
 * (the point the NorMuon paper section 2.2 calls O_t: after the iterations,
 * before NorMuon, the shape scale and the learning rate).  `slice` indexes
 * mo_plan_slices' table; `ws` is the workspace that step used.  On success
 * *o is a device pointer inside `ws` to a (rows, cols) row-major matrix in
 * the stored orientation with row stride *ld elements and element type
 * *dtype (MO_BF16 or MO_F32, the NS precision's storage).  The values stay
 * valid until the next step or ns call on that workspace.  Host only; no
 * device work.  MO_EINVAL for a bad index, a slice whose param had no
 * gradient, or a plan that has not run a step on `ws`. */
mo_status mo_plan_ns_output(const mo_plan* plan, int32_t slice, const void* ws, void** o,
                            int64_t* ld, int32_t* dtype);
/* Whether grouped steps keep O in the workspace.  By default (keep = 0) a
 * plan whose every active slice allows it applies the Muon update
 * W <- W (1 - lr wd) - lr scale O (the Muon post on OMN, update paragraph)
 * inside the last Newton-Schulz launch, from the same bf16-rounded O and
 * with the same arithmetic as the separate row pass, so the weights are
 * bit-identical either way; O is then not stored and mo_plan_ns_output
 * fails (MO_EINVAL) for that step.  Allowed when the NS precision is bf16,
 * NorMuon is off, and every slice has cols % 8 == 0 with 16-byte aligned
 * weight rows.  keep = 1 always runs the separate pass and keeps O.
 * Host only; takes effect from the next step.  MO_EINVAL for a NULL plan. */
mo_status mo_plan_keep_ns_output(mo_plan* plan, int32_t keep);
/* 1 if the next grouped step will apply the update inside the last
 * Newton-Schulz launch (see mo_plan_keep_ns_output), else 0 (also for NULL). */
int32_t mo_plan_fuses_update(const mo_plan* plan);
/* 1 if the plan runs any slice in Gram space, else 0 (also for NULL).  The
 * choice is made at plan creation by the rule of mo_ns_options (gram_space
 * option, bf16 path, coefficient-table gain, slice shape). */
int32_t mo_plan_gram_space(const mo_plan* plan);
/* How each slice of mo_plan_slices' table runs its Newton-Schulz iterations,
 * one int per slice: bit 0 set when in Gram space; bits 1-2 the kernel,
 * 0 = batched GEMM on 128 x 128 tiles, 1 = batched GEMM on 256 x 256 tiles,
 * 2 = slice-resident kernel; -1 for a slice whose param has no gradient.
 * Host only.  MO_EINVAL for a NULL pointer or n below the slice count. */
mo_status mo_plan_slice_algorithms(const mo_plan* plan, int32_t* out, int32_t n);

/* ------------------------------------------------------------------------
 * Kernel timing (diagnostics).  While enabled, every kernel launch of this
 * library is bracketed by two HIP events recorded on the launch's own
 * stream.  mo_timing_read waits for the recorded events of one kernel class
 * and returns their summed duration (ms) and launch count.  Enabling (on=1)
 * or disabling (on=0) clears earlier records.  While enabled, the grouped
 * step also keeps its AdamW kernels on the caller's stream instead of the
 * overlapping side stream, so that each duration is one kernel's alone.
 * Host thread safe.
 * ------------------------------------------------------------------------ */
typedef enum mo_kernel_class {
  MO_KC_MOMENTUM = 0, MO_KC_NS_STATS = 1, MO_KC_NS_SCALE = 2, MO_KC_NS_PREP = 3,
  MO_KC_NS_GEMM = 4, MO_KC_NS_FINAL = 5, MO_KC_ROWS = 6, MO_KC_ADAM_SUMSQ = 7,
  MO_KC_ADAM_NORM = 8, MO_KC_ADAM_APPLY = 9, MO_KC_NS_SMALL = 10, MO_KC_SPECTRAL = 11,
  MO_KC_COUNT = 12
} mo_kernel_class;

mo_status mo_timing_enable(int32_t on);
mo_status mo_timing_read(int32_t kclass, double* total_ms, int64_t* launches);

/* Plain device-to-device copy of `bytes` bytes by a kernel of this library
 * (k_diag_copy), enqueued on `stream`: a transfer of known size against which
 * hardware byte counters (FETCH_SIZE, WRITE_SIZE) are calibrated.  `src` and
 * `dst` are device pointers, 16-byte aligned, not overlapping; `bytes` is a
 * multiple of 16.  MO_EINVAL / MO_EALIGN otherwise.  Not part of the
 * optimizer step. */
mo_status mo_diag_copy(const void* src, void* dst, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MUON_ADAMW_H */
