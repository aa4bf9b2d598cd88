/*
 * amc.h - attention-matching KV compaction on one MI355X (gfx950).
 *
 * C ABI of libamc.  The method is "Fast KV Compaction via Attention
 * Matching" (arXiv 2602.16284) as described on the pages that summarise it:
 *
 *   - problem statement: compact a block of keys/values (K, V) of length T to
 *     t << T entries (C_k, beta, C_v) so that, on reference queries, the
 *     compacted block reproduces the local attention output and the attention
 *     mass (xinfinite.net article, section 1; youleyou.com rewrite, "the
 *     math", formulas 1 and 2; zhichai.net deep-dive, section 1.3);
 *   - C_k is a subset of the original keys, chosen by greedy orthogonal
 *     matching pursuit on the mass features Phi_ij = exp(q_i . k_j), with an
 *     NNLS refit of non-negative weights w after each pick and beta = log w
 *     (zhichai.net deep-dive, section 1.6; xinfinite.net article, section 2,
 *     step 2 and Fig. 1);
 *   - the batched variant takes the top k keys per iteration and refits only
 *     every R iterations (xinfinite.net article, section 3, Table 1);
 *   - C_v is the ordinary least squares fit of the attention output with C_k
 *     and beta fixed (xinfinite.net article, section 2, step 3);
 *   - beta is an additive per-token logit bias, one scalar per compacted
 *     token (zhichai.net deep-dive, sections 1.4 and 4.1);
 *   - heads with different budgets are packed flat, varlen, without padding
 *     (zhichai.net deep-dive, section 4.2).
 *
 * Conventions used by every entry point:
 *
 *   - Heads are independent problems.  Head h owns rows cu_q[h]..cu_q[h+1]-1
 *     of Q and rows cu_k[h]..cu_k[h+1]-1 of K, V (and of beta_in).  Q, K and V
 *     are row-major with head_dim contiguous elements per row.
 *   - The logit of query i and key j is  l_ij = scale * q_i . k_j + beta_in_j
 *     (scale defaults to 1/sqrt(head_dim), the model's own logit scale).
 *   - Outputs are packed by cu_budgets (amc_output_offsets): head h owns
 *     output rows cu_budgets[h]..cu_budgets[h+1]-1, in ascending original key
 *     index.  A compacted key whose NNLS weight is zero keeps its slot with
 *     beta = -inf and a zero value row.
 *   - All device buffers belong to the caller; the library never allocates
 *     device memory.  Host arrays are read only during the call.
 *   - Calls that take a stream enqueue work on it and return without
 *     synchronising.  Argument, shape and workspace errors are detected before
 *     anything is enqueued (no partial output).  A failed launch returns
 *     AMC_ERR_HIP.
 *   - Data-dependent numeric events are reported per head in head_status
 *     (device int32[H], optional) as AMC_HS_* bits; the call still completes.
 *   - The library holds no global mutable state apart from the per-device
 *     static workspace of amc_compact_noalloc; calls are reentrant.  Two calls
 *     that share a workspace (or, for amc_compact_noalloc, a GPU) must not
 *     overlap in time.
 */
#ifndef AMC_H
#define AMC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AMC_VERSION 1

typedef enum {
  AMC_OK = 0,
  AMC_ERR_INVALID_ARG = 1, /* a pointer, size, shape or option is invalid */
  AMC_ERR_UNSUPPORTED = 2, /* valid but outside what this build implements */
  AMC_ERR_WORKSPACE = 3,   /* workspace or trace buffer too small / misaligned */
  AMC_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} amc_status;

typedef enum { AMC_F32 = 0, AMC_BF16 = 1 } amc_dtype;

typedef enum {
  AMC_SEL_OMP = 0,         /* one key per iteration, NNLS refit after each */
  AMC_SEL_OMP_BATCHED = 1, /* top-k keys per iteration, refit every R iterations */
  AMC_SEL_HIGHEST = 2      /* AM-Highest: the t keys with the largest attention summed over the
                            * reference queries, sum_i Phi_ij / m_i (ties to the lower index),
                            * then one NNLS refit and the value fit (zhichai.net English summary,
                            * "Method Family and Trade-offs"; youleyou.com, the highest-attention
                            * keys method).  topk and refit_every must be 1; one cycle per head.
                            * The picks are recorded in ascending key order. */
} amc_select;

/* head_status bits */
#define AMC_HS_CHOL_JITTER 1u    /* the value fit needed a diagonal shift */
#define AMC_HS_NNLS_CAP 2u       /* an NNLS refit hit its iteration cap */
#define AMC_HS_NONFINITE 4u      /* Q, K, V or beta_in produced a non-finite logit or output */
#define AMC_HS_NNLS_SINGULAR 8u  /* a candidate key was linearly dependent on the active set */
#define AMC_HS_NNLS_QR 16u       /* the head's refits and value fit went through orthogonal
                                  * factorisations of Phi_S (amc_options.exact_refit) */

/* amc_options.flags */
#define AMC_FLAG_TRACE 1u /* fill the trace buffer (selection order, scores, weights) */

/* Kernel classes reported by the timer (amc_timer_read). */
typedef enum {
  AMC_K_INIT = 0,
  AMC_K_SHIFT = 1,   /* per-head logit maximum */
  AMC_K_PHI = 2,     /* mass features, target mass, attention output */
  AMC_K_SWEEP = 3,   /* r^T Phi correlation sweep with block top-k */
  AMC_K_MERGE = 4,   /* per-head top-k merge and selection update */
  AMC_K_PANEL = 5,   /* float64 columns of the selected keys */
  AMC_K_GRAM = 6,    /* Gram matrix and right-hand side update */
  AMC_K_NNLS = 7,    /* NNLS refit */
  AMC_K_RESID = 8,   /* residual r = m - Phi_S w */
  AMC_K_OLS_NORMAL = 9, /* normal equations of the value fit */
  AMC_K_OLS_SOLVE = 10, /* Cholesky solve of the value fit */
  AMC_K_PACK = 11,   /* sorted, packed outputs */
  AMC_K_SWEEP_EXACT = 12, /* float32 sweep of the heads whose candidate band overflowed */
  AMC_K_RESCORE = 13, /* float64 scores and columns of the band's candidates */
  AMC_K_PRUNE = 14,   /* per-cycle bound that drops keys from the bounded sweep */
  AMC_K_DIGITS = 15,  /* bf16 rows in exact base-256 digit form for the int8 logits */
  AMC_K_PHI_F64 = 16, /* float64-MFMA mass features of the heads off the digit grid */
  AMC_NUM_KERNEL_CLASSES = 17
} amc_kernel_class;

typedef struct {
  int32_t num_heads;      /* H >= 1 */
  int32_t head_dim;       /* d in {64, 128}; else AMC_ERR_UNSUPPORTED */
  const int64_t *cu_q;    /* HOST int64[H+1], cu_q[0] = 0, strictly increasing */
  const int64_t *cu_k;    /* HOST int64[H+1], cu_k[0] = 0, strictly increasing */
  const int64_t *budgets; /* HOST int64[H], 1 <= budgets[h] <= min(T_h, 16384) (else
                           * AMC_ERR_UNSUPPORTED); budgets above 176 keep the NNLS
                           * state and above 192 the value-fit factor in the workspace */
  amc_dtype in_dtype;     /* storage type of Q, K, V (C_k is written in it too) */
  float scale;            /* logit scale; 0 means 1/sqrt(head_dim) */
} amc_problem;

typedef struct {
  amc_select select;
  int32_t topk;           /* k: keys taken per iteration (1 for AMC_SEL_OMP) */
  int32_t refit_every;    /* R: refit after every R-th iteration (1 for AMC_SEL_OMP) */
  int32_t nnls_max_iters; /* active-set iteration cap per refit (0 = 3 * budget + 30) */
  int32_t nnls_polish;    /* refinement refits after the last key (default 1) */
  double nnls_tol;        /* KKT entering tolerance of the Gram solver, relative to max |b| in
                           * unit-diagonal form (0 = automatic: 10 eps t in the Gram-form
                           * refits of the selection; eps / 2, any gradient the float64 data
                           * resolve, in the polish refits after the last key of budgets up
                           * to 2048, in every refit that warm-starts the exact refit, and in
                           * amc_nnls) */
  uint64_t phi_budget_bytes; /* Phi is stored when sum_h n_h ceil8(T_h) * 4 <= this, as two
                              * 16-bit planes (the high and low halves of its float32
                              * values): a sweep reads the high plane, bounds every score,
                              * and rescores the keys whose bounds reach the top k R + 1 in
                              * float64 (when more than 128 do, that head's sweep reads
                              * both planes).  Else every sweep recomputes its Phi tiles
                              * from Q and K.  The picks are the same either way. */
  amc_dtype cv_dtype;     /* C_v output type (default AMC_F32) */
  int32_t head_groups;    /* amc_compact splits the heads into this many groups of
                           * consecutive heads (at most H are used), each run on a
                           * stream of its own created for the call and joined back
                           * to the caller's stream: the groups' mass-feature passes
                           * (matrix-core bound) overlap the selection loops of the
                           * groups before them.  Results are the same bits for any
                           * value.  0 = automatic (4 for H >= 256 with H a multiple
                           * of 32, else 1); 1..8; 9..16 AMC_ERR_UNSUPPORTED (a
                           * 16-group run of the 60k-token stack left no result; the
                           * cause was not established); else AMC_ERR_INVALID_ARG. */
  int32_t exact_refit;    /* which heads' NNLS refits (and value fit) leave the Gram form
                           * Phi_S^T Phi_S for orthogonal factorisations of Phi_S itself
                           * (Lawson-Hanson on the triangular factor of [Phi_S m]; the value
                           * fit from the factor of [A Y]), which resolve the minimiser when
                           * the selected keys are nearly collinear or the mass is almost
                           * fitted (zhichai.net deep-dive, section 1.6; xinfinite.net
                           * article, section 2, steps 2 and 3).  Heads with budget up to
                           * 640 and at most 8192 queries only; the others keep the Gram form.
                           * 3 (default): every such head, from its first refit, each refit
                           * warm-started from the Gram solver's weights for the same keys
                           * (run first; the same minimiser, reached in fewer active-set
                           * steps); 0: every such head, from its first refit, warm-started
                           * from the previous refit's weights only;
                           * 1: a head moves there, for the rest of the call, at the first
                           * refit whose last relative mass residual is below 1e-6 or whose
                           * Gram solve met a singular candidate or the iteration cap (faster
                           * where few heads need it, but the Gram form can miss the
                           * minimiser without either sign); 2: never.  Such heads carry
                           * AMC_HS_NNLS_QR. */
  int32_t digits_in_panel; /* recompute mode with bf16 inputs: 1 (default) lets the int8 digit
                           * rows and value tiles of the mass-feature pass share the panel's
                           * first bytes (every head group's pass is enqueued before any
                           * group's selection, which waits for all of them); 0 keeps them
                           * apart (a larger workspace).  The outputs are the same bits. */
  uint32_t flags;         /* AMC_FLAG_* */
  void *timer;            /* optional amc_timer_create() handle; NULL = none */
} amc_options;

/* Offsets, in bytes from the start of the trace buffer, of its sections.
 * Sections (each 256-byte aligned):
 *   shift      double [H]          the per-head logit shift s used for Phi
 *   pick       int32  [sum t_h]    original key index, in selection order, at cu_budgets[h]
 *   pick_score double [sum t_h]    r^T Phi[:, j] of each pick in the sweep that took it
 *                                  (float64 Phi columns, or the float32 Phi of an exact
 *                                  sweep: within float32 rounding of each other)
 *   weight     double [sum t_h]    final NNLS weight w of each pick (selection order)
 *   runner_up  double [sum c_h]    best score not taken by each cycle, at cu_cycles[h]
 *   nnls_iters int32  [sum c_h]    active-set iterations of the refit closing each cycle
 *   swept_keys int32  [sum c_h]    keys whose stored Phi columns the cycle's bounded sweep
 *                                  read (T_h when every key is read; 0 when Phi is not
 *                                  stored)
 *   swept_keys8 int32 [sum c_h]    keys whose columns of the 8-bit copy of Phi the cycle's
 *                                  second pruning stage read (0 where it did not run)
 *   relres     double [sum c_h]    relative mass residual ||m - Phi_S w|| / ||m|| after the
 *                                  cycle's refit (float64 residual; the last cycle's entry
 *                                  after the polish refits)
 * where a "cycle" is the R iterations between two refits; head h has
 * c_h = ceil(t_h / (k R)) cycles (amc_cycle_offsets). */
typedef struct {
  uint64_t shift, pick, pick_score, weight, runner_up, nnls_iters, swept_keys, swept_keys8, relres;
  uint64_t total_bytes;
} amc_trace_layout;

/* Fills *o with the defaults: plain OMP (k = R = 1), automatic NNLS cap and
 * tolerance, one polish refit, 64 GiB Phi budget, float32 C_v, automatic head
 * groups and exact-refit gate, digit rows in the panel, no trace, no timer.  Every refit starts from the previous refit's exact minimiser and
 * from the gradient Phi_S^T r of its float64 residual; a polish refit repeats
 * that once with no new key. */
void amc_default_options(amc_options *o);

/* Workspace bytes amc_compact needs for this problem (device memory,
 * 256-byte aligned).  Errors: AMC_ERR_INVALID_ARG for an invalid problem or
 * options, AMC_ERR_UNSUPPORTED for a shape outside this build. */
amc_status amc_workspace_size(const amc_problem *p, const amc_options *o, uint64_t *bytes);

/* cu_budgets (HOST int64[H+1]): exclusive prefix sum of the budgets; the
 * output row range of each head.  Selection-batch sizes do not change it. */
amc_status amc_output_offsets(const amc_problem *p, int64_t *cu_budgets);

/* cu_cycles (HOST int64[H+1]): exclusive prefix sum of the per-head number of
 * refit cycles ceil(t_h / (k R)); indexes the per-cycle trace sections. */
amc_status amc_cycle_offsets(const amc_problem *p, const amc_options *o, int64_t *cu_cycles);

/* Trace buffer layout for this problem and these options. */
amc_status amc_trace_layout_for(const amc_problem *p, const amc_options *o, amc_trace_layout *layout);

/* Compacts every head.  Device pointers:
 *   Q        [sum n_h][d]  in_dtype
 *   K, V     [sum T_h][d]  in_dtype
 *   beta_in  [sum T_h]     float32, nullable (all zero); an existing per-key
 *                          logit bias, e.g. from an earlier compaction
 *   Ck       [sum t_h][d]  in_dtype, exact copies of the selected keys
 *   beta     [sum t_h]     float32, beta_in_j + log w_j (-inf where w_j = 0)
 *   Cv       [sum t_h][d]  cv_dtype
 *   sel_idx  [sum t_h]     int32, nullable: selected original index (within the head)
 *   head_status [H]        int32, nullable: AMC_HS_* bits
 *   trace    trace_bytes   nullable unless AMC_FLAG_TRACE (layout: amc_trace_layout_for)
 *   workspace workspace_bytes (>= amc_workspace_size, 256-byte aligned)
 * stream is a hipStream_t (NULL: the default stream). */
amc_status amc_compact(const amc_problem *p, const amc_options *o, const void *Q, const void *K,
                       const void *V, const float *beta_in, void *Ck, float *beta, void *Cv,
                       int32_t *sel_idx, int32_t *head_status, void *trace, uint64_t trace_bytes,
                       void *workspace, uint64_t workspace_bytes, void *stream);

/* amc_compact without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The workspace is a static device array of the
 * library, amc_noalloc_max_workspace() bytes (256 MiB) per GPU, held until the
 * process ends; the call itself allocates nothing (no hipMalloc/hipFree, no
 * streams or events: the heads run as one group, and options.timer and
 * options.head_groups are ignored).  The first call on a device looks up that
 * device's copy of the array (hipGetSymbolAddress).  Outputs, trace and
 * arguments as for amc_compact; results are the same bits as amc_compact with
 * head_groups = 1.  Errors: AMC_ERR_WORKSPACE when amc_workspace_size for this
 * problem exceeds amc_noalloc_max_workspace() (nothing is enqueued); the others
 * as for amc_compact.  Every call on one GPU shares its array: calls that
 * overlap in time on one GPU (other streams or threads) race and must be
 * serialised by the caller. */
amc_status amc_compact_noalloc(const amc_problem *p, const amc_options *o, const void *Q, const void *K,
                               const void *V, const float *beta_in, void *Ck, float *beta, void *Cv,
                               int32_t *sel_idx, int32_t *head_status, void *trace, uint64_t trace_bytes,
                               void *stream);

/* Bytes of the static workspace amc_compact_noalloc uses on each GPU. */
uint64_t amc_noalloc_max_workspace(void);

/* Stage 1 alone: the per-head shift s_h (logit maximum, float64[H]), the mass
 * features Phi = exp(l - s) (float32 [n_h][T_h] per head, packed at
 * sum_{g<h} n_g T_g; nullable), the target mass m = Phi 1 (float64[sum n_h])
 * and the attention output Y = Phi V / m (float32 [sum n_h][d])
 * (zhichai.net deep-dive, section 1.6: Phi and m; xinfinite.net article,
 * section 2, step 3: the output to match).  workspace as for amc_compact. */
amc_status amc_mass_features(const amc_problem *p, const void *Q, const void *K, const void *V,
                             const float *beta_in, double *shift, float *phi, double *m, float *Y,
                             int32_t *head_status, void *workspace, uint64_t workspace_bytes,
                             void *stream);

/* Workspace bytes for amc_mass_features. */
amc_status amc_mass_features_workspace(const amc_problem *p, uint64_t *bytes);

/* Batched NNLS: for each problem b, w_b = argmin_{w >= 0} 0.5 w^T G_b w - g_b^T w
 * with G_b symmetric positive semi-definite (the Gram form of the bias fit,
 * zhichai.net deep-dive, section 1.6; projected gradient, xinfinite.net
 * article, Fig. 2; exact active-set polish).  Device pointers:
 *   G      float64, problem b at G + cu_t2[b] (dense t_b x t_b, row-major)
 *   g      float64[sum t_b] at cu_t[b];  w  float64[sum t_b] (in: warm start
 *          if warm != 0, out: solution)
 *   iters  int32[num] nullable: active-set iterations used
 *   status int32[num] nullable: AMC_HS_NNLS_* bits
 * cu_t (HOST int64[num+1]) gives the sizes; cu_t2 is derived (sum of t_b^2).
 * t_b <= 176 in this build (else AMC_ERR_UNSUPPORTED). */
amc_status amc_nnls(int32_t num, const int64_t *cu_t, const double *G, const double *g, double *w,
                    int32_t warm, int32_t pg_iters, int32_t max_iters, double tol, int32_t *iters,
                    int32_t *status, void *stream);

/* Non-uniform per-head budgets by greedy swaps (zhichai.net deep-dive, section
 * 4.2: sensitivity curves rank the heads once, a greedy-swap algorithm gives
 * each head its own compression; xinfinite.net article, section 4, Fig. 3 and
 * 4).  Host only; no device work.
 *   loss     HOST double [H][J]: head h's sensitivity (e.g. its reconstruction
 *            loss) when it keeps (j + 1) * unit keys, j = 0..J-1
 *   unit     keys per budget step (>= 1)
 *   total    the budgets' sum, a multiple of unit with H * unit <= total <= H * J * unit
 *   budgets  HOST int64 [H] out
 *   swaps    HOST int64 out, nullable: the unit moves made
 * Every head starts with total / (H unit) units, the remainder one unit each
 * to the lowest heads; then, while it lowers the summed loss, one unit moves
 * to the head whose loss falls most by receiving it from the other head whose
 * loss rises least by giving it up (ties to the lower head), a head keeping
 * between 1 and J units.  With curves that fall by less at each further step
 * (the usual shape) no single move then improves the sum, which makes it the
 * minimum.  Errors:
 * AMC_ERR_INVALID_ARG for a null pointer, non-finite loss or a total out of
 * range. */
amc_status amc_greedy_swap_budgets(int32_t num_heads, int32_t steps, const double *loss, int64_t unit,
                                   int64_t total, int64_t *budgets, int64_t *swaps);

/* Kernel timer: HIP events recorded around every launch of an amc_compact
 * call whose options carry the handle.  Reading synchronises on the events. */
amc_status amc_timer_create(void **timer);
amc_status amc_timer_reset(void *timer);
/* Launch count and summed duration (ms) of one kernel class since the last reset. */
amc_status amc_timer_read(void *timer, int32_t kernel_class, int64_t *launches, double *total_ms);
void amc_timer_destroy(void *timer);

const char *amc_status_string(amc_status s);
int amc_version(void);

#ifdef __cplusplus
}
#endif

#endif /* AMC_H */
