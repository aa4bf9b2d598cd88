// Internal declarations shared by the libamc host planner and its HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "amc.h"

namespace amc {

// Tile sizes fixed by the kernels.
constexpr int kShiftRows = 128;  // queries per block of the logit-maximum kernel
constexpr int kPhiRows = 64;     // queries per block of the mass-feature kernel
constexpr int kPhiKeys = 64;     // keys per tile of the mass-feature kernel
constexpr int kPhi16Rows = 128;  // queries per block of the bf16 mass-feature kernel
constexpr int kSweepCols = 256;  // columns per block of the correlation sweep
constexpr int kMaxCycle = 255;   // largest k * R (keys per refit cycle)
constexpr int kLdsMaxT = 192;    // largest budget of the LDS-resident value fit
constexpr int kNnlsLdsT = 176;   // largest budget whose NNLS state fits in LDS (larger: global memory)
constexpr int kNnlsVecPerSlot = 15;  // float64 words of global NNLS state per budget slot
constexpr int kMaxBudget = 16384;  // largest budget per head (packed triangles indexed in int32)
constexpr int kMaxSweepBlocks = 1024;  // sweep column blocks per head the merge handles
constexpr int kBandCap = 128;    // candidates per head the float64 rescoring takes (more: exact sweep)
constexpr int kRescoreRows = 256; // queries per block of the rescoring kernel
constexpr int kStoredMaxN = 8192; // longest head (queries) the stored-Phi path takes
constexpr int kQrMaxT = 640;     // largest budget the orthogonal-factorisation refit takes
constexpr int kQrMaxN = 8192;    // most queries it takes (the append kernel holds a head's rows in registers)
constexpr int kQrChunk = 8;      // slots per block reflector of its factorisation
constexpr double kQrRelResid = 1e-6;  // relative mass residual below which they do
constexpr int kResidRows = 256;  // queries per block of the residual kernel (one partial sum each)

// Per-head descriptor, computed on the host and copied to the device once per call.
// All offsets are in elements of the array they index.
struct HeadDesc {
  int64_t n, T, t;        // queries, keys, budget
  int64_t q_off;          // first row of the head in Q
  int64_t k_off;          // first row of the head in K, V, beta_in; first entry in sel_slot
  int64_t ldT;            // row stride of the head's Phi (T rounded up to 4 for the float32
                          // output, to 64 for the stored planes: whole 64-key tiles)
  int64_t phi_off;        // first element of the head's Phi
  int64_t n_off;          // first entry in the per-query arrays (m, r, mhat, rows of Y)
  int64_t t_off;          // first entry in the per-slot arrays (= cu_budgets[h])
  int64_t tt_off;         // first element of the head's t x t matrices (G, normal matrix)
  int64_t panel_off;      // first element of the head's float64 panel [t][n]
  int64_t cblk_off;       // first sweep column block of the head in the candidate arrays
  int64_t n_cblk;         // sweep column blocks of the head
  int64_t sblk_off;       // first logit-maximum block of the head
  int64_t n_sblk;         // logit-maximum blocks of the head
  int64_t cyc_off;        // first cycle of the head in the per-cycle trace arrays
  int64_t vt_off;         // first element of the head's transposed value tiles (bf16 inputs)
  int64_t kt_off;         // first row of the head in the arrays of keys padded to whole 64-key tiles
  int64_t ldN;            // stored planes: column stride (n rounded up to 64)
  int64_t qr_off;         // first element of the head's exact-refit state (-1: none), laid out
                          // by qr_layout
  int64_t out_off;        // mass-feature stage: first element of the head in the caller's dense
                          // float32 Phi ([n][T] per head, packed)
};
static_assert(sizeof(HeadDesc) == 21 * 8, "HeadDesc layout");

// Float64 words of one head's exact-refit state, in this order (each part to a
// multiple of 32 words): V [t][n] Householder vectors, Rb [t][t] triangular
// factor (column-packed), cb [t] leading part of the rotated mass, Tw [t / 4][8][8]
// block-reflector factors, mt [n] rotated mass, W: the work area of the
// Lawson-Hanson steps (a packed triangle) and of the value fit ((t + 129)^2
// triangle and t x 128 solution).
struct QrLayout {
  int64_t V, Rb, cb, Tw, mt, W, total;
};
__host__ __device__ inline QrLayout qr_layout(int64_t t, int64_t n) {
  const auto pad = [](int64_t x) { return (x + 31) & ~int64_t(31); };
  const int64_t ld = t + 129;
  QrLayout L;
  L.V = 0;
  L.Rb = pad(t * n);
  L.cb = L.Rb + pad(t * t);
  L.Tw = L.cb + pad(t);
  L.mt = L.Tw + pad((t + 3) / 4 * kQrChunk * kQrChunk);  // chunks of 4 slots at the most
  L.W = L.mt + pad(n);
  // the larger of the value fit's (triangle and solution) and the Lawson-Hanson
  // steps' (packed free block, right-hand side and t full-height columns)
  const int64_t ols = ld * ld + t * 128, lh = t * (t + 3) / 2 + t + t * t + 64;
  L.total = L.W + pad(ols > lh ? ols : lh);
  return L;
}

// Device pointers of the workspace carve-up and of the caller's buffers.
struct Buffers {
  const HeadDesc *desc;
  const void *Q, *K, *V;
  const float *beta_in;
  float *shift_part;   // [sum n_sblk]
  double *shift;       // [H]
  float *phi;          // [sum n*ldT] float32 Phi (the mass-feature entry point's output)
  uint16_t *phi16;     // per head at 2*phi_off: high plane [ldT keys][ldN queries], then low plane
                       // [ldT][ldN] (key columns; queries from n to ldN and keys past T are zero)
  float *colsum;       // per head at kt_off * qb128: [128-query block][keys, T rounded up to 64]
                       // sums of the high plane, rounded down (written by the first sweep)
  float *rpn;          // [sum n][2] float32 positive and negative parts of r (per cycle)
  double *rabs;        // [H] sum |r| (per cycle)
  int32_t *surv_list;  // per head at kt_off: keys that pass the cycle's first pruning stage
  int32_t *surv_cnt;   // [H] their number, -1: every key
  double *prune_L;     // [H] the first stage's threshold (-inf: every key kept)
  uint8_t *q8;         // per head at phi_off: 8-bit plane [ldT keys][ldN queries] (null: no
                       // second stage)
  int32_t *q8_bad;     // [H] 1: the head's 8-bit plane is out of range (stage skipped)
  int32_t *surv2_list; // per head at kt_off: keys that pass both stages (the bounded sweep's list)
  int32_t *surv2_cnt;  // [H] their number, -1: every key
  uint16_t *vt;        // bf16 inputs: per head at vt_off, [T/64 tiles][d][72] values, key-permuted
                       // (64 per row and a pad of 8, the layout the mass-feature kernels stage)
  int8_t *qdig;        // bf16 inputs: rows of Q as five base-256 digit rows ([rows][5][d]); null:
                       // every head takes the float64 logit kernel
  int32_t *qexp;       // [rows of Q] row exponents of the digit form
  int8_t *kdig;        // per head at kt_off rows: K rows padded to whole tiles, each row its five
                       // digit rows and 16 bytes of pad ([rows][5 d + 16])
  uint8_t *ktab;       // per head at kt_off / 64: per 64-key tile 1 KiB, float64 (bias - shift)
                       // of each key (-inf past T), then its int32 row exponent, in stored order
  int32_t *f64_heads;  // [H] 1: a row of the head is not exact in digit form (float64 logits)
  int32_t *f64_list;   // [H] those heads, listed per launch (a group's from its first entry)
  int32_t *f64_cnt;    // [H] the list's length, at the launch's first head
  double *m, *r, *mhat;  // [sum n]
  float *Y;            // [sum n][d]
  int32_t *sel_slot;   // [sum T]  0 = unselected, else 1 + slot
  int32_t *sel_list;   // [sum t]  key index of each slot
  double *panel;       // [sum t*n] row a = float64 column of slot a over the queries
  double *G;           // [sum t*t]
  double *bvec;        // [sum t]
  double *gA;          // [sum t]  Phi_S^T r from the float64 panel and residual
  double *w;           // [sum t]
  double *rhs;         // [sum t][d]
  float *cv_sel;       // [sum t][d]
  int32_t *pos_of_slot;  // [sum t]
  int32_t *ols_flist;  // [sum t]  slots with w > 0, ascending
  int32_t *ols_fcount; // [H]
  double *ols_dn;      // [sum t]  diagonal scaling of the normal matrix
  double *ols_L;       // packed Cholesky factor of the scaled normal matrix, at tt_off (shares nn_L)
  double *nn_L;        // [sum t*t] NNLS factor of the free set, kept between refits (at tt_off)
  int32_t *nn_P;       // [sum t]  NNLS free set in factor order
  int32_t *nn_np;      // [H]      NNLS free-set size
  double *nn_vec;      // [sum t][kNnlsVecPerSlot] NNLS vectors of heads above kNnlsLdsT (else null)
  double *cand_val;    // [sum n_cblk][kMaxCycle + 1]  block top-(kR+1) scores, or band upper bounds
  int32_t *cand_idx;   // [sum n_cblk][kMaxCycle + 1]
  double *sw_up, *sw_lo;  // per head at kt_off: bounded-sweep bounds of the listed keys, in list order
  int32_t *sw_key;     // per head at kt_off: the listed keys
  int32_t *band_list;  // [H][kBandCap] key indices of the head's candidate band
  int32_t *band_cnt;   // [H]
  int32_t *exact;      // [H] 1: the head's band overflowed; this cycle takes the exact sweep
  double *stage;       // [sum n][kBandCap] float64 Phi columns of the band, per head [kBandCap][n]
  double *part;        // [H][kBandCap][max_qblk] partial scores of the band per query block
  int32_t *head_status;  // [H] or null
  int32_t *qr_flag;    // [H] exact refit: 0 Gram form, 1 flagged at this refit, 2 every later refit,
                       // bit 4: the value fit too (null: the path is off; heads with qr_off < 0
                       // keep the Gram form)
  int32_t *qr_built;   // [H] slots of the head's orthogonal factorisation that are current
  double *qrbuf;       // per head at qr_off: the exact refit's factorisation and work triangles
  double *rpart;       // [H][nrb][2] per 256-query block: sum r^2 and sum m^2 of the last residual
  double *score_all;   // [sum T] AM-Highest: every key's score from the sweep (null otherwise)
  // trace (all null when tracing is off)
  double *tr_shift, *tr_pick_score, *tr_weight, *tr_runner;
  int32_t *tr_pick, *tr_iters, *tr_swept, *tr_swept8;
  double *tr_relres;
};

struct Dims {
  int H, d;
  int in_bf16;         // 1: Q/K/V are bfloat16, 0: float32
  double scale;
  int64_t max_n, max_T, max_t, min_t;
  int64_t n_lo, n_hi;  // fewest and most queries of the heads a launch covers (the exact refit
                       // launches one kernel per class of n)
  int64_t max_sblk, max_cblk, max_qblk;
  int band_cap;        // largest band the rescoring takes (<= kBandCap)
  int64_t qb128;       // 128-query blocks of the longest head (column sums per key)
  int64_t total_sblk;
  int64_t nrb;         // residual blocks per head (max n / kResidRows, rounded up)
};

struct NnlsParams {
  int pg_iters;   // projected-gradient warm-up (stand-alone solver)
  int max_iters;  // 0: automatic
  double tol;     // 0: automatic
};

// Event-pair recorder used by the launch wrappers when a timer is attached.
struct Timer;
void timer_begin(Timer *t, int cls, hipStream_t s);
void timer_end(Timer *t, int cls, hipStream_t s);

// Kernel launchers (each returns hipSuccess or the launch error).
hipError_t launch_fill_i32(int32_t *p, int64_t count, int32_t value, hipStream_t s);
hipError_t launch_shift(const Dims &dm, const Buffers &b, hipStream_t s);
// store: 0 = no Phi, 1 = float32 Phi to b.phi, 2 = the two 16-bit planes to b.phi16.
// bf16 inputs with b.vt set (store 0 or 2) take the tiled kernel, after launch_vt.
hipError_t launch_phi(const Dims &dm, const Buffers &b, int store, hipStream_t s);
hipError_t launch_vt(const Dims &dm, const Buffers &b, hipStream_t s);
// bf16 inputs with b.qdig set: the digit form of the rows, before launch_phi; after it, the
// float64 kernel over the heads off the digit grid
hipError_t launch_digits(const Dims &dm, const Buffers &b, hipStream_t s);
hipError_t launch_phi_fallback(const Dims &dm, const Buffers &b, int store, hipStream_t s);
// the two 16-bit planes of the stored Phi to the caller's dense float32 Phi (at out_off)
hipError_t launch_planes_to_phi(const Dims &dm, const Buffers &b, hipStream_t s);
// gated: only the heads with b.exact[h] != 0 (else every head)
hipError_t launch_sweep(const Dims &dm, const Buffers &b, int cycle, int cyc_keys, int gated, hipStream_t s);
hipError_t launch_sweep_rc(const Dims &dm, const Buffers &b, int cycle, int cyc_keys, hipStream_t s);
hipError_t launch_sweep_band(const Dims &dm, const Buffers &b, int cycle, int cyc_keys, hipStream_t s);
// per cycle of the stored-Phi selection: r's parts and the keys the bounded sweep reads
hipError_t launch_prune(const Dims &dm, const Buffers &b, int cycle, int cyc_keys, hipStream_t s);
// second pruning stage from the 8-bit plane, then the list the bounded sweep reads
hipError_t launch_sweep_q8(const Dims &dm, const Buffers &b, int cycle, int cyc_keys, hipStream_t s);
hipError_t launch_q8_compact(const Dims &dm, const Buffers &b, int cycle, int cyc_keys, hipStream_t s);
hipError_t launch_band_merge(const Dims &dm, const Buffers &b, int cycle, int cyc_keys, hipStream_t s);
hipError_t launch_rescore(const Dims &dm, const Buffers &b, int cycle, int cyc_keys, hipStream_t s);
hipError_t launch_choose(const Dims &dm, const Buffers &b, int cycle, int cyc_keys, hipStream_t s);
hipError_t launch_merge(const Dims &dm, const Buffers &b, int cycle, int cyc_keys, int gated, hipStream_t s);
hipError_t launch_panel(const Dims &dm, const Buffers &b, int cycle, int cyc_keys, int gated, hipStream_t s);
hipError_t launch_gram(const Dims &dm, const Buffers &b, int cycle, int cyc_keys, int polish, hipStream_t s);
hipError_t launch_nnls(const Dims &dm, const Buffers &b, int cycle, int cyc_keys, int polish,
                       const NnlsParams &np, hipStream_t s);
// the workspace-resident refits (heads above kNnlsLdsT), called by launch_nnls
hipError_t launch_nnls_global(const Dims &dm, const Buffers &b, int cycle, int cyc_keys, int polish,
                              const NnlsParams &np, hipStream_t s);
hipError_t launch_resid(const Dims &dm, const Buffers &b, int cycle, int cyc_keys, int polish, hipStream_t s);
// AM-Highest: 1 / m into b.mhat (the sweep, given it as r, then scores sum_i Phi_ij / m_i
// into b.score_all), and
// the top t of those scores per head (ties to the lower key) as the cycle's picks
hipError_t launch_recip(const Dims &dm, const Buffers &b, hipStream_t s);
hipError_t launch_topt(const Dims &dm, const Buffers &b, hipStream_t s);
// trace only (no-op without it): relative mass residual of each head after the refit
hipError_t launch_relres(const Dims &dm, const Buffers &b, int cycle, int cyc_keys, int polish, hipStream_t s);
hipError_t launch_ols_normal(const Dims &dm, const Buffers &b, hipStream_t s);
hipError_t launch_pack(const Dims &dm, const Buffers &b, void *Ck, float *beta, void *Cv,
                       int cv_bf16, int32_t *sel_idx, hipStream_t s);
// Stand-alone batched NNLS on caller-provided Gram systems.
// h_cu_t / h_cu_t2 are HOST prefix sums of t_b and t_b^2; they travel as kernel arguments.
hipError_t launch_nnls_batched(int num, const int64_t *h_cu_t, const int64_t *h_cu_t2, int64_t max_t,
                               const double *G, const double *g, double *w, int warm,
                               const NnlsParams &np, int32_t *iters, int32_t *status, hipStream_t s);
hipError_t launch_copy_words(uint64_t *dst, const uint64_t *src, int64_t count, hipStream_t s);
hipError_t launch_ols_factor(const Dims &dm, const Buffers &b, hipStream_t s);
hipError_t launch_ols_trsm(const Dims &dm, const Buffers &b, hipStream_t s);
// exact refit and value fit of the heads flagged in b.qr_flag (no-ops when it is null)
hipError_t launch_nnls_qr(const Dims &dm, const Buffers &b, int cycle, int cyc_keys, int polish, hipStream_t s);
hipError_t launch_ols_qr(const Dims &dm, const Buffers &b, hipStream_t s);

}  // namespace amc
