// libamc host side: argument validation, workspace planning, launch sequencing
// and the kernel timer.  Nothing here touches the GPU before validation has
// passed, so every argument error returns with nothing enqueued.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "amc.h"
#include "amc_internal.h"

namespace amc {

// ---------------------------------------------------------------------------
// timer
// ---------------------------------------------------------------------------
struct Timer {
  std::vector<hipEvent_t> start, stop;
  std::vector<int> cls;
  size_t used = 0;
  bool failed = false;
};

void timer_begin(Timer *t, int c, hipStream_t s) {
  if (!t || t->failed) return;
  if (t->used == t->start.size()) {
    hipEvent_t a, b;
    if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) {
      t->failed = true;
      return;
    }
    t->start.push_back(a);
    t->stop.push_back(b);
    t->cls.push_back(c);
  }
  t->cls[t->used] = c;
  if (hipEventRecord(t->start[t->used], s) != hipSuccess) t->failed = true;
}

void timer_end(Timer *t, int c, hipStream_t s) {
  (void)c;
  if (!t || t->failed) return;
  if (hipEventRecord(t->stop[t->used], s) != hipSuccess) t->failed = true;
  t->used++;
}

// ---------------------------------------------------------------------------
// planning
// ---------------------------------------------------------------------------
static inline uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

static inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Plan {
  Dims dm{};
  std::vector<HeadDesc> desc;
  int kR = 1;
  int64_t max_cycles = 0, sum_t = 0, sum_cycles = 0, sum_n = 0, sum_T = 0;
  bool store_phi = true;
  bool highest = false;  // AM-Highest selection: one cycle with every key of each head
  // byte offsets in the workspace
  uint64_t o_desc = 0, o_shift_part = 0, o_shift = 0, o_phi = 0, o_m = 0, o_r = 0, o_mhat = 0,
           o_Y = 0, o_sel_slot = 0, o_sel_list = 0, o_panel = 0, o_G = 0, o_bvec = 0, o_w = 0,
           o_rhs = 0, o_cvsel = 0, o_pos = 0, o_cand_val = 0, o_cand_idx = 0, o_flist = 0, o_fcount = 0,
           o_dn = 0, o_L = 0, o_nnL = 0, o_nnP = 0, o_nnnp = 0, o_gA = 0, o_nnvec = 0, o_cand_lo = 0,
           o_cand_lidx = 0, o_cand_cnt = 0, o_band_list = 0, o_band_cnt = 0, o_exact = 0, o_stage = 0,
           o_part = 0, o_vt = 0, o_qdig = 0, o_kdig = 0, o_qexp = 0, o_ktab = 0, o_f64h = 0, o_colsum = 0, o_rpn = 0, o_rabs = 0,
           o_surv = 0, o_survcnt = 0, o_pruneL = 0, o_q8 = 0, o_q8bad = 0, o_surv2 = 0, o_surv2cnt = 0,
           o_qrflag = 0, o_qrbuilt = 0, o_qrbuf = 0, o_rpart = 0, o_score = 0, total = 0;
  bool exact_path = false;  // some head may take the orthogonal-factorisation refit
  bool store_q8 = false;  // the 8-bit plane of the second pruning stage fits the budget too
  bool alias_digits = false;  // digit rows and value tiles lie in the panel (recompute mode)
};

// AMC_PRUNE_Q8=0 leaves the 8-bit plane and the second pruning stage out
// (the selection is the same either way; for testing and measurement).
static bool q8_stage_enabled() {
  const char *e = std::getenv("AMC_PRUNE_Q8");
  return !(e && std::strcmp(e, "0") == 0);
}

static amc_status check_problem(const amc_problem *p) {
  if (!p || p->num_heads < 1 || !p->cu_q || !p->cu_k || !p->budgets) return AMC_ERR_INVALID_ARG;
  if (p->in_dtype != AMC_F32 && p->in_dtype != AMC_BF16) return AMC_ERR_INVALID_ARG;
  if (!(std::isfinite(p->scale)) || p->scale < 0.0f) return AMC_ERR_INVALID_ARG;
  if (p->head_dim != 64 && p->head_dim != 128) {
    return p->head_dim > 0 ? AMC_ERR_UNSUPPORTED : AMC_ERR_INVALID_ARG;
  }
  if (p->cu_q[0] != 0 || p->cu_k[0] != 0) return AMC_ERR_INVALID_ARG;
  for (int h = 0; h < p->num_heads; ++h) {
    const int64_t n = p->cu_q[h + 1] - p->cu_q[h];
    const int64_t T = p->cu_k[h + 1] - p->cu_k[h];
    const int64_t t = p->budgets[h];
    if (n < 1 || T < 1 || t < 1 || t > T) return AMC_ERR_INVALID_ARG;
    if (T > (int64_t(1) << 30) || n > (int64_t(1) << 30)) return AMC_ERR_UNSUPPORTED;
  }
  return AMC_OK;
}

static amc_status check_options(const amc_options *o) {
  if (!o) return AMC_ERR_INVALID_ARG;
  if (o->select != AMC_SEL_OMP && o->select != AMC_SEL_OMP_BATCHED && o->select != AMC_SEL_HIGHEST)
    return AMC_ERR_INVALID_ARG;
  if (o->topk < 1 || o->refit_every < 1) return AMC_ERR_INVALID_ARG;
  if ((o->select == AMC_SEL_OMP || o->select == AMC_SEL_HIGHEST) && (o->topk != 1 || o->refit_every != 1))
    return AMC_ERR_INVALID_ARG;
  if (int64_t(o->topk) * o->refit_every > kMaxCycle) return AMC_ERR_UNSUPPORTED;
  if (o->nnls_max_iters < 0 || o->nnls_polish < 0 || o->nnls_polish > 8) return AMC_ERR_INVALID_ARG;
  if (o->head_groups < 0 || o->head_groups > 16) return AMC_ERR_INVALID_ARG;
  if (o->head_groups > 8) return AMC_ERR_UNSUPPORTED;
  if (o->exact_refit < 0 || o->exact_refit > 3) return AMC_ERR_INVALID_ARG;
  if (o->digits_in_panel != 0 && o->digits_in_panel != 1) return AMC_ERR_INVALID_ARG;
  if (!(o->nnls_tol >= 0.0) || !std::isfinite(o->nnls_tol)) return AMC_ERR_INVALID_ARG;
  if (o->cv_dtype != AMC_F32 && o->cv_dtype != AMC_BF16) return AMC_ERR_INVALID_ARG;
  if (o->flags & ~uint32_t(AMC_FLAG_TRACE)) return AMC_ERR_INVALID_ARG;
  return AMC_OK;
}

// Builds the plan.  features_only: the amc_mass_features stage (no selection state).
static amc_status make_plan(const amc_problem *p, const amc_options *o, bool features_only, Plan &pl) {
  amc_status st = check_problem(p);
  if (st != AMC_OK) return st;
  if (!features_only) {
    st = check_options(o);
    if (st != AMC_OK) return st;
  }
  const int H = p->num_heads;
  const int d = p->head_dim;
  pl.kR = features_only ? 1 : o->topk * o->refit_every;
  pl.highest = !features_only && o->select == AMC_SEL_HIGHEST;
  if (pl.highest) {
    // one cycle per head takes all of its keys
    int64_t tmax = 1;
    for (int h = 0; h < p->num_heads; ++h) tmax = std::max<int64_t>(tmax, p->budgets[h]);
    pl.kR = int(std::min<int64_t>(tmax, kMaxBudget));
  }
  Dims &dm = pl.dm;
  dm.H = H;
  dm.d = d;
  dm.in_bf16 = p->in_dtype == AMC_BF16;
  dm.scale = p->scale > 0.0f ? double(p->scale) : 1.0 / std::sqrt(double(d));
  pl.desc.assign(H, HeadDesc{});
  int64_t phi = 0, nn = 0, tt = 0, t2 = 0, panel = 0, cblk = 0, sblk = 0, cyc = 0, TT = 0, vt = 0, ktr = 0, qrb = 0;
  int64_t dense = 0;
  for (int h = 0; h < H; ++h) {
    HeadDesc &D = pl.desc[h];
    D.n = p->cu_q[h + 1] - p->cu_q[h];
    D.T = p->cu_k[h + 1] - p->cu_k[h];
    D.t = features_only ? 1 : p->budgets[h];
    D.q_off = p->cu_q[h];
    D.k_off = p->cu_k[h];
    // rows of the stored Phi: float32 rows for the mass-feature entry point on
    // float32 inputs (4-key segments), 16-bit planes otherwise (whole 64-key
    // tiles; the mass-feature entry point then unpacks them)
    D.ldT = (features_only && !dm.in_bf16) ? (D.T + 3) / 4 * 4 : (D.T + 63) / 64 * 64;
    D.out_off = dense;
    dense += D.n * D.T;
    D.ldN = (D.n + 63) / 64 * 64;
    D.vt_off = vt;
    D.kt_off = ktr;
    D.phi_off = phi;
    D.n_off = nn;
    D.t_off = tt;
    D.tt_off = t2;
    D.panel_off = panel;
    D.cblk_off = cblk;
    D.n_cblk = ceil_div(D.T, kSweepCols);
    D.sblk_off = sblk;
    D.n_sblk = ceil_div(D.n, kShiftRows);
    D.cyc_off = cyc;
    D.qr_off = -1;
    if (!features_only && o->exact_refit != 2 && D.t <= kQrMaxT && D.n <= kQrMaxN) {
      D.qr_off = qrb;
      qrb += qr_layout(D.t, D.n).total;
      pl.exact_path = true;
    }
    if (!features_only) {
      if (D.t > kMaxBudget) return AMC_ERR_UNSUPPORTED;
      if (D.n_cblk > kMaxSweepBlocks) return AMC_ERR_UNSUPPORTED;
    }
    const int64_t cycles = ceil_div(D.t, pl.kR);
    phi += (features_only && !dm.in_bf16 ? D.n : D.ldN) * D.ldT;
    vt += (D.T + 63) / 64 * 72 * d;
    ktr += (D.T + 63) / 64 * 64;
    nn += D.n;
    tt += D.t;
    t2 += D.t * D.t;
    panel += D.t * D.n;
    cblk += D.n_cblk;
    sblk += D.n_sblk;
    cyc += cycles;
    TT += D.T;
    dm.max_n = std::max(dm.max_n, D.n);
    dm.max_T = std::max(dm.max_T, D.T);
    dm.max_t = std::max(dm.max_t, D.t);
    dm.min_t = h == 0 ? D.t : std::min(dm.min_t, D.t);
    dm.n_lo = h == 0 ? D.n : std::min(dm.n_lo, D.n);
    dm.n_hi = std::max(dm.n_hi, D.n);
    dm.max_sblk = std::max(dm.max_sblk, D.n_sblk);
    dm.max_cblk = std::max(dm.max_cblk, D.n_cblk);
    pl.max_cycles = std::max(pl.max_cycles, cycles);
  }
  dm.total_sblk = sblk;
  dm.max_qblk = ceil_div(dm.max_n, kRescoreRows);
  dm.qb128 = ceil_div(dm.max_n, 128);
  dm.nrb = ceil_div(dm.max_n, kResidRows);
  pl.sum_t = tt;
  pl.sum_cycles = cyc;
  pl.sum_n = nn;
  pl.sum_T = TT;
  const uint64_t phi_bytes = uint64_t(phi) * 4;
  if (!features_only) {
    // else every sweep recomputes Phi
    pl.store_phi = phi_bytes <= o->phi_budget_bytes && dm.max_n <= kStoredMaxN;
    pl.store_q8 = pl.store_phi && phi_bytes + uint64_t(phi) <= o->phi_budget_bytes && q8_stage_enabled();
  }

  uint64_t off = 0;
  auto take = [&](uint64_t bytes) {
    const uint64_t at = off;
    off = align256(off + bytes);
    return at;
  };
  pl.o_desc = take(sizeof(HeadDesc) * H);
  pl.o_shift_part = take(4ull * sblk);
  pl.o_shift = take(8ull * H);
  if (features_only) {
    if (dm.in_bf16) {
      // the selection's own mass-feature kernels: value tiles, digit rows,
      // the two Phi planes
      pl.o_phi = take(phi_bytes);
      pl.o_vt = take(2ull * vt);
      pl.o_qdig = take(5ull * d * nn);
      pl.o_qexp = take(4ull * nn);
      pl.o_kdig = take((5ull * d + 16) * ktr);
      pl.o_ktab = take(16ull * ktr);
      pl.o_f64h = take(4ull * 3 * H);
    }
    pl.total = off;
    return AMC_OK;
  }
  pl.o_phi = take(pl.store_phi ? phi_bytes : 0);
  pl.o_m = take(8ull * nn);
  pl.o_r = take(8ull * nn);
  pl.o_mhat = take(8ull * nn);
  pl.o_Y = take(4ull * nn * d);
  pl.o_sel_slot = take(4ull * TT);
  pl.o_sel_list = take(4ull * tt);
  pl.o_panel = take(8ull * panel);
  pl.o_G = take(8ull * t2);
  pl.o_bvec = take(8ull * tt);
  pl.o_w = take(8ull * tt);
  pl.o_rhs = take(8ull * tt * d);
  pl.o_cvsel = take(4ull * tt * d);
  pl.o_pos = take(4ull * tt);
  pl.o_cand_val = take(8ull * cblk * (kMaxCycle + 1));
  pl.o_cand_idx = take(4ull * cblk * (kMaxCycle + 1));
  pl.o_flist = take(4ull * tt);
  pl.o_fcount = take(4ull * H);
  pl.o_dn = take(8ull * tt);
  pl.o_nnL = take(8ull * t2);  // rows of t entries (slotted rows above kNnlsLdsT)
  // The value fit's packed factor of a head takes the first t(t+1)/2 entries
  // of that head's NNLS factor: it is formed after the head's last refit, on
  // the same stream, and the NNLS factor is not read again in the call.
  pl.o_L = pl.o_nnL;
  pl.o_nnP = take(4ull * tt);
  pl.o_nnnp = take(4ull * H);
  pl.o_gA = take(8ull * tt);
  pl.o_nnvec = dm.max_t > kNnlsLdsT ? take(8ull * kNnlsVecPerSlot * tt) : 0;
  pl.o_rpart = take(16ull * H * dm.nrb);
  if (pl.highest) pl.o_score = take(8ull * TT);  // every key's AM-Highest score
  if (pl.exact_path) {
    pl.o_qrflag = take(4ull * H);
    pl.o_qrbuilt = take(4ull * H);
    pl.o_qrbuf = take(8ull * uint64_t(qrb));
  }
  if (pl.store_phi) {  // bounded sweep, band and rescoring state
    pl.o_cand_lo = take(8ull * ktr);   // sweep upper bounds
    pl.o_cand_lidx = take(8ull * ktr); // sweep lower bounds
    pl.o_cand_cnt = take(4ull * ktr);  // swept keys
    pl.o_band_list = take(4ull * H * kBandCap);
    pl.o_band_cnt = take(4ull * H);
    pl.o_exact = take(4ull * H);
    pl.o_stage = take(8ull * nn * kBandCap);
    pl.o_part = take(8ull * H * kBandCap * dm.max_qblk);
    pl.o_colsum = take(4ull * ktr * dm.qb128);
    pl.o_rpn = take(8ull * nn);
    pl.o_rabs = take(8ull * H);
    pl.o_surv = take(4ull * ktr);
    pl.o_survcnt = take(4ull * H);
    pl.o_pruneL = take(8ull * H);
    if (pl.store_q8) {
      pl.o_q8 = take(uint64_t(phi));
      pl.o_q8bad = take(4ull * H);
      pl.o_surv2 = take(4ull * ktr);
      pl.o_surv2cnt = take(4ull * H);
    }
  }
  if (dm.in_bf16) {
    // In recompute mode the digit rows and the value tiles serve only the
    // mass-feature pass, which every head group finishes before any group
    // writes its first panel rows (amc_compact orders the groups so): then
    // they take the start of the panel when they fit there.
    const uint64_t dig_bytes = align256(2ull * vt) + align256(5ull * d * nn) + align256(4ull * nn) +
                               align256((5ull * d + 16) * ktr) + align256(16ull * ktr);
    pl.alias_digits = !features_only && !pl.store_phi && dig_bytes <= 8ull * uint64_t(panel) && o->digits_in_panel != 0;
    const uint64_t resume = off;
    if (pl.alias_digits) off = pl.o_panel;
    pl.o_vt = take(2ull * vt);  // transposed value tiles of the mass-feature kernel
    // digit form of the rows for the int8 logits
    pl.o_qdig = take(5ull * d * nn);
    pl.o_qexp = take(4ull * nn);
    pl.o_kdig = take((5ull * d + 16) * ktr);
    pl.o_ktab = take(16ull * ktr);
    if (pl.alias_digits) off = resume;
    pl.o_f64h = take(4ull * 3 * H);  // flags, the list of flagged heads, its length (per head group)
  }
  pl.total = off;
  return AMC_OK;
}

static void trace_layout(const Plan &pl, amc_trace_layout *L) {
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) {
    const uint64_t at = off;
    off = align256(off + bytes);
    return at;
  };
  L->shift = take(8ull * pl.dm.H);
  L->pick = take(4ull * pl.sum_t);
  L->pick_score = take(8ull * pl.sum_t);
  L->weight = take(8ull * pl.sum_t);
  L->runner_up = take(8ull * pl.sum_cycles);
  L->nnls_iters = take(4ull * pl.sum_cycles);
  L->swept_keys = take(4ull * pl.sum_cycles);
  L->swept_keys8 = take(4ull * pl.sum_cycles);
  L->relres = take(8ull * pl.sum_cycles);
  L->total_bytes = off;
}

// Copies the head descriptors to the device through kernel arguments, so the
// host vector may die as soon as the call returns (no pageable async copy).
static amc_status upload_desc(const Plan &pl, HeadDesc *d_desc, hipStream_t s) {
  const uint64_t *words = reinterpret_cast<const uint64_t *>(pl.desc.data());
  const int64_t n = int64_t(pl.desc.size()) * int64_t(sizeof(HeadDesc) / 8);
  if (launch_copy_words(reinterpret_cast<uint64_t *>(d_desc), words, n, s) != hipSuccess) return AMC_ERR_HIP;
  return AMC_OK;
}

static bool sync_check_enabled() {
  const char *e = std::getenv("AMC_SYNC_CHECK");
  return e && e[0] == '1';
}

// Head groups of one call (each on its own stream): the option, else four for
// stacks of at least 256 heads that split into multiples of 8 (the XCD
// mapping of the tiled kernels), else one; never more than H.
static int head_groups(int requested, int H) {
  const int g = requested > 0 ? requested : ((H >= 256 && H % 32 == 0) ? 4 : 1);
  return g < H ? g : H;
}

// First head of group g: the groups shrink by a factor 0.8 one to the next
// (the last group's selection loop runs alone at the end, so a smaller last
// group shortens that tail), with bounds on multiples of 8 heads when the
// count allows (the mass-feature kernels map heads to XCDs in eights).
static int group_bound(int H, int ngroups, int g) {
  if (g <= 0) return 0;
  if (g >= ngroups) return H;
  double tot = 0.0, acc = 0.0;
  for (int i = 0; i < ngroups; ++i) tot += std::pow(0.8, i);
  for (int i = 0; i < g; ++i) acc += std::pow(0.8, i);
  const double x = double(H) * acc / tot;
  int b = (H % 8 == 0 && H >= 8 * ngroups) ? 8 * int(std::lround(x / 8.0)) : int(std::lround(x));
  const int lo = group_bound(H, ngroups, g - 1) + 1, hi = H - (ngroups - g);  // every group keeps a head
  return b < lo ? lo : (b > hi ? hi : b);
}

// The buffers of heads [h0, ...): the descriptor table and the arrays indexed
// by head number start at h0; everything else is reached through the
// descriptors' offsets.
static Buffers head_range(const Buffers &b, int h0, int64_t max_qblk, int64_t nrb) {
  Buffers r = b;
  r.desc = b.desc + h0;
  r.shift = b.shift + h0;
  if (b.head_status) r.head_status = b.head_status + h0;
  if (b.tr_shift) r.tr_shift = b.tr_shift + h0;
  r.nn_np = b.nn_np + h0;
  r.ols_fcount = b.ols_fcount + h0;
  if (b.band_list) r.band_list = b.band_list + int64_t(h0) * kBandCap;
  if (b.band_cnt) r.band_cnt = b.band_cnt + h0;
  if (b.exact) r.exact = b.exact + h0;
  if (b.part) r.part = b.part + int64_t(h0) * kBandCap * max_qblk;
  if (b.f64_heads) {
    r.f64_heads = b.f64_heads + h0;
    r.f64_list = b.f64_list + h0;  // a group's list holds its own heads (group-relative numbers)
    r.f64_cnt = b.f64_cnt + h0;
  }
  if (b.rabs) r.rabs = b.rabs + h0;
  if (b.surv_cnt) r.surv_cnt = b.surv_cnt + h0;
  if (b.prune_L) r.prune_L = b.prune_L + h0;
  if (b.q8_bad) r.q8_bad = b.q8_bad + h0;
  if (b.surv2_cnt) r.surv2_cnt = b.surv2_cnt + h0;
  if (b.qr_flag) r.qr_flag = b.qr_flag + h0;
  if (b.qr_built) r.qr_built = b.qr_built + h0;
  if (b.rpart) r.rpart = b.rpart + int64_t(h0) * 2 * nrb;
  return r;
}

// AMC_PHI_LOGITS=f64 sends every head of a bf16 call to the float64-MFMA
// logit kernel (the int8 digit kernel is the default).
static bool phi_logits_f64() {
  const char *e = std::getenv("AMC_PHI_LOGITS");
  return e && std::strcmp(e, "f64") == 0;
}

// Largest candidate band the float64 rescoring takes; AMC_BAND_CAP lowers it
// (0 sends every head through the float32 sweep), for testing that path.
static int band_cap_setting() {
  const char *e = std::getenv("AMC_BAND_CAP");
  if (!e || !e[0]) return kBandCap;
  const long v = std::strtol(e, nullptr, 10);
  return v < 0 ? 0 : (v > kBandCap ? kBandCap : int(v));
}

// ---------------------------------------------------------------------------
// static scratch of the allocation-free entry point
// ---------------------------------------------------------------------------
// amc_compact_noalloc carves its workspace out of this array instead of a
// caller buffer.  Each GPU the library runs on holds its own copy, at its own
// address, until the process ends.  In host code `scratch` names a host-side
// stand-in, never the device memory: the device address comes from
// hipGetSymbolAddress, once per device, and only that pointer is used.
constexpr uint64_t kScratchBytes = 256ull << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void *g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device (nullptr on error).
static void *scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace amc

using namespace amc;

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
extern "C" {

void amc_default_options(amc_options *o) {
  if (!o) return;
  std::memset(o, 0, sizeof(*o));
  o->select = AMC_SEL_OMP;
  o->topk = 1;
  o->refit_every = 1;
  o->nnls_max_iters = 0;
  o->nnls_polish = 1;
  o->nnls_tol = 0.0;
  o->phi_budget_bytes = 64ull << 30;
  o->cv_dtype = AMC_F32;
  o->head_groups = 0;
  o->exact_refit = 3;
  o->digits_in_panel = 1;
  o->flags = 0;
  o->timer = nullptr;
}

amc_status amc_workspace_size(const amc_problem *p, const amc_options *o, uint64_t *bytes) {
  if (!bytes) return AMC_ERR_INVALID_ARG;
  Plan pl;
  amc_status st = make_plan(p, o, false, pl);
  if (st != AMC_OK) return st;
  *bytes = pl.total;
  return AMC_OK;
}

amc_status amc_mass_features_workspace(const amc_problem *p, uint64_t *bytes) {
  if (!bytes) return AMC_ERR_INVALID_ARG;
  Plan pl;
  amc_status st = make_plan(p, nullptr, true, pl);
  if (st != AMC_OK) return st;
  *bytes = pl.total;
  return AMC_OK;
}

amc_status amc_output_offsets(const amc_problem *p, int64_t *cu_budgets) {
  if (!cu_budgets) return AMC_ERR_INVALID_ARG;
  amc_status st = check_problem(p);
  if (st != AMC_OK) return st;
  cu_budgets[0] = 0;
  for (int h = 0; h < p->num_heads; ++h) cu_budgets[h + 1] = cu_budgets[h] + p->budgets[h];
  return AMC_OK;
}

amc_status amc_cycle_offsets(const amc_problem *p, const amc_options *o, int64_t *cu_cycles) {
  if (!cu_cycles) return AMC_ERR_INVALID_ARG;
  amc_status st = check_problem(p);
  if (st != AMC_OK) return st;
  st = check_options(o);
  if (st != AMC_OK) return st;
  const int64_t kR = int64_t(o->topk) * o->refit_every;
  cu_cycles[0] = 0;
  for (int h = 0; h < p->num_heads; ++h)
    cu_cycles[h + 1] = cu_cycles[h] + (o->select == AMC_SEL_HIGHEST ? 1 : ceil_div(p->budgets[h], kR));
  return AMC_OK;
}

amc_status amc_trace_layout_for(const amc_problem *p, const amc_options *o, amc_trace_layout *layout) {
  if (!layout) return AMC_ERR_INVALID_ARG;
  Plan pl;
  amc_status st = make_plan(p, o, false, pl);
  if (st != AMC_OK) return st;
  trace_layout(pl, layout);
  return AMC_OK;
}

#define AMC_LAUNCH(cls, expr)                                                     \
  do {                                                                            \
    if (timer) timer_begin(timer, (cls), stream);                                 \
    hipError_t e_ = (expr);                                                       \
    if (timer) timer_end(timer, (cls), stream);                                   \
    if (e_ != hipSuccess) return AMC_ERR_HIP;                                     \
    if (sync_check) {                                                             \
      if (hipStreamSynchronize(stream) != hipSuccess || hipGetLastError() != hipSuccess) \
        return AMC_ERR_HIP;                                                       \
    }                                                                             \
  } while (0)

static amc_status compact_impl(const amc_problem *p, const amc_options *o, const void *Q, const void *K,
                               const void *V, const float *beta_in, void *Ck, float *beta, void *Cv,
                               int32_t *sel_idx, int32_t *head_status, void *trace, uint64_t trace_bytes,
                               void *workspace, uint64_t workspace_bytes, void *stream_ptr) {
  Plan pl;
  amc_status st = make_plan(p, o, false, pl);
  if (st != AMC_OK) return st;
  if (!Q || !K || !V || !Ck || !beta || !Cv) return AMC_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < pl.total) return AMC_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return AMC_ERR_WORKSPACE;
  amc_trace_layout tl{};
  const bool tracing = (o->flags & AMC_FLAG_TRACE) != 0;
  if (tracing) {
    trace_layout(pl, &tl);
    if (!trace || trace_bytes < tl.total_bytes) return AMC_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(trace) & 255) return AMC_ERR_WORKSPACE;
  }
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
  Timer *timer = reinterpret_cast<Timer *>(o->timer);
  const bool sync_check = sync_check_enabled();

  char *ws = static_cast<char *>(workspace);
  Buffers b{};
  b.desc = reinterpret_cast<const HeadDesc *>(ws + pl.o_desc);
  b.Q = Q;
  b.K = K;
  b.V = V;
  b.beta_in = beta_in;
  b.shift_part = reinterpret_cast<float *>(ws + pl.o_shift_part);
  b.shift = reinterpret_cast<double *>(ws + pl.o_shift);
  b.phi = nullptr;
  b.phi16 = pl.store_phi ? reinterpret_cast<uint16_t *>(ws + pl.o_phi) : nullptr;
  b.vt = pl.dm.in_bf16 ? reinterpret_cast<uint16_t *>(ws + pl.o_vt) : nullptr;
  if (pl.dm.in_bf16 && !phi_logits_f64()) {
    b.qdig = reinterpret_cast<int8_t *>(ws + pl.o_qdig);
    b.qexp = reinterpret_cast<int32_t *>(ws + pl.o_qexp);
    b.kdig = reinterpret_cast<int8_t *>(ws + pl.o_kdig);
    b.ktab = reinterpret_cast<uint8_t *>(ws + pl.o_ktab);
    b.f64_heads = reinterpret_cast<int32_t *>(ws + pl.o_f64h);
    b.f64_list = b.f64_heads + pl.dm.H;
    b.f64_cnt = b.f64_heads + 2 * pl.dm.H;
  }
  b.m = reinterpret_cast<double *>(ws + pl.o_m);
  b.r = reinterpret_cast<double *>(ws + pl.o_r);
  b.mhat = reinterpret_cast<double *>(ws + pl.o_mhat);
  b.Y = reinterpret_cast<float *>(ws + pl.o_Y);
  b.sel_slot = reinterpret_cast<int32_t *>(ws + pl.o_sel_slot);
  b.sel_list = reinterpret_cast<int32_t *>(ws + pl.o_sel_list);
  b.panel = reinterpret_cast<double *>(ws + pl.o_panel);
  b.G = reinterpret_cast<double *>(ws + pl.o_G);
  b.bvec = reinterpret_cast<double *>(ws + pl.o_bvec);
  b.w = reinterpret_cast<double *>(ws + pl.o_w);
  b.rhs = reinterpret_cast<double *>(ws + pl.o_rhs);
  b.cv_sel = reinterpret_cast<float *>(ws + pl.o_cvsel);
  b.pos_of_slot = reinterpret_cast<int32_t *>(ws + pl.o_pos);
  b.cand_val = reinterpret_cast<double *>(ws + pl.o_cand_val);
  b.cand_idx = reinterpret_cast<int32_t *>(ws + pl.o_cand_idx);
  b.ols_flist = reinterpret_cast<int32_t *>(ws + pl.o_flist);
  b.ols_fcount = reinterpret_cast<int32_t *>(ws + pl.o_fcount);
  b.ols_dn = reinterpret_cast<double *>(ws + pl.o_dn);
  b.ols_L = reinterpret_cast<double *>(ws + pl.o_L);
  b.nn_L = reinterpret_cast<double *>(ws + pl.o_nnL);
  b.nn_P = reinterpret_cast<int32_t *>(ws + pl.o_nnP);
  b.nn_np = reinterpret_cast<int32_t *>(ws + pl.o_nnnp);
  b.nn_vec = pl.dm.max_t > kNnlsLdsT ? reinterpret_cast<double *>(ws + pl.o_nnvec) : nullptr;
  b.gA = reinterpret_cast<double *>(ws + pl.o_gA);
  if (pl.store_phi) {
    b.sw_up = reinterpret_cast<double *>(ws + pl.o_cand_lo);
    b.sw_lo = reinterpret_cast<double *>(ws + pl.o_cand_lidx);
    b.sw_key = reinterpret_cast<int32_t *>(ws + pl.o_cand_cnt);
    b.band_list = reinterpret_cast<int32_t *>(ws + pl.o_band_list);
    b.band_cnt = reinterpret_cast<int32_t *>(ws + pl.o_band_cnt);
    b.exact = reinterpret_cast<int32_t *>(ws + pl.o_exact);
    b.stage = reinterpret_cast<double *>(ws + pl.o_stage);
    b.part = reinterpret_cast<double *>(ws + pl.o_part);
    b.colsum = reinterpret_cast<float *>(ws + pl.o_colsum);
    b.rpn = reinterpret_cast<float *>(ws + pl.o_rpn);
    b.rabs = reinterpret_cast<double *>(ws + pl.o_rabs);
    b.surv_list = reinterpret_cast<int32_t *>(ws + pl.o_surv);
    b.surv_cnt = reinterpret_cast<int32_t *>(ws + pl.o_survcnt);
    b.prune_L = reinterpret_cast<double *>(ws + pl.o_pruneL);
    if (pl.store_q8) {
      b.q8 = reinterpret_cast<uint8_t *>(ws + pl.o_q8);
      b.q8_bad = reinterpret_cast<int32_t *>(ws + pl.o_q8bad);
      b.surv2_list = reinterpret_cast<int32_t *>(ws + pl.o_surv2);
      b.surv2_cnt = reinterpret_cast<int32_t *>(ws + pl.o_surv2cnt);
    }
  }
  b.head_status = head_status;
  b.rpart = reinterpret_cast<double *>(ws + pl.o_rpart);
  b.score_all = pl.highest ? reinterpret_cast<double *>(ws + pl.o_score) : nullptr;
  if (pl.exact_path) {
    b.qr_flag = reinterpret_cast<int32_t *>(ws + pl.o_qrflag);
    b.qr_built = reinterpret_cast<int32_t *>(ws + pl.o_qrbuilt);
    b.qrbuf = reinterpret_cast<double *>(ws + pl.o_qrbuf);
  }
  if (tracing) {
    char *tr = static_cast<char *>(trace);
    b.tr_shift = reinterpret_cast<double *>(tr + tl.shift);
    b.tr_pick = reinterpret_cast<int32_t *>(tr + tl.pick);
    b.tr_pick_score = reinterpret_cast<double *>(tr + tl.pick_score);
    b.tr_weight = reinterpret_cast<double *>(tr + tl.weight);
    b.tr_runner = reinterpret_cast<double *>(tr + tl.runner_up);
    b.tr_iters = reinterpret_cast<int32_t *>(tr + tl.nnls_iters);
    b.tr_swept = reinterpret_cast<int32_t *>(tr + tl.swept_keys);
    b.tr_swept8 = reinterpret_cast<int32_t *>(tr + tl.swept_keys8);
    b.tr_relres = reinterpret_cast<double *>(tr + tl.relres);
  }
  NnlsParams np{0, o->nnls_max_iters, o->nnls_tol};
  pl.dm.band_cap = band_cap_setting();
  const Dims &dm = pl.dm;

  AMC_LAUNCH(AMC_K_INIT, (upload_desc(pl, const_cast<HeadDesc *>(b.desc), stream) == AMC_OK
                              ? hipSuccess
                              : hipErrorLaunchFailure));
  AMC_LAUNCH(AMC_K_INIT, launch_fill_i32(b.sel_slot, pl.sum_T, 0, stream));
  if (head_status) AMC_LAUNCH(AMC_K_INIT, launch_fill_i32(head_status, dm.H, 0, stream));
  if (b.tr_swept && !pl.store_phi) AMC_LAUNCH(AMC_K_INIT, launch_fill_i32(b.tr_swept, pl.sum_cycles, 0, stream));
  if (b.tr_swept8) AMC_LAUNCH(AMC_K_INIT, launch_fill_i32(b.tr_swept8, pl.sum_cycles, 0, stream));
  if (b.q8_bad) AMC_LAUNCH(AMC_K_INIT, launch_fill_i32(b.q8_bad, dm.H, 0, stream));
  // exact refit: 2 sends every eligible head there from its first refit
  // (with bit 8, the Gram solver runs first and gives each refit its warm
  // start); 0 leaves it to the Gram solver until that flags the head
  const int qr_init = o->exact_refit == 0 ? 2 : o->exact_refit == 3 ? 2 | 8 : 0;
  if (b.qr_flag) AMC_LAUNCH(AMC_K_INIT, launch_fill_i32(b.qr_flag, dm.H, qr_init, stream));
  if (b.qr_built) AMC_LAUNCH(AMC_K_INIT, launch_fill_i32(b.qr_built, dm.H, 0, stream));

  // The heads run in groups, each on a stream of its own (the caller's for the
  // first), joined back to the caller's stream by events: the groups' mass
  // features run one after another, each overlapping the selection loops of
  // the groups before it (MFMA-bound against HBM- and latency-bound work).
  const int ngroups = head_groups(o->head_groups, dm.H);
  std::vector<hipStream_t> gs(size_t(ngroups), stream);
  std::vector<hipEvent_t> ev;
  auto cleanup = [&]() {
    for (hipEvent_t e : ev) (void)hipEventDestroy(e);
    for (int g = 1; g < ngroups; ++g)
      if (gs[size_t(g)] != stream) (void)hipStreamDestroy(gs[size_t(g)]);
  };
  auto new_event = [&](hipEvent_t *e) {
    if (hipEventCreateWithFlags(e, hipEventDisableTiming) != hipSuccess) return false;
    ev.push_back(*e);
    return true;
  };
  hipEvent_t ev_start = nullptr;
  std::vector<hipEvent_t> ev_phi(size_t(ngroups), nullptr), ev_done(size_t(ngroups), nullptr),
      ev_pre(size_t(ngroups), nullptr);
  if (ngroups > 1) {
    bool ok = new_event(&ev_start) && hipEventRecord(ev_start, stream) == hipSuccess;
    for (int g = 1; ok && g < ngroups; ++g) {
      ok = hipStreamCreateWithFlags(&gs[size_t(g)], hipStreamNonBlocking) == hipSuccess;
      if (!ok) gs[size_t(g)] = stream;
      ok = ok && hipStreamWaitEvent(gs[size_t(g)], ev_start, 0) == hipSuccess;
    }
    for (int g = 0; ok && g < ngroups; ++g)
      ok = new_event(&ev_phi[size_t(g)]) && new_event(&ev_done[size_t(g)]) &&
           (!pl.alias_digits || new_event(&ev_pre[size_t(g)]));
    if (!ok) {
      cleanup();
      return AMC_ERR_HIP;
    }
  }
  amc_status result = AMC_OK;
  // With the digit rows in the panel, every group's mass-feature pass is
  // enqueued first (pass 0) and every group's selection waits for all of them
  // (pass 1); otherwise one pass does both.
  const int npass = pl.alias_digits ? 2 : 1;
  for (int pass = 0; pass < npass && result == AMC_OK; ++pass)
  for (int g = 0; g < ngroups && result == AMC_OK; ++g) {
    const bool do_phi = pass == 0, do_sel = pass == npass - 1;
    const int h0 = group_bound(dm.H, ngroups, g), h1 = group_bound(dm.H, ngroups, g + 1);
    const Buffers bg = head_range(b, h0, dm.max_qblk, dm.nrb);
    Dims dg = dm;
    dg.H = h1 - h0;
    int64_t cycles = 0;
    dg.n_lo = pl.desc[size_t(h0)].n;
    dg.n_hi = 0;
    for (int h = h0; h < h1; ++h) {
      cycles = std::max(cycles, ceil_div(pl.desc[size_t(h)].t, pl.kR));
      dg.n_lo = std::min(dg.n_lo, pl.desc[size_t(h)].n);
      dg.n_hi = std::max(dg.n_hi, pl.desc[size_t(h)].n);
    }
    result = [&]() -> amc_status {
      hipStream_t stream = gs[size_t(g)];
      // the shift, value tiles and digit rows of a group run beside the
      // previous group's mass features; its own wait for them (one at a time,
      // matrix-bound) comes just before them, and the float64 fallback heads
      // run beside the next group's
      if (do_phi) {
        AMC_LAUNCH(AMC_K_SHIFT, launch_shift(dg, bg, stream));
        if (bg.vt) AMC_LAUNCH(AMC_K_INIT, launch_vt(dg, bg, stream));
        if (bg.qdig) AMC_LAUNCH(AMC_K_DIGITS, launch_digits(dg, bg, stream));
        if (g > 0 && hipStreamWaitEvent(stream, ev_phi[size_t(g - 1)], 0) != hipSuccess) return AMC_ERR_HIP;
        AMC_LAUNCH(AMC_K_PHI, launch_phi(dg, bg, pl.store_phi ? 2 : 0, stream));
        if (ngroups > 1 && hipEventRecord(ev_phi[size_t(g)], stream) != hipSuccess) return AMC_ERR_HIP;
        if (bg.qdig) AMC_LAUNCH(AMC_K_PHI_F64, launch_phi_fallback(dg, bg, pl.store_phi ? 2 : 0, stream));
        if (npass > 1 && ngroups > 1 && hipEventRecord(ev_pre[size_t(g)], stream) != hipSuccess) return AMC_ERR_HIP;
      }
      if (!do_sel) return AMC_OK;
      if (npass > 1)
        for (int g2 = 0; g2 < ngroups; ++g2)
          if (g2 != g && hipStreamWaitEvent(stream, ev_pre[size_t(g2)], 0) != hipSuccess) return AMC_ERR_HIP;
      for (int c = 0; c < cycles; ++c) {
        if (pl.highest) {
          // one sweep scores every key by its attention summed over the
          // queries (r = 1 / m), then each head's top t are the picks
          Buffers bh = bg;
          bh.r = bg.mhat;  // 1 / m (r itself stays m, the Gram solver's gradient)
          AMC_LAUNCH(AMC_K_SWEEP, launch_recip(dg, bg, stream));
          if (pl.store_phi) AMC_LAUNCH(AMC_K_SWEEP_EXACT, launch_sweep(dg, bh, c, pl.kR, 0, stream));
          else AMC_LAUNCH(AMC_K_SWEEP, launch_sweep_rc(dg, bh, c, pl.kR, stream));
          AMC_LAUNCH(AMC_K_MERGE, launch_topt(dg, bg, stream));
          AMC_LAUNCH(AMC_K_PANEL, launch_panel(dg, bg, c, pl.kR, 0, stream));
        } else if (pl.store_phi) {
          // bounded sweep and float64 rescoring of the band; the heads whose
          // band overflowed take the float32 sweep, merge and panel
          // (after the first cycle, with the 8-bit plane, a second pruning stage
          // narrows the list the bounded sweep reads)
          AMC_LAUNCH(AMC_K_PRUNE, launch_prune(dg, bg, c, pl.kR, stream));
          Buffers bs = bg;
          if (bg.q8 && c > 0) {
            AMC_LAUNCH(AMC_K_SWEEP, launch_sweep_q8(dg, bg, c, pl.kR, stream));
            AMC_LAUNCH(AMC_K_PRUNE, launch_q8_compact(dg, bg, c, pl.kR, stream));
            bs.surv_list = bg.surv2_list;
            bs.surv_cnt = bg.surv2_cnt;
          }
          AMC_LAUNCH(AMC_K_SWEEP, launch_sweep_band(dg, bs, c, pl.kR, stream));
          AMC_LAUNCH(AMC_K_MERGE, launch_band_merge(dg, bs, c, pl.kR, stream));
          AMC_LAUNCH(AMC_K_SWEEP_EXACT, launch_sweep(dg, bg, c, pl.kR, 1, stream));
          AMC_LAUNCH(AMC_K_MERGE, launch_merge(dg, bg, c, pl.kR, 1, stream));
          AMC_LAUNCH(AMC_K_RESCORE, launch_rescore(dg, bg, c, pl.kR, stream));
          AMC_LAUNCH(AMC_K_MERGE, launch_choose(dg, bg, c, pl.kR, stream));
          AMC_LAUNCH(AMC_K_PANEL, launch_panel(dg, bg, c, pl.kR, 1, stream));
        } else {
          AMC_LAUNCH(AMC_K_SWEEP, launch_sweep_rc(dg, bg, c, pl.kR, stream));
          AMC_LAUNCH(AMC_K_MERGE, launch_merge(dg, bg, c, pl.kR, 0, stream));
          AMC_LAUNCH(AMC_K_PANEL, launch_panel(dg, bg, c, pl.kR, 0, stream));
        }
        AMC_LAUNCH(AMC_K_GRAM, launch_gram(dg, bg, c, pl.kR, 0, stream));
        AMC_LAUNCH(AMC_K_NNLS, launch_nnls(dg, bg, c, pl.kR, 0, np, stream));
        if (bg.qr_flag) AMC_LAUNCH(AMC_K_NNLS, launch_nnls_qr(dg, bg, c, pl.kR, 0, stream));
        AMC_LAUNCH(AMC_K_RESID, launch_resid(dg, bg, c, pl.kR, 0, stream));
        if (bg.tr_relres) AMC_LAUNCH(AMC_K_RESID, launch_relres(dg, bg, c, pl.kR, 0, stream));
      }
      for (int r = 0; r < o->nnls_polish; ++r) {
        AMC_LAUNCH(AMC_K_GRAM, launch_gram(dg, bg, 0, pl.kR, 1, stream));
        AMC_LAUNCH(AMC_K_NNLS, launch_nnls(dg, bg, 0, pl.kR, 1, np, stream));
        if (bg.qr_flag) AMC_LAUNCH(AMC_K_NNLS, launch_nnls_qr(dg, bg, 0, pl.kR, 1, stream));
        AMC_LAUNCH(AMC_K_RESID, launch_resid(dg, bg, 0, pl.kR, 1, stream));
        if (bg.tr_relres) AMC_LAUNCH(AMC_K_RESID, launch_relres(dg, bg, 0, pl.kR, 1, stream));
      }
      AMC_LAUNCH(AMC_K_OLS_NORMAL, launch_ols_normal(dg, bg, stream));
      AMC_LAUNCH(AMC_K_OLS_SOLVE, launch_ols_factor(dg, bg, stream));
      AMC_LAUNCH(AMC_K_OLS_SOLVE, launch_ols_trsm(dg, bg, stream));
      if (bg.qr_flag) AMC_LAUNCH(AMC_K_OLS_SOLVE, launch_ols_qr(dg, bg, stream));
      AMC_LAUNCH(AMC_K_PACK, launch_pack(dg, bg, Ck, beta, Cv, o->cv_dtype == AMC_BF16, sel_idx, stream));
      if (ngroups > 1 && g > 0 && hipEventRecord(ev_done[size_t(g)], stream) != hipSuccess) return AMC_ERR_HIP;
      return AMC_OK;
    }();
  }
  // the caller's stream waits for every group (also after a failed launch, so
  // that nothing is left running apart from it)
  for (int g = 1; g < ngroups; ++g)
    if (hipStreamWaitEvent(stream, ev_done[size_t(g)], 0) != hipSuccess && result == AMC_OK) result = AMC_ERR_HIP;
  cleanup();
  return result;
}

amc_status amc_compact(const amc_problem *p, const amc_options *o, const void *Q, const void *K,
                       const void *V, const float *beta_in, void *Ck, float *beta, void *Cv,
                       int32_t *sel_idx, int32_t *head_status, void *trace, uint64_t trace_bytes,
                       void *workspace, uint64_t workspace_bytes, void *stream_ptr) {
  return compact_impl(p, o, Q, K, V, beta_in, Ck, beta, Cv, sel_idx, head_status, trace, trace_bytes, workspace,
                      workspace_bytes, stream_ptr);
}

amc_status amc_compact_noalloc(const amc_problem *p, const amc_options *o, const void *Q, const void *K,
                               const void *V, const float *beta_in, void *Ck, float *beta, void *Cv,
                               int32_t *sel_idx, int32_t *head_status, void *trace, uint64_t trace_bytes,
                               void *stream_ptr) {
  if (!o) return AMC_ERR_INVALID_ARG;
  // one head group (no streams or events created) and no timer (its events)
  amc_options oo = *o;
  if (oo.head_groups < 0 || oo.head_groups > 16) return AMC_ERR_INVALID_ARG;
  oo.head_groups = 1;
  oo.timer = nullptr;
  Plan pl;
  amc_status st = make_plan(p, &oo, false, pl);
  if (st != AMC_OK) return st;
  if (pl.total > kScratchBytes) return AMC_ERR_WORKSPACE;
  void *ws = scratch_on_current_device();
  if (!ws) return AMC_ERR_HIP;
  return compact_impl(p, &oo, Q, K, V, beta_in, Ck, beta, Cv, sel_idx, head_status, trace, trace_bytes, ws,
                      kScratchBytes, stream_ptr);
}

uint64_t amc_noalloc_max_workspace(void) { return kScratchBytes; }

amc_status amc_mass_features(const amc_problem *p, const void *Q, const void *K, const void *V,
                             const float *beta_in, double *shift, float *phi, double *m, float *Y,
                             int32_t *head_status, void *workspace, uint64_t workspace_bytes,
                             void *stream_ptr) {
  Plan pl;
  amc_status st = make_plan(p, nullptr, true, pl);
  if (st != AMC_OK) return st;
  if (!Q || !K || !V || !shift || !m || !Y) return AMC_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < pl.total) return AMC_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return AMC_ERR_WORKSPACE;
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
  Timer *timer = nullptr;
  const bool sync_check = sync_check_enabled();
  // The caller's Phi is packed densely ([n][T] per head).  float32 inputs: the
  // kernel writes rows of stride ldT, so a caller Phi is only accepted when
  // every T is a multiple of 4.  bfloat16 inputs run the selection's kernels
  // (int8 digit logits, float64 fallback heads) into the 16-bit planes, which
  // are then unpacked.
  if (phi && !pl.dm.in_bf16) {
    for (const HeadDesc &D : pl.desc)
      if (D.ldT != D.T) return AMC_ERR_UNSUPPORTED;
  }
  char *ws = static_cast<char *>(workspace);
  Buffers b{};
  b.desc = reinterpret_cast<const HeadDesc *>(ws + pl.o_desc);
  b.Q = Q;
  b.K = K;
  b.V = V;
  b.beta_in = beta_in;
  b.shift_part = reinterpret_cast<float *>(ws + pl.o_shift_part);
  b.shift = shift;
  b.phi = phi;
  b.m = m;
  b.r = nullptr;
  b.Y = Y;
  b.head_status = head_status;
  AMC_LAUNCH(AMC_K_INIT, (upload_desc(pl, const_cast<HeadDesc *>(b.desc), stream) == AMC_OK
                              ? hipSuccess
                              : hipErrorLaunchFailure));
  if (head_status) AMC_LAUNCH(AMC_K_INIT, launch_fill_i32(head_status, pl.dm.H, 0, stream));
  if (pl.dm.in_bf16) {
    b.phi = phi;
    b.phi16 = reinterpret_cast<uint16_t *>(ws + pl.o_phi);
    b.vt = reinterpret_cast<uint16_t *>(ws + pl.o_vt);
    if (!phi_logits_f64()) {
      b.qdig = reinterpret_cast<int8_t *>(ws + pl.o_qdig);
      b.qexp = reinterpret_cast<int32_t *>(ws + pl.o_qexp);
      b.kdig = reinterpret_cast<int8_t *>(ws + pl.o_kdig);
      b.ktab = reinterpret_cast<uint8_t *>(ws + pl.o_ktab);
      b.f64_heads = reinterpret_cast<int32_t *>(ws + pl.o_f64h);
      b.f64_list = b.f64_heads + pl.dm.H;
      b.f64_cnt = b.f64_heads + 2 * pl.dm.H;
    }
    const int store = phi ? 2 : 0;
    AMC_LAUNCH(AMC_K_SHIFT, launch_shift(pl.dm, b, stream));
    AMC_LAUNCH(AMC_K_INIT, launch_vt(pl.dm, b, stream));
    if (b.qdig) AMC_LAUNCH(AMC_K_DIGITS, launch_digits(pl.dm, b, stream));
    AMC_LAUNCH(AMC_K_PHI, launch_phi(pl.dm, b, store, stream));
    if (b.qdig) AMC_LAUNCH(AMC_K_PHI_F64, launch_phi_fallback(pl.dm, b, store, stream));
    if (phi) AMC_LAUNCH(AMC_K_PACK, launch_planes_to_phi(pl.dm, b, stream));
    return AMC_OK;
  }
  AMC_LAUNCH(AMC_K_SHIFT, launch_shift(pl.dm, b, stream));
  AMC_LAUNCH(AMC_K_PHI, launch_phi(pl.dm, b, phi != nullptr, stream));
  return AMC_OK;
}

amc_status amc_greedy_swap_budgets(int32_t num_heads, int32_t steps, const double *loss, int64_t unit,
                                   int64_t total, int64_t *budgets, int64_t *swaps) {
  if (num_heads < 1 || steps < 1 || !loss || !budgets || unit < 1) return AMC_ERR_INVALID_ARG;
  const int64_t H = num_heads, J = steps;
  if (total % unit != 0) return AMC_ERR_INVALID_ARG;
  const int64_t units = total / unit;
  if (units < H || units > H * J) return AMC_ERR_INVALID_ARG;
  for (int64_t e = 0; e < H * J; ++e)
    if (!std::isfinite(loss[e])) return AMC_ERR_INVALID_ARG;
  // u[h]: head h's units, 1..J; loss at u units is loss[h][u - 1]
  std::vector<int64_t> u(size_t(H), units / H);
  for (int64_t h = 0; h < units % H; ++h) ++u[size_t(h)];
  int64_t moves = 0;
  for (;;) {
    // the most valuable unit to receive, and the cheapest one to give up
    // among the other heads
    int64_t donor = -1, recv = -1;
    double cost = 0.0, gain = 0.0;
    for (int64_t h = 0; h < H; ++h) {
      const double *lh = loss + h * J;
      const int64_t k = u[size_t(h)];
      if (k < J) {
        const double g = lh[k - 1] - lh[k];  // fall of the loss with one unit more
        if (recv < 0 || g > gain) {
          recv = h;
          gain = g;
        }
      }
    }
    if (recv < 0) break;
    for (int64_t h = 0; h < H; ++h) {
      const int64_t k = u[size_t(h)];
      if (h == recv || k <= 1) continue;
      const double *lh = loss + h * J;
      const double c = lh[k - 2] - lh[k - 1];  // rise of the loss with one unit less
      if (donor < 0 || c < cost) {
        donor = h;
        cost = c;
      }
    }
    if (donor < 0 || !(gain > cost)) break;
    --u[size_t(donor)];
    ++u[size_t(recv)];
    ++moves;
    if (moves > H * J * J) break;  // cannot happen while each move lowers the sum; a guard only
  }
  for (int64_t h = 0; h < H; ++h) budgets[h] = u[size_t(h)] * unit;
  if (swaps) *swaps = moves;
  return AMC_OK;
}

amc_status amc_nnls(int32_t num, const int64_t *cu_t, const double *G, const double *g, double *w,
                    int32_t warm, int32_t pg_iters, int32_t max_iters, double tol, int32_t *iters,
                    int32_t *status, void *stream_ptr) {
  if (num < 1 || !cu_t || !G || !g || !w) return AMC_ERR_INVALID_ARG;
  if (pg_iters < 0 || max_iters < 0 || !(tol >= 0.0) || !std::isfinite(tol)) return AMC_ERR_INVALID_ARG;
  if (cu_t[0] != 0) return AMC_ERR_INVALID_ARG;
  int64_t max_t = 0;
  std::vector<int64_t> cu2(num + 1, 0);
  for (int i = 0; i < num; ++i) {
    const int64_t t = cu_t[i + 1] - cu_t[i];
    if (t < 1) return AMC_ERR_INVALID_ARG;
    if (t > kNnlsLdsT) return AMC_ERR_UNSUPPORTED;
    max_t = std::max(max_t, t);
    cu2[i + 1] = cu2[i] + t * t;
  }
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
  NnlsParams np{pg_iters, max_iters, tol};
  // The size tables travel as kernel arguments in chunks; see launch_nnls_batched.
  hipError_t e = launch_nnls_batched(num, cu_t, cu2.data(), max_t, G, g, w, warm, np, iters, status, stream);
  if (e != hipSuccess) return AMC_ERR_HIP;
  if (sync_check_enabled()) {
    if (hipStreamSynchronize(stream) != hipSuccess || hipGetLastError() != hipSuccess) return AMC_ERR_HIP;
  }
  return AMC_OK;
}

amc_status amc_timer_create(void **timer) {
  if (!timer) return AMC_ERR_INVALID_ARG;
  Timer *t = new (std::nothrow) Timer();
  if (!t) return AMC_ERR_INVALID_ARG;
  *timer = t;
  return AMC_OK;
}

amc_status amc_timer_reset(void *timer) {
  if (!timer) return AMC_ERR_INVALID_ARG;
  Timer *t = static_cast<Timer *>(timer);
  t->used = 0;
  t->failed = false;
  return AMC_OK;
}

amc_status amc_timer_read(void *timer, int32_t kernel_class, int64_t *launches, double *total_ms) {
  if (!timer || !launches || !total_ms) return AMC_ERR_INVALID_ARG;
  if (kernel_class < 0 || kernel_class >= AMC_NUM_KERNEL_CLASSES) return AMC_ERR_INVALID_ARG;
  Timer *t = static_cast<Timer *>(timer);
  if (t->failed) return AMC_ERR_HIP;
  int64_t cnt = 0;
  double tot = 0.0;
  for (size_t i = 0; i < t->used; ++i) {
    if (t->cls[i] != kernel_class) continue;
    if (hipEventSynchronize(t->stop[i]) != hipSuccess) return AMC_ERR_HIP;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, t->start[i], t->stop[i]) != hipSuccess) return AMC_ERR_HIP;
    ++cnt;
    tot += ms;
  }
  *launches = cnt;
  *total_ms = tot;
  return AMC_OK;
}

void amc_timer_destroy(void *timer) {
  if (!timer) return;
  Timer *t = static_cast<Timer *>(timer);
  for (hipEvent_t e : t->start) (void)hipEventDestroy(e);
  for (hipEvent_t e : t->stop) (void)hipEventDestroy(e);
  delete t;
}

const char *amc_status_string(amc_status s) {
  switch (s) {
    case AMC_OK: return "ok";
    case AMC_ERR_INVALID_ARG: return "invalid argument";
    case AMC_ERR_UNSUPPORTED: return "unsupported by this build";
    case AMC_ERR_WORKSPACE: return "workspace or trace buffer too small or misaligned";
    case AMC_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int amc_version(void) { return AMC_VERSION; }

}  // extern "C"
