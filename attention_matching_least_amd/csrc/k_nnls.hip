// NNLS bias fit: w = argmin_{w >= 0} 0.5 w^T G w - b^T w, the Gram form of
// min ||Phi_S w - m|| (zhichai.net deep-dive, section 1.6: refit w by NNLS
// after every pick; xinfinite.net article, section 2, step 2).
//
// The pages' GPU solver is projected gradient (xinfinite.net article,
// Fig. 2).  On these Gram matrices (condition numbers 1e9 and beyond)
// projected gradient alone does not reach the minimiser, so the exact
// minimiser is found by an active-set method on the Gram form (Bro and
// De Jong's fast NNLS): zero variables with a positive gradient enter, the
// least-squares solution on the free set is computed from a Cholesky factor,
// and if it leaves the feasible set the iterate steps back and the blocking
// variables leave.  Projected gradient survives as the warm-up of the
// stand-alone solver (amc_nnls).
//
// Accuracy.  Everything is float64 in unit-diagonal form (w = u / sqrt(diag
// G)).  The solver keeps the gradient g = b - G u explicitly.  Each refit of
// a compaction starts from g = Phi_S^T r computed from the float64 panel and
// the float64 residual of the previous refit (the corrected semi-normal
// equations of Bjorck), and a final refit with no new key refines the weights
// once more.  Within a refit the rows of the free set follow the factor's
// model: the step d solves L L^T d = g_P, so moving a fraction alpha along d
// scales g_P by (1 - alpha), and y = L^-1 g_P scales with it.  The rows of
// zero variables are brought up to date only when candidates are chosen, by
// the exact increment from a snapshot: g_a = g_a(snap) - G_a (u - u_snap).
//
// The factor is updated, not recomputed.  Up to eight candidates enter
// together: one blocked forward substitution with several right-hand sides
// gives their factor rows and L^-1 g for the following solve, and a small
// Cholesky of the block finishes the rows.  A variable that leaves is deleted
// by a row shift plus a blocked rank-one update of the trailing rows (Givens
// rotations, applied to y as well, so no forward substitution is needed
// between entries).  Between the refits of one compaction the factor and the
// free set persist in the workspace.
//
// GPU mapping: one block per system (256 threads; 512 for the workspace-
// resident state of large budgets, whose passes over global memory are
// latency-bound, so more rows are in flight at once).  Triangular work runs in
// 16-row blocks: one wave solves the 16 x 16 diagonal block in registers
// (v_readlane broadcasts), then every thread updates one of the rows beyond
// it.  The state lives in LDS for budgets up to kNnlsLdsT; above that the same
// code runs on the workspace copy in global memory, with the two solve vectors
// still in LDS.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <climits>
#include <cmath>
#include <type_traits>

#include "amc_internal.h"

#define AMC_NNLS_NT 256
namespace amc {
namespace {
#include "k_nnls_body.h"
}  // namespace

hipError_t launch_nnls(const Dims &dm, const Buffers &b, int cycle, int kR, int polish, const NnlsParams &np,
                       hipStream_t s) {
  if (dm.min_t <= kNnlsLdsT) {
    const int maxp = int(dm.max_t < kNnlsLdsT ? dm.max_t : kNnlsLdsT);
    const size_t bytes = nnls_smem_bytes(maxp);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_nnls_cycle<false>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(bytes));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_nnls_cycle<false>, dim3(unsigned(dm.H)), dim3(NT), bytes, s, b.desc, b.G, b.bvec, b.gA,
                       b.w, cycle, kR, polish, np, maxp, b.nn_L, b.nn_P, b.nn_np, b.nn_vec, b.tr_iters, b.tr_weight,
                       b.head_status, b.qr_flag, b.rpart, int(dm.nrb));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (dm.max_t > kNnlsLdsT) return launch_nnls_global(dm, b, cycle, kR, polish, np, s);
  return hipSuccess;
}

hipError_t launch_nnls_batched(int num, const int64_t *h_cu_t, const int64_t *h_cu_t2, int64_t max_t,
                               const double *G, const double *g, double *w, int warm, const NnlsParams &np,
                               int32_t *iters, int32_t *status, hipStream_t s) {
  const int maxp = int(max_t);
  const size_t bytes = nnls_smem_bytes(maxp);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_nnls_batched),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, int(bytes));
  if (e != hipSuccess) return e;
  for (int base = 0; base < num; base += 64) {
    NnlsChunk ch;
    ch.count = num - base < 64 ? num - base : 64;
    for (int i = 0; i <= ch.count; ++i) {
      ch.cu_t[i] = h_cu_t[base + i] - h_cu_t[base];
      ch.cu_t2[i] = h_cu_t2[base + i] - h_cu_t2[base];
    }
    hipLaunchKernelGGL(k_nnls_batched, dim3(unsigned(ch.count)), dim3(NT), bytes, s, ch, base,
                       G + h_cu_t2[base], g + h_cu_t[base], w + h_cu_t[base], warm, np, maxp, iters, status);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace amc
