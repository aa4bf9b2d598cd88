// Workspace-resident NNLS refits (budgets above kNnlsLdsT) with 512-thread
// blocks; the solver itself is k_nnls_body.h, documented in k_nnls.hip.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <climits>
#include <cmath>
#include <type_traits>

#include "amc_internal.h"

#define AMC_NNLS_NT 512
namespace amc {
namespace {
#include "k_nnls_body.h"
}  // namespace

hipError_t launch_nnls_global(const Dims &dm, const Buffers &b, int cycle, int kR, int polish, const NnlsParams &np,
                              hipStream_t s) {
  const size_t bytes = nnls_global_smem_bytes(dm.max_t);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_nnls_cycle<true>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, int(bytes));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_nnls_cycle<true>, dim3(unsigned(dm.H)), dim3(NT), bytes, s, b.desc, b.G, b.bvec, b.gA, b.w,
                     cycle, kR, polish, np, nnls_global_vec_bytes(dm.max_t) ? int(dm.max_t) : 0, b.nn_L, b.nn_P, b.nn_np, b.nn_vec, b.tr_iters,
                     b.tr_weight, b.head_status, b.qr_flag, b.rpart, int(dm.nrb));
  return hipGetLastError();
}

}  // namespace amc
