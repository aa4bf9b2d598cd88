// NNLS bias fit: w = argmin_{w >= 0} 0.5 w^T G w - b^T w, the Gram form of
// min ||Phi_S w - m|| (zhichai.net deep-dive, section 1.6: refit w by NNLS
// after every pick; xinfinite.net article, section 2, step 2).
//
// The pages' GPU solver is projected gradient (xinfinite.net article,
// Fig. 2).  On these Gram matrices (condition numbers ~1e9) projected
// gradient alone does not reach the minimiser, so it only warms up the active
// set here; an exact active-set polish (the Gram-form method of Bro and
// De Jong, with a Cholesky solve of the free block in LDS) finishes the fit.
// Everything runs in float64 in unit-diagonal form (w = u / sqrt(diag G)),
// which leaves the minimiser unchanged and makes the tolerance meaningful for
// columns of very different norm.
//
// One 256-thread block solves one system; the packed Cholesky factor of the
// free block (p <= 192) lives in LDS.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <climits>
#include <cmath>

#include "amc_internal.h"

namespace amc {
namespace {

constexpr int NT = 256;
constexpr unsigned char F_PASSIVE = 1, F_BLOCKED = 2;

__device__ __forceinline__ int tri(int r) { return r * (r + 1) / 2; }

__device__ __forceinline__ void decode_tri(int e, int *r, int *c) {
  int rr = int((sqrtf(8.0f * float(e) + 1.0f) - 1.0f) * 0.5f);
  while (tri(rr + 1) <= e) ++rr;
  while (tri(rr) > e) --rr;
  *r = rr;
  *c = e - tri(rr);
}

struct Red {
  double v[NT / 64];
  int i[NT / 64];
};

// Block max of v (ties to the lower index); returns the winning index, -1 if none valid.
__device__ int block_argmax(double v, int idx, Red *red, double *out_v) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const double ov = __shfl_xor(v, off);
    const int oi = __shfl_xor(idx, off);
    if (oi >= 0 && (idx < 0 || ov > v || (ov == v && oi < idx))) {
      v = ov;
      idx = oi;
    }
  }
  __syncthreads();
  if (lane == 0) {
    red->v[wave] = v;
    red->i[wave] = idx;
  }
  __syncthreads();
  v = red->v[0];
  idx = red->i[0];
  for (int w = 1; w < NT / 64; ++w) {
    const double ov = red->v[w];
    const int oi = red->i[w];
    if (oi >= 0 && (idx < 0 || ov > v || (ov == v && oi < idx))) {
      v = ov;
      idx = oi;
    }
  }
  *out_v = v;
  return idx;
}

__device__ double block_sum(double v, Red *red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  __syncthreads();
  if (lane == 0) red->v[wave] = v;
  __syncthreads();
  double s = 0.0;
  for (int w = 0; w < NT / 64; ++w) s += red->v[w];
  return s;
}

struct Smem {
  double *L, *u, *y, *g, *dg, *bs, *v;
  int *plist;
  unsigned char *flag;
};

__device__ Smem carve(char *base, int maxp) {
  Smem s;
  double *d = reinterpret_cast<double *>(base);
  s.L = d;
  d += tri(maxp);
  s.u = d;
  d += maxp;
  s.y = d;
  d += maxp;
  s.g = d;
  d += maxp;
  s.dg = d;
  d += maxp;
  s.bs = d;
  d += maxp;
  s.v = d;
  d += maxp;
  s.plist = reinterpret_cast<int *>(d);
  s.flag = reinterpret_cast<unsigned char *>(s.plist + maxp);
  return s;
}

// g = bs - Gs u with Gs = D^-1 G D^-1 (D = diag(dg)), using v = u / dg.
__device__ void grad(const double *G, int64_t ld, int p, const Smem &S) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int a = tid; a < p; a += NT) S.v[a] = S.u[a] / S.dg[a];
  __syncthreads();
  for (int a = wave; a < p; a += NT / 64) {
    double acc = 0.0;
    for (int b = lane; b < p; b += 64) acc = fma(G[a * ld + b], S.v[b], acc);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) S.g[a] = S.bs[a] - acc / S.dg[a];
  }
  __syncthreads();
}

// Least squares on the passive set with feasibility back-tracking.  Returns
// with u optimal on its (possibly reduced) passive set.  just_added: the
// variable that entered last (or -1); if its own solution component is not
// positive on the first solve it is blocked for this fit (the safeguard of
// Lawson and Hanson against cycling on round-off).
__device__ void solve_passive(const double *G, int64_t ld, int p, const Smem &S, int just_added, int *status,
                              Red *red) {
  __shared__ int sh_np, sh_fail, sh_kmin, sh_first;
  __shared__ double sh_alpha;
  const int tid = threadIdx.x;
  if (tid == 0) sh_first = 1;
  for (int guard = 0; guard < 2 * p + 4; ++guard) {
    __syncthreads();
    if (tid == 0) {
      int k = 0;
      for (int a = 0; a < p; ++a)
        if (S.flag[a] & F_PASSIVE) S.plist[k++] = a;
      sh_np = k;
      sh_fail = -1;
    }
    __syncthreads();
    const int np = sh_np;
    if (np == 0) {
      for (int a = tid; a < p; a += NT) S.u[a] = 0.0;
      __syncthreads();
      return;
    }
    const int ne = tri(np);
    for (int e = tid; e < ne; e += NT) {
      int r, c;
      decode_tri(e, &r, &c);
      const int ar = S.plist[r], ac = S.plist[c];
      S.L[e] = G[ar * ld + ac] / (S.dg[ar] * S.dg[ac]);
    }
    __syncthreads();
    // right-looking Cholesky of the packed free block
    for (int k = 0; k < np; ++k) {
      if (tid == 0) {
        const double piv = S.L[tri(k) + k];
        if (!(piv > 1e-14)) sh_fail = k;
        else S.L[tri(k) + k] = sqrt(piv);
      }
      __syncthreads();
      if (sh_fail >= 0) break;
      const double dkk = S.L[tri(k) + k];
      for (int r = k + 1 + tid; r < np; r += NT) S.L[tri(r) + k] /= dkk;
      __syncthreads();
      const int mm = np - k - 1;
      const int nt = tri(mm);
      for (int e = tid; e < nt; e += NT) {
        int r, c;
        decode_tri(e, &r, &c);
        r += k + 1;
        c += k + 1;
        S.L[tri(r) + c] -= S.L[tri(r) + k] * S.L[tri(c) + k];
      }
      __syncthreads();
    }
    if (sh_fail >= 0) {
      // the failing variable depends linearly on the ones before it: drop it for this fit
      if (tid == 0) {
        const int a = S.plist[sh_fail];
        S.flag[a] = F_BLOCKED;
        S.u[a] = 0.0;
        *status |= int(AMC_HS_NNLS_SINGULAR);
        sh_first = 0;
      }
      continue;
    }
    // forward then backward substitution: y = L^-T L^-1 bs_P
    for (int k = tid; k < np; k += NT) S.y[k] = S.bs[S.plist[k]];
    __syncthreads();
    for (int k = 0; k < np; ++k) {
      if (tid == 0) S.y[k] /= S.L[tri(k) + k];
      __syncthreads();
      const double yk = S.y[k];
      for (int r = k + 1 + tid; r < np; r += NT) S.y[r] -= S.L[tri(r) + k] * yk;
      __syncthreads();
    }
    for (int k = np - 1; k >= 0; --k) {
      if (tid == 0) S.y[k] /= S.L[tri(k) + k];
      __syncthreads();
      const double yk = S.y[k];
      for (int r = tid; r < k; r += NT) S.y[r] -= S.L[tri(k) + r] * yk;
      __syncthreads();
    }
    // feasibility
    double ratio = INFINITY;
    int kk = -1;
    for (int k = tid; k < np; k += NT) {
      if (S.y[k] <= 0.0) {
        const double ua = S.u[S.plist[k]];
        const double den = ua - S.y[k];
        const double rt = den > 0.0 ? ua / den : 0.0;
        if (kk < 0 || rt < ratio) {
          ratio = rt;
          kk = k;
        }
      }
    }
    double best;
    const int kmin = block_argmax(kk >= 0 ? -ratio : -INFINITY, kk, red, &best);
    if (kmin < 0) {
      for (int a = tid; a < p; a += NT) S.u[a] = 0.0;
      __syncthreads();
      for (int k = tid; k < np; k += NT) S.u[S.plist[k]] = S.y[k];
      __syncthreads();
      return;
    }
    if (tid == 0) {
      sh_alpha = -best;
      sh_kmin = kmin;
    }
    __syncthreads();
    if (sh_first && just_added >= 0 && S.plist[sh_kmin] == just_added && S.u[just_added] == 0.0) {
      // the entering variable does not take a positive value: block it, keep u
      __syncthreads();
      if (tid == 0) {
        S.flag[just_added] = F_BLOCKED;
        S.u[just_added] = 0.0;
      }
      __syncthreads();
      return;
    }
    const double alpha = sh_alpha;
    for (int k = tid; k < np; k += NT) {
      const int a = S.plist[k];
      S.u[a] += alpha * (S.y[k] - S.u[a]);
    }
    __syncthreads();
    if (tid == 0) {
      S.u[S.plist[sh_kmin]] = 0.0;
      sh_first = 0;
    }
    __syncthreads();
    for (int k = tid; k < np; k += NT) {
      const int a = S.plist[k];
      if (!(S.u[a] > 0.0)) {
        S.u[a] = 0.0;
        S.flag[a] &= ~F_PASSIVE;
      }
    }
  }
  __syncthreads();
}

// Solves one system.  nwarm: entries of w used as the warm start (the rest start at 0).
__device__ void nnls_block(const double *G, int64_t ld, int p, const double *b, double *w, int nwarm,
                           const NnlsParams np_, char *smem, int maxp, int *iters_out, int *status_out) {
  __shared__ Red red;
  __shared__ int sh_status, sh_iters;
  const int tid = threadIdx.x;
  Smem S = carve(smem, maxp);
  if (tid == 0) {
    sh_status = 0;
    sh_iters = 0;
  }
  double bl = 0.0;
  for (int a = tid; a < p; a += NT) {
    const double gaa = G[a * ld + a];
    unsigned char f = 0;
    double dg = sqrt(gaa);
    if (!(dg > 0.0) || !isfinite(dg)) {
      dg = 1.0;
      f = F_BLOCKED;
    }
    S.dg[a] = dg;
    const double bs = f ? 0.0 : b[a] / dg;
    S.bs[a] = bs;
    const double u0 = (a < nwarm && !f) ? fmax(w[a], 0.0) * dg : 0.0;
    S.u[a] = u0 > 0.0 ? u0 : 0.0;
    S.flag[a] = f;
    bl = fmax(bl, fabs(bs));
  }
  double bmax;
  (void)block_argmax(bl, 0, &red, &bmax);
  const double tol = (np_.tol > 0.0 ? np_.tol : 10.0 * DBL_EPSILON * double(p)) * bmax;
  const int cap = np_.max_iters > 0 ? np_.max_iters : 3 * p + 30;

  if (bmax > 0.0 && isfinite(bmax)) {
    // projected-gradient warm-up, step 1/L with L a Gershgorin bound of Gs
    if (np_.pg_iters > 0) {
      double rs = 0.0;
      const int lane = tid & 63, wave = tid >> 6;
      double rowmax = 0.0;
      for (int a = wave; a < p; a += NT / 64) {
        double acc = 0.0;
        for (int c = lane; c < p; c += 64) acc += fabs(G[a * ld + c]) / S.dg[c];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
        if (!(S.flag[a] & F_BLOCKED)) rowmax = fmax(rowmax, acc / S.dg[a]);
      }
      (void)rs;
      double Lmax;
      (void)block_argmax(rowmax, 0, &red, &Lmax);
      const double step = Lmax > 0.0 ? 1.0 / Lmax : 0.0;
      for (int it = 0; it < np_.pg_iters; ++it) {
        grad(G, ld, p, S);
        for (int a = tid; a < p; a += NT)
          if (!(S.flag[a] & F_BLOCKED)) S.u[a] = fmax(0.0, S.u[a] + step * S.g[a]);
        __syncthreads();
      }
    }
    for (int a = tid; a < p; a += NT)
      if (S.u[a] > 0.0) S.flag[a] |= F_PASSIVE;
    __syncthreads();
    int anyp = 0;
    for (int a = tid; a < p; a += NT) anyp |= (S.flag[a] & F_PASSIVE) ? 1 : 0;
    if (block_sum(double(anyp), &red) > 0.0) solve_passive(G, ld, p, S, -1, &sh_status, &red);
    int iters = 0;
    for (;;) {
      grad(G, ld, p, S);
      double gv = -INFINITY;
      int gi = -1;
      for (int a = tid; a < p; a += NT) {
        if (!(S.flag[a] & (F_PASSIVE | F_BLOCKED)) && (gi < 0 || S.g[a] > gv)) {
          gv = S.g[a];
          gi = a;
        }
      }
      double best;
      const int j = block_argmax(gv, gi, &red, &best);
      if (j < 0 || !(best > tol)) break;
      if (iters >= cap) {
        if (tid == 0) sh_status |= int(AMC_HS_NNLS_CAP);
        break;
      }
      ++iters;
      __syncthreads();
      if (tid == 0) S.flag[j] |= F_PASSIVE;
      __syncthreads();
      solve_passive(G, ld, p, S, j, &sh_status, &red);
    }
    if (tid == 0) sh_iters = iters;
  } else {
    for (int a = tid; a < p; a += NT) S.u[a] = 0.0;
  }
  __syncthreads();
  for (int a = tid; a < p; a += NT) w[a] = S.u[a] / S.dg[a];
  if (tid == 0) {
    *iters_out = sh_iters;
    *status_out = sh_status;
  }
}

__host__ __device__ constexpr size_t nnls_smem_bytes(int maxp) {
  return size_t(8) * (size_t(maxp) * (maxp + 1) / 2 + 6 * size_t(maxp)) + 4 * size_t(maxp) + size_t(maxp) + 16;
}

__global__ __launch_bounds__(NT) void k_nnls_cycle(const HeadDesc *__restrict__ desc, const double *__restrict__ G,
                                                   const double *__restrict__ bvec, double *__restrict__ w, int cycle,
                                                   int kR, NnlsParams np_, int maxp, int32_t *__restrict__ tr_iters,
                                                   double *__restrict__ tr_weight,
                                                   int32_t *__restrict__ head_status) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int h = blockIdx.x;
  const HeadDesc D = desc[h];
  const int64_t S0 = int64_t(cycle) * kR;
  if (S0 >= D.t) return;
  const int Kc = int(D.t - S0 < kR ? D.t - S0 : kR);
  const int p = int(S0) + Kc;
  int iters = 0, status = 0;
  nnls_block(G + D.tt_off, D.t, p, bvec + D.t_off, w + D.t_off, int(S0), np_, smem, maxp, &iters, &status);
  __syncthreads();
  if (threadIdx.x == 0) {
    if (tr_iters) tr_iters[D.cyc_off + cycle] = iters;
    if (status && head_status) atomicOr(head_status + h, status);
  }
  if (tr_weight)
    for (int a = threadIdx.x; a < p; a += NT) tr_weight[D.t_off + a] = w[D.t_off + a];
}

struct NnlsChunk {
  int count;
  int64_t cu_t[65];
  int64_t cu_t2[65];
};

__global__ __launch_bounds__(NT) void k_nnls_batched(NnlsChunk ch, int base, const double *__restrict__ G,
                                                     const double *__restrict__ g, double *__restrict__ w, int warm,
                                                     NnlsParams np_, int maxp, int32_t *__restrict__ iters,
                                                     int32_t *__restrict__ status) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int i = blockIdx.x;
  if (i >= ch.count) return;
  const int64_t t0 = ch.cu_t[i];
  const int p = int(ch.cu_t[i + 1] - t0);
  int it = 0, st = 0;
  nnls_block(G + ch.cu_t2[i], p, p, g + t0, w + t0, warm ? p : 0, np_, smem, maxp, &it, &st);
  if (threadIdx.x == 0) {
    if (iters) iters[base + i] = it;
    if (status) status[base + i] = st;
  }
}

}  // namespace

hipError_t launch_nnls(const Dims &dm, const Buffers &b, int cycle, int kR, const NnlsParams &np,
                       hipStream_t s) {
  const int maxp = int(dm.max_t);
  const size_t bytes = nnls_smem_bytes(maxp);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_nnls_cycle),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, int(bytes));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_nnls_cycle, dim3(unsigned(dm.H)), dim3(NT), bytes, s, b.desc, b.G, b.bvec, b.w, cycle, kR,
                     np, maxp, b.tr_iters, b.tr_weight, b.head_status);
  return hipGetLastError();
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
