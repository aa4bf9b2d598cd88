// NNLS bias fit: w = argmin_{w >= 0} 0.5 w^T G w - b^T w, the Gram form of
// min ||Phi_S w - m|| (zhichai.net deep-dive, section 1.6: refit w by NNLS
// after every pick; xinfinite.net article, section 2, step 2).
//
// The pages' GPU solver is projected gradient (xinfinite.net article,
// Fig. 2).  On these Gram matrices (condition numbers 1e9 and beyond)
// projected gradient alone does not reach the minimiser, so the exact
// minimiser is found by an active-set method on the Gram form (Bro and
// De Jong's fast NNLS): the most violating zero variable enters, the
// least-squares solution on the free set is computed from a Cholesky factor,
// and if it leaves the feasible set the iterate steps back and the blocking
// variables leave.  Projected gradient survives as the warm-up of the
// stand-alone solver (amc_nnls).
//
// Accuracy.  Everything is float64 in unit-diagonal form (w = u / sqrt(diag
// G)).  The solver works in correction form: it keeps the gradient
// g = b - G u explicitly, moves by corrections d = G_PP^-1 g_P solved with the
// factor, and updates g by -G d.  Inside a compaction each refit starts from
// g = Phi_S^T r computed from the float64 panel and the float64 residual of
// the previous refit (the corrected semi-normal equations of Bjorck), so the
// gradient never suffers the cancellation of b - G u, and a final refit with
// no new key refines the weights once more.
//
// The factor is updated, not recomputed: a variable that enters appends one
// row (a forward substitution); a variable that leaves is deleted by a row
// shift plus a rank-one update of the trailing block.  Between the refits of
// one compaction the factor and the free set persist in the workspace.  The
// sequential passes run in one wave with vectors spread over the lanes'
// registers (index i lives in lane i % 64, slot i / 64); the mat-vecs use the
// whole block.  The packed factor of up to 192 variables lives in LDS.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <climits>
#include <cmath>

#include "amc_internal.h"

namespace amc {
namespace {

constexpr int NT = 256;
constexpr int NR = (kLdsMaxT + 63) / 64;  // register slots per lane for a vector of length <= kLdsMaxT
constexpr unsigned char F_PASSIVE = 1, F_BLOCKED = 2;
constexpr double PIV_TOL = 1e-14;  // smallest acceptable squared pivot in unit-diagonal form

__device__ __forceinline__ int tri(int r) { return r * (r + 1) / 2; }

__device__ __forceinline__ void wsync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// element k of a lane-distributed vector, broadcast to every lane.  Written
// as selects over all slots so the vector stays in registers.
__device__ __forceinline__ double getv(const double (&r)[NR], int k) {
  const int s = k >> 6;
  double x = r[0];
#pragma unroll
  for (int m = 1; m < NR; ++m) x = (s == m) ? r[m] : x;
  return __shfl(x, k & 63);
}

__device__ __forceinline__ void setv(double (&r)[NR], int k, double v) {
  const bool mine = lane_id() == (k & 63);
  const int s = k >> 6;
#pragma unroll
  for (int m = 0; m < NR; ++m) r[m] = (mine && s == m) ? v : r[m];
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
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

// LDS state of one solve
struct St {
  double *L;      // packed lower factor of Gs_PP, rows in free-set order
  double *rdiag;  // 1 / L_kk
  double *u;      // scaled iterate, per variable
  double *g;      // scaled gradient bs - Gs u, per variable
  double *dg;     // sqrt(G_aa)
  double *bs;     // b_a / dg_a
  double *delta;  // step of the free variables, in factor order
  int *plist;     // free set in factor order
  int *np;        // free-set size
  int *ctl;       // wave-0 decision broadcast to the block
  unsigned char *flag;
};

__device__ St carve(char *base, int maxp) {
  St s;
  double *d = reinterpret_cast<double *>(base);
  s.L = d;
  d += tri(maxp);
  s.rdiag = d;
  d += maxp;
  s.u = d;
  d += maxp;
  s.g = d;
  d += maxp;
  s.dg = d;
  d += maxp;
  s.bs = d;
  d += maxp;
  s.delta = d;
  d += maxp;
  s.plist = reinterpret_cast<int *>(d);
  s.np = s.plist + maxp;
  s.ctl = s.np + 1;
  s.flag = reinterpret_cast<unsigned char *>(s.ctl + 1);
  return s;
}

__host__ __device__ constexpr size_t nnls_smem_bytes(int maxp) {
  return size_t(8) * (size_t(maxp) * (maxp + 1) / 2 + 6 * size_t(maxp)) + 4 * (size_t(maxp) + 2) + size_t(maxp) + 16;
}

// ---- wave-0 routines ------------------------------------------------------

// L x = r (forward), leading n rows
__device__ __forceinline__ void fwd(const St &S, int n, double (&r)[NR]) {
  const int lane = lane_id();
  for (int k = 0; k < n; ++k) {
    const double xk = getv(r, k) * S.rdiag[k];
    setv(r, k, xk);
#pragma unroll
    for (int m = 0; m < NR; ++m) {
      const int i = lane + 64 * m;
      if (i > k && i < n) r[m] = fma(-S.L[tri(i) + k], xk, r[m]);
    }
  }
}

// L^T x = r (backward), leading n rows
__device__ __forceinline__ void bwd(const St &S, int n, double (&r)[NR]) {
  const int lane = lane_id();
  for (int k = n - 1; k >= 0; --k) {
    const double xk = getv(r, k) * S.rdiag[k];
    setv(r, k, xk);
    const int base = tri(k);
#pragma unroll
    for (int m = 0; m < NR; ++m) {
      const int i = lane + 64 * m;
      if (i < k) r[m] = fma(-S.L[base + i], xk, r[m]);
    }
  }
}

// Appends variable j to the factor.  Returns false (and changes nothing) if
// its column is numerically dependent on the free set.
__device__ __forceinline__ bool append(const St &S, const double *G, int64_t ld, int j) {
  const int lane = lane_id();
  const int np = *S.np;
  const double dj = S.dg[j];
  double c[NR];
#pragma unroll
  for (int m = 0; m < NR; ++m) {
    const int k = lane + 64 * m;
    double v = 0.0;
    if (k < np) {
      const int a = S.plist[k];
      v = G[int64_t(j) * ld + a] / (S.dg[a] * dj);
    }
    c[m] = v;
  }
  fwd(S, np, c);
  double ss = 0.0;
#pragma unroll
  for (int m = 0; m < NR; ++m) {
    const int k = lane + 64 * m;
    if (k < np) ss = fma(c[m], c[m], ss);
  }
  ss = wave_sum(ss);
  const double gjj = G[int64_t(j) * ld + j] / (dj * dj);
  const double d2 = gjj - ss;
  if (!(d2 > PIV_TOL)) return false;
  const double djj = sqrt(d2);
  const int base = tri(np);
#pragma unroll
  for (int m = 0; m < NR; ++m) {
    const int k = lane + 64 * m;
    if (k < np) S.L[base + k] = c[m];
  }
  if (lane == 0) {
    S.L[base + np] = djj;
    S.rdiag[np] = 1.0 / djj;
    S.plist[np] = j;
    S.flag[j] |= F_PASSIVE;
    *S.np = np + 1;
  }
  wsync();
  return true;
}

// Deletes factor position q: rows below shift up without column q, then the
// trailing block absorbs the removed column by a rank-one update.
__device__ __forceinline__ void remove_at(const St &S, int q) {
  const int lane = lane_id();
  const int np = *S.np;
  double x[NR];
#pragma unroll
  for (int m = 0; m < NR; ++m) x[m] = 0.0;
  for (int i = q + 1; i < np; ++i) {
    double v[NR];
#pragma unroll
    for (int m = 0; m < NR; ++m) {
      const int c = lane + 64 * m;
      v[m] = c <= i ? S.L[tri(i) + c] : 0.0;
    }
    const double xi = S.L[tri(i) + q];
    // new row i-1, entry c' = old entry c' (c' < q) or old entry c'+1 (c' >= q)
    double nv[NR];
#pragma unroll
    for (int m = 0; m < NR; ++m) {
      const double right_same = __shfl(v[m], (lane + 1) & 63);
      const double right_next = (m + 1 < NR) ? __shfl(v[m + 1 < NR ? m + 1 : m], 0) : 0.0;
      const double right = lane == 63 ? right_next : right_same;
      const int cp = lane + 64 * m;
      nv[m] = cp < q ? v[m] : right;
    }
    wsync();
    const int nb = tri(i - 1);
#pragma unroll
    for (int m = 0; m < NR; ++m) {
      const int cp = lane + 64 * m;
      if (cp <= i - 1) S.L[nb + cp] = nv[m];
    }
    setv(x, i - 1, xi);
    wsync();
  }
  int pv[NR];
#pragma unroll
  for (int m = 0; m < NR; ++m) {
    const int k = lane + 64 * m;
    pv[m] = (k + 1 < np) ? S.plist[k + 1] : 0;
  }
  wsync();
#pragma unroll
  for (int m = 0; m < NR; ++m) {
    const int k = lane + 64 * m;
    if (k >= q && k < np - 1) S.plist[k] = pv[m];
  }
  if (lane == 0) *S.np = np - 1;
  wsync();
  const int n2 = np - 1;
  // rank-one update: L33' L33'^T = L33 L33^T + x x^T on positions q..n2-1
  for (int k = q; k < n2; ++k) {
    const double lkk = S.L[tri(k) + k];
    const double xk = getv(x, k);
    const double r = sqrt(lkk * lkk + xk * xk);
    const double cc = r / lkk, s = xk / lkk;
#pragma unroll
    for (int m = 0; m < NR; ++m) {
      const int i = lane + 64 * m;
      if (i > k && i < n2) {
        const double lik = (S.L[tri(i) + k] + s * x[m]) / cc;
        S.L[tri(i) + k] = lik;
        x[m] = cc * x[m] - s * lik;
      }
    }
    if (lane == 0) {
      S.L[tri(k) + k] = r;
      S.rdiag[k] = 1.0 / r;
    }
    wsync();
  }
}

// ---- block routines -------------------------------------------------------

// g_a -= sum_k Gs[a][P_k] delta_k for every variable a < p (G is symmetric, so
// row P_k of G is read contiguously).
__device__ void grad_update(const St &S, const double *G, int64_t ld, int p) {
  const int np = *S.np;
  for (int a = threadIdx.x; a < p; a += NT) {
    double acc = 0.0;
    for (int k = 0; k < np; ++k) {
      const double dk = S.delta[k];
      if (dk != 0.0) {
        const int c = S.plist[k];
        acc = fma(G[int64_t(c) * ld + a], dk / S.dg[c], acc);
      }
    }
    S.g[a] -= acc / S.dg[a];
  }
}

enum { CTL_DONE = 1, CTL_PARTIAL = 2, CTL_DROP = 3 };

// Least squares on the free set in correction form, with feasibility
// back-tracking, starting from a feasible u whose support is the free set.
// entering: the variable that just entered (or -1); if on the first solve it
// alone blocks, it is set aside for the rest of this fit (Lawson and Hanson's
// guard against cycling on round-off).
__device__ void settle(const St &S, const double *G, int64_t ld, int p, int entering) {
  const int tid = threadIdx.x, wave = tid >> 6;
  bool first = true;
  for (int guard = 0; guard < kLdsMaxT + 4; ++guard) {
    __syncthreads();
    if (wave == 0) {
      const int lane = lane_id();
      const int np = *S.np;
      double d[NR];
#pragma unroll
      for (int m = 0; m < NR; ++m) {
        const int k = lane + 64 * m;
        d[m] = k < np ? S.g[S.plist[k]] : 0.0;
      }
      fwd(S, np, d);
      bwd(S, np, d);  // d = Gs_PP^-1 g_P: the step to the free-set optimum
      double best = INFINITY;
      int kb = -1;
#pragma unroll
      for (int m = 0; m < NR; ++m) {
        const int k = lane + 64 * m;
        if (k < np) {
          const double ua = S.u[S.plist[k]];
          const double z = ua + d[m];
          if (z <= 0.0) {
            const double rt = d[m] < 0.0 ? ua / (-d[m]) : 0.0;
            if (kb < 0 || rt < best) {
              best = rt;
              kb = k;
            }
          }
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const double ob = __shfl_xor(best, off);
        const int ok = __shfl_xor(kb, off);
        if (ok >= 0 && (kb < 0 || ob < best || (ob == best && ok < kb))) {
          best = ob;
          kb = ok;
        }
      }
      int ctl;
      if (kb < 0) {
        ctl = CTL_DONE;
#pragma unroll
        for (int m = 0; m < NR; ++m) {
          const int k = lane + 64 * m;
          if (k < np) S.delta[k] = d[m];
        }
      } else if (first && entering >= 0 && kb == np - 1 && S.plist[kb] == entering && S.u[entering] == 0.0) {
        ctl = CTL_DROP;
      } else {
        ctl = CTL_PARTIAL;
        const double alpha = best < 1.0 ? best : 1.0;
#pragma unroll
        for (int m = 0; m < NR; ++m) {
          const int k = lane + 64 * m;
          if (k < np) {
            const double ua = S.u[S.plist[k]];
            double un = (k == kb) ? 0.0 : fma(alpha, d[m], ua);
            if (!(un > 0.0)) un = 0.0;
            S.delta[k] = un - ua;
          }
        }
      }
      if (lane == 0) *S.ctl = ctl;
      wsync();
    }
    __syncthreads();
    const int ctl = *S.ctl;
    if (ctl == CTL_DROP) {
      if (tid == 0) {
        *S.np = *S.np - 1;
        S.flag[entering] = F_BLOCKED;
      }
      __syncthreads();
      return;
    }
    grad_update(S, G, ld, p);
    const int np = *S.np;
    for (int k = tid; k < np; k += NT) {
      const int a = S.plist[k];
      const double un = S.u[a] + S.delta[k];
      S.u[a] = un > 0.0 ? un : 0.0;
    }
    __syncthreads();
    if (ctl == CTL_DONE) return;
    first = false;
    if (wave == 0) {
      // every free variable that reached zero leaves (highest position first)
      for (int k = *S.np - 1; k >= 0; --k) {
        const int a = S.plist[k];
        if (!(S.u[a] > 0.0)) {
          wsync();
          if (lane_id() == 0) {
            S.u[a] = 0.0;
            S.flag[a] &= ~F_PASSIVE;
          }
          wsync();
          remove_at(S, k);
        }
      }
    }
  }
  __syncthreads();
}

// One block solves one system.
//   gA     : accurate unscaled gradient b - G w at the warm start (nullable:
//            then it is formed from G and b)
//   np_in, plist_in, L_in : persisted free set and factor (np_in = 0: none)
//   pg     : projected-gradient warm-up iterations (stand-alone solver only)
__device__ __forceinline__ void nnls_solve(const double *G, int64_t ld, int p, const double *b, const double *gA,
                                           double *w, int nwarm, const NnlsParams prm, char *smem, int maxp,
                                           int np_in, const int32_t *plist_in, const double *L_in, int pg,
                                           int *iters_out, int *status_out) {
  __shared__ Red red;
  __shared__ int sh_status;
  const int tid = threadIdx.x, wave = tid >> 6;
  St S = carve(smem, maxp);
  if (tid == 0) {
    sh_status = 0;
    *S.np = np_in;
  }
  double bl = 0.0;
  for (int a = tid; a < p; a += NT) {
    const double gaa = G[int64_t(a) * ld + a];
    double dg = sqrt(gaa);
    unsigned char f = 0;
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
  for (int e = tid; e < tri(np_in); e += NT) S.L[e] = L_in[e];
  __syncthreads();
  for (int k = tid; k < np_in; k += NT) {
    const int a = plist_in[k];
    S.plist[k] = a;
    S.flag[a] |= F_PASSIVE;
    S.rdiag[k] = 1.0 / S.L[tri(k) + k];
  }
  __syncthreads();
  // initial gradient
  if (gA) {
    for (int a = tid; a < p; a += NT) S.g[a] = (S.flag[a] & F_BLOCKED) ? 0.0 : gA[a] / S.dg[a];
  } else {
    for (int a = tid; a < p; a += NT) {
      double acc = 0.0;
      for (int c = 0; c < p; ++c) acc = fma(G[int64_t(c) * ld + a], S.u[c] / S.dg[c], acc);
      S.g[a] = S.bs[a] - acc / S.dg[a];
    }
  }
  double bmax;
  (void)block_argmax(bl, 0, &red, &bmax);
  const double tol = (prm.tol > 0.0 ? prm.tol : 10.0 * DBL_EPSILON * double(p)) * bmax;
  const int cap = prm.max_iters > 0 ? prm.max_iters : 3 * p + 30;
  int iters = 0;

  if (bmax > 0.0 && isfinite(bmax)) {
    if (pg > 0) {
      // projected-gradient warm-up (step 1/L, L a Gershgorin bound of Gs)
      double rowmax = 0.0;
      for (int a = tid; a < p; a += NT) {
        double acc = 0.0;
        for (int c = 0; c < p; ++c) acc += fabs(G[int64_t(c) * ld + a]) / S.dg[c];
        if (!(S.flag[a] & F_BLOCKED)) rowmax = fmax(rowmax, acc / S.dg[a]);
      }
      double Lmax;
      (void)block_argmax(rowmax, 0, &red, &Lmax);
      const double step = Lmax > 0.0 ? 1.0 / Lmax : 0.0;
      for (int it = 0; it < pg; ++it) {
        __syncthreads();
        for (int a = tid; a < p; a += NT)
          S.delta[a] = (S.flag[a] & F_BLOCKED) ? 0.0 : fmax(0.0, S.u[a] + step * S.g[a]) - S.u[a];
        __syncthreads();
        for (int a = tid; a < p; a += NT) {
          double acc = 0.0;
          for (int c = 0; c < p; ++c) acc = fma(G[int64_t(c) * ld + a], S.delta[c] / S.dg[c], acc);
          S.g[a] -= acc / S.dg[a];
        }
        __syncthreads();
        for (int a = tid; a < p; a += NT) S.u[a] += S.delta[a];
      }
      __syncthreads();
    }
    if (np_in == 0) {
      // the support of the warm start becomes the free set
      if (wave == 0) {
        for (int a = 0; a < p; ++a) {
          if (S.u[a] > 0.0 && !(S.flag[a] & F_PASSIVE) && !append(S, G, ld, a)) {
            if (lane_id() == 0) S.flag[a] = F_BLOCKED;
            wsync();
          }
        }
      }
      __syncthreads();
      // a dependent variable dropped here still carries weight: take it out of u and g
      for (int a = tid; a < p; a += NT) S.delta[a] = ((S.flag[a] & F_BLOCKED) && S.u[a] > 0.0) ? -S.u[a] : 0.0;
      __syncthreads();
      for (int a = tid; a < p; a += NT) {
        double acc = 0.0;
        for (int c = 0; c < p; ++c)
          if (S.delta[c] != 0.0) acc = fma(G[int64_t(c) * ld + a], S.delta[c] / S.dg[c], acc);
        S.g[a] -= acc / S.dg[a];
      }
      __syncthreads();
      for (int a = tid; a < p; a += NT)
        if (S.flag[a] & F_BLOCKED) S.u[a] = 0.0;
      __syncthreads();
      if (*S.np > 0) settle(S, G, ld, p, -1);
    } else {
      settle(S, G, ld, p, -1);  // refine the persisted optimum with the accurate gradient
    }
    for (;;) {
      __syncthreads();
      double gv = -INFINITY;
      int gi = -1;
      for (int a = tid; a < p; a += NT) {
        if (S.flag[a] & (F_PASSIVE | F_BLOCKED)) continue;
        if (gi < 0 || S.g[a] > gv) {
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
      if (wave == 0) {
        const bool ok = append(S, G, ld, j);
        if (lane_id() == 0) {
          *S.ctl = ok ? 1 : 0;
          if (!ok) {
            S.flag[j] = F_BLOCKED;
            sh_status |= int(AMC_HS_NNLS_SINGULAR);
          }
        }
        wsync();
      }
      __syncthreads();
      if (*S.ctl) settle(S, G, ld, p, j);
    }
  }
  __syncthreads();
  for (int a = tid; a < p; a += NT) w[a] = S.u[a] / S.dg[a];
  if (tid == 0) {
    *iters_out = iters;
    *status_out = sh_status;
  }
}

// One refit per head.  polish: no new key; refine the last fit (p = t).
__global__ __launch_bounds__(NT) void k_nnls_cycle(const HeadDesc *__restrict__ desc, const double *__restrict__ G,
                                                   const double *__restrict__ bvec, const double *__restrict__ gA,
                                                   double *__restrict__ w, int cycle, int kR, int polish,
                                                   NnlsParams prm, int maxp, double *__restrict__ nn_L,
                                                   int32_t *__restrict__ nn_P, int32_t *__restrict__ nn_np,
                                                   int32_t *__restrict__ tr_iters, double *__restrict__ tr_weight,
                                                   int32_t *__restrict__ head_status) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int h = blockIdx.x;
  const HeadDesc D = desc[h];
  int64_t S0;
  int Kc;
  if (polish) {
    S0 = D.t;
    Kc = 0;
  } else {
    S0 = int64_t(cycle) * kR;
    if (S0 >= D.t) return;
    Kc = int(D.t - S0 < kR ? D.t - S0 : kR);
  }
  const int p = int(S0) + Kc;
  const int np_in = S0 == 0 ? 0 : nn_np[h];
  int iters = 0, status = 0;
  nnls_solve(G + D.tt_off, D.t, p, bvec + D.t_off, gA + D.t_off, w + D.t_off, int(S0), prm, smem, maxp, np_in,
             nn_P + D.t_off, nn_L + D.tri_off, 0, &iters, &status);
  St S = carve(smem, maxp);
  __syncthreads();
  const int np = *S.np;
  for (int e = threadIdx.x; e < tri(np); e += NT) nn_L[D.tri_off + e] = S.L[e];
  for (int k = threadIdx.x; k < np; k += NT) nn_P[D.t_off + k] = S.plist[k];
  if (threadIdx.x == 0) {
    nn_np[h] = np;
    if (tr_iters && !polish) tr_iters[D.cyc_off + cycle] = iters;
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
                                                     NnlsParams prm, int maxp, int32_t *__restrict__ iters,
                                                     int32_t *__restrict__ status) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int i = blockIdx.x;
  if (i >= ch.count) return;
  const int64_t t0 = ch.cu_t[i];
  const int p = int(ch.cu_t[i + 1] - t0);
  int it = 0, st = 0;
  nnls_solve(G + ch.cu_t2[i], p, p, g + t0, nullptr, w + t0, warm ? p : 0, prm, smem, maxp, 0, nullptr, nullptr,
             prm.pg_iters, &it, &st);
  if (threadIdx.x == 0) {
    if (iters) iters[base + i] = it;
    if (status) status[base + i] = st;
  }
}

}  // namespace

hipError_t launch_nnls(const Dims &dm, const Buffers &b, int cycle, int kR, int polish, const NnlsParams &np,
                       hipStream_t s) {
  const int maxp = int(dm.max_t);
  const size_t bytes = nnls_smem_bytes(maxp);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_nnls_cycle),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, int(bytes));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_nnls_cycle, dim3(unsigned(dm.H)), dim3(NT), bytes, s, b.desc, b.G, b.bvec, b.gA, b.w, cycle,
                     kR, polish, np, maxp, b.nn_L, b.nn_P, b.nn_np, b.tr_iters, b.tr_weight, b.head_status);
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
