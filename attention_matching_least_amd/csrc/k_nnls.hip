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
// The factor is updated, not recomputed.  Up to eight zero variables with a
// positive gradient enter together: one forward substitution with several
// right-hand sides gives their new factor rows and L^-1 g for the following
// solve, and a small Cholesky of the block finishes the rows.  A variable
// that leaves is deleted by a row shift plus a rank-one update of the
// trailing block.  Between the refits of one compaction the factor and the
// free set persist in the workspace.  The sequential passes run in one wave
// with vectors spread over the lanes' registers (index i lives in lane i % 64,
// slot i / 64, broadcast with v_readlane); the mat-vecs use the whole block.
// The packed factor of up to 192 variables lives in LDS.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <climits>
#include <cmath>
#include <type_traits>

#include "amc_internal.h"

namespace amc {
namespace {

constexpr int NT = 256;
constexpr int NR = (kLdsMaxT + 63) / 64;  // register slots per lane for a vector of length <= kLdsMaxT
constexpr int NB = 8;  // zero variables that may enter together
constexpr unsigned char F_PASSIVE = 1, F_BLOCKED = 2, F_NEW = 4;
constexpr double PIV_TOL = 1e-14;  // smallest acceptable squared pivot in unit-diagonal form

__device__ __forceinline__ int tri(int r) { return r * (r + 1) / 2; }

__device__ __forceinline__ void wsync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Compile-time loop: f(integral_constant<int, I>) for I in [B, E).  Register
// arrays indexed only through it keep constant indices from the front end
// on, so they are never demoted to scratch memory.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// double broadcast from a (wave-uniform) lane
__device__ __forceinline__ double rl(double x, int lane) {
  const int lo = __builtin_amdgcn_readlane(__double2loint(x), lane);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(x), lane);
  return __hiloint2double(hi, lo);
}

// element k of a lane-distributed vector, broadcast to every lane
__device__ __forceinline__ double getv(const double (&r)[NR], int k) {
  const int s = k >> 6;
  double x = r[0];
  static_for<1, NR>([&](auto M) {
    constexpr int m = M;
    x = (s == m) ? r[m] : x;
  });
  return rl(x, k & 63);
}

__device__ __forceinline__ void setv(double (&r)[NR], int k, double v) {
  const bool mine = lane_id() == (k & 63);
  const int s = k >> 6;
  static_for<0, NR>([&](auto M) {
    constexpr int m = M;
    r[m] = (mine && s == m) ? v : r[m];
  });
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
__device__ __forceinline__ int block_argmax(double v, int idx, Red *red, double *out_v) {
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
  double *blk;    // block-append scratch: dot products and block rows
  int *plist;     // free set in factor order
  int *cand;      // entering candidates
  int *np;        // free-set size
  int *ctl;       // wave-0 decisions broadcast to the block: [0] settle step, [1] candidates,
                  // [2] free-set size, [3] enter one at a time from now on
  unsigned char *flag;
};

constexpr int BLK_DOUBLES = (NB + 1) * (NB + 1) + NB * NB + 2 * NB;

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
  s.blk = d;
  d += BLK_DOUBLES;
  s.plist = reinterpret_cast<int *>(d);
  s.cand = s.plist + maxp;
  s.np = s.cand + NB;
  s.ctl = s.np + 1;
  s.flag = reinterpret_cast<unsigned char *>(s.ctl + 4);
  return s;
}

__host__ __device__ constexpr size_t nnls_smem_bytes(int maxp) {
  return size_t(8) * (size_t(maxp) * (maxp + 1) / 2 + 6 * size_t(maxp) + BLK_DOUBLES) +
         4 * (size_t(maxp) + NB + 5) + size_t(maxp) + 16;
}

// ---- wave-0 routines ------------------------------------------------------

// L x = r (forward) for B right-hand sides at once, leading n rows.  The
// column of L for the next step is loaded while the current one is applied.
template <int B>
__device__ __forceinline__ void fwd_multi(const St &S, int n, double (&r)[B][NR]) {
  const int lane = lane_id();
  double nxt[NR];
  static_for<0, NR>([&](auto I_m) {
    constexpr int m = decltype(I_m)::value;
    const int i = lane + 64 * m;
    nxt[m] = (i > 0 && i < n) ? S.L[tri(i)] : 0.0;
  });
  for (int k = 0; k < n; ++k) {
    double cur[NR];
    static_for<0, NR>([&](auto I_m) {
      constexpr int m = decltype(I_m)::value;
      cur[m] = nxt[m];
    });
    if (k + 1 < n) {
      static_for<0, NR>([&](auto I_m) {
        constexpr int m = decltype(I_m)::value;
        const int i = lane + 64 * m;
        nxt[m] = (i > k + 1 && i < n) ? S.L[tri(i) + k + 1] : 0.0;
      });
    }
    const double rk = S.rdiag[k];
    static_for<0, B>([&](auto I_b) {
      constexpr int b = decltype(I_b)::value;
      const double xk = getv(r[b], k) * rk;
      setv(r[b], k, xk);
      static_for<0, NR>([&](auto I_m) {
        constexpr int m = decltype(I_m)::value;
        r[b][m] = fma(-cur[m], xk, r[b][m]);
      });
    });
  }
}

// L^T x = r (backward), leading n rows
__device__ __forceinline__ void bwd(const St &S, int n, double (&r)[NR]) {
  const int lane = lane_id();
  double nxt[NR];
  static_for<0, NR>([&](auto I_m) {
    constexpr int m = decltype(I_m)::value;
    const int i = lane + 64 * m;
    nxt[m] = (n > 0 && i < n - 1) ? S.L[tri(n - 1) + i] : 0.0;
  });
  for (int k = n - 1; k >= 0; --k) {
    double cur[NR];
    static_for<0, NR>([&](auto I_m) {
      constexpr int m = decltype(I_m)::value;
      cur[m] = nxt[m];
    });
    if (k > 0) {
      static_for<0, NR>([&](auto I_m) {
        constexpr int m = decltype(I_m)::value;
        const int i = lane + 64 * m;
        nxt[m] = (i < k - 1) ? S.L[tri(k - 1) + i] : 0.0;
      });
    }
    const double xk = getv(r, k) * S.rdiag[k];
    setv(r, k, xk);
    static_for<0, NR>([&](auto I_m) {
      constexpr int m = decltype(I_m)::value;
      r[m] = fma(-cur[m], xk, r[m]);
    });
  }
}

__device__ __forceinline__ double gs(const St &S, const double *G, int64_t ld, int a, int c) {
  return G[int64_t(a) * ld + c] / (S.dg[a] * S.dg[c]);
}

// Appends the nc <= NB candidates in S.cand (zero, not blocked) to the free
// set.  One forward pass over the current factor gives each candidate's row
// l = L^-1 Gs[P, j] and y_P = L^-1 g_P; the rows are finished by a Cholesky
// of the block (candidates whose pivot vanishes are blocked).  Returns
// y = L^-1 g_P over the extended free set in registers.
__device__ __forceinline__ void block_append(const St &S, const double *G, int64_t ld, int nc, double (&y)[NR],
                                             int *status) {
  const int lane = lane_id();
  const int np0 = *S.np;
  double r[NB + 1][NR];
  static_for<0, NR>([&](auto I_m) {
    constexpr int m = decltype(I_m)::value;
    const int k = lane + 64 * m;
    const int a = k < np0 ? S.plist[k] : 0;
    r[0][m] = k < np0 ? S.g[a] : 0.0;
    static_for<0, NB>([&](auto I_b) {
      constexpr int b = decltype(I_b)::value;
      r[b + 1][m] = (k < np0 && b < nc) ? gs(S, G, ld, S.cand[b], a) : 0.0;
    });
  });
  fwd_multi<NB + 1>(S, np0, r);
  // Gram of the block rows over the old columns: dots[b1][b2] = <r_b1, r_b2>, b = 0 is y
  double *dots = S.blk;                        // (NB+1) x (NB+1)
  double *E = S.blk + (NB + 1) * (NB + 1);     // NB x NB: block-row entries by accepted order
  double *Dg = E + NB * NB;                    // NB: diagonal of accepted rows
  double *yb = Dg + NB;                        // NB: y of accepted rows
  static_for<0, NB + 1>([&](auto I_b1) {
    constexpr int b1 = decltype(I_b1)::value;
    static_for<0, b1 + 1>([&](auto I_b2) {
      constexpr int b2 = decltype(I_b2)::value;
      if (b1 > nc || b2 > nc) return;
      double v = 0.0;
      static_for<0, NR>([&](auto I_m) {
        constexpr int m = decltype(I_m)::value;
        v = fma(r[b1][m], r[b2][m], v);
      });
      v = wave_sum(v);
      if (lane == 0) dots[b1 * (NB + 1) + b2] = v;
    });
  });
  wsync();
  // Cholesky of the block, identical in every lane (wave-uniform values);
  // loops are unrolled so the small arrays stay in registers
  int rank[NB], idx_of[NB];
  int nacc = 0;
  static_for<0, NB>([&](auto I_b) {
    constexpr int b = decltype(I_b)::value;
    rank[b] = -1;
    idx_of[b] = 0;
  });
  static_for<0, NB>([&](auto I_b) {
    constexpr int b = decltype(I_b)::value;
    if (b < nc) {
      const int j = S.cand[b];
      double row[NB];
      double ss = dots[(b + 1) * (NB + 1) + (b + 1)];
      double yy = S.g[j] - dots[(b + 1) * (NB + 1)];
      static_for<0, NB>([&](auto I_a) {
        constexpr int a = decltype(I_a)::value;
        row[a] = 0.0;
        if (a < nacc) {
          const int bb = idx_of[a];
          double v = gs(S, G, ld, j, S.cand[bb]) - dots[(b + 1) * (NB + 1) + (bb + 1)];
          static_for<0, a>([&](auto I_a2) {
            constexpr int a2 = decltype(I_a2)::value;
            v -= row[a2] * E[a * NB + a2];
          });
          v /= Dg[a];
          row[a] = v;
          ss += v * v;
          yy -= v * yb[a];
        }
      });
      const double d2 = gs(S, G, ld, j, j) - ss;
      if (d2 > PIV_TOL) {
        const double dd = sqrt(d2);
        rank[b] = nacc;
        static_for<0, NB>([&](auto I_a) {
          constexpr int a = decltype(I_a)::value;
          if (a == nacc) idx_of[a] = b;
        });
        if (lane == 0) {
          static_for<0, NB>([&](auto I_a) {
            constexpr int a = decltype(I_a)::value;
            if (a < nacc) E[nacc * NB + a] = row[a];
          });
          Dg[nacc] = dd;
          yb[nacc] = yy / dd;
        }
        wsync();
        ++nacc;
      } else {
        if (lane == 0) {
          S.flag[j] = F_BLOCKED;
          *status |= int(AMC_HS_NNLS_SINGULAR);
        }
        wsync();
      }
    }
  });
  // write the accepted rows
  static_for<0, NB>([&](auto I_b) {
    constexpr int b = decltype(I_b)::value;
    if (b >= nc || rank[b] < 0) return;
    const int pos = np0 + rank[b];
    const int base = tri(pos);
    static_for<0, NR>([&](auto I_m) {
      constexpr int m = decltype(I_m)::value;
      const int k = lane + 64 * m;
      if (k < np0) S.L[base + k] = r[b + 1][m];
    });
    const int ra = rank[b];
    for (int a = lane; a < ra; a += 64) S.L[base + np0 + a] = E[ra * NB + a];
    if (lane == 0) {
      S.L[base + pos] = Dg[ra];
      S.rdiag[pos] = 1.0 / Dg[ra];
      S.plist[pos] = S.cand[b];
      S.flag[S.cand[b]] |= F_PASSIVE | F_NEW;
    }
  });
  static_for<0, NR>([&](auto I_m) {
    constexpr int m = decltype(I_m)::value;
    y[m] = r[0][m];
  });
  for (int a = 0; a < nacc; ++a) setv(y, np0 + a, yb[a]);
  if (lane == 0) *S.np = np0 + nacc;
  wsync();
}

// Deletes factor position q: rows below shift up without column q, then the
// trailing block absorbs the removed column by a rank-one update.
__device__ __forceinline__ void remove_at(const St &S, int q) {
  const int lane = lane_id();
  const int np = *S.np;
  double x[NR];
  static_for<0, NR>([&](auto I_m) {
    constexpr int m = decltype(I_m)::value;
    x[m] = 0.0;
  });
  for (int i = q + 1; i < np; ++i) {
    double v[NR];
    static_for<0, NR>([&](auto I_m) {
      constexpr int m = decltype(I_m)::value;
      const int c = lane + 64 * m;
      v[m] = c <= i ? S.L[tri(i) + c] : 0.0;
    });
    const double xi = S.L[tri(i) + q];
    // new row i-1, entry c' = old entry c' (c' < q) or old entry c'+1 (c' >= q)
    double nv[NR];
    static_for<0, NR>([&](auto I_m) {
      constexpr int m = decltype(I_m)::value;
      const double right_same = __shfl(v[m], (lane + 1) & 63);
      const double right_next = (m + 1 < NR) ? __shfl(v[m + 1 < NR ? m + 1 : m], 0) : 0.0;
      const double right = lane == 63 ? right_next : right_same;
      const int cp = lane + 64 * m;
      nv[m] = cp < q ? v[m] : right;
    });
    wsync();
    const int nb = tri(i - 1);
    static_for<0, NR>([&](auto I_m) {
      constexpr int m = decltype(I_m)::value;
      const int cp = lane + 64 * m;
      if (cp <= i - 1) S.L[nb + cp] = nv[m];
    });
    setv(x, i - 1, xi);
    wsync();
  }
  int pv[NR];
  static_for<0, NR>([&](auto I_m) {
    constexpr int m = decltype(I_m)::value;
    const int k = lane + 64 * m;
    pv[m] = (k + 1 < np) ? S.plist[k + 1] : 0;
  });
  wsync();
  static_for<0, NR>([&](auto I_m) {
    constexpr int m = decltype(I_m)::value;
    const int k = lane + 64 * m;
    if (k >= q && k < np - 1) S.plist[k] = pv[m];
  });
  if (lane == 0) *S.np = np - 1;
  wsync();
  const int n2 = np - 1;
  // rank-one update: L33' L33'^T = L33 L33^T + x x^T on positions q..n2-1
  for (int k = q; k < n2; ++k) {
    const double lkk = S.L[tri(k) + k];
    const double xk = getv(x, k);
    const double r = sqrt(lkk * lkk + xk * xk);
    const double cc = r / lkk, s = xk / lkk;
    static_for<0, NR>([&](auto I_m) {
      constexpr int m = decltype(I_m)::value;
      const int i = lane + 64 * m;
      if (i > k && i < n2) {
        const double lik = (S.L[tri(i) + k] + s * x[m]) / cc;
        S.L[tri(i) + k] = lik;
        x[m] = cc * x[m] - s * lik;
      }
    });
    if (lane == 0) {
      S.L[tri(k) + k] = r;
      S.rdiag[k] = 1.0 / r;
    }
    wsync();
  }
}

// ---- block routines -------------------------------------------------------

// g_a -= sum_k Gs[a][P_k] delta_k for every variable a < p (G is symmetric, so
// row P_k of G is read contiguously across the threads).  Eight independent
// partial sums keep eight loads in flight per thread.
__device__ __forceinline__ void grad_update(const St &S, const double *G, int64_t ld, int p) {
  const int np = *S.np;
  for (int a = threadIdx.x; a < p; a += NT) {
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int k = 0;
    for (; k + 8 <= np; k += 8) {
      static_for<0, 8>([&](auto I_u) {
        constexpr int u = decltype(I_u)::value;
        const int c = S.plist[k + u];
        acc[u] = fma(G[int64_t(c) * ld + a], S.delta[k + u] / S.dg[c], acc[u]);
      });
    }
    for (; k < np; ++k) {
      const int c = S.plist[k];
      acc[0] = fma(G[int64_t(c) * ld + a], S.delta[k] / S.dg[c], acc[0]);
    }
    const double s = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
    S.g[a] -= s / S.dg[a];
  }
}

enum { CTL_DONE = 1, CTL_PARTIAL = 2, CTL_DROP = 3 };
constexpr unsigned char F_DROP = 8;

// Least squares on the free set in correction form, with feasibility
// back-tracking, starting from a feasible u whose support is the free set;
// variables that just entered sit at zero, flagged F_NEW.  have_y: y holds
// L^-1 g_P already.
//  - An entering variable whose solution is not positive leaves again before
//    any step is taken.  If it entered alone it is set aside for the rest of
//    this fit (Lawson and Hanson's guard against cycling on round-off);
//    otherwise ctl[3] is raised so that later candidates enter one at a time.
//  - Otherwise the iterate moves toward the solution, as far as feasibility
//    allows, and the variables that reach zero leave.
__device__ __forceinline__ void settle(const St &S, const double *G, int64_t ld, int p, double (&y)[NR], bool have_y,
                                       bool single) {
  const int tid = threadIdx.x, wave = tid >> 6;
  for (int guard = 0; guard < 2 * kLdsMaxT + 4; ++guard) {
    __syncthreads();
    if (wave == 0) {
      const int lane = lane_id();
      const int np = *S.np;
      double d[1][NR];
      if (have_y) {
        static_for<0, NR>([&](auto I_m) {
          constexpr int m = decltype(I_m)::value;
          d[0][m] = y[m];
        });
      } else {
        static_for<0, NR>([&](auto I_m) {
          constexpr int m = decltype(I_m)::value;
          const int k = lane + 64 * m;
          d[0][m] = k < np ? S.g[S.plist[k]] : 0.0;
        });
        fwd_multi<1>(S, np, d);
      }
      bwd(S, np, d[0]);  // d = Gs_PP^-1 g_P: the step to the free-set optimum
      // entering variables that do not turn positive
      int ndrop = 0;
      static_for<0, NR>([&](auto I_m) {
        constexpr int m = decltype(I_m)::value;
        const int k = lane + 64 * m;
        if (k < np) {
          const int a = S.plist[k];
          if ((S.flag[a] & F_NEW) && S.u[a] == 0.0 && !(d[0][m] > 0.0)) {
            S.flag[a] |= F_DROP;
            ++ndrop;
          }
        }
      });
      ndrop = int(wave_sum(double(ndrop)));
      int ctl;
      if (ndrop > 0) {
        ctl = CTL_DROP;
      } else {
        double best = INFINITY;
        int kb = -1;
        static_for<0, NR>([&](auto I_m) {
          constexpr int m = decltype(I_m)::value;
          const int k = lane + 64 * m;
          if (k < np) {
            const double ua = S.u[S.plist[k]];
            if (ua + d[0][m] <= 0.0) {
              const double rt = d[0][m] < 0.0 ? ua / (-d[0][m]) : 0.0;
              if (kb < 0 || rt < best) {
                best = rt;
                kb = k;
              }
            }
          }
        });
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
          const double ob = __shfl_xor(best, off);
          const int ok = __shfl_xor(kb, off);
          if (ok >= 0 && (kb < 0 || ob < best || (ob == best && ok < kb))) {
            best = ob;
            kb = ok;
          }
        }
        ctl = kb < 0 ? CTL_DONE : CTL_PARTIAL;
        const double alpha = kb < 0 ? 1.0 : (best < 1.0 ? best : 1.0);
        static_for<0, NR>([&](auto I_m) {
          constexpr int m = decltype(I_m)::value;
          const int k = lane + 64 * m;
          if (k < np) {
            const double ua = S.u[S.plist[k]];
            double un = (k == kb) ? 0.0 : fma(alpha, d[0][m], ua);
            if (!(un > 0.0)) un = 0.0;
            S.delta[k] = ctl == CTL_DONE ? d[0][m] : un - ua;
          }
        });
      }
      if (lane == 0) S.ctl[0] = ctl;
      wsync();
    }
    have_y = false;
    __syncthreads();
    const int ctl = S.ctl[0];
    if (ctl == CTL_DROP) {
      if (wave == 0) {
        for (int k = *S.np - 1; k >= 0; --k) {
          const int a = S.plist[k];
          if (S.flag[a] & F_DROP) {
            wsync();
            if (lane_id() == 0) {
              S.flag[a] = single ? F_BLOCKED : 0;
              if (!single) S.ctl[3] = 1;
            }
            wsync();
            remove_at(S, k);
          }
        }
      }
      continue;
    }
    grad_update(S, G, ld, p);
    const int np = *S.np;
    for (int k = tid; k < np; k += NT) {
      const int a = S.plist[k];
      const double un = S.u[a] + S.delta[k];
      S.u[a] = un > 0.0 ? un : 0.0;
    }
    __syncthreads();
    if (wave == 0) {
      if (ctl == CTL_PARTIAL) {
        // every free variable that reached zero leaves (highest position first)
        for (int k = *S.np - 1; k >= 0; --k) {
          const int a = S.plist[k];
          if (!(S.u[a] > 0.0)) {
            wsync();
            if (lane_id() == 0) {
              S.u[a] = 0.0;
              S.flag[a] &= ~(F_PASSIVE | F_NEW);
            }
            wsync();
            remove_at(S, k);
          }
        }
      }
      for (int k = lane_id(); k < *S.np; k += 64) S.flag[S.plist[k]] &= ~F_NEW;
      wsync();
    }
    if (ctl == CTL_DONE) break;
  }
  __syncthreads();
}

// Top-NB zero variables by gradient above tol (wave 0); returns the count.
__device__ __forceinline__ int pick_candidates(const St &S, int p, double tol, int maxc) {
  const int lane = lane_id();
  double v[NR];
  static_for<0, NR>([&](auto I_m) {
    constexpr int m = decltype(I_m)::value;
    const int a = lane + 64 * m;
    v[m] = (a < p && !(S.flag[a] & (F_PASSIVE | F_BLOCKED)) && S.g[a] > tol) ? S.g[a] : -INFINITY;
  });
  int nc = 0;
  for (int b = 0; b < maxc; ++b) {
    double bv = -INFINITY;
    int bi = -1;
    static_for<0, NR>([&](auto I_m) {
      constexpr int m = decltype(I_m)::value;
      const int a = lane + 64 * m;
      if (v[m] > bv || (v[m] == bv && bi >= 0 && a < bi && v[m] > -INFINITY)) {
        if (v[m] > -INFINITY) {
          bv = v[m];
          bi = a;
        }
      }
    });
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const double ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (oi >= 0 && (bi < 0 || ov > bv || (ov == bv && oi < bi))) {
        bv = ov;
        bi = oi;
      }
    }
    if (bi < 0) break;
    if (lane == 0) S.cand[nc] = bi;
    static_for<0, NR>([&](auto I_m) {
      constexpr int m = decltype(I_m)::value;
      if (lane + 64 * m == bi) v[m] = -INFINITY;
    });
    ++nc;
  }
  wsync();
  return nc;
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
    S.ctl[3] = 0;
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
  double y[NR];
  static_for<0, NR>([&](auto I_m) {
    constexpr int m = decltype(I_m)::value;
    y[m] = 0.0;
  });

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
      // the support of the warm start becomes the free set, NB variables at a time
      if (wave == 0) {
        int a0 = 0;
        for (;;) {
          int nc = 0;
          for (; a0 < p && nc < NB; ++a0)
            if (S.u[a0] > 0.0 && !(S.flag[a0] & (F_PASSIVE | F_BLOCKED))) {
              if (lane_id() == 0) S.cand[nc] = a0;
              ++nc;
            }
          wsync();
          if (nc == 0) break;
          block_append(S, G, ld, nc, y, &sh_status);
        }
        for (int k = lane_id(); k < *S.np; k += 64) S.flag[S.plist[k]] &= ~F_NEW;
        wsync();
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
      if (*S.np > 0) settle(S, G, ld, p, y, false, false);
    } else {
      settle(S, G, ld, p, y, false, false);  // refine the persisted optimum with the accurate gradient
    }
    for (;;) {
      __syncthreads();
      if (wave == 0) {
        const int nc = pick_candidates(S, p, tol, S.ctl[3] ? 1 : NB);
        if (lane_id() == 0) S.ctl[1] = nc;
        wsync();
      }
      __syncthreads();
      const int nc = S.ctl[1];
      if (nc == 0) break;
      if (iters >= cap) {
        if (tid == 0) sh_status |= int(AMC_HS_NNLS_CAP);
        break;
      }
      ++iters;
      if (wave == 0) {
        block_append(S, G, ld, nc, y, &sh_status);
        if (lane_id() == 0) S.ctl[2] = *S.np;
        wsync();
      }
      __syncthreads();
      if (S.ctl[2] > 0) settle(S, G, ld, p, y, true, nc == 1);
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
