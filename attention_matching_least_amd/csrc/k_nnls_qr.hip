// Exact refit through orthogonal factorisations, for the heads whose Gram
// form cannot resolve the NNLS minimiser (zhichai.net deep-dive, section 1.6:
// refit w by NNLS after every pick; xinfinite.net article, section 2, step 2:
// the bias fit is an NNLS problem; step 3: the value fit is a least-squares
// problem).
//
// When the selected keys are nearly collinear and the mass is almost fitted,
// the Gram matrix Phi_S^T Phi_S (whose conditioning is the square of
// Phi_S's) no longer determines the minimiser in float64: its KKT tests are
// decided by gradients at the level of rounding, and its steps lose the
// small singular directions.  These kernels never form it.
//
// k_nnls_qr, one block per head (the heads the Gram solver flagged):
//   1. The columns of [Phi_S D^-1 | m] (D the column norms), ordered [free |
//      zero | m], are reduced to their upper-triangular factor T by Householder
//      reflections applied to row blocks of 8..64 queries at a time (the
//      block goes through LDS; only T is kept, never Q).  ||Phi_S D^-1 u - m||
//      then equals ||T u - c|| up to a constant, with c = T's last column.
//   2. Lawson and Hanson's active-set steps run on T.  Its leading block
//      solves the free set's least squares by back substitution; a free
//      variable that would turn non-positive makes the iterate step back to
//      feasibility and leave; otherwise the zero column whose part below the
//      free rows makes the largest cosine with the residual's part there
//      enters, if that cosine exceeds kCosTol.  A free column whose diagonal
//      falls below kDepTol (unit columns) is dependent on the columns before it
//      and leaves for good.
//   3. Moving a column in or out changes only the rows of T from its position
//      on: those rows are factored again (the same row-block reflections on
//      the trailing block of T, in the new column order), the rows above are
//      copied with their columns permuted.
//
// k_ols_qr: the value fit of the same heads, C_v[F] = argmin ||A C - Y|| with
// A = Phi_F diag(w_F) / mhat, from the triangular factor of [A | Y] (step 1
// with these columns) and back substitution.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>

#include "amc_internal.h"

namespace amc {
namespace {

constexpr int NT = 256;
constexpr int NW = NT / 64;
constexpr double kCosTol = 1e-10;  // smallest cosine of an entering column with the residual
constexpr double kDepTol = 1e-12;  // smallest diagonal of a free (unit) column
constexpr int kQrLdsBytes = 96 * 1024;  // LDS for the row block of the reduction

__device__ __forceinline__ double wsum(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

struct RedQ {
  double v[NW];
  int i[NW];
};

__device__ __forceinline__ double block_sum(double v, RedQ *red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wsum(v);
  __syncthreads();
  if (lane == 0) red->v[wave] = v;
  __syncthreads();
  double s = 0.0;
  for (int w = 0; w < NW; ++w) s += red->v[w];
  return s;
}

// Largest v over the block (ties to the lower idx; idx < 0 is empty); every
// thread gets the winning index and *out its value.
__device__ __forceinline__ int block_best(double v, int idx, RedQ *red, double *out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int o = 32; o > 0; o >>= 1) {
    const double ov = __shfl_xor(v, o);
    const int oi = __shfl_xor(idx, o);
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
  for (int w = 1; w < NW; ++w) {
    const double ov = red->v[w];
    const int oi = red->i[w];
    if (oi >= 0 && (idx < 0 || ov > v || (ov == v && oi < idx))) {
      v = ov;
      idx = oi;
    }
  }
  *out = v;
  return idx;
}

// Rows per LDS block of the reduction for ncol columns.
__device__ __forceinline__ int rows_per_block(int ncol) {
  int b = kQrLdsBytes / (8 * ncol);
  b = b > 64 ? 64 : b;
  return b < 1 ? 1 : b;
}

// Householder reduction of the rows produced by src(i, j) (i < nrows, j in
// [k0, ncol)) into rows and columns k0..ncol-1 of the upper-triangular R
// (row stride ld).  Row blocks of at most rows_per_block(ncol - k0) rows pass
// through B (LDS); R's rows k0..ncol-1 start at zero.  For every column j the
// reflection that zeroes the block's column j against R[j][j] is applied to
// R's row j and to the block's later columns (one thread per column).
template <class Src>
__device__ void rb_reduce(const Src &src, int nrows, int k0, int ncol, double *R, int ld, double *B) {
  const int tid = threadIdx.x;
  const int w = ncol - k0;
  if (w <= 0) return;
  for (int e = tid; e < w * w; e += NT) {
    const int r = e / w, c = e % w;
    R[int64_t(k0 + r) * ld + k0 + c] = 0.0;
  }
  const int bm = rows_per_block(w);
  for (int i0 = 0; i0 < nrows; i0 += bm) {
    const int nb = nrows - i0 < bm ? nrows - i0 : bm;
    __syncthreads();
    for (int e = tid; e < nb * w; e += NT) {
      const int r = e % nb, c = e / nb;
      B[r * w + c] = src(i0 + r, k0 + c);
    }
    __syncthreads();
    for (int j = 0; j < w; ++j) {
      double sig = 0.0;
      for (int r = 0; r < nb; ++r) sig = fma(B[r * w + j], B[r * w + j], sig);
      const double x0 = R[int64_t(k0 + j) * ld + k0 + j];
      if (sig == 0.0) continue;  // the block's column is already zero (same for every thread)
      const double nrm = sqrt(fma(x0, x0, sig));
      const double beta = x0 >= 0.0 ? -nrm : nrm;
      const double tau = (beta - x0) / beta;
      const double sc = 1.0 / (x0 - beta);
      __syncthreads();  // every thread has read R[j][j]
      for (int c = j + 1 + tid; c < w; c += NT) {
        double s = 0.0;
        for (int r = 0; r < nb; ++r) s = fma(B[r * w + j], B[r * w + c], s);
        double *rc = &R[int64_t(k0 + j) * ld + k0 + c];
        s = tau * fma(s, sc, *rc);
        *rc -= s;
        const double ss = s * sc;
        for (int r = 0; r < nb; ++r) B[r * w + c] = fma(-ss, B[r * w + j], B[r * w + c]);
      }
      if (tid == 0) R[int64_t(k0 + j) * ld + k0 + j] = beta;
      __syncthreads();
    }
  }
  __syncthreads();
}

// Source of the initial reduction: row i of [Phi_perm D^-1 | m] from the
// float64 panel (row a of the panel = column of slot a over the queries).
struct PanelSrc {
  const double *P;   // the head's panel
  const double *m;   // the head's target mass
  const int *perm;   // slot of each column position (LDS)
  const double *dgi; // 1 / column norm of each slot (LDS)
  int64_t n;
  int ncol;          // columns including m (last)
  __device__ __forceinline__ double operator()(int i, int j) const {
    if (j == ncol - 1) return m[i];
    const int a = perm[j];
    return P[int64_t(a) * n + i] * dgi[a];
  }
};

// Source of a trailing re-factorisation: rows k0.. of the old factor with its
// columns in the new order (cmap: old position of each new position).
struct TriSrc {
  const double *T;
  int ld;
  int k0;
  const int *cmap;
  __device__ __forceinline__ double operator()(int i, int j) const {
    const int oc = cmap[j];
    const int row = k0 + i;
    return oc >= row ? T[int64_t(row) * ld + oc] : 0.0;
  }
};

// New factor Tn from the old To after a change of column order from
// position k0 on (cmap[q] = old position of new position q, ncol_new columns
// including the right-hand side): rows above k0 are copied with their
// columns permuted; rows k0.. of the old factor, restricted to the new
// columns, are reduced again.  nrow_old: rows of To that may be nonzero.
__device__ void refactor_from(const double *To, double *Tn, int ld, int k0, int ncol_new, int nrow_old,
                              const int *cmap, double *B) {
  const int tid = threadIdx.x;
  for (int e = tid; e < k0 * ncol_new; e += NT) {
    const int r = e / ncol_new, q = e % ncol_new;
    if (q >= r) Tn[int64_t(r) * ld + q] = To[int64_t(r) * ld + cmap[q]];
  }
  TriSrc src{To, ld, k0, cmap};
  rb_reduce(src, nrow_old - k0, k0, ncol_new, Tn, ld, B);
}

// ---------------------------------------------------------------------------
// k_nnls_qr
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(NT) void k_nnls_qr(const HeadDesc *__restrict__ desc, const double *__restrict__ panel,
                                                const double *__restrict__ m, const double *__restrict__ G,
                                                double *__restrict__ w, int cycle, int kR, int polish,
                                                int32_t *__restrict__ qr_flag, double *__restrict__ qrbuf,
                                                int32_t *__restrict__ tr_iters, double *__restrict__ tr_weight,
                                                int32_t *__restrict__ head_status) {
  extern __shared__ __attribute__((aligned(16))) double B[];
  __shared__ int perm[kQrMaxT + 1];   // slot of each column position: free, then zero
  __shared__ int cmap[kQrMaxT + 1];   // old position of each new position
  __shared__ double u[kQrMaxT];       // scaled iterate, by slot
  __shared__ double dgi[kQrMaxT];     // 1 / column norm, by slot (0: blocked)
  __shared__ double z[kQrMaxT];       // free-set solution, by position
  __shared__ RedQ red;
  __shared__ int ptmp[kQrMaxT + 1];   // scratch positions
  __shared__ int sh_f, sh_nz, sh_k0, sh_status;
  const int h = blockIdx.x;
  const int flag = qr_flag[h];
  if (flag == 0) return;
  const HeadDesc D = desc[h];
  if (D.t > kQrMaxT || D.qr_off < 0) return;
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
  const int tid = threadIdx.x;
  const int ld = int(D.t + 1 + 128);  // row stride of the factors (value fit: t + d + 1 columns)
  double *Ta = qrbuf + D.qr_off;
  double *Tb = Ta + int64_t(ld) * ld;
  // warm start: the weights of the previous refit; a head flagged by the Gram
  // solver at this refit also has its weights for the new keys
  const int nwarm = flag == 1 ? p : int(S0);
  const double *Gh = G + D.tt_off;
  for (int a = tid; a < p; a += NT) {
    const double gaa = Gh[int64_t(a) * D.t + a];
    const double dg = sqrt(gaa);
    const bool ok = dg > 0.0 && isfinite(dg);
    dgi[a] = ok ? 1.0 / dg : 0.0;
    const double wa = a < nwarm ? w[D.t_off + a] : 0.0;
    u[a] = (ok && wa > 0.0) ? wa * dg : 0.0;
  }
  if (tid == 0) sh_status = 0;
  __syncthreads();
  // column order: free slots ascending, then zero slots ascending (blocked left out)
  if (tid == 0) {
    int f = 0;
    for (int a = 0; a < p; ++a)
      if (dgi[a] > 0.0 && u[a] > 0.0) perm[f++] = a;
    int nz = 0;
    for (int a = 0; a < p; ++a)
      if (dgi[a] > 0.0 && !(u[a] > 0.0)) perm[f + nz++] = a;
    sh_f = f;
    sh_nz = nz;
  }
  __syncthreads();
  int f = sh_f, nz = sh_nz;
  int ncol = f + nz + 1;
  {
    PanelSrc src{panel + D.panel_off, m + D.n_off, perm, dgi, D.n, ncol};
    rb_reduce(src, int(D.n), 0, ncol, Ta, ld, B);
  }
  int nrow = int(D.n) < ncol ? int(D.n) : ncol;  // rows of T that may be nonzero
  double *T = Ta, *Tn = Tb;
  const int cap = 3 * p + 30;
  int iters = 0;
  for (;;) {
    if (iters >= cap) {
      if (tid == 0) sh_status |= int(AMC_HS_NNLS_CAP);
      break;
    }
    ++iters;
    // a free column dependent on the ones before it leaves for good
    int dep = -1;
    {
      double v;
      int cand = -1;
      for (int k = tid; k < f; k += NT)
        if (cand < 0 && !(fabs(T[int64_t(k) * ld + k]) > kDepTol)) cand = k;
      dep = block_best(cand >= 0 ? -double(cand) : -INFINITY, cand, &red, &v);
    }
    if (dep >= 0) {
      for (int q = tid; q < ncol - 1; q += NT) cmap[q] = q < dep ? q : q + 1;
      __syncthreads();
      if (tid == 0) {
        const int a = perm[dep];
        u[a] = 0.0;
        dgi[a] = 0.0;
        for (int q = dep; q < ncol - 1; ++q) perm[q] = perm[q + 1];
      }
      __syncthreads();
      refactor_from(T, Tn, ld, dep, ncol - 1, nrow, cmap, B);
      double *x = T;
      T = Tn;
      Tn = x;
      --f;
      --ncol;
      nrow = nrow < ncol ? nrow : ncol;
      if (tid == 0) sh_status |= int(AMC_HS_NNLS_SINGULAR);
      continue;
    }
    // least squares on the free set: T_FF z = c_F (column-oriented back substitution)
    for (int k = tid; k < f; k += NT) z[k] = T[int64_t(k) * ld + ncol - 1];
    __syncthreads();
    for (int k = f - 1; k >= 0; --k) {
      const double zk = z[k] / T[int64_t(k) * ld + k];
      __syncthreads();
      for (int i = tid; i < k; i += NT) z[i] = fma(-T[int64_t(i) * ld + k], zk, z[i]);
      if (tid == 0) z[k] = zk;
      __syncthreads();
    }
    // infeasible: step from u toward z until the first free variable reaches zero
    int ib;
    double best;
    {
      int cand = -1;
      double bv = INFINITY;
      for (int k = tid; k < f; k += NT) {
        if (!(z[k] > 0.0)) {
          const double ua = u[perm[k]];
          const double rt = ua > 0.0 ? ua / (ua - z[k]) : 0.0;
          if (cand < 0 || rt < bv) {
            bv = rt;
            cand = k;
          }
        }
      }
      double nb;
      ib = block_best(cand >= 0 ? -bv : -INFINITY, cand, &red, &nb);
      best = -nb;
    }
    if (ib >= 0) {
      const double alpha = best;
      for (int k = tid; k < f; k += NT) {
        const int a = perm[k];
        const double un = k == ib ? 0.0 : fma(alpha, z[k] - u[a], u[a]);
        u[a] = un > 0.0 ? un : 0.0;
      }
      __syncthreads();
      // the free variables now at zero move to the zero set (at their slot's
      // place among the zero columns), one refactorisation for all of them
      if (tid == 0) {
        int nf = 0, first = -1, nl = 0;
        for (int k = 0; k < f; ++k) {
          if (u[perm[k]] > 0.0) {
            cmap[nf++] = k;
          } else {
            if (first < 0) first = k;
            ptmp[nl++] = k;  // leaving positions, ascending slots (free slots are not sorted: sort below)
          }
        }
        for (int x = 1; x < nl; ++x) {
          const int v = ptmp[x];
          int y = x - 1;
          while (y >= 0 && perm[ptmp[y]] > perm[v]) {
            ptmp[y + 1] = ptmp[y];
            --y;
          }
          ptmp[y + 1] = v;
        }
        // zero columns: the old ones (positions f.., ascending slots) merged with the leaving ones
        int iz = f, il = 0, q = nf;
        while (iz < f + nz || il < nl) {
          const bool take_old = il >= nl || (iz < f + nz && perm[iz] < perm[ptmp[il]]);
          cmap[q++] = take_old ? iz++ : ptmp[il++];
        }
        cmap[q] = ncol - 1;
        sh_f = nf;
        sh_nz = nz + nl;
        sh_k0 = first;
      }
      __syncthreads();
      const int k0 = sh_k0;
      // new column order (perm is read through cmap before it is rewritten)
      for (int q = tid; q < ncol - 1; q += NT) ptmp[q] = perm[cmap[q]];
      __syncthreads();
      for (int q = tid; q < ncol - 1; q += NT) perm[q] = ptmp[q];
      __syncthreads();
      refactor_from(T, Tn, ld, k0, ncol, nrow, cmap, B);
      double *x = T;
      T = Tn;
      Tn = x;
      f = sh_f;
      nz = sh_nz;
      continue;
    }
    for (int k = tid; k < f; k += NT) u[perm[k]] = z[k];
    // residual below the free rows and every zero column's part there
    double rr = 0.0;
    for (int r = f + tid; r < nrow && r < ncol - 1; r += NT) {
      const double v = T[int64_t(r) * ld + ncol - 1];
      rr = fma(v, v, rr);
    }
    const double nr = sqrt(block_sum(rr, &red));
    int enter = -1;
    if (nr > 0.0) {
      int cand = -1;
      double bv = kCosTol;
      for (int q = tid; q < nz; q += NT) {
        const int col = f + q;
        double num = 0.0, den = 0.0;
        for (int r = f; r <= col && r < nrow; ++r) {
          const double tv = T[int64_t(r) * ld + col];
          num = fma(tv, T[int64_t(r) * ld + ncol - 1], num);
          den = fma(tv, tv, den);
        }
        den = sqrt(den);
        if (den > kDepTol) {
          const double cs = num / (den * nr);
          if (cs > bv) {
            bv = cs;
            cand = q;
          }
        }
      }
      double v;
      enter = block_best(cand >= 0 ? bv : -INFINITY, cand, &red, &v);
    }
    if (enter < 0) break;
    // the entering column moves to position f
    for (int q = tid; q < ncol; q += NT) {
      int oc;
      if (q < f) oc = q;
      else if (q == f) oc = f + enter;
      else if (q <= f + enter) oc = q - 1;
      else oc = q;
      cmap[q] = oc;
    }
    __syncthreads();
    if (tid == 0) {
      const int a = perm[f + enter];
      for (int q = f + enter; q > f; --q) perm[q] = perm[q - 1];
      perm[f] = a;
    }
    __syncthreads();
    refactor_from(T, Tn, ld, f, ncol, nrow, cmap, B);
    double *x = T;
    T = Tn;
    Tn = x;
    ++f;
    --nz;
  }
  __syncthreads();
  for (int a = tid; a < p; a += NT) {
    const double wa = dgi[a] > 0.0 ? u[a] * dgi[a] : 0.0;
    w[D.t_off + a] = wa;
    if (tr_weight) tr_weight[D.t_off + a] = wa;
  }
  if (tid == 0) {
    qr_flag[h] = 2;
    if (tr_iters && !polish) tr_iters[D.cyc_off + cycle] = iters;
    if (head_status) atomicOr(head_status + h, sh_status | int(AMC_HS_NNLS_QR));
  }
}

// ---------------------------------------------------------------------------
// k_ols_qr: C_v[F] = argmin ||A C - Y||, A = Phi_F diag(w_F) / mhat
// ---------------------------------------------------------------------------
struct OlsSrc {
  const double *P;    // panel
  const double *mh;   // mhat
  const float *Y;     // rows of Y (d columns)
  const int *fl;      // slots of F (LDS)
  const double *wf;   // their weights (LDS)
  int64_t n;
  int f, d;
  __device__ __forceinline__ double operator()(int i, int j) const {
    if (j < f) return P[int64_t(fl[j]) * n + i] * wf[j] / mh[i];
    return double(Y[int64_t(i) * d + (j - f)]);
  }
};

template <int D>
__global__ __launch_bounds__(NT) void k_ols_qr(const HeadDesc *__restrict__ desc, const double *__restrict__ panel,
                                               const double *__restrict__ w, const double *__restrict__ mhat,
                                               const float *__restrict__ Y, const int32_t *__restrict__ qr_flag,
                                               double *__restrict__ qrbuf, float *__restrict__ cv_sel,
                                               int32_t *__restrict__ head_status) {
  extern __shared__ __attribute__((aligned(16))) double B[];
  __shared__ int fl[kQrMaxT];
  __shared__ double wf[kQrMaxT];
  __shared__ int sh_f, sh_bad;
  const int h = blockIdx.x;
  if (qr_flag[h] == 0) return;
  const HeadDesc Dh = desc[h];
  if (Dh.t > kQrMaxT || Dh.qr_off < 0) return;
  const int tid = threadIdx.x;
  const int t = int(Dh.t);
  const int ld = int(Dh.t + 1 + 128);
  double *T = qrbuf + Dh.qr_off;
  if (tid == 0) {
    int f = 0;
    for (int a = 0; a < t; ++a) {
      const double wa = w[Dh.t_off + a];
      if (wa > 0.0) {
        fl[f] = a;
        wf[f] = wa;
        ++f;
      }
    }
    sh_f = f;
    sh_bad = 0;
  }
  // keys with w = 0 get a zero value row
  for (int e = tid; e < t * D; e += NT) {
    const int a = e / D;
    if (!(w[Dh.t_off + a] > 0.0)) cv_sel[(Dh.t_off + a) * D + e % D] = 0.0f;
  }
  __syncthreads();
  const int f = sh_f;
  if (f == 0) return;
  const int ncol = f + D;
  OlsSrc src{panel + Dh.panel_off, mhat + Dh.n_off, Y + Dh.n_off * D, fl, wf, Dh.n, f, D};
  rb_reduce(src, int(Dh.n), 0, ncol, T, ld, B);
  // back substitution T_FF X = T_FY, one value column per thread (X in
  // float64 after the factor); a diagonal at rounding level (a column
  // dependent on the ones before it) gets x = 0
  double *X = T + int64_t(ld) * ld;
  for (int c = tid; c < D; c += NT) {
    for (int k = f - 1; k >= 0; --k) {
      double s = T[int64_t(k) * ld + f + c];
      for (int i = k + 1; i < f; ++i) s = fma(-T[int64_t(k) * ld + i], X[int64_t(i) * D + c], s);
      const double dk = T[int64_t(k) * ld + k];
      double x = 0.0;
      if (fabs(dk) > kDepTol * 1e-3) {
        x = s / dk;
      } else {
        sh_bad = 1;
      }
      X[int64_t(k) * D + c] = x;
      cv_sel[(Dh.t_off + fl[k]) * D + c] = float(x);
    }
  }
  __syncthreads();
  if (tid == 0 && sh_bad && head_status) atomicOr(head_status + h, int(AMC_HS_CHOL_JITTER));
}

}  // namespace

static size_t qr_lds(int64_t max_t, int d) {
  (void)max_t;
  (void)d;
  return size_t(kQrLdsBytes);
}

hipError_t launch_nnls_qr(const Dims &dm, const Buffers &b, int cycle, int kR, int polish, hipStream_t s) {
  if (!b.qr_flag) return hipSuccess;
  const size_t bytes = qr_lds(dm.max_t, dm.d);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_nnls_qr),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, int(bytes));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_nnls_qr, dim3(unsigned(dm.H)), dim3(NT), bytes, s, b.desc, b.panel, b.m, b.G, b.w, cycle, kR,
                     polish, b.qr_flag, b.qrbuf, b.tr_iters, b.tr_weight, b.head_status);
  return hipGetLastError();
}

hipError_t launch_ols_qr(const Dims &dm, const Buffers &b, hipStream_t s) {
  if (!b.qr_flag) return hipSuccess;
  const size_t bytes = qr_lds(dm.max_t, dm.d);
  if (dm.d == 128) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_ols_qr<128>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(bytes));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_ols_qr<128>, dim3(unsigned(dm.H)), dim3(NT), bytes, s, b.desc, b.panel, b.w, b.mhat, b.Y,
                       b.qr_flag, b.qrbuf, b.cv_sel, b.head_status);
  } else {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_ols_qr<64>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(bytes));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_ols_qr<64>, dim3(unsigned(dm.H)), dim3(NT), bytes, s, b.desc, b.panel, b.w, b.mhat, b.Y,
                       b.qr_flag, b.qrbuf, b.cv_sel, b.head_status);
  }
  return hipGetLastError();
}

}  // namespace amc
