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
// Per head that the Gram solver flagged (or every eligible head, on request):
//   k_qr_append keeps a Householder factorisation Phi_S D^-1 = H [Rb; 0] of
//   the selected columns (D the column norms) in slot order, with cb the
//   leading entries of H^T m: each refit's new columns take the reflections
//   already stored, then one new reflection each, so the work per refit is
//   linear in the keys already selected and the factor stays orthogonal to
//   working precision however dependent the columns are (a dependent column
//   leaves a diagonal of Rb at rounding level, which the steps below treat as
//   dependent).
//   ||Phi_S D^-1 u - m|| then equals ||Rb u - cb|| up to a constant.
//   k_nnls_qr (one wave) runs Lawson and Hanson's active-set steps on that
//   triangle: the columns ordered [free | zero | cb] are made triangular again
//   (T) by one Householder reflection per column over the rows below its
//   diagonal; the leading block gives the free set's least squares by back
//   substitution; a free variable that would turn non-positive makes the
//   iterate step back to feasibility and moves behind the zero columns;
//   otherwise the zero column whose part below the free rows makes the largest
//   cosine (above kCosTol) with the residual's part there enters.  Moving a
//   column disturbs T only from its position on, where the same reflections
//   restore it (a band of one row for a deleted column, the entering column's
//   own rows for an entering one).
//
// k_ols_qr: the value fit of heads whose free columns are nearly dependent
// (smallest free pivot below kOlsPivot), C_v[F] = argmin ||A C - Y|| with
// A = Phi_F diag(w_F) / mhat, from the triangular factor of [A | Y], reduced
// by Householder reflections over row blocks of queries staged in LDS, and
// back substitution.  Other heads keep the normal equations.
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
constexpr int kQrLdsBytes = 96 * 1024;  // LDS for the row block of the value fit's reduction
constexpr double kOlsPivot = 1e-6;  // smallest free pivot (unit columns) the normal-equation value fit takes

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

// ---------------------------------------------------------------------------
// Per-head state of the exact refit (qr_layout).  Rb is column-packed (poff).
// Row a of V is v_a itself
// (zero before a, one at a): H_a = I - tau_a v_a v_a^T.  The slots form
// chunks of CW (8, or 4 for heads above 4096 queries); the reflections of
// chunk c multiply to I - V_c T_c V_c^T (compact WY form: T_c upper
// triangular with the tau on its diagonal), T_c kept at Tw + 64 c for the
// slots the chunk has so far.
// ---------------------------------------------------------------------------
// Column-packed triangles: column q holds rows 0..q+1 (the last a subdiagonal
// entry, zero between steps) from word poff(q) on.
__host__ __device__ constexpr int poff(int q) { return q * (q + 3) / 2; }

struct QrState {
  double *V, *Rb, *cb, *Tw, *mt, *W;
  int ld;  // row stride of the value fit's triangle
};
__device__ __forceinline__ QrState qr_state(const HeadDesc &D, double *qrbuf) {
  const QrLayout L = qr_layout(D.t, D.n);
  double *b = qrbuf + D.qr_off;
  return QrState{b + L.V, b + L.Rb, b + L.cb, b + L.Tw, b + L.mt, b + L.W, int(D.t + 129)};
}

constexpr int NA = 512;       // threads of the append kernel (one block per head)
constexpr int NAW = NA / 64;  // its waves
constexpr int RED_RES = NAW * 32;  // start of the block sums in the reduction buffer

// One halving step of wave_sum_scatter: lanes with bit O set keep the upper
// half of v[0..SZ), the others the lower half, each adding its partner's.
template <int SZ, int O, int NV>
__device__ __forceinline__ void scatter_step(double (&v)[NV], int lane) {
  if constexpr (SZ > 1) {
    const bool up = (lane & O) != 0;
#pragma unroll
    for (int j = 0; j < SZ / 2; ++j) {
      const double send = up ? v[j] : v[j + SZ / 2];
      const double keep = up ? v[j + SZ / 2] : v[j];
      v[j] = keep + __shfl_xor(send, O);
    }
    scatter_step<SZ / 2, O / 2, NV>(v, lane);
  }
}

// Wave sum of each of v[0..NV) (NV a power of two), scattered: afterwards
// lane l holds (returns) the sum of the value with index l / (64 / NV).
template <int NV>
__device__ __forceinline__ double wave_sum_scatter(double (&v)[NV]) {
  const int lane = threadIdx.x & 63;
  scatter_step<NV, 32, NV>(v, lane);
  double r = v[0];
#pragma unroll
  for (int o = 32 / NV; o > 0; o >>= 1) r += __shfl_xor(r, o);
  return r;
}

// Sums of v[0..NV) over the block (NV a power of two, at most 32); every
// thread gets them.
template <int NV>
__device__ __forceinline__ void block_sums(double (&v)[NV], double *red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const double s = wave_sum_scatter<NV>(v);
  if ((lane & (64 / NV - 1)) == 0) red[wave * NV + lane / (64 / NV)] = s;
  __syncthreads();
  if (threadIdx.x < NV) {
    double acc = 0.0;
    for (int w2 = 0; w2 < NAW; ++w2) acc += red[w2 * NV + threadIdx.x];
    red[RED_RES + threadIdx.x] = acc;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < NV; ++k) v[k] = red[RED_RES + k];
}

struct AppendLds {
  double mt[kQrMaxN];  // the rotated mass H^T m of the head (each thread keeps its own rows)
  double red[RED_RES + 32];
  double wpart[NAW][kQrChunk][kQrChunk];
  double Wl[kQrChunk][kQrChunk];
  double Zl[kQrChunk][kQrChunk];
  double Tl[kQrChunk][kQrChunk];
  double dgs[kQrChunk];
  double x0;
};

// X := Q_c^T X for the chunk c whose first len reflections start at slot c0:
// Q_c^T = I - V_c T_c^T V_c^T.  W = V_c^T X, Z = T_c^T W, X -= V_c Z.
template <int RPT, int CW>
__device__ __forceinline__ void apply_block(double (&X)[RPT][CW], const double *V, const double *Tc, int n,
                                            int c0, int len, AppendLds &L) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll 1
  for (int l = 0; l < len; ++l) {
    const double *vr = V + int64_t(c0 + l) * n;
    double acc[CW];
#pragma unroll
    for (int k = 0; k < CW; ++k) acc[k] = 0.0;
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int i = tid + r * NA;
      const double v = i < n ? vr[i] : 0.0;
#pragma unroll
      for (int k = 0; k < CW; ++k) acc[k] = fma(v, X[r][k], acc[k]);
    }
    const double s = wave_sum_scatter<CW>(acc);
    if ((lane & (64 / CW - 1)) == 0) L.wpart[wave][l][lane / (64 / CW)] = s;
  }
  __syncthreads();
  if (tid < len * CW) {
    const int l = tid / CW, k = tid % CW;
    double s = 0.0;
    for (int w2 = 0; w2 < NAW; ++w2) s += L.wpart[w2][l][k];
    L.Wl[l][k] = s;
  }
  __syncthreads();
  if (tid < len * CW) {
    const int l = tid / CW, k = tid % CW;
    double z = 0.0;
    for (int j = 0; j <= l; ++j) z = fma(Tc[j * kQrChunk + l], L.Wl[j][k], z);
    L.Zl[l][k] = z;
  }
  __syncthreads();
#pragma unroll 1
  for (int l = 0; l < len; ++l) {
    const double *vr = V + int64_t(c0 + l) * n;
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int i = tid + r * NA;
      const double v = i < n ? vr[i] : 0.0;
#pragma unroll
      for (int k = 0; k < CW; ++k) X[r][k] = fma(-v, L.Zl[l][k], X[r][k]);
    }
  }
}

// Brings V, Rb, cb, Tw, mt of one head from qr_built slots to p.  Per chunk:
// the new columns of Phi_S D^-1 (panel rows times 1 / sqrt(G_aa)) take the
// block reflectors already stored, all together in registers, and wait in
// their own rows of V; then, one column at a time, each takes the
// reflections made before it in this call (the same compact WY form, on the
// diagonal block of T_c for those slots) and gets one new reflection of its
// own (Householder QR: stable however dependent the columns are), which m
// takes too.
template <int RPT, int CW>
__device__ void qr_append_head(const HeadDesc &D, const QrState &S, const double *__restrict__ P,
                               const double *__restrict__ m, const double *__restrict__ Gh, int from, int p,
                               AppendLds &L) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = int(D.t);
  const int n = int(D.n);
  // the rotated mass stays in LDS (a thread reads and writes only its own
  // rows), keeping registers for the columns
  double *mtr = L.mt;
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const int i = tid + r * NA;
    if (i < n) mtr[i] = from == 0 ? m[i] : S.mt[i];
  }
#pragma unroll 1
  for (int cidx = from / CW; cidx * CW < p; ++cidx) {
    const int c0 = cidx * CW;
    const int lo = from > c0 ? from - c0 : 0;  // first new slot of the chunk (relative)
    const int hi = p - c0 < CW ? p - c0 : CW;  // end of the chunk's slots (relative)
    double *Tc = S.Tw + int64_t(cidx) * kQrChunk * kQrChunk;
    __syncthreads();
    if (tid < CW) {
      double dg = 0.0;
      if (tid >= lo && tid < hi) {
        const double gaa = Gh[int64_t(c0 + tid) * t + c0 + tid];
        const double sq = sqrt(gaa);
        dg = (sq > 0.0 && isfinite(sq)) ? 1.0 / sq : 0.0;
      }
      L.dgs[tid] = dg;
    }
    if (tid < kQrChunk * kQrChunk) L.Tl[tid / kQrChunk][tid % kQrChunk] = Tc[tid];
    __syncthreads();
    {
      double X[RPT][CW];
#pragma unroll
      for (int k = 0; k < CW; ++k) {
        const bool live = k >= lo && k < hi;
        const double dg = L.dgs[k];
        const double *pr = P + int64_t(c0 + k) * n;
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
          const int i = tid + r * NA;
          X[r][k] = (live && i < n) ? pr[i] * dg : 0.0;
        }
      }
      // the complete chunks before this one, then this chunk's stored reflections
#pragma unroll 1
      for (int cc = 0; cc < cidx; ++cc)
        apply_block<RPT, CW>(X, S.V, S.Tw + int64_t(cc) * kQrChunk * kQrChunk, n, cc * CW, CW, L);
      if (lo > 0) apply_block<RPT, CW>(X, S.V, Tc, n, c0, lo, L);
#pragma unroll
      for (int k = 0; k < CW; ++k) {
        if (k < lo || k >= hi) continue;  // same for every thread
        double *vr = S.V + int64_t(c0 + k) * n;
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
          const int i = tid + r * NA;
          if (i < n) vr[i] = X[r][k];
        }
      }
    }
#pragma unroll 1
    for (int kc = lo; kc < hi; ++kc) {
      const int a = c0 + kc;
      double *va = S.V + int64_t(a) * n;
      __syncthreads();  // rows of V written by other threads
      double xc[RPT];
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        const int i = tid + r * NA;
        xc[r] = i < n ? va[i] : 0.0;
      }
      if (kc > lo) {
        // the reflections lo..kc-1 of this call: x -= V_s T_s^T (V_s^T x)
        double wv[CW];
#pragma unroll
        for (int j = 0; j < CW; ++j) wv[j] = 0.0;
#pragma unroll
        for (int j = 0; j < CW; ++j) {
          if (j < lo || j >= kc) continue;  // same for every thread
          const double *vj = S.V + int64_t(c0 + j) * n;
#pragma unroll
          for (int r = 0; r < RPT; ++r) {
            const int i = tid + r * NA;
            if (i < n) wv[j] = fma(vj[i], xc[r], wv[j]);
          }
        }
        block_sums<CW>(wv, L.red);
        double zv[CW];
#pragma unroll
        for (int l = 0; l < CW; ++l) {
          double z = 0.0;
#pragma unroll
          for (int j = 0; j < CW; ++j)
            if (j >= lo && j <= l) z = fma(L.Tl[j][l], wv[j], z);
          zv[l] = (l >= lo && l < kc) ? z : 0.0;
        }
#pragma unroll
        for (int l = 0; l < CW; ++l) {
          if (l < lo || l >= kc) continue;  // same for every thread
          const double *vl = S.V + int64_t(c0 + l) * n;
#pragma unroll
          for (int r = 0; r < RPT; ++r) {
            const int i = tid + r * NA;
            if (i < n) xc[r] = fma(-vl[i], zv[l], xc[r]);
          }
        }
      }
      // norm of the column below its slot, and its entry at the slot
      double sg[1] = {0.0};
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        const int i = tid + r * NA;
        if (i > a && i < n) sg[0] = fma(xc[r], xc[r], sg[0]);
        if (i == a) L.x0 = xc[r];
      }
      if (tid == 0 && a >= n) L.x0 = 0.0;
      block_sums<1>(sg, L.red);
      const double sig = sg[0];
      const double x0 = L.x0;
      // column a of Rb above the diagonal
      double *Ra = S.Rb + poff(a);
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        const int i = tid + r * NA;
        if (i < a && i < n) Ra[i] = xc[r];
      }
      for (int i = n + tid; i < a; i += NA) Ra[i] = 0.0;
      double tau, diag, sc;
      if (sig == 0.0) {
        tau = 0.0;
        diag = x0;
        sc = 0.0;
      } else {
        const double nrm = sqrt(fma(x0, x0, sig));
        diag = x0 >= 0.0 ? -nrm : nrm;
        sc = 1.0 / (x0 - diag);
        tau = (diag - x0) / diag;
      }
      if (tid == 0) {
        Ra[a] = diag;
        Ra[a + 1] = 0.0;
      }
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        const int i = tid + r * NA;
        const double v = i < a ? 0.0 : (i == a ? 1.0 : xc[r] * sc);
        xc[r] = i < n ? v : 0.0;
      }
      // dots of v_a with mt (dv[0]) and with the chunk's earlier reflections
      // (dv[1 + j], j < kc <= CW - 1, for T_c's new column)
      double dv[CW];
#pragma unroll
      for (int k = 0; k < CW; ++k) dv[k] = 0.0;
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        const int i = tid + r * NA;
        dv[0] = fma(xc[r], i < n ? mtr[i] : 0.0, dv[0]);
      }
#pragma unroll
      for (int j = 0; j < CW - 1; ++j) {
        if (j >= kc) continue;  // same for every thread
        const double *vj = S.V + int64_t(c0 + j) * n;
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
          const int i = tid + r * NA;
          if (i < n) dv[1 + j] = fma(vj[i], xc[r], dv[1 + j]);
        }
      }
      block_sums<CW>(dv, L.red);
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        const int i = tid + r * NA;
        if (i < n) va[i] = xc[r];
        if (i < n) {
          const double mv = fma(-tau * dv[0], xc[r], mtr[i]);
          mtr[i] = mv;
          if (i == a) S.cb[a] = mv;
        }
      }
      if (tid == 0 && a >= n) S.cb[a] = 0.0;
      // T_c column kc: tau on the diagonal, -tau T_c[l][0..kc) e above it
      if (tid <= kc) {
        double s2 = 0.0;
#pragma unroll
        for (int j = 0; j < CW - 1; ++j)
          if (j >= tid && j < kc) s2 = fma(L.Tl[tid][j], dv[1 + j], s2);
        L.Tl[tid][kc] = tid == kc ? tau : -tau * s2;
      }
    }
    __syncthreads();
    if (tid < kQrChunk * kQrChunk) Tc[tid] = L.Tl[tid / kQrChunk][tid % kQrChunk];
  }
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const int i = tid + r * NA;
    if (i < n) S.mt[i] = mtr[i];
  }
  (void)lane;
  (void)wave;
}

// One launch per row count class: RPT rows of every thread, heads with
// n in (NA * RPT / 2, NA * RPT] (the first class from n = 1).  The chunk's
// columns stay in registers (RPT x CW words a thread).
template <int RPT, int CW>
__global__ __launch_bounds__(NA) void k_qr_append(const HeadDesc *__restrict__ desc, const double *__restrict__ panel,
                                                  const double *__restrict__ m, const double *__restrict__ G,
                                                  int cycle, int kR, int polish, const int32_t *__restrict__ qr_flag,
                                                  int32_t *__restrict__ qr_built, double *__restrict__ qrbuf) {
  __shared__ AppendLds L;
  const int h = blockIdx.x;
  if (qr_flag[h] == 0) return;
  const HeadDesc D = desc[h];
  if (D.t > kQrMaxT || D.n > kQrMaxN || D.qr_off < 0) return;
  if (D.n > int64_t(NA) * RPT || (RPT > 2 && D.n <= int64_t(NA) * RPT / 2)) return;
  int p;
  if (polish) {
    p = int(D.t);
  } else {
    const int64_t S0 = int64_t(cycle) * kR;
    if (S0 >= D.t) return;
    p = int(D.t - S0 < kR ? D.t : S0 + kR);
  }
  const int from = qr_built[h];
  if (from >= p) return;
  const QrState S = qr_state(D, qrbuf);
  qr_append_head<RPT, CW>(D, S, panel + D.panel_off, m + D.n_off, G + D.tt_off, from, p, L);
  if (threadIdx.x == 0) qr_built[h] = p;
}

// ---------------------------------------------------------------------------
// k_nnls_qr: Lawson-Hanson on the reduced triangle, one wave per head.
//
// Work pool (LDS when it fits, else the head's work area), cap words:
//   [0, poff(f))           the free block, column-packed and upper triangular
//                          (column q: rows 0..q, and a zero subdiagonal word)
//   ... free ...
//   zero columns           full height (p rows), slot k at cap - p (k + 2)
//   [cap - p, cap)         the right-hand side c
// All columns and c share one orthogonal row basis (the Householder basis of
// the slots, then the rotations of these steps).  Rows f..p-1 are the
// orthogonal complement of the free columns within the slots' span: the
// residual's part is c[f..p), a zero column's part there decides whether it
// enters (its cosine with the residual).
// ---------------------------------------------------------------------------
constexpr int NQ = 64;  // one wave
constexpr int kLhLdsBytes = 156 * 1024;  // dynamic LDS of the Lawson-Hanson kernel

__device__ __forceinline__ double wave_max_abs_idx(double v, int idx, int *out_idx) {
  for (int o = 32; o > 0; o >>= 1) {
    const double ov = __shfl_xor(v, o);
    const int oi = __shfl_xor(idx, o);
    if (oi >= 0 && (idx < 0 || ov > v || (ov == v && oi < idx))) {
      v = ov;
      idx = oi;
    }
  }
  *out_idx = idx;
  return v;
}

// The pool of one head: base B (LDS or the work area), cap words, p slots.
struct LhPool {
  double *B;
  int64_t cap;
  int p;
  __device__ __forceinline__ double *c() const { return B + cap - p; }
  __device__ __forceinline__ double *zc(int k) const { return B + cap - int64_t(p) * (k + 2); }
  __device__ __forceinline__ double *fc(int q) const { return B + poff(q); }
  // room for f free columns, nz zero columns and c
  __device__ __forceinline__ bool fits(int f, int nz) const {
    return int64_t(poff(f)) + 2 + int64_t(p) * (nz + 1) <= cap;
  }
};

// Householder reflection of rows r0..r1 of x (r0 < r1) that zeroes rows
// r0+1..r1: x[r0] gets the diagonal, x[r0+1..r1] the vector v (v[r0] = 1).
// Returns tau (0: nothing to do).
__device__ __forceinline__ double lh_reflect(double *x, int r0, int r1) {
  const int lane = threadIdx.x;
  double sg = 0.0;
  for (int r = r0 + 1 + lane; r <= r1; r += NQ) sg = fma(x[r], x[r], sg);
  sg = wsum(sg);
  __syncthreads();
  if (sg == 0.0) return 0.0;
  const double x0 = x[r0];
  const double nrm = sqrt(fma(x0, x0, sg));
  const double diag = x0 >= 0.0 ? -nrm : nrm;
  const double sc = 1.0 / (x0 - diag);
  __syncthreads();
  for (int r = r0 + 1 + lane; r <= r1; r += NQ) x[r] *= sc;
  if (lane == 0) x[r0] = diag;
  __syncthreads();
  return (diag - x0) / diag;
}

// Applies (I - tau v v^T), v = [1, x[r0+1..r1]], to rows r0..r1 of y (four
// partial sums, so the loads of one lane overlap).
__device__ __forceinline__ void lh_apply(const double *x, double tau, int r0, int r1, double *y) {
  double s0 = y[r0], s1 = 0.0, s2 = 0.0, s3 = 0.0;
  int r = r0 + 1;
  for (; r + 3 <= r1; r += 4) {
    s0 = fma(x[r], y[r], s0);
    s1 = fma(x[r + 1], y[r + 1], s1);
    s2 = fma(x[r + 2], y[r + 2], s2);
    s3 = fma(x[r + 3], y[r + 3], s3);
  }
  for (; r <= r1; ++r) s0 = fma(x[r], y[r], s0);
  const double s = tau * ((s0 + s1) + (s2 + s3));
  y[r0] -= s;
  r = r0 + 1;
  for (; r + 3 <= r1; r += 4) {
    const double a0 = y[r], a1 = y[r + 1], a2 = y[r + 2], a3 = y[r + 3];
    const double v0 = x[r], v1 = x[r + 1], v2 = x[r + 2], v3 = x[r + 3];
    y[r] = fma(-s, v0, a0);
    y[r + 1] = fma(-s, v1, a1);
    y[r + 2] = fma(-s, v2, a2);
    y[r + 3] = fma(-s, v3, a3);
  }
  for (; r <= r1; ++r) y[r] = fma(-s, x[r], y[r]);
}

// Value of lane `ln` (uniform) of v, in every lane.
__device__ __forceinline__ double read_lane(double v, int ln) {
  const unsigned long long b = __builtin_bit_cast(unsigned long long, v);
  const unsigned lo = __builtin_amdgcn_readlane(unsigned(b), ln);
  const unsigned hi = __builtin_amdgcn_readlane(unsigned(b >> 32), ln);
  return __builtin_bit_cast(double, (static_cast<unsigned long long>(hi) << 32) | lo);
}

// Back substitution T_FF z = c_F over the packed free block (f <= 64 NS):
// lane l holds z at rows l, l + 64, ...; each step reads its entry from the
// owning lane (a scalar read) and updates the rows above it.
template <int NS>
__device__ __forceinline__ void lh_backsub(const double *B, const double *c, const double *rd, double *z, int f) {
  const int lane = threadIdx.x;
  double zr[NS];
#pragma unroll
  for (int s2 = 0; s2 < NS; ++s2) {
    const int i = lane + 64 * s2;
    zr[s2] = i < f ? c[i] : 0.0;
  }
  for (int k = f - 1; k >= 0; --k) {
    const int sk = k >> 6;
    const double *C = B + poff(k);
    double cv[NS];
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2) {
      const int i = lane + 64 * s2;
      cv[s2] = i < k ? C[i] : 0.0;
    }
    double mine = zr[0];
#pragma unroll
    for (int s2 = 1; s2 < NS; ++s2)
      if (s2 == sk) mine = zr[s2];
    const double zk = read_lane(mine, k & 63) * rd[k];
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2) {
      const int i = lane + 64 * s2;
      zr[s2] = i == k ? zk : fma(-cv[s2], zk, zr[s2]);
    }
  }
#pragma unroll
  for (int s2 = 0; s2 < NS; ++s2) {
    const int i = lane + 64 * s2;
    if (i < f) z[i] = zr[s2];
  }
}

// The Givens chain of a leaving free column k (see lh_solve's leave): the
// free columns k+1..f-1 move down one place, each restored by a rotation of
// rows q, q+1 that zeroes the subdiagonal entry of the column arriving at q.
// Rotation q needs that column's row q after rotation q-1, so the chain is
// serial; every lane carries the current row q of the targets it owns (the
// moved columns, the zero columns, c and, when kept, the leaving column in
// its new zero slot), and only the rotation itself waits on the previous one.
// Targets, by index tg: [0, nm) the moved columns (old position k+1+tg), then
// the nz zero columns, c, and the new zero slot (when ntar = nm + nz + 2).
// Offsets are from B; `last` is the step at which a moved column is the
// pivot (INT_MAX: never; -1: no target).
template <int KS>
__device__ __forceinline__ void lh_chain(double *B, int64_t cap, int p, int k, int f, int nm, int nz, int ntar) {
  const int lane = threadIdx.x;
  int so[KS], dof[KS], last[KS];
  double carry[KS], bn[KS];
#pragma unroll
  for (int s2 = 0; s2 < KS; ++s2) {
    const int tg = lane + 64 * s2;
    if (tg < nm) {
      so[s2] = poff(k + 1 + tg);
      dof[s2] = poff(k + tg);
      last[s2] = k + tg;
    } else if (tg < ntar) {
      const int m = tg - nm;  // zero column m, then c (m = nz), then the new zero slot (m = nz + 1)
      so[s2] = int(cap - int64_t(p) * (m == nz ? 1 : (m < nz ? m + 2 : nz + 2)));
      dof[s2] = so[s2];
      last[s2] = INT_MAX;
    } else {
      so[s2] = 0;
      dof[s2] = 0;
      last[s2] = -1;
    }
    carry[s2] = last[s2] >= 0 ? B[so[s2] + k] : 0.0;
    bn[s2] = last[s2] > k ? B[so[s2] + k + 1] : 0.0;
  }
  for (int q = k; q < f - 1; ++q) {
    const int tp = q - k;  // the pivot: the moved column arriving at q
    double mine = carry[0];
#pragma unroll
    for (int s2 = 1; s2 < KS; ++s2)
      if (s2 == (tp >> 6)) mine = carry[s2];
    const double x = read_lane(mine, tp & 63);
    const double y = B[poff(q + 1) + q + 1];  // its diagonal, not yet rotated
    const double rr = sqrt(fma(x, x, y * y));
    const double inv = rr > 0.0 ? 1.0 / rr : 0.0;
    const double cs = rr > 0.0 ? x * inv : 1.0, sn = y * inv;
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      const int l = last[s2];
      if (l < q) continue;  // done, or no target (same for the whole slot's loop bounds)
      if (l == q) {
        B[dof[s2] + q] = rr;
        B[dof[s2] + q + 1] = 0.0;
        continue;
      }
      const double b0 = bn[s2];
      bn[s2] = (l > q + 1 && q + 2 < p) ? B[so[s2] + q + 2] : 0.0;
      B[dof[s2] + q] = fma(cs, carry[s2], sn * b0);
      carry[s2] = fma(cs, b0, -sn * carry[s2]);
    }
  }
#pragma unroll
  for (int s2 = 0; s2 < KS; ++s2)
    if (last[s2] == INT_MAX) B[dof[s2] + f - 1] = carry[s2];
}

// Per-slot state of the Lawson-Hanson steps (LDS).
struct LhSlots {
  double *u;     // scaled iterate, by slot
  double *dgi;   // 1 / column norm, by slot (0: left out)
  double *z;     // free-set solution by position; the leaving column
  double *rd;    // 1 / diagonal of the free block
  int *perm;     // slot of each free position
  int *zslot;    // slot of each zero column
};

struct LhResult {
  int iters, status, f;
  double pmin;
};

// The whole refit of one head on the pool at base B (cap words): false when
// the pool overflowed (then nothing was written).  kLds: B is in LDS (the
// compiler then addresses it as such).
template <bool kLds>
__device__ __forceinline__ bool lh_solve(double *B, int64_t cap, const HeadDesc &D, const QrState &St,
                                         const double *__restrict__ Gh, const double *__restrict__ w, int p,
                                         int nwarm, const LhSlots &L, LhResult &R) {
  const int lane = threadIdx.x;
  const int t = int(D.t);
  double *u = L.u, *dgi = L.dgi, *z = L.z, *rd = L.rd;
  int *perm = L.perm, *zslot = L.zslot;
  LhPool P{B, cap, p};
  int nzc = 0;
  for (int a = lane; a < p; a += NQ) {
    const double gaa = Gh[int64_t(a) * t + a];
    const double dg = sqrt(gaa);
    const bool ok = dg > 0.0 && isfinite(dg) && St.Rb[poff(a) + a] != 0.0;
    dgi[a] = ok ? 1.0 / dg : 0.0;
    const double wa = a < nwarm ? w[D.t_off + a] : 0.0;
    u[a] = (ok && wa > 0.0) ? wa * dg : 0.0;
    nzc += (ok && !(wa > 0.0)) ? 1 : 0;
  }
  for (int o = 32; o > 0; o >>= 1) nzc += __shfl_xor(nzc, o);
  if (!P.fits(p, nzc)) return false;
  // the triangle in slot order (Rb's first p columns, same packing) and c
  {
    const int total = poff(p);
    // sixteen loads in flight per lane (one wave copies the whole triangle)
    for (int e0 = 0; e0 < total; e0 += 16 * NQ) {
      double v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int e = e0 + j * NQ + lane;
        v[j] = St.Rb[e < total ? e : total - 1];  // unconditional load; the store below is guarded
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int e = e0 + j * NQ + lane;
        if (e < total) B[e] = v[j];
      }
    }
    double *c = P.c();
    for (int a = lane; a < p; a += NQ) c[a] = St.cb[a];
  }
  __syncthreads();
  // free block in slot order: a free slot after zero ones takes one reflection
  // of rows f..a, which the later slots, the zero columns and c take too
  int f = 0, nz = 0;
  for (int a = 0; a < p; ++a) {
    double *col = B + poff(a);
    if (!(dgi[a] > 0.0)) continue;  // left out (same for every lane)
    if (!(u[a] > 0.0)) {
      double *zk = P.zc(nz);
      for (int r = lane; r < p; r += NQ) zk[r] = r <= a ? col[r] : 0.0;
      if (lane == 0) zslot[nz] = a;
      ++nz;
      __syncthreads();
      continue;
    }
    if (a > f) {
      const double tau = lh_reflect(col, f, a);
      if (tau != 0.0) {
        const int nlater = p - 1 - a;
        const int ntar = nlater + nz + 1;
        for (int j = lane; j < ntar; j += NQ) {
          double *y = j < nlater ? B + poff(a + 1 + j) : (j < nlater + nz ? P.zc(j - nlater) : P.c());
          lh_apply(col, tau, f, a, y);
        }
        __syncthreads();
      }
      double *dst = P.fc(f);
      for (int r = lane; r <= f; r += NQ) dst[r] = col[r];
      if (lane == 0) dst[f + 1] = 0.0;
    }
    if (lane == 0) perm[f] = a;
    ++f;
    __syncthreads();
  }
  const int cap_it = 3 * p + 30;
  int iters = 0, status = 0;
  bool overflow = false;
  // removes free column k (to a new zero column if keep); the later free
  // columns shift down, each restored by a rotation (lh_chain)
  auto leave = [&](int k, bool keep) {
    if (keep && !P.fits(f - 1, nz + 1)) {
      overflow = true;
      return;
    }
    const int slot = perm[k];
    const int nm = f - 1 - k;
    if (keep) {
      double *zk = P.zc(nz);
      const double *ck = P.fc(k);
      for (int r = lane; r < p; r += NQ) zk[r] = r <= k ? ck[r] : 0.0;
    }
    __syncthreads();
    if (lane == 0)
      for (int q = k; q < f - 1; ++q) perm[q] = perm[q + 1];
    // rows above k move unchanged, in increasing order (a column's new place
    // is the old place of the one before it)
    for (int j = k + 1; j < f; ++j) {
      const double *src = P.fc(j);
      double *dst = P.fc(j - 1);
      for (int r = lane; r < k; r += NQ) dst[r] = src[r];
    }
    __syncthreads();
    const int ntar = nm + nz + 1 + (keep ? 1 : 0);
    switch ((ntar + 63) >> 6) {
      case 1: lh_chain<1>(B, P.cap, p, k, f, nm, nz, ntar); break;
      case 2: lh_chain<2>(B, P.cap, p, k, f, nm, nz, ntar); break;
      case 3: lh_chain<3>(B, P.cap, p, k, f, nm, nz, ntar); break;
      case 4: lh_chain<4>(B, P.cap, p, k, f, nm, nz, ntar); break;
      case 5: lh_chain<5>(B, P.cap, p, k, f, nm, nz, ntar); break;
      case 6: lh_chain<6>(B, P.cap, p, k, f, nm, nz, ntar); break;
      case 7: lh_chain<7>(B, P.cap, p, k, f, nm, nz, ntar); break;
      case 8: lh_chain<8>(B, P.cap, p, k, f, nm, nz, ntar); break;
      case 9: lh_chain<9>(B, P.cap, p, k, f, nm, nz, ntar); break;
      case 10: lh_chain<10>(B, P.cap, p, k, f, nm, nz, ntar); break;
      default: lh_chain<11>(B, P.cap, p, k, f, nm, nz, ntar); break;
    }
    __syncthreads();
    --f;
    if (keep) {
      if (lane == 0) zslot[nz] = slot;
      ++nz;
    }
    __syncthreads();
  };
  for (;;) {
    if (iters >= cap_it) {
      status |= int(AMC_HS_NNLS_CAP);
      break;
    }
    ++iters;
    // a free column dependent on the ones before it leaves for good
    int dep = -1;
    {
      int cand = -1;
      for (int k = lane; k < f && cand < 0; k += NQ)
        if (!(fabs(P.fc(k)[k]) > kDepTol)) cand = k;
      (void)wave_max_abs_idx(cand >= 0 ? -double(cand) : -INFINITY, cand, &dep);
    }
    if (dep >= 0) {
      const int a = perm[dep];
      __syncthreads();
      if (lane == 0) {
        dgi[a] = 0.0;
        u[a] = 0.0;
      }
      leave(dep, false);
      status |= int(AMC_HS_NNLS_SINGULAR);
      continue;
    }
    // least squares on the free set: T_FF z = c_F
    {
      const double *c = P.c();
      for (int k = lane; k < f; k += NQ) rd[k] = 1.0 / P.fc(k)[k];
      __syncthreads();
      switch ((f + 63) >> 6) {
        case 0: break;
        case 1: lh_backsub<1>(B, c, rd, z, f); break;
        case 2: lh_backsub<2>(B, c, rd, z, f); break;
        case 3: lh_backsub<3>(B, c, rd, z, f); break;
        case 4: lh_backsub<4>(B, c, rd, z, f); break;
        case 5: lh_backsub<5>(B, c, rd, z, f); break;
        case 6: lh_backsub<6>(B, c, rd, z, f); break;
        case 7: lh_backsub<7>(B, c, rd, z, f); break;
        case 8: lh_backsub<8>(B, c, rd, z, f); break;
        case 9: lh_backsub<9>(B, c, rd, z, f); break;
        default: lh_backsub<10>(B, c, rd, z, f); break;
      }
      __syncthreads();
    }
    // infeasible: step from u toward z until the first free variable reaches zero
    int ib = -1;
    double best;
    {
      int cand = -1;
      double bv = INFINITY;
      for (int k = lane; k < f; k += NQ) {
        if (!(z[k] > 0.0)) {
          const double ua = u[perm[k]];
          const double rt = ua > 0.0 ? ua / (ua - z[k]) : 0.0;
          if (cand < 0 || rt < bv) {
            bv = rt;
            cand = k;
          }
        }
      }
      best = -wave_max_abs_idx(cand >= 0 ? -bv : -INFINITY, cand, &ib);
    }
    if (ib >= 0) {
      for (int k = lane; k < f; k += NQ) {
        const int a = perm[k];
        const double un = k == ib ? 0.0 : fma(best, z[k] - u[a], u[a]);
        u[a] = un > 0.0 ? un : 0.0;
      }
      __syncthreads();
      // each free variable now at zero leaves the free block (the highest position first)
      for (int k = f - 1; k >= 0; --k) {
        if (u[perm[k]] > 0.0) continue;  // same for every lane
        leave(k, true);
        if (overflow) return false;
      }
      continue;
    }
    for (int k = lane; k < f; k += NQ) u[perm[k]] = z[k];
    __syncthreads();
    // residual below the free rows, and the cosine of every zero column's part there with it
    const double *c = P.c();
    double rr = 0.0;
    for (int r = f + lane; r < p; r += NQ) rr = fma(c[r], c[r], rr);
    const double nr = sqrt(wsum(rr));
    int enter = -1;
    if (nr > 0.0) {
      double bv = -INFINITY;
      int bs = -1, bq = -1;
      for (int k = lane; k < nz; k += NQ) {
        const double *Z = P.zc(k);
        double n0 = 0.0, n1 = 0.0, d0 = 0.0, d1 = 0.0;
        int r = f;
        for (; r + 1 < p; r += 2) {
          const double z0 = Z[r], z1 = Z[r + 1];
          n0 = fma(z0, c[r], n0);
          n1 = fma(z1, c[r + 1], n1);
          d0 = fma(z0, z0, d0);
          d1 = fma(z1, z1, d1);
        }
        if (r < p) {
          n0 = fma(Z[r], c[r], n0);
          d0 = fma(Z[r], Z[r], d0);
        }
        const double num = n0 + n1;
        double den = sqrt(d0 + d1);
        if (den > kDepTol) {
          const double cs = num / (den * nr);
          const int sl = zslot[k];
          if (cs > kCosTol && (bs < 0 || cs > bv || (cs == bv && sl < bs))) {
            bv = cs;
            bs = sl;
            bq = k;
          }
        }
      }
      for (int o = 32; o > 0; o >>= 1) {
        const double ov = __shfl_xor(bv, o);
        const int os = __shfl_xor(bs, o), oq = __shfl_xor(bq, o);
        if (os >= 0 && (bs < 0 || ov > bv || (ov == bv && os < bs))) {
          bv = ov;
          bs = os;
          bq = oq;
        }
      }
      enter = bq;
    }
    if (enter < 0) break;
    // the entering column: one reflection of rows f..p-1 (which the other zero
    // columns and c take too) leaves it triangular at position f
    double *Ze = P.zc(enter);
    const int slot = zslot[enter];
    if (f + 1 < p) {
      const double tau = lh_reflect(Ze, f, p - 1);
      if (tau != 0.0) {
        for (int j = lane; j <= nz; j += NQ)
          if (j != enter) lh_apply(Ze, tau, f, p - 1, j < nz ? P.zc(j) : P.c());
        __syncthreads();
      }
    }
    for (int r = lane; r <= f; r += NQ) z[r] = Ze[r];
    __syncthreads();
    // the last zero column takes the entering one's place
    if (enter != nz - 1) {
      const double *Zl = P.zc(nz - 1);
      for (int r = lane; r < p; r += NQ) Ze[r] = Zl[r];
      if (lane == 0) zslot[enter] = zslot[nz - 1];
    }
    --nz;
    __syncthreads();
    if (!P.fits(f + 1, nz)) return false;
    double *dst = P.fc(f);
    for (int r = lane; r <= f; r += NQ) dst[r] = z[r];
    if (lane == 0) {
      dst[f + 1] = 0.0;
      perm[f] = slot;
    }
    ++f;
    __syncthreads();
  }
  __syncthreads();
  double pmin = INFINITY;
  for (int k = lane; k < f; k += NQ) pmin = fmin(pmin, fabs(P.fc(k)[k]));
  for (int o = 32; o > 0; o >>= 1) pmin = fmin(pmin, __shfl_xor(pmin, o));
  R.iters = iters;
  R.status = status;
  R.f = f;
  R.pmin = pmin;
  return true;
}

__global__ __launch_bounds__(NQ) void k_nnls_qr(const HeadDesc *__restrict__ desc, const double *__restrict__ G,
                                                double *__restrict__ w, int cycle, int kR, int polish,
                                                int32_t *__restrict__ qr_flag, double *__restrict__ qrbuf,
                                                int32_t *__restrict__ tr_iters, double *__restrict__ tr_weight,
                                                int32_t *__restrict__ head_status, int lds_words) {
  extern __shared__ __attribute__((aligned(16))) double lds[];
  const int h = blockIdx.x;
  const int flag = qr_flag[h];
  if (flag == 0) return;
  const HeadDesc D = desc[h];
  if (D.t > kQrMaxT || D.n > kQrMaxN || D.qr_off < 0) return;
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
  const int lane = threadIdx.x;
  const QrState St = qr_state(D, qrbuf);
  const QrLayout QL = qr_layout(D.t, D.n);
  // per-slot arrays at the bottom of the dynamic LDS, then the pool
  LhSlots L;
  L.u = lds;
  L.dgi = lds + p;
  L.z = lds + 2 * p;
  L.rd = lds + 3 * p;
  L.perm = reinterpret_cast<int *>(lds + 4 * p);
  L.zslot = L.perm + p;
  // warm start: the weights of the previous refit; a head flagged by the Gram
  // solver at this refit, or whose every refit the Gram solver runs first
  // (flag bit 8), also has its weights for the new keys
  const int nwarm = ((flag & 3) == 1 || (flag & 8)) ? p : int(S0);
  const double *Gh = G + D.tt_off;
  LhResult R;
  if (!lh_solve<true>(lds + 5 * p, int64_t(lds_words) - 5 * p, D, St, Gh, w, p, nwarm, L, R)) {
    __syncthreads();
    (void)lh_solve<false>(St.W, QL.total - QL.W, D, St, Gh, w, p, nwarm, L, R);  // holds every state
  }
  __syncthreads();
  for (int a = lane; a < p; a += NQ) {
    const double wa = L.dgi[a] > 0.0 ? L.u[a] * L.dgi[a] : 0.0;
    w[D.t_off + a] = wa;
    if (tr_weight) tr_weight[D.t_off + a] = wa;
  }
  // the value fit leaves the normal equations when the free columns are
  // nearly dependent: smallest pivot of the free block below 1e-6
  if (lane == 0) {
    qr_flag[h] = 2 | (flag & 8) | (((flag & 4) || (polish && R.pmin < kOlsPivot)) ? 4 : 0);
    if (tr_iters && !polish) tr_iters[D.cyc_off + cycle] = R.iters;
    if (head_status) atomicOr(head_status + h, R.status | int(AMC_HS_NNLS_QR));
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
  if ((qr_flag[h] & 4) == 0) return;
  const HeadDesc Dh = desc[h];
  if (Dh.t > kQrMaxT || Dh.qr_off < 0) return;
  const int tid = threadIdx.x;
  const int t = int(Dh.t);
  const QrState St = qr_state(Dh, qrbuf);
  const int ld = St.ld;
  double *T = St.W;
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
  double *X = St.W + int64_t(ld) * ld;
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

hipError_t launch_nnls_qr(const Dims &dm, const Buffers &b, int cycle, int kR, int polish, hipStream_t s) {
  if (!b.qr_flag) return hipSuccess;
  // one launch per row-count class present among the launch's heads: class
  // RPT takes n in (NA RPT / 2, NA RPT] (the first class from n = 1)
  const int64_t lo = dm.n_lo, hi = dm.n_hi < kQrMaxN ? dm.n_hi : kQrMaxN;
  auto has = [&](int64_t a, int64_t b_) { return lo <= b_ && hi > a; };
  if (has(0, 2 * NA))
    hipLaunchKernelGGL((k_qr_append<2, 8>), dim3(unsigned(dm.H)), dim3(NA), 0, s, b.desc, b.panel, b.m, b.G, cycle,
                       kR, polish, b.qr_flag, b.qr_built, b.qrbuf);
  if (has(2 * NA, 4 * NA))
    hipLaunchKernelGGL((k_qr_append<4, 8>), dim3(unsigned(dm.H)), dim3(NA), 0, s, b.desc, b.panel, b.m, b.G, cycle,
                       kR, polish, b.qr_flag, b.qr_built, b.qrbuf);
  if (has(4 * NA, 8 * NA))
    hipLaunchKernelGGL((k_qr_append<8, 8>), dim3(unsigned(dm.H)), dim3(NA), 0, s, b.desc, b.panel, b.m, b.G, cycle,
                       kR, polish, b.qr_flag, b.qr_built, b.qrbuf);
  if (has(8 * NA, 16 * NA))
    hipLaunchKernelGGL((k_qr_append<16, 4>), dim3(unsigned(dm.H)), dim3(NA), 0, s, b.desc, b.panel, b.m, b.G, cycle,
                       kR, polish, b.qr_flag, b.qr_built, b.qrbuf);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t tq = dm.max_t < kQrMaxT ? dm.max_t : kQrMaxT;
  // per-slot arrays (5 words a slot) and the whole pool of the largest head, within kLhLdsBytes
  int64_t words = 5 * tq + tq * (tq + 3) / 2 + tq + 2 + tq * tq;
  if (words * 8 > kLhLdsBytes) words = kLhLdsBytes / 8;
  e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_nnls_qr), hipFuncAttributeMaxDynamicSharedMemorySize,
                          int(words * 8));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_nnls_qr, dim3(unsigned(dm.H)), dim3(NQ), size_t(words * 8), s, b.desc, b.G, b.w, cycle, kR,
                     polish, b.qr_flag, b.qrbuf, b.tr_iters, b.tr_weight, b.head_status, int(words));
  return hipGetLastError();
}

hipError_t launch_ols_qr(const Dims &dm, const Buffers &b, hipStream_t s) {
  if (!b.qr_flag) return hipSuccess;
  const size_t bytes = size_t(kQrLdsBytes);
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
