// Value fit and packing (xinfinite.net article, section 2, step 3: with C_k
// and beta fixed, C_v is an ordinary least-squares solution).
//
// The compacted block's attention output for query i is sum_j A_ij C_v[j]
// with A_ij = Phi_ij w_j / mhat_i over the keys with w_j > 0 (a key with
// w_j = 0 has beta = -inf and contributes nothing).  C_v solves the normal
// equations (A^T A) C_v = A^T Y; A^T A is formed in float64 from the float64
// panel and factored by Cholesky in unit-diagonal form (condition numbers
// reach ~1e9 here), with a small diagonal shift as the fallback when a pivot
// vanishes (then AMC_HS_CHOL_JITTER is reported).
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <type_traits>

#include "amc_internal.h"

namespace amc {
namespace {

constexpr int NT = 256;

__device__ __forceinline__ int tri(int r) { return r * (r + 1) / 2; }

__device__ __forceinline__ void decode_tri(int e, int *r, int *c) {
  int rr = int((sqrtf(8.0f * float(e) + 1.0f) - 1.0f) * 0.5f);
  while (tri(rr + 1) <= e) ++rr;
  while (tri(rr) > e) --rr;
  *r = rr;
  *c = e - tri(rr);
}

// ---------------------------------------------------------------------------
// normal equations: N = At At^T and rhs = At Y with At[a][i] = P[a][i] w_a / mhat_i,
// formed as N[a][b] = w_a w_b sum_i X[a][i] X[b][i] and rhs[a][d] = w_a sum_i
// X[a][i] Y[i][d] with X[a][i] = P[a][i] / mhat_i, on float64 MFMA.
// Block tile: 64 rows a x 64 columns, of N (column tiles below tx = ceil(t /
// 64)) or of rhs (the D columns after them); each wave takes 16 rows; the
// queries are staged through LDS 64 at a time, the next stage prefetched into
// registers.  N is symmetric and its readers take the lower triangle, so the
// tiles wholly above the diagonal are skipped.
// ---------------------------------------------------------------------------
typedef double f64x4o __attribute__((ext_vector_type(4)));

template <int D>
__global__ __launch_bounds__(NT) void k_ols_normal(const HeadDesc *__restrict__ desc, const double *__restrict__ panel,
                                                   const double *__restrict__ w, const double *__restrict__ mhat,
                                                   const float *__restrict__ Y, double *__restrict__ N,
                                                   double *__restrict__ rhs, int H, int tx, int ty, int xcd_map,
    const int32_t *__restrict__ qr_flag) {
  constexpr int CH = 64;       // queries per stage
  constexpr int STR = CH + 1;  // padded row, in doubles
  __shared__ double xs[64 * STR];
  __shared__ double zs[64 * STR];
  __shared__ double minv[2][CH];
  // tx * ty tiles per head; with xcd_map (H a multiple of 8) the tiles of a
  // head go to one XCD, so its panel is fetched into one L2
  int h, j;
  {
    const int b = blockIdx.x, per = tx * ty;
    if (xcd_map) {
      const int slot = b >> 3;
      h = (b & 7) + 8 * (slot / per);
      j = slot % per;
    } else {
      h = b / per;
      j = b % per;
    }
  }
  if (h >= H) return;
  const HeadDesc Dh = desc[h];
  if (qr_flag && (qr_flag[h] & 4)) return;  // the value fit of k_ols_qr
  const int64_t t = Dh.t, n = Dh.n;
  const int64_t a0 = int64_t(j % tx) * 64;
  const int bt = j / tx;
  const bool isN = bt < tx;
  const int64_t b0 = isN ? int64_t(bt) * 64 : int64_t(bt - tx) * 64;  // N column or rhs column
  if (a0 >= t || (isN && (b0 >= t || b0 > a0)) || (!isN && b0 >= D)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  const double *P = Dh.panel_off + panel;
  // staged values before scaling by 1/mhat: 16 row and 16 column values per thread
  double xr[16], zr[16];
  double mr = 1.0;
  auto fetch = [&](int64_t i0) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = tid + NT * u;
      const int rr = e / CH, c = e % CH;
      const int64_t i = i0 + c;
      const int64_t a = a0 + rr, b = b0 + rr;
      xr[u] = (i < n && a < t) ? P[a * n + i] : 0.0;
      zr[u] = (isN && i < n && b < t) ? P[b * n + i] : 0.0;
    }
    if (tid < CH) mr = i0 + tid < n ? mhat[Dh.n_off + i0 + tid] : 1.0;
  };
  static_assert(64 * CH == 16 * NT, "stage size");
  f64x4o acc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] = f64x4o{0.0, 0.0, 0.0, 0.0};
  fetch(0);
  int buf = 0;
  for (int64_t i0 = 0; i0 < n; i0 += CH) {
    if (tid < CH) minv[buf][tid] = 1.0 / mr;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = tid + NT * u;
      const int rr = e / CH, c = e % CH;
      const double iv = minv[buf][c];
      xs[rr * STR + c] = xr[u] * iv;
      const int64_t b = b0 + rr;
      if (isN) {
        zs[rr * STR + c] = zr[u] * iv;
      } else {
        const int64_t i = i0 + c;
        zs[rr * STR + c] = (b < D && i < n) ? double(Y[(Dh.n_off + i) * D + b]) : 0.0;
      }
    }
    __syncthreads();
    if (i0 + CH < n) fetch(i0 + CH);
    const double *xa = &xs[(wave * 16 + c16) * STR + g];
#pragma unroll
    for (int k = 0; k < CH / 4; ++k) {
      const double av = xa[4 * k];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        acc[q] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, zs[(16 * q + c16) * STR + 4 * k + g], acc[q], 0, 0, 0);
    }
    buf ^= 1;
  }
  // element e of lane group g: row wave*16 + g + 4e; tile q: column 16 q + c16
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t a = a0 + wave * 16 + g + 4 * e;
    if (a >= t) continue;
    const double wa = w[Dh.t_off + a];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t b = b0 + 16 * q + c16;
      if (isN) {
        if (b < t) N[Dh.tt_off + a * t + b] = acc[q][e] * wa * w[Dh.t_off + b];
      } else if (b < D) {
        rhs[(Dh.t_off + a) * D + b] = acc[q][e] * wa;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// factor: unit-diagonal Cholesky of N restricted to F = {a : w_a > 0}.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(NT) void k_ols_factor(const HeadDesc *__restrict__ desc, const double *__restrict__ N,
                                                   const double *__restrict__ w, int32_t *__restrict__ flist,
                                                   int32_t *__restrict__ fcount, double *__restrict__ dn,
                                                   double *__restrict__ Lout, int32_t *__restrict__ head_status,
    const int32_t *__restrict__ qr_flag) {
  extern __shared__ __attribute__((aligned(16))) double Ls[];
  __shared__ int sf[kLdsMaxT];
  __shared__ double sdn[kLdsMaxT];
  __shared__ int sh_f, sh_fail;
  const int h = blockIdx.x;
  const HeadDesc Dh = desc[h];
  if (qr_flag && (qr_flag[h] & 4)) return;  // the value fit of k_ols_qr
  if (Dh.t > kLdsMaxT) return;  // k_ols_factor_g
  const int t = int(Dh.t);
  const int tid = threadIdx.x;
  if (tid == 0) {
    int k = 0;
    for (int a = 0; a < t; ++a)
      if (w[Dh.t_off + a] > 0.0) sf[k++] = a;
    sh_f = k;
  }
  __syncthreads();
  const int f = sh_f;
  for (int k = tid; k < f; k += NT) {
    const double v = N[Dh.tt_off + int64_t(sf[k]) * t + sf[k]];
    sdn[k] = (v > 0.0 && isfinite(v)) ? sqrt(v) : 1.0;
  }
  __syncthreads();
  double jitter = 0.0;
  for (int attempt = 0; attempt < 6; ++attempt) {
    const int ne = tri(f);
    for (int e = tid; e < ne; e += NT) {
      int r, c;
      decode_tri(e, &r, &c);
      double v = N[Dh.tt_off + int64_t(sf[r]) * t + sf[c]] / (sdn[r] * sdn[c]);
      if (r == c) v += jitter;
      Ls[e] = v;
    }
    if (tid == 0) sh_fail = -1;
    __syncthreads();
    for (int k = 0; k < f; ++k) {
      if (tid == 0) {
        const double piv = Ls[tri(k) + k];
        if (!(piv > 1e-15)) sh_fail = k;
        else Ls[tri(k) + k] = sqrt(piv);
      }
      __syncthreads();
      if (sh_fail >= 0) break;
      const double dkk = Ls[tri(k) + k];
      for (int r = k + 1 + tid; r < f; r += NT) Ls[tri(r) + k] /= dkk;
      __syncthreads();
      const int mm = f - k - 1;
      const int nt = tri(mm);
      for (int e = tid; e < nt; e += NT) {
        int r, c;
        decode_tri(e, &r, &c);
        r += k + 1;
        c += k + 1;
        Ls[tri(r) + c] -= Ls[tri(r) + k] * Ls[tri(c) + k];
      }
      __syncthreads();
    }
    if (sh_fail < 0) break;
    jitter = jitter == 0.0 ? 1e-13 : jitter * 100.0;
    if (tid == 0 && head_status) atomicOr(head_status + h, int32_t(AMC_HS_CHOL_JITTER));
    __syncthreads();
  }
  for (int e = tid; e < tri(f); e += NT) Lout[Dh.tt_off + e] = Ls[e];
  for (int k = tid; k < f; k += NT) {
    flist[Dh.t_off + k] = sf[k];
    dn[Dh.t_off + k] = sdn[k];
  }
  if (tid == 0) fcount[h] = f;
}

// ---------------------------------------------------------------------------
// triangular solves, 32 right-hand-side columns per block and 8 per wave; each
// wave substitutes column by column with no block barriers: lane l holds rows
// l, l + 64 and l + 128 of its 8 columns, x_k = r_k / L_kk comes from its
// lane, and column k of L (forward) or row k (backward) is applied to the rows
// still open.  C_v[F] = D^-1 X.
// ---------------------------------------------------------------------------
__device__ __forceinline__ double rl64(double x, int lane) {
  const int lo = __builtin_amdgcn_readlane(__double2loint(x), lane);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(x), lane);
  return __hiloint2double(hi, lo);
}

template <int D>
__global__ __launch_bounds__(NT) void k_ols_trsm(const HeadDesc *__restrict__ desc, const double *__restrict__ rhs,
                                                 const int32_t *__restrict__ flist,
                                                 const int32_t *__restrict__ fcount, const double *__restrict__ dn,
                                                 const double *__restrict__ Lg, const double *__restrict__ w,
                                                 float *__restrict__ cv_sel,
    const int32_t *__restrict__ qr_flag) {
  constexpr int NCB = 32, NCW = 8;
  static_assert(kLdsMaxT <= 192, "three rows per lane");
  extern __shared__ __attribute__((aligned(16))) double sm[];
  const int h = blockIdx.y;
  const HeadDesc Dh = desc[h];
  if (qr_flag && (qr_flag[h] & 4)) return;  // the value fit of k_ols_qr
  if (Dh.t > kLdsMaxT) return;  // k_ols_trsm_g
  const int t = int(Dh.t);
  const int c0 = blockIdx.x * NCB;
  const int f = fcount[h];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  double *Ls = sm;
  for (int e = tid; e < tri(f); e += NT) Ls[e] = Lg[Dh.tt_off + e];
  // keys with w = 0 get a zero value row
  for (int e = tid; e < t * NCB; e += NT) {
    const int a = e / NCB, c = e % NCB;
    if (!(w[Dh.t_off + a] > 0.0)) cv_sel[(Dh.t_off + a) * D + c0 + c] = 0.0f;
  }
  __syncthreads();
  const int cw = c0 + NCW * wave;
  int rbase[3];
  double rd[3], xv[NCW][3];
#pragma unroll
  for (int m = 0; m < 3; ++m) {
    const int i = lane + 64 * m;
    rbase[m] = i < f ? tri(i) : 0;
    rd[m] = i < f ? 1.0 / Ls[rbase[m] + i] : 0.0;
    const int64_t row = i < f ? (Dh.t_off + flist[Dh.t_off + i]) * D : 0;
    const double di = i < f ? dn[Dh.t_off + i] : 1.0;
#pragma unroll
    for (int q = 0; q < NCW; ++q) xv[q][m] = i < f ? rhs[row + cw + q] / di : 0.0;
  }
  // forward: L y = x, column k of L below row k
#pragma unroll
  for (int M = 0; M < 3; ++M) {
    const int k1 = f < 64 * M + 64 ? f : 64 * M + 64;
    for (int k = 64 * M; k < k1; ++k) {
      const int kl = k - 64 * M;
      double lc[3];
#pragma unroll
      for (int m = 0; m < 3; ++m)
        lc[m] = (m >= M && (m > M || lane > kl) && lane + 64 * m < f) ? Ls[rbase[m] + k] : 0.0;
#pragma unroll
      for (int q = 0; q < NCW; ++q) {
        const double xk = rl64(xv[q][M] * rd[M], kl);
#pragma unroll
        for (int m = M; m < 3; ++m) xv[q][m] = fma(-lc[m], xk, xv[q][m]);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < NCW; ++q)
#pragma unroll
    for (int m = 0; m < 3; ++m) xv[q][m] *= rd[m];
  // backward: L^T z = y, row k of L left of column k
#pragma unroll
  for (int MM = 0; MM < 3; ++MM) {
    const int M = 2 - MM;
    for (int k = (f < 64 * M + 64 ? f : 64 * M + 64) - 1; k >= 64 * M; --k) {
      const int kl = k - 64 * M;
      const double *Lk = Ls + tri(k);
      double lr[3];
#pragma unroll
      for (int m = 0; m < 3; ++m) lr[m] = m < M ? Lk[lane + 64 * m] : (m == M && lane < kl ? Lk[lane + 64 * M] : 0.0);
#pragma unroll
      for (int q = 0; q < NCW; ++q) {
        const double xk = rl64(xv[q][M] * rd[M], kl);
#pragma unroll
        for (int m = 0; m <= M; ++m) xv[q][m] = fma(-lr[m], xk, xv[q][m]);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < 3; ++m) {
    const int i = lane + 64 * m;
    if (i < f) {
      const int64_t row = (Dh.t_off + flist[Dh.t_off + i]) * D;
      const double di = dn[Dh.t_off + i];
#pragma unroll
      for (int q = 0; q < NCW; ++q) cv_sel[row + cw + q] = float(xv[q][m] * rd[m] / di);
    }
  }
}

// ---------------------------------------------------------------------------
// pack: ascending original index; C_k copy, beta = beta_in + log w, C_v, sel_idx
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

template <int D, bool BF16>
__global__ __launch_bounds__(NT) void k_pack(const HeadDesc *__restrict__ desc, const int32_t *__restrict__ sel_slot,
                                             const int32_t *__restrict__ sel_list, const double *__restrict__ w,
                                             const float *__restrict__ beta_in, const void *__restrict__ Kv,
                                             const float *__restrict__ cv_sel, void *__restrict__ Ckv,
                                             float *__restrict__ beta, void *__restrict__ Cvv, int cv_bf16,
                                             int32_t *__restrict__ sel_idx, int32_t *__restrict__ pos_of_slot) {
  using E = typename std::conditional<BF16, uint16_t, float>::type;
  __shared__ int cnt[NT];
  const int h = blockIdx.x;
  const HeadDesc Dh = desc[h];
  const int tid = threadIdx.x;
  const int64_t T = Dh.T;
  const int64_t chunk = (T + NT - 1) / NT;
  const int64_t j0 = tid * chunk, j1 = (j0 + chunk < T) ? j0 + chunk : T;
  int32_t *spos = pos_of_slot + Dh.t_off;
  for (int64_t a = tid; a < Dh.t; a += NT) spos[a] = -1;
  int c = 0;
  for (int64_t j = j0; j < j1; ++j) c += sel_slot[Dh.k_off + j] != 0;
  cnt[tid] = c;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < NT; ++i) {
      const int v = cnt[i];
      cnt[i] = run;
      run += v;
    }
  }
  __syncthreads();
  int pos = cnt[tid];
  const int64_t out = Dh.t_off;
  for (int64_t j = j0; j < j1; ++j) {
    const int s = sel_slot[Dh.k_off + j];
    if (s <= 0 || s > Dh.t || pos >= Dh.t) continue;
    const int slot = s - 1;
    spos[slot] = pos;
    if (sel_idx) sel_idx[out + pos] = int32_t(j);
    const double wv = w[Dh.t_off + slot];
    const double bi = beta_in ? double(beta_in[Dh.k_off + j]) : 0.0;
    beta[out + pos] = wv > 0.0 ? float(bi + log(wv)) : -INFINITY;
    ++pos;
  }
  __syncthreads();
  const E *K = static_cast<const E *>(Kv);
  E *Ck = static_cast<E *>(Ckv);
  const int64_t t = Dh.t;
  for (int64_t e = tid; e < t * D; e += NT) {
    const int64_t a = e / D, col = e % D;
    const int sp = spos[a];
    const int j = sel_list[Dh.t_off + a];
    if (sp < 0 || j < 0 || j >= Dh.T) continue;
    const int64_t row = out + sp;
    Ck[row * D + col] = K[(Dh.k_off + j) * D + col];
    const float v = cv_sel[(Dh.t_off + a) * D + col];
    if (cv_bf16) static_cast<uint16_t *>(Cvv)[row * D + col] = f32_to_bf16_rne(v);
    else static_cast<float *>(Cvv)[row * D + col] = v;
  }
}

// ---------------------------------------------------------------------------
// Budgets above kLdsMaxT: the same value fit with the factor in global memory.
// ---------------------------------------------------------------------------
constexpr int TBO = 16;  // panel width of the blocked factorisation and solves

template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

__device__ __forceinline__ double rl(double x, int lane) {
  const int lo = __builtin_amdgcn_readlane(__double2loint(x), lane);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(x), lane);
  return __hiloint2double(hi, lo);
}

// F = {a : w_a > 0} ascending, its size, and the diagonal scaling of N_FF.
__global__ __launch_bounds__(NT) void k_ols_flist_g(const HeadDesc *__restrict__ desc, const double *__restrict__ N,
                                                    const double *__restrict__ w, int32_t *__restrict__ flist,
                                                    int32_t *__restrict__ fcount, double *__restrict__ dn,
    const int32_t *__restrict__ qr_flag) {
  __shared__ int wcnt[NT / 64];
  const int h = blockIdx.x;
  const HeadDesc Dh = desc[h];
  if (qr_flag && (qr_flag[h] & 4)) return;  // the value fit of k_ols_qr
  if (Dh.t <= kLdsMaxT) return;
  const int t = int(Dh.t);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t *fl = flist + Dh.t_off;
  int base = 0;
  for (int a0 = 0; a0 < t; a0 += NT) {
    const int a = a0 + tid;
    const bool pred = a < t && w[Dh.t_off + a] > 0.0;
    const unsigned long long bal = __ballot(pred);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wcnt[wave] = __popcll(bal);
    __syncthreads();
    int off = base;
    for (int v = 0; v < wave; ++v) off += wcnt[v];
    if (pred) fl[off + before] = a;
    for (int v = 0; v < NT / 64; ++v) base += wcnt[v];
    __syncthreads();
  }
  for (int k = tid; k < base; k += NT) {
    const int a = fl[k];
    const double v = N[Dh.tt_off + int64_t(a) * t + a];
    dn[Dh.t_off + k] = (v > 0.0 && isfinite(v)) ? sqrt(v) : 1.0;
  }
  if (tid == 0) fcount[h] = base;
}

// Blocked right-looking Cholesky of the scaled N_FF in the packed factor
// storage: per panel of 16 columns, wave 0 factors the diagonal block in
// registers, every thread then solves one row of the panel below it, and the
// trailing triangle takes the panel's rank-16 update in 4 x 4 tiles.
__global__ __launch_bounds__(NT) void k_ols_factor_g(const HeadDesc *__restrict__ desc, const double *__restrict__ N,
                                                     const int32_t *__restrict__ flist,
                                                     const int32_t *__restrict__ fcount, const double *__restrict__ dn,
                                                     double *__restrict__ L, int32_t *__restrict__ head_status,
    const int32_t *__restrict__ qr_flag) {
  __shared__ double Db[TBO * TBO];
  __shared__ int sh_fail;
  const int h = blockIdx.x;
  const HeadDesc Dh = desc[h];
  if (qr_flag && (qr_flag[h] & 4)) return;  // the value fit of k_ols_qr
  if (Dh.t <= kLdsMaxT) return;
  const int t = int(Dh.t);
  const int f = fcount[h];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t *fl = flist + Dh.t_off;
  const double *dnh = dn + Dh.t_off;
  const double *Nh = N + Dh.tt_off;
  double *Lh = L + Dh.tt_off;
  double jitter = 0.0;
  for (int attempt = 0; attempt < 6; ++attempt) {
    for (int e = tid; e < tri(f); e += NT) {
      int r, c;
      decode_tri(e, &r, &c);
      double v = Nh[int64_t(fl[r]) * t + fl[c]] / (dnh[r] * dnh[c]);
      if (r == c) v += jitter;
      Lh[e] = v;
    }
    if (tid == 0) sh_fail = -1;
    __syncthreads();
    for (int k0 = 0; k0 < f; k0 += TBO) {
      const int e = f - k0 < TBO ? f - k0 : TBO;
      if (wave == 0 && lane < TBO) {
        const int i = lane;
        const bool act = i < e;
        const int rb = act ? tri(k0 + i) + k0 : 0;
        double Lr[TBO];
        static_for<0, TBO>([&](auto J) {
          constexpr int j = decltype(J)::value;
          Lr[j] = (act && j <= i) ? Lh[rb + j] : 0.0;
        });
        bool bad = false;
        static_for<0, TBO>([&](auto K) {
          constexpr int kk = decltype(K)::value;
          if (kk < e) {
            const double piv = rl(Lr[kk], kk);
            if (!(piv > 1e-15)) bad = true;
            const double d = sqrt(piv > 1e-15 ? piv : 1.0);
            const double rdd = 1.0 / d;
            if (i == kk) Lr[kk] = d;
            else if (i > kk) Lr[kk] *= rdd;
            static_for<kk + 1, TBO>([&](auto J) {
              constexpr int j = decltype(J)::value;
              if (j < e) {
                const double ljk = rl(Lr[kk], j);
                if (i >= j) Lr[j] = fma(-Lr[kk], ljk, Lr[j]);
              }
            });
          }
        });
        if (act) {
          static_for<0, TBO>([&](auto J) {
            constexpr int j = decltype(J)::value;
            if (j <= i) {
              Lh[rb + j] = Lr[j];
              Db[i * TBO + j] = Lr[j];
            }
          });
        }
        if (bad && lane == 0) sh_fail = k0;
      }
      __syncthreads();
      if (sh_fail >= 0) break;
      if (k0 + TBO >= f) continue;
      // panel rows below the block: L[r, k0:k0+16] = A[r, k0:k0+16] L_blk^-T
      for (int r = k0 + TBO + tid; r < f; r += NT) {
        const int rb = tri(r) + k0;
        double x[TBO];
        static_for<0, TBO>([&](auto K) {
          constexpr int kk = decltype(K)::value;
          x[kk] = Lh[rb + kk];
        });
        static_for<0, TBO>([&](auto K) {
          constexpr int kk = decltype(K)::value;
          double v = x[kk];
          static_for<0, kk>([&](auto J) {
            constexpr int j = decltype(J)::value;
            v = fma(-x[j], Db[kk * TBO + j], v);
          });
          x[kk] = v / Db[kk * TBO + kk];
        });
        static_for<0, TBO>([&](auto K) {
          constexpr int kk = decltype(K)::value;
          Lh[rb + kk] = x[kk];
        });
      }
      __syncthreads();
      // trailing update A[r][c] -= sum_j L[r][k0+j] L[c][k0+j], r >= c >= k0 + 16, in 4 x 4 tiles
      const int s0 = k0 + TBO;
      const int m = f - s0;
      const int nb = (m + 3) / 4;
      const int ntiles = nb * (nb + 1) / 2;
      for (int ti = tid; ti < ntiles; ti += NT) {
        int R, C;
        decode_tri(ti, &R, &C);
        int rr[4], cc[4];
        static_for<0, 4>([&](auto Q) {
          constexpr int q = decltype(Q)::value;
          const int r = s0 + 4 * R + q, c = s0 + 4 * C + q;
          rr[q] = r < f ? r : f - 1;
          cc[q] = c < f ? c : f - 1;
        });
        double acc[4][4];
        static_for<0, 4>([&](auto Q) {
          static_for<0, 4>([&](auto U) { acc[decltype(Q)::value][decltype(U)::value] = 0.0; });
        });
        for (int j = 0; j < TBO; ++j) {
          double pr[4], pc[4];
          static_for<0, 4>([&](auto Q) {
            constexpr int q = decltype(Q)::value;
            pr[q] = Lh[tri(rr[q]) + k0 + j];
            pc[q] = Lh[tri(cc[q]) + k0 + j];
          });
          static_for<0, 4>([&](auto Q) {
            constexpr int q = decltype(Q)::value;
            static_for<0, 4>([&](auto U) {
              constexpr int u = decltype(U)::value;
              acc[q][u] = fma(pr[q], pc[u], acc[q][u]);
            });
          });
        }
        static_for<0, 4>([&](auto Q) {
          constexpr int q = decltype(Q)::value;
          const int r = s0 + 4 * R + q;
          static_for<0, 4>([&](auto U) {
            constexpr int u = decltype(U)::value;
            const int c = s0 + 4 * C + u;
            if (r < f && c <= r) Lh[tri(r) + c] -= acc[q][u];
          });
        });
      }
      __syncthreads();
    }
    __syncthreads();
    if (sh_fail < 0) break;
    jitter = jitter == 0.0 ? 1e-13 : jitter * 100.0;
    if (tid == 0 && head_status) atomicOr(head_status + h, int32_t(AMC_HS_CHOL_JITTER));
    __syncthreads();
  }
}

// Triangular solves with the global factor, 8 right-hand-side columns per
// block, in place in the rhs rows of F: L Y = X / dn, L^T Z = Y, C_v = Z / dn.
template <int D>
__global__ __launch_bounds__(NT) void k_ols_trsm_g(const HeadDesc *__restrict__ desc, double *__restrict__ rhs,
                                                   const int32_t *__restrict__ flist,
                                                   const int32_t *__restrict__ fcount, const double *__restrict__ dn,
                                                   const double *__restrict__ L, const double *__restrict__ w,
                                                   float *__restrict__ cv_sel,
    const int32_t *__restrict__ qr_flag) {
  constexpr int NC = 8;
  __shared__ double Db[TBO * TBO];
  __shared__ double Xb[TBO * NC];
  const int h = blockIdx.y;
  const HeadDesc Dh = desc[h];
  if (qr_flag && (qr_flag[h] & 4)) return;  // the value fit of k_ols_qr
  if (Dh.t <= kLdsMaxT) return;
  const int t = int(Dh.t);
  const int c0 = blockIdx.x * NC;
  const int f = fcount[h];
  const int tid = threadIdx.x;
  const int32_t *fl = flist + Dh.t_off;
  const double *dnh = dn + Dh.t_off;
  const double *Lh = L + Dh.tt_off;
  auto X = [&](int k) -> double * { return rhs + (Dh.t_off + fl[k]) * D + c0; };
  for (int e = tid; e < t * NC; e += NT) {
    const int a = e / NC, c = e % NC;
    if (!(w[Dh.t_off + a] > 0.0)) cv_sel[(Dh.t_off + a) * D + c0 + c] = 0.0f;
  }
  for (int e = tid; e < f * NC; e += NT) X(e / NC)[e % NC] /= dnh[e / NC];
  __syncthreads();
  // forward
  for (int k0 = 0; k0 < f; k0 += TBO) {
    const int e = f - k0 < TBO ? f - k0 : TBO;
    for (int q = tid; q < TBO * TBO; q += NT) {
      const int i = q / TBO, j = q % TBO;
      Db[q] = (i < e && j <= i) ? Lh[tri(k0 + i) + k0 + j] : 0.0;
    }
    for (int q = tid; q < e * NC; q += NT) Xb[q] = X(k0 + q / NC)[q % NC];
    __syncthreads();
    if (tid < NC) {
      for (int i = 0; i < e; ++i) {
        double v = Xb[i * NC + tid];
        for (int j = 0; j < i; ++j) v = fma(-Db[i * TBO + j], Xb[j * NC + tid], v);
        Xb[i * NC + tid] = v / Db[i * TBO + i];
      }
    }
    __syncthreads();
    for (int q = tid; q < e * NC; q += NT) X(k0 + q / NC)[q % NC] = Xb[q];
    for (int r = k0 + TBO + tid; r < f; r += NT) {
      const int rb = tri(r) + k0;
      double lr[TBO];
      static_for<0, TBO>([&](auto J) {
        constexpr int j = decltype(J)::value;
        lr[j] = Lh[rb + j];
      });
      double *xr = X(r);
      static_for<0, NC>([&](auto Cc) {
        constexpr int c = decltype(Cc)::value;
        double acc = 0.0;
        static_for<0, TBO>([&](auto J) {
          constexpr int j = decltype(J)::value;
          acc = fma(lr[j], Xb[j * NC + c], acc);
        });
        xr[c] -= acc;
      });
    }
    __syncthreads();
  }
  // backward
  for (int k0 = ((f - 1) / TBO) * TBO; f > 0 && k0 >= 0; k0 -= TBO) {
    const int e = f - k0 < TBO ? f - k0 : TBO;
    for (int q = tid; q < TBO * TBO; q += NT) {
      const int i = q / TBO, j = q % TBO;
      Db[q] = (i < e && j <= i) ? Lh[tri(k0 + i) + k0 + j] : 0.0;
    }
    for (int q = tid; q < e * NC; q += NT) Xb[q] = X(k0 + q / NC)[q % NC];
    __syncthreads();
    if (tid < NC) {
      for (int i = e - 1; i >= 0; --i) {
        double v = Xb[i * NC + tid];
        for (int j = i + 1; j < e; ++j) v = fma(-Db[j * TBO + i], Xb[j * NC + tid], v);
        Xb[i * NC + tid] = v / Db[i * TBO + i];
      }
    }
    __syncthreads();
    for (int q = tid; q < e * NC; q += NT) X(k0 + q / NC)[q % NC] = Xb[q];
    for (int r = tid; r < k0; r += NT) {
      double *xr = X(r);
      double acc[NC];
      static_for<0, NC>([&](auto Cc) { acc[decltype(Cc)::value] = 0.0; });
      for (int j = 0; j < e; ++j) {
        const double l = Lh[tri(k0 + j) + r];
        static_for<0, NC>([&](auto Cc) {
          constexpr int c = decltype(Cc)::value;
          acc[c] = fma(l, Xb[j * NC + c], acc[c]);
        });
      }
      static_for<0, NC>([&](auto Cc) {
        constexpr int c = decltype(Cc)::value;
        xr[c] -= acc[c];
      });
    }
    __syncthreads();
  }
  for (int e = tid; e < f * NC; e += NT) {
    const int k = e / NC, c = e % NC;
    cv_sel[(Dh.t_off + fl[k]) * D + c0 + c] = float(X(k)[c] / dnh[k]);
  }
}

}  // namespace

hipError_t launch_ols_normal(const Dims &dm, const Buffers &b, hipStream_t s) {
  const int tx = int((dm.max_t + 63) / 64), ty = tx + int((dm.d + 63) / 64);
  const int xcd_map = dm.H % 8 == 0 ? 1 : 0;
  dim3 grid(unsigned(tx * ty * dm.H));
  if (dm.d == 128)
    hipLaunchKernelGGL((k_ols_normal<128>), grid, dim3(NT), 0, s, b.desc, b.panel, b.w, b.mhat, b.Y, b.G, b.rhs,
                       dm.H, tx, ty, xcd_map, b.qr_flag);
  else
    hipLaunchKernelGGL((k_ols_normal<64>), grid, dim3(NT), 0, s, b.desc, b.panel, b.w, b.mhat, b.Y, b.G, b.rhs,
                       dm.H, tx, ty, xcd_map, b.qr_flag);
  return hipGetLastError();
}

hipError_t launch_ols_factor(const Dims &dm, const Buffers &b, hipStream_t s) {
  if (dm.min_t <= kLdsMaxT) {
    const int64_t mt = dm.max_t < kLdsMaxT ? dm.max_t : kLdsMaxT;
    const size_t bytes = size_t(8) * size_t(mt) * size_t(mt + 1) / 2 + 16;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_ols_factor),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(bytes));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_ols_factor, dim3(unsigned(dm.H)), dim3(NT), bytes, s, b.desc, b.G, b.w, b.ols_flist,
                       b.ols_fcount, b.ols_dn, b.ols_L, b.head_status, b.qr_flag);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (dm.max_t > kLdsMaxT) {
    hipLaunchKernelGGL(k_ols_flist_g, dim3(unsigned(dm.H)), dim3(NT), 0, s, b.desc, b.G, b.w, b.ols_flist,
                       b.ols_fcount, b.ols_dn, b.qr_flag);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_ols_factor_g, dim3(unsigned(dm.H)), dim3(NT), 0, s, b.desc, b.G, b.ols_flist, b.ols_fcount,
                       b.ols_dn, b.ols_L, b.head_status, b.qr_flag);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_ols_trsm(const Dims &dm, const Buffers &b, hipStream_t s) {
  dim3 grid(unsigned(dm.d / 8), unsigned(dm.H));
  if (dm.max_t > kLdsMaxT) {
    if (dm.d == 128)
      hipLaunchKernelGGL((k_ols_trsm_g<128>), grid, dim3(NT), 0, s, b.desc, b.rhs, b.ols_flist, b.ols_fcount,
                         b.ols_dn, b.ols_L, b.w, b.cv_sel, b.qr_flag);
    else
      hipLaunchKernelGGL((k_ols_trsm_g<64>), grid, dim3(NT), 0, s, b.desc, b.rhs, b.ols_flist, b.ols_fcount,
                         b.ols_dn, b.ols_L, b.w, b.cv_sel, b.qr_flag);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || dm.min_t > kLdsMaxT) return e;
  }
  const int64_t mt = dm.max_t < kLdsMaxT ? dm.max_t : kLdsMaxT;
  const size_t bytes = size_t(8) * (size_t(mt) * size_t(mt + 1) / 2) + 16;
  grid = dim3(unsigned(dm.d / 32), unsigned(dm.H));
  hipError_t e;
  if (dm.d == 128) {
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_ols_trsm<128>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(bytes));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_ols_trsm<128>), grid, dim3(NT), bytes, s, b.desc, b.rhs, b.ols_flist, b.ols_fcount,
                       b.ols_dn, b.ols_L, b.w, b.cv_sel, b.qr_flag);
  } else {
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_ols_trsm<64>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(bytes));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_ols_trsm<64>), grid, dim3(NT), bytes, s, b.desc, b.rhs, b.ols_flist, b.ols_fcount,
                       b.ols_dn, b.ols_L, b.w, b.cv_sel, b.qr_flag);
  }
  return hipGetLastError();
}

hipError_t launch_pack(const Dims &dm, const Buffers &b, void *Ck, float *beta, void *Cv, int cv_bf16,
                       int32_t *sel_idx, hipStream_t s) {
#define AMC_PACK_ARGS \
  b.desc, b.sel_slot, b.sel_list, b.w, b.beta_in, b.K, b.cv_sel, Ck, beta, Cv, cv_bf16, sel_idx, b.pos_of_slot
  if (dm.d == 128) {
    if (dm.in_bf16) hipLaunchKernelGGL((k_pack<128, true>), dim3(unsigned(dm.H)), dim3(NT), 0, s, AMC_PACK_ARGS);
    else hipLaunchKernelGGL((k_pack<128, false>), dim3(unsigned(dm.H)), dim3(NT), 0, s, AMC_PACK_ARGS);
  } else {
    if (dm.in_bf16) hipLaunchKernelGGL((k_pack<64, true>), dim3(unsigned(dm.H)), dim3(NT), 0, s, AMC_PACK_ARGS);
    else hipLaunchKernelGGL((k_pack<64, false>), dim3(unsigned(dm.H)), dim3(NT), 0, s, AMC_PACK_ARGS);
  }
#undef AMC_PACK_ARGS
  return hipGetLastError();
}

}  // namespace amc
