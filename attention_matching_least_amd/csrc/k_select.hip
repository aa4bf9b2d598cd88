// Greedy key selection kernels (zhichai.net deep-dive, section 1.6; batched
// top-k selection with delayed refit, xinfinite.net article, section 3):
//
//   sweep  : c_j = r^T Phi[:, j] over the unselected keys, block-local top-(K+1)
//   merge  : per-head top-(K+1) of the block candidates; appends the K picks
//   panel  : float64 columns Phi[:, j] of the new picks, recomputed from Q, K
//
// With Phi stored, the sweep that runs every cycle is a bounded one: it reads
// the high 16-bit plane of the stored float32 Phi (Phi truncated to bfloat16,
// half the bytes) and gives every key an interval that holds its score, the
// band merge keeps the keys whose interval reaches the (K+1)-th best lower
// bound, the rescoring computes their float64 columns and exact scores from
// Q and K, and the choice takes the top K+1 of those (the same keys the full
// scores would give) and moves the picks' columns into the panel.  A head
// whose band holds more than kBandCap keys takes the float32 sweep over both
// planes, the merge and the panel in the same cycle.
//   gram   : new columns of G = Phi_S^T Phi_S and of b = Phi_S^T m
//   resid  : mhat = Phi_S w and r = m - mhat
//
// A "cycle" is the R iterations between two refits.  Within a cycle the
// residual does not change, so the R top-k picks of the cycle are the top
// k*R keys of a single sweep; the sweep runs once per cycle.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <climits>
#include <cmath>
#include <type_traits>

#include "amc_internal.h"

namespace amc {
namespace {

constexpr int KP_STRIDE = kMaxCycle + 1;  // candidate slots per sweep block
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bool better(double va, int ia, double vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// Sorts 256 (value, index) pairs in LDS, best first (value descending, index
// ascending).  Threads at or above 256 only take part in the barriers.
__device__ void block_sort256(double *v, int *ix) {
  const int tid = threadIdx.x;
  for (int k = 2; k <= 256; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      const int p = tid ^ j;
      if (tid < 256 && p > tid) {
        const double va = v[tid], vb = v[p];
        const int ia = ix[tid], ib = ix[p];
        const bool first_better = better(va, ia, vb, ib);
        const bool want_first_better = (tid & k) == 0;
        if (first_better != want_first_better) {
          v[tid] = vb;
          v[p] = va;
          ix[tid] = ib;
          ix[p] = ia;
        }
      }
      __syncthreads();
    }
  }
}

// Stored Phi planes keep each 64-key tile in the order the mass-feature
// kernel writes it: position 32 (kb / 2) + 8 g + 4 (kb % 2) + e holds key
// 16 kb + g + 4 e.
__device__ __forceinline__ int64_t key_at(int64_t pos) {
  const int p = int(pos & 63);
  const int kb = 2 * (p >> 5) + ((p >> 2) & 1), g = (p >> 3) & 3, e = p & 3;
  return (pos & ~int64_t(63)) + 16 * kb + g + 4 * e;
}

__device__ __forceinline__ int cycle_keys(const HeadDesc &D, int cycle, int kR, int64_t *S0) {
  const int64_t s0 = int64_t(cycle) * kR;
  *S0 = s0;
  if (s0 >= D.t) return 0;
  const int64_t left = D.t - s0;
  return int(left < kR ? left : kR);
}

// ---------------------------------------------------------------------------
// sweep over the float32 Phi, rebuilt exactly from its two 16-bit planes: one
// block = 256 columns of one head, 4 waves split the rows.  gate: only the
// heads with gate[h] != 0.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 join_planes(u32x2 hv, u32x2 lv) {
  f32x4 x;
  x.x = __uint_as_float((hv.x << 16) | (lv.x & 0xffffu));
  x.y = __uint_as_float((hv.x & 0xffff0000u) | (lv.x >> 16));
  x.z = __uint_as_float((hv.y << 16) | (lv.y & 0xffffu));
  x.w = __uint_as_float((hv.y & 0xffff0000u) | (lv.y >> 16));
  return x;
}

__global__ __launch_bounds__(256) void k_sweep(const HeadDesc *__restrict__ desc, const uint16_t *__restrict__ phi16,
                                               const double *__restrict__ r, const int32_t *__restrict__ sel_slot,
                                               int cycle, int kR, const int32_t *__restrict__ gate,
                                               double *__restrict__ cand_val,
                                               int32_t *__restrict__ cand_idx, int32_t *__restrict__ head_status) {
  __shared__ double red[4][256];
  __shared__ double sv[256];
  __shared__ int si[256];
  const int h = blockIdx.y;
  const HeadDesc D = desc[h];
  const int blk = blockIdx.x;
  if (blk >= D.n_cblk) return;
  int64_t S0;
  const int Kc = cycle_keys(D, cycle, kR, &S0);
  if (Kc == 0) return;
  if (gate && gate[h] == 0) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t j0 = int64_t(blk) * kSweepCols + 4 * lane;  // stored position
  double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
  if (j0 < D.ldT) {  // ldT is a multiple of 64: the 8-byte segments lie within the row
    const uint16_t *ph = phi16 + 2 * D.phi_off + j0;
    const uint16_t *pl = ph + D.n * D.ldT;
    const double *rr = r + D.n_off;
    const int64_t ld = D.ldT;
    int64_t i = wave;
    for (; i + 28 < D.n; i += 32) {
      f32x4 x[8];
      double rv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t at = (i + 4 * u) * ld;
        x[u] = join_planes(__builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(ph + at)),
                           __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(pl + at)));
        rv[u] = rr[i + 4 * u];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        a0 = fma(rv[u], double(x[u].x), a0);
        a1 = fma(rv[u], double(x[u].y), a1);
        a2 = fma(rv[u], double(x[u].z), a2);
        a3 = fma(rv[u], double(x[u].w), a3);
      }
    }
    for (; i < D.n; i += 4) {
      const f32x4 x = join_planes(*reinterpret_cast<const u32x2 *>(ph + i * ld),
                                  *reinterpret_cast<const u32x2 *>(pl + i * ld));
      const double rv = rr[i];
      a0 = fma(rv, double(x.x), a0);
      a1 = fma(rv, double(x.y), a1);
      a2 = fma(rv, double(x.z), a2);
      a3 = fma(rv, double(x.w), a3);
    }
  }
  red[wave][4 * lane + 0] = a0;
  red[wave][4 * lane + 1] = a1;
  red[wave][4 * lane + 2] = a2;
  red[wave][4 * lane + 3] = a3;
  __syncthreads();
  const int64_t pos = int64_t(blk) * kSweepCols + tid;
  const int64_t col = key_at(pos);
  double c = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
  int idx = int(col);
  if (pos >= D.ldT || col >= D.T || sel_slot[D.k_off + col] != 0) {
    c = -INFINITY;
    idx = INT_MAX;
  } else if (!isfinite(c)) {
    if (head_status) atomicOr(head_status + h, int32_t(AMC_HS_NONFINITE));
    c = -DBL_MAX;  // still a valid, selectable key
  }
  sv[tid] = c;
  si[tid] = idx;
  __syncthreads();
  block_sort256(sv, si);
  if (tid <= Kc) {
    const int64_t o = (D.cblk_off + blk) * KP_STRIDE + tid;
    cand_val[o] = sv[tid];
    cand_idx[o] = si[tid];
  }
}

// ---------------------------------------------------------------------------
// recompute sweep (Phi not stored): the same scores c_j = r^T Phi[:, j], with
// each Phi tile rebuilt from Q and K as the mass-feature stage builds it:
// float64 MFMA logits S^T = K Q^T from the exact inputs and a float64 exp
// (the scores are summed from the float64 Phi, before any float32 rounding).
// One block = 256 keys of one head in 8 waves of 32 keys; each wave keeps its
// keys' MFMA operands in registers and the queries stream through LDS 64 at
// a time.
// ---------------------------------------------------------------------------
typedef double f64x4 __attribute__((ext_vector_type(4)));
constexpr int RC_THREADS = 512;

template <typename T>
struct InRc;
template <>
struct InRc<uint16_t> {
  __device__ static float f(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }
};
template <>
struct InRc<float> {
  __device__ static float f(float v) { return v; }
};

// Elements 16 u + 4 g + v (u < D / 16, v < 4) of the row at element offset
// `off`, as float64, at k-step 4 u + v: 8-byte loads of 4 bf16 (16 bytes of
// float32), issued unconditionally (the caller passes a valid row), zeroed
// when !keep.
template <int D, typename E>
__device__ __forceinline__ void load_row4(const E *__restrict__ base, int64_t off, int g, bool keep, double *out) {
#pragma unroll
  for (int u = 0; u < D / 16; ++u) {
    const int64_t at = off + 16 * u + 4 * g;
    float x[4];
    if constexpr (std::is_same<E, uint16_t>::value) {
      const u32x2 w = *reinterpret_cast<const u32x2 *>(base + at);
      x[0] = __uint_as_float(w.x << 16);
      x[1] = __uint_as_float(w.x & 0xffff0000u);
      x[2] = __uint_as_float(w.y << 16);
      x[3] = __uint_as_float(w.y & 0xffff0000u);
    } else {
      const f32x4 w = *reinterpret_cast<const f32x4 *>(base + at);
      x[0] = w.x;
      x[1] = w.y;
      x[2] = w.z;
      x[3] = w.w;
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) out[4 * u + v] = keep ? double(x[v]) : 0.0;
  }
}

template <int D, bool BF16>
__global__ __launch_bounds__(RC_THREADS) void k_sweep_rc(
    const HeadDesc *__restrict__ desc, const void *__restrict__ Qv, const void *__restrict__ Kv,
    const float *__restrict__ beta_in, double scale, const double *__restrict__ shift, const double *__restrict__ r,
    const int32_t *__restrict__ sel_slot, int cycle, int kR, double *__restrict__ cand_val,
    int32_t *__restrict__ cand_idx, int32_t *__restrict__ head_status) {
  using E = typename std::conditional<BF16, uint16_t, float>::type;
  constexpr int NS = D / 4;    // MFMA k-steps over the head dimension
  constexpr int QT = 64;       // queries per LDS stage
  constexpr int QSTR = D + 4;  // elements per staged query row
  constexpr int KB = 2;        // 16-key tiles per wave
  static_assert(RC_THREADS / 64 * KB * 16 == kSweepCols, "one block covers one sweep column block");
  __shared__ __attribute__((aligned(16))) E qs[QT * QSTR];
  __shared__ double rs[QT];
  __shared__ double sv[256];
  __shared__ int si[256];
  const E *Q = static_cast<const E *>(Qv);
  const E *K = static_cast<const E *>(Kv);
  const int h = blockIdx.y;
  const HeadDesc Dh = desc[h];
  const int blk = blockIdx.x;
  if (blk >= Dh.n_cblk) return;
  int64_t S0;
  const int Kc = cycle_keys(Dh, cycle, kR, &S0);
  if (Kc == 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  const double s = shift[h];
  const int64_t kbase = int64_t(blk) * kSweepCols + wave * (KB * 16);
  // A operands: key kbase + 16 kb + c16, head dims 16 u + 4 g + v at k-step 4 u + v
  double kf[KB][NS];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int64_t key = kbase + kb * 16 + c16;
    load_row4<D>(K, (Dh.k_off + (key < Dh.T ? key : Dh.T - 1)) * D, g, key < Dh.T, kf[kb]);
  }
  // output rows of tile kb: key kbase + 16 kb + g + 4 e (keys past T contribute exp(-inf) = 0)
  double bb[KB][4], sc[KB][4];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t key = kbase + kb * 16 + g + 4 * e;
      bb[kb][e] = key < Dh.T ? (beta_in ? double(beta_in[Dh.k_off + key]) : 0.0) : -INFINITY;
      sc[kb][e] = 0.0;
    }

  for (int64_t i0 = 0; i0 < Dh.n; i0 += QT) {
    __syncthreads();
    for (int gi = tid; gi < QT * D / 4; gi += RC_THREADS) {
      // 4 elements per access, from a real row (rows past n are zeroed)
      const int qq = gi / (D / 4), c4 = gi % (D / 4);
      const bool ok = i0 + qq < Dh.n;
      const int64_t src = (Dh.q_off + (ok ? i0 + qq : Dh.n - 1)) * D + 4 * c4;
      if constexpr (BF16) {
        u32x2 w = *reinterpret_cast<const u32x2 *>(Q + src);
        if (!ok) w = u32x2{0u, 0u};
        *reinterpret_cast<u32x2 *>(&qs[qq * QSTR + 4 * c4]) = w;
      } else {
        f32x4 w = *reinterpret_cast<const f32x4 *>(Q + src);
        if (!ok) w = f32x4{0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<f32x4 *>(&qs[qq * QSTR + 4 * c4]) = w;
      }
    }
    if (tid < QT) rs[tid] = i0 + tid < Dh.n ? r[Dh.n_off + i0 + tid] : 0.0;
    __syncthreads();
#pragma unroll 1
    for (int qt = 0; qt < QT / 16; ++qt) {
      f64x4 acc[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) acc[kb] = f64x4{0.0, 0.0, 0.0, 0.0};
      const E *qp = &qs[(qt * 16 + c16) * QSTR + 4 * g];
#pragma unroll
      for (int u = 0; u < NS / 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const double bq = double(InRc<E>::f(qp[16 * u + v]));
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
            acc[kb] = __builtin_amdgcn_mfma_f64_16x16x4f64(kf[kb][4 * u + v], bq, acc[kb], 0, 0, 0);
        }
      // output column c16 is query i0 + 16 qt + c16
      const double rq = rs[qt * 16 + c16];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[kb][e] = fma(rq, exp(scale * acc[kb][e] + bb[kb][e] - s), sc[kb][e]);
    }
  }
  // sum over the 16 query columns of each lane group, then one score per key
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      double v = sc[kb][e];
      v += __shfl_xor(v, 1);
      v += __shfl_xor(v, 2);
      v += __shfl_xor(v, 4);
      v += __shfl_xor(v, 8);
      if (c16 == 0) sv[wave * (KB * 16) + kb * 16 + g + 4 * e] = v;
    }
  __syncthreads();
  if (tid < 256) {
    const int64_t col = int64_t(blk) * kSweepCols + tid;
    double c = sv[tid];
    int idx = int(col);
    if (col >= Dh.T || sel_slot[Dh.k_off + col] != 0) {
      c = -INFINITY;
      idx = INT_MAX;
    } else if (!isfinite(c)) {
      if (head_status) atomicOr(head_status + h, int32_t(AMC_HS_NONFINITE));
      c = -DBL_MAX;  // still a valid, selectable key
    }
    sv[tid] = c;
    si[tid] = idx;
  }
  __syncthreads();
  block_sort256(sv, si);
  if (tid <= Kc) {
    const int64_t o = (Dh.cblk_off + blk) * KP_STRIDE + tid;
    cand_val[o] = sv[tid];
    cand_idx[o] = si[tid];
  }
}

// ---------------------------------------------------------------------------
// Tournament over the sorted candidate lists of one head (list l at
// (base + l) * KP_STRIDE, best first, read up to position last): on_rank(rank,
// value, index) runs on thread 0 for the ranks 0..last in order.  Every thread
// of the block must call it.
// ---------------------------------------------------------------------------
template <typename F>
__device__ void tournament(const double *__restrict__ val, const int32_t *__restrict__ idx, int64_t base, int nl,
                           int last, F on_rank) {
  __shared__ double wv[4];
  __shared__ int wi[4], wl[4];
  __shared__ int win_list;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // each thread owns lists tid, tid+256, tid+512, tid+768
  int pos[4] = {0, 0, 0, 0};
  for (int rank = 0; rank <= last; ++rank) {
    double bv = -INFINITY;
    int bi = INT_MAX, bl = -1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int l = tid + 256 * q;
      if (l < nl && pos[q] <= last) {
        const int64_t o = (base + l) * KP_STRIDE + pos[q];
        const double v = val[o];
        const int ix = idx[o];
        if (bl < 0 || better(v, ix, bv, bi)) {
          bv = v;
          bi = ix;
          bl = l;
        }
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const double ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      const int ol = __shfl_xor(bl, off);
      if (ol >= 0 && (bl < 0 || better(ov, oi, bv, bi))) {
        bv = ov;
        bi = oi;
        bl = ol;
      }
    }
    if (lane == 0) {
      wv[wave] = bv;
      wi[wave] = bi;
      wl[wave] = bl;
    }
    __syncthreads();
    if (tid == 0) {
      double v = wv[0];
      int ix = wi[0], l = wl[0];
      for (int w = 1; w < 4; ++w)
        if (wl[w] >= 0 && (l < 0 || better(wv[w], wi[w], v, ix))) {
          v = wv[w];
          ix = wi[w];
          l = wl[w];
        }
      win_list = l;
      on_rank(rank, v, ix);
    }
    __syncthreads();
    const int l = win_list;
    if (l >= 0 && (l & 255) == tid) pos[l >> 8]++;
  }
}

// ---------------------------------------------------------------------------
// merge: one block per head; the tournament's first Kc winners are the picks,
// the next one the runner-up.  gate: only the heads with gate[h] != 0.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_merge(const HeadDesc *__restrict__ desc, int cycle, int kR,
                                               const int32_t *__restrict__ gate,
                                               const double *__restrict__ cand_val,
                                               const int32_t *__restrict__ cand_idx, int32_t *__restrict__ sel_slot,
                                               int32_t *__restrict__ sel_list, int32_t *__restrict__ tr_pick,
                                               double *__restrict__ tr_pick_score, double *__restrict__ tr_runner) {
  const int h = blockIdx.x;
  const HeadDesc D = desc[h];
  int64_t S0;
  const int Kc = cycle_keys(D, cycle, kR, &S0);
  if (Kc == 0) return;
  if (gate && gate[h] == 0) return;
  tournament(cand_val, cand_idx, D.cblk_off, int(D.n_cblk), Kc, [&](int rank, double v, int ix) {
    if (rank < Kc) {
      const int64_t slot = S0 + rank;
      if (ix >= 0 && ix < D.T) {
        sel_list[D.t_off + slot] = ix;
        sel_slot[D.k_off + ix] = int32_t(slot + 1);
      }
      if (tr_pick) {
        tr_pick[D.t_off + slot] = ix;
        tr_pick_score[D.t_off + slot] = v;
      }
    } else if (tr_runner) {
      tr_runner[D.cyc_off + cycle] = (ix >= 0 && ix < D.T) ? v : -INFINITY;
    }
  });
}

// ---------------------------------------------------------------------------
// bounded sweep over the high plane (Phi truncated to bfloat16).  For a key j
// with stored float32 values x_ij, high halves h_ij and exact Phi_ij:
//   0 <= x_ij - h_ij < 2^-7 h_ij           (7 explicit significand bits kept)
//   |Phi_ij - x_ij| <= 2^-24 Phi_ij         (float32 rounding of float64 Phi)
// so with P_j = sum_{r_i > 0} r_i h_ij and N_j = sum_{r_i < 0} r_i h_ij,
//   P_j + N_j + 2^-7 N_j - e_j <= r^T Phi[:, j] <= P_j + N_j + 2^-7 P_j + e_j,
// where e_j covers the float32 accumulation of P and N (same-sign sums, so a
// relative error of (terms per lane + 2) 2^-24 each), the float32 rounding of
// Phi and of r, the float64 rescoring's own rounding, and an absolute term for
// values below float32's normal range.  One block = 256 keys: each lane takes
// 8 keys of every 8th row (16-byte loads), P and N accumulate in float32 per
// lane and in float64 across the 8 row streams; each column is a stored
// position, mapped to its key at the end.  Out: the block's top-(Kc+1)
// lower bounds, sorted (cand_lo / cand_lidx), and in key order every key whose
// upper bound reaches the (Kc+1)-th of them (cand_val = upper bound,
// cand_idx, cand_cnt = their number, -1 if a bound is not finite).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void band_accum(const u32x4 &x, double rv, float (&P)[8], float (&N)[8], double &ra) {
  const float rp = float(fmax(rv, 0.0)), rn = float(fmin(rv, 0.0));
  ra += fabs(rv);  // NaN in r reaches the bounds through this sum
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float v0 = __uint_as_float(w[c] << 16);
    const float v1 = __uint_as_float(w[c] & 0xffff0000u);
    P[2 * c] = fmaf(rp, v0, P[2 * c]);
    N[2 * c] = fmaf(rn, v0, N[2 * c]);
    P[2 * c + 1] = fmaf(rp, v1, P[2 * c + 1]);
    N[2 * c + 1] = fmaf(rn, v1, N[2 * c + 1]);
  }
}

__global__ __launch_bounds__(256) void k_sweep_band(const HeadDesc *__restrict__ desc,
                                                    const uint16_t *__restrict__ phi16, const double *__restrict__ r,
                                                    const int32_t *__restrict__ sel_slot, int cycle, int kR,
                                                    double *__restrict__ cand_val, int32_t *__restrict__ cand_idx,
                                                    int32_t *__restrict__ cand_cnt, double *__restrict__ cand_lo,
                                                    int32_t *__restrict__ cand_lidx) {
  __shared__ __attribute__((aligned(16))) float ps_p[8][256];
  __shared__ __attribute__((aligned(16))) float ps_n[8][256];
  __shared__ double ra_s[8];
  __shared__ double sv[256];
  __shared__ int si[256];
  __shared__ int wcnt[4];
  const int h = blockIdx.y;
  const HeadDesc D = desc[h];
  const int blk = blockIdx.x;
  if (blk >= D.n_cblk) return;
  int64_t S0;
  const int Kc = cycle_keys(D, cycle, kR, &S0);
  if (Kc == 0) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cg = lane & 31;
  const int stream = 2 * wave + (lane >> 5);  // rows stream, stream + 8, ...
  const int64_t j0 = int64_t(blk) * kSweepCols + 8 * cg;
  float P[8], N[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) P[k] = N[k] = 0.0f;
  double ra = 0.0;
  if (j0 < D.ldT) {  // ldT is a multiple of 64: the 16-byte segment lies within the row
    const uint16_t *p = phi16 + 2 * D.phi_off + j0;
    const double *rr = r + D.n_off;
    const int64_t ld = D.ldT;
    int64_t i = stream;
    for (; i + 56 < D.n; i += 64) {
      u32x4 x[8];
      double rv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        x[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p + (i + 8 * u) * ld));
        rv[u] = rr[i + 8 * u];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) band_accum(x[u], rv[u], P, N, ra);
    }
    for (; i < D.n; i += 8) band_accum(*reinterpret_cast<const u32x4 *>(p + i * ld), rr[i], P, N, ra);
  }
  *reinterpret_cast<float4 *>(&ps_p[stream][8 * cg]) = make_float4(P[0], P[1], P[2], P[3]);
  *reinterpret_cast<float4 *>(&ps_p[stream][8 * cg + 4]) = make_float4(P[4], P[5], P[6], P[7]);
  *reinterpret_cast<float4 *>(&ps_n[stream][8 * cg]) = make_float4(N[0], N[1], N[2], N[3]);
  *reinterpret_cast<float4 *>(&ps_n[stream][8 * cg + 4]) = make_float4(N[4], N[5], N[6], N[7]);
  if (cg == 0) ra_s[stream] = ra;  // lane cg = 0 always reads (block start < T <= ldT)
  __syncthreads();
  const int64_t pos = int64_t(blk) * kSweepCols + tid;  // stored position of this thread's key
  const int64_t col = key_at(pos);
  double Pd = 0.0, Nd = 0.0, rs = 0.0;
#pragma unroll
  for (int st = 0; st < 8; ++st) {
    Pd += double(ps_p[st][tid]);
    Nd += double(ps_n[st][tid]);
    rs += ra_s[st];
  }
  const bool valid = pos < D.ldT && col < D.T && sel_slot[D.k_off + col] == 0;
  const double crel = 2.0 * (double(D.n) * 0.125 + 16.0) * 0x1p-24 + 0x1p-22;
  const double slack = crel * (Pd - Nd) + (rs + double(D.n)) * 0x1p-120;
  const double c7 = 0x1.00001p-7;
  const double up = (Pd + Nd) + c7 * Pd + slack;
  const double lo = (Pd + Nd) + c7 * Nd - slack;
  const bool bad = valid && !(isfinite(up) && isfinite(lo));
  sv[tid] = valid ? lo : -INFINITY;
  si[tid] = valid ? int(col) : INT_MAX;
  const int any_bad = __syncthreads_or(int(bad));
  block_sort256(sv, si);
  const double Lb = sv[Kc];
  const int64_t o = (D.cblk_off + blk) * KP_STRIDE;
  if (tid <= Kc) {
    cand_lo[o + tid] = sv[tid];
    cand_lidx[o + tid] = si[tid];
  }
  const bool take = valid && up >= Lb;
  const uint64_t m = __ballot(take);
  if (lane == 0) wcnt[wave] = __popcll(m);
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wcnt[w];
  if (take) {
    const int at = base + __popcll(m & ((uint64_t(1) << lane) - 1));
    cand_val[o + at] = up;
    cand_idx[o + at] = int(col);
  }
  if (tid == 0) cand_cnt[D.cblk_off + blk] = any_bad ? -1 : wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
}

// ---------------------------------------------------------------------------
// band merge: one block per head.  L = the (Kc+1)-th best lower bound over
// all blocks (the tournament over the blocks' sorted lists); the band is every
// key whose upper bound reaches L, in block and key order.  It holds the true
// top Kc+1: each of those scores at least L, and its upper bound at least its
// score.  exact[h] = 1 when the band overflows kBandCap (or a bound was not
// finite): the head takes the float32 sweep this cycle.  band_cap <= kBandCap
// (lower only to exercise the exact path).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_band_merge(const HeadDesc *__restrict__ desc, int cycle, int kR,
                                                    const double *__restrict__ cand_val,
                                                    const int32_t *__restrict__ cand_idx,
                                                    const int32_t *__restrict__ cand_cnt,
                                                    const double *__restrict__ cand_lo,
                                                    const int32_t *__restrict__ cand_lidx,
                                                    int band_cap, int32_t *__restrict__ band_list,
                                                    int32_t *__restrict__ band_cnt, int32_t *__restrict__ exact) {
  __shared__ double s_L;
  __shared__ int wcnt[4];
  const int h = blockIdx.x;
  const HeadDesc D = desc[h];
  int64_t S0;
  const int Kc = cycle_keys(D, cycle, kR, &S0);
  if (Kc == 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nl = int(D.n_cblk);
  int bad = 0;
  for (int l = tid; l < nl; l += 256) bad |= cand_cnt[D.cblk_off + l] < 0;
  if (__syncthreads_or(bad)) {
    if (tid == 0) {
      band_cnt[h] = 0;
      exact[h] = 1;
    }
    return;
  }
  double *Lp = &s_L;
  tournament(cand_lo, cand_lidx, D.cblk_off, nl, Kc, [&](int rank, double v, int ix) {
    if (rank == Kc) *Lp = ix != INT_MAX ? v : -INFINITY;
  });
  const double L = s_L;
  int total = 0;
  int32_t *out = band_list + int64_t(h) * kBandCap;
  for (int l = 0; l < nl; ++l) {
    const int64_t o = (D.cblk_off + l) * KP_STRIDE;
    const int cnt = cand_cnt[D.cblk_off + l];
    for (int e0 = 0; e0 < cnt; e0 += 256) {
      const int e = e0 + tid;
      bool take = false;
      int ix = 0;
      if (e < cnt) {
        ix = cand_idx[o + e];
        take = ix != INT_MAX && cand_val[o + e] >= L;
      }
      const uint64_t m = __ballot(take);
      if (lane == 0) wcnt[wave] = __popcll(m);
      __syncthreads();
      int at = total;
      for (int w = 0; w < wave; ++w) at += wcnt[w];
      at += __popcll(m & ((uint64_t(1) << lane) - 1));
      if (take && at < kBandCap) out[at] = ix;
      total += wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
      __syncthreads();
    }
  }
  if (tid == 0) {
    band_cnt[h] = total;
    exact[h] = (total > band_cap || total < Kc) ? 1 : 0;
  }
}

// ---------------------------------------------------------------------------
// panel: float64 Phi columns of the new picks; one block = 64 queries
// ---------------------------------------------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(256) void k_panel(const HeadDesc *__restrict__ desc, const void *__restrict__ Qv,
                                               const void *__restrict__ Kv, const float *__restrict__ beta_in,
                                               double scale, const double *__restrict__ shift,
                                               const int32_t *__restrict__ sel_list, int cycle, int kR,
                                               const int32_t *__restrict__ gate, double *__restrict__ panel) {
  using E = typename std::conditional<BF16, uint16_t, float>::type;
  constexpr int VEC = 16 / int(sizeof(E));  // elements per 16-byte load
  __shared__ float qs[64][D + 1];
  __shared__ float kbuf[4][D];
  const E *Q = static_cast<const E *>(Qv);
  const E *K = static_cast<const E *>(Kv);
  const int h = blockIdx.y;
  const HeadDesc Dh = desc[h];
  int64_t S0;
  const int Kc = cycle_keys(Dh, cycle, kR, &S0);
  if (Kc == 0) return;
  if (gate && gate[h] == 0) return;
  const int64_t q0 = int64_t(blockIdx.x) * 64;
  if (q0 >= Dh.n) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  auto cvt = [](E v) -> float {
    if constexpr (BF16) return __uint_as_float(uint32_t(v) << 16);
    else return v;
  };
  for (int gi = tid; gi < 64 * D / VEC; gi += 256) {
    const int rr = gi / (D / VEC), cv = gi % (D / VEC);
    E x[VEC];
    if (q0 + rr < Dh.n) {
      *reinterpret_cast<uint4 *>(x) = *reinterpret_cast<const uint4 *>(Q + (Dh.q_off + q0 + rr) * D + VEC * cv);
    } else {
#pragma unroll
      for (int u = 0; u < VEC; ++u) x[u] = E(0);
    }
#pragma unroll
    for (int u = 0; u < VEC; ++u) qs[rr][VEC * cv + u] = cvt(x[u]);
  }
  __syncthreads();
  const double s = shift[h];
  const int64_t q = q0 + lane;
  for (int kk = wave; kk < Kc; kk += 4) {
    const int j = sel_list[Dh.t_off + S0 + kk];
    const bool jok = j >= 0 && j < Dh.T;
    for (int c = lane; c < D; c += 64) kbuf[wave][c] = jok ? cvt(K[(Dh.k_off + j) * D + c]) : 0.0f;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // products of the float32 inputs are exact in float64; four partial sums
    double d0 = 0.0, d1 = 0.0, d2 = 0.0, d3 = 0.0;
#pragma unroll 8
    for (int c = 0; c < D; c += 4) {
      d0 = fma(double(qs[lane][c]), double(kbuf[wave][c]), d0);
      d1 = fma(double(qs[lane][c + 1]), double(kbuf[wave][c + 1]), d1);
      d2 = fma(double(qs[lane][c + 2]), double(kbuf[wave][c + 2]), d2);
      d3 = fma(double(qs[lane][c + 3]), double(kbuf[wave][c + 3]), d3);
    }
    const double dot = (d0 + d1) + (d2 + d3);
    const double bias = (beta_in && jok) ? double(beta_in[Dh.k_off + j]) : 0.0;
    if (q < Dh.n) panel[Dh.panel_off + (S0 + kk) * Dh.n + q] = jok ? exp(scale * dot + bias - s) : 0.0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// ---------------------------------------------------------------------------
// rescoring: float64 Phi columns of the head's band keys, as the panel
// computes them (float64 MFMA logits from the exact inputs, float64 exp),
// written to the stage, and their partial scores r^T Phi[:, j] over the
// block's queries.  One block = kRescoreRows = 256 queries, 4 waves of 64;
// each 16-key group of the band keeps its keys' MFMA operands in registers
// (keys as rows of v_mfma_f64_16x16x4f64) while a wave walks its four
// 16-query tiles (each over two accumulation chains, even and odd k-steps).
// ---------------------------------------------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(256) void k_rescore(const HeadDesc *__restrict__ desc, const void *__restrict__ Qv,
                                                 const void *__restrict__ Kv, const float *__restrict__ beta_in,
                                                 double scale, const double *__restrict__ shift,
                                                 const double *__restrict__ r, int cycle, int kR,
                                                 const int32_t *__restrict__ band_list,
                                                 const int32_t *__restrict__ band_cnt,
                                                 const int32_t *__restrict__ exact, int64_t max_qblk,
                                                 double *__restrict__ stage, double *__restrict__ part) {
  using E = typename std::conditional<BF16, uint16_t, float>::type;
  constexpr int NS = D / 4;  // MFMA k-steps over the head dimension
  static_assert(kRescoreRows == 256, "4 waves x 4 tiles of 16 queries");
  __shared__ double red[4][16];
  const E *Q = static_cast<const E *>(Qv);
  const E *K = static_cast<const E *>(Kv);
  const int h = blockIdx.y;
  const HeadDesc Dh = desc[h];
  int64_t S0;
  const int Kc = cycle_keys(Dh, cycle, kR, &S0);
  if (Kc == 0) return;
  if (exact[h] != 0) return;
  const int qb = blockIdx.x;
  const int64_t q0 = int64_t(qb) * kRescoreRows;
  if (q0 >= Dh.n) return;
  const int U = band_cnt[h];  // <= kBandCap when exact[h] == 0
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  const double s = shift[h];
  const int64_t qw = q0 + 64 * wave + c16;  // this lane's query in tile qt: qw + 16 qt
  double *stg = stage + Dh.n_off * kBandCap;
  for (int g0 = 0; g0 < U; g0 += 16) {
    const int ui = g0 + c16;
    const bool uok = ui < U;
    const int j = uok ? band_list[int64_t(h) * kBandCap + ui] : 0;
    const double bj = (uok && beta_in) ? double(beta_in[Dh.k_off + j]) : 0.0;
    // A operand: head dims 16 u + 4 g + v of key j at k-step 4 u + v (every
    // lane loads a real row, 4 elements at a time; lanes past the band zero it)
    double kd[NS];
    load_row4<D>(K, (Dh.k_off + j) * D, g, uok, kd);
    double be[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) be[e] = __shfl(bj, g + 4 * e);  // bias of band key g0 + g + 4 e
    double vs[4] = {0.0, 0.0, 0.0, 0.0};  // r_q Phi_qj summed over this lane's queries
#pragma unroll 1
    for (int qt = 0; qt < 4; ++qt) {
      const int64_t qa = qw + 16 * qt;
      const bool va = qa < Dh.n;
      double xa[NS];
      load_row4<D>(Q, (Dh.q_off + (va ? qa : Dh.n - 1)) * D, g, va, xa);
      const double ra = va ? r[Dh.n_off + qa] : 0.0;
      // two accumulation chains over the even and odd k-steps
      f64x4 a0 = {0.0, 0.0, 0.0, 0.0}, a1 = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int k = 0; k < NS; k += 2) {
        a0 = __builtin_amdgcn_mfma_f64_16x16x4f64(kd[k], xa[k], a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f64_16x16x4f64(kd[k + 1], xa[k + 1], a1, 0, 0, 0);
      }
      // element e: band key g0 + g + 4 e, query qa
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ue = g0 + g + 4 * e;
        if (ue < U && va) {
          const double p = exp(scale * (a0[e] + a1[e]) + be[e] - s);
          stg[int64_t(ue) * Dh.n + qa] = p;
          vs[e] = fma(ra, p, vs[e]);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      double v = vs[e];
      v += __shfl_xor(v, 1);
      v += __shfl_xor(v, 2);
      v += __shfl_xor(v, 4);
      v += __shfl_xor(v, 8);
      if (c16 == 0) red[wave][g + 4 * e] = v;
    }
    __syncthreads();
    if (tid < 16 && g0 + tid < U)
      part[(int64_t(h) * kBandCap + g0 + tid) * max_qblk + qb] = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// choice: the band's exact scores (partials summed in query-block order), the
// top Kc picks and the runner-up (score descending, key index ascending), the
// selection update (block 0), and the picks' staged columns copied into their
// panel rows (all blocks of the head, a share each).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_choose(const HeadDesc *__restrict__ desc, int cycle, int kR,
                                                const int32_t *__restrict__ band_list,
                                                const int32_t *__restrict__ band_cnt,
                                                const int32_t *__restrict__ exact, int64_t max_qblk,
                                                const double *__restrict__ part, const double *__restrict__ stage,
                                                int32_t *__restrict__ sel_slot, int32_t *__restrict__ sel_list,
                                                double *__restrict__ panel, int32_t *__restrict__ tr_pick,
                                                double *__restrict__ tr_pick_score, double *__restrict__ tr_runner,
                                                int32_t *__restrict__ head_status) {
  __shared__ double sc[kBandCap];
  __shared__ int ix[kBandCap];
  __shared__ int pick_u[kMaxCycle + 1];
  const int h = blockIdx.y;
  const HeadDesc D = desc[h];
  int64_t S0;
  const int Kc = cycle_keys(D, cycle, kR, &S0);
  if (Kc == 0) return;
  if (exact[h] != 0) return;
  const int U = band_cnt[h];  // Kc <= U <= kBandCap when exact[h] == 0
  const int tid = threadIdx.x;
  const int64_t nqb = (D.n + kRescoreRows - 1) / kRescoreRows;
  if (tid < U) {
    const double *pp = part + (int64_t(h) * kBandCap + tid) * max_qblk;
    double sum = 0.0;
    for (int64_t b = 0; b < nqb; ++b) sum += pp[b];
    if (!isfinite(sum)) {
      if (head_status && blockIdx.x == 0) atomicOr(head_status + h, int32_t(AMC_HS_NONFINITE));
      sum = -DBL_MAX;  // still a valid, selectable key
    }
    sc[tid] = sum;
    ix[tid] = band_list[int64_t(h) * kBandCap + tid];
  }
  __syncthreads();
  if (tid < U) {
    int rank = 0;
    for (int v = 0; v < U; ++v) rank += better(sc[v], ix[v], sc[tid], ix[tid]) ? 1 : 0;
    if (rank <= Kc) pick_u[rank] = tid;
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    if (tid < Kc) {
      const int u = pick_u[tid];
      const int j = ix[u];
      const int64_t slot = S0 + tid;
      sel_list[D.t_off + slot] = j;
      sel_slot[D.k_off + j] = int32_t(slot + 1);
      if (tr_pick) {
        tr_pick[D.t_off + slot] = j;
        tr_pick_score[D.t_off + slot] = sc[u];
      }
    }
    if (tid == 0 && tr_runner) tr_runner[D.cyc_off + cycle] = U > Kc ? sc[pick_u[Kc]] : -INFINITY;
  }
  const int64_t n = D.n;
  const double *stg = stage + D.n_off * kBandCap;
  double *pan = panel + D.panel_off + S0 * n;
  const int64_t total = int64_t(Kc) * n;
  for (int64_t e = int64_t(blockIdx.x) * 256 + tid; e < total; e += int64_t(gridDim.x) * 256) {
    const int rk = int(e / n);
    const int64_t qq = e - int64_t(rk) * n;
    pan[e] = stg[int64_t(pick_u[rk]) * n + qq];
  }
}

// ---------------------------------------------------------------------------
// gram: dot products over the n queries of the rows [panel rows 0..Snew-1, m]
// with the columns [new keys S0..Snew-1, r], on float64 MFMA
// (v_mfma_f64_16x16x4f64).  They give the new columns of G = Phi_S^T Phi_S
// (written to both halves), b = Phi_S^T m for the new keys (the m row), and
// gA = Phi_S^T r (the r column).  polish: no new key, only the r column.
// One block = 64 rows x 16 columns, the queries staged through LDS 64 at a
// time; each wave takes 16 rows.
// ---------------------------------------------------------------------------
typedef double f64x4g __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_gram(const HeadDesc *__restrict__ desc, const double *__restrict__ panel,
                                              const double *__restrict__ m, const double *__restrict__ r, int cycle,
                                              int kR, int polish, double *__restrict__ G, double *__restrict__ bvec,
                                              double *__restrict__ gA) {
  constexpr int CH = 64;       // queries per LDS stage
  constexpr int STR = CH + 1;  // padded row, in doubles
  __shared__ double xs[64 * STR];
  __shared__ double zs[16 * STR];
  const int h = blockIdx.z;
  const HeadDesc D = desc[h];
  int64_t S0;
  int Kc;
  if (polish) {
    S0 = D.t;
    Kc = 0;
  } else {
    Kc = cycle_keys(D, cycle, kR, &S0);
    if (Kc == 0) return;
  }
  const int64_t Snew = S0 + Kc;
  const int64_t nrows = Kc > 0 ? Snew + 1 : Snew;  // row Snew is m
  const int ncols = Kc + 1;                         // column Kc is r
  const int64_t a0 = int64_t(blockIdx.x) * 64;
  const int c0 = blockIdx.y * 16;
  if (a0 >= nrows || c0 >= ncols) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  const double *P = panel + D.panel_off;
  const int64_t n = D.n;
  // each thread stages 16 row values and 4 column values per LDS stage; the
  // next stage's loads are issued before the current stage's MFMAs
  double xr[16], zr[4];
  auto fetch = [&](int64_t i0) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = tid + 256 * u;
      const int rr = e / CH, c = e % CH;
      const int64_t a = a0 + rr, i = i0 + c;
      double v = 0.0;
      if (i < n) {
        if (a < Snew) v = P[a * n + i];
        else if (a == Snew && Kc > 0) v = m[D.n_off + i];
      }
      xr[u] = v;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + 256 * u;
      const int cc = e / CH, c = e % CH;
      const int col = c0 + cc;
      const int64_t i = i0 + c;
      double v = 0.0;
      if (i < n) {
        if (col < Kc) v = P[(S0 + col) * n + i];
        else if (col == Kc) v = r[D.n_off + i];
      }
      zr[u] = v;
    }
  };
  static_assert(64 * CH == 16 * 256 && 16 * CH == 4 * 256, "stage sizes");
  f64x4g acc = {0.0, 0.0, 0.0, 0.0};
  fetch(0);
  for (int64_t i0 = 0; i0 < n; i0 += CH) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = tid + 256 * u;
      xs[(e / CH) * STR + e % CH] = xr[u];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + 256 * u;
      zs[(e / CH) * STR + e % CH] = zr[u];
    }
    __syncthreads();
    if (i0 + CH < n) fetch(i0 + CH);
    const double *xa = &xs[(wave * 16 + c16) * STR + g];
    const double *zb = &zs[c16 * STR + g];
#pragma unroll
    for (int k = 0; k < CH / 4; ++k) acc = __builtin_amdgcn_mfma_f64_16x16x4f64(xa[4 * k], zb[4 * k], acc, 0, 0, 0);
  }
  // element e of lane group g holds row wave*16 + g + 4e, column c16
  const int64_t ld = D.t;
  const int col = c0 + c16;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t a = a0 + wave * 16 + g + 4 * e;
    if (col < Kc) {
      const int64_t b = S0 + col;
      if (a < Snew) {
        G[D.tt_off + a * ld + b] = acc[e];
        G[D.tt_off + b * ld + a] = acc[e];
      } else if (a == Snew) {
        bvec[D.t_off + b] = acc[e];
      }
    } else if (col == Kc && a < Snew) {
      gA[D.t_off + a] = acc[e];
    }
  }
}

// ---------------------------------------------------------------------------
// residual: mhat = Phi_S w, r = m - mhat (float64)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_resid(const HeadDesc *__restrict__ desc, const double *__restrict__ panel,
                                               const double *__restrict__ w, const double *__restrict__ m, int cycle,
                                               int kR, int polish, double *__restrict__ r, double *__restrict__ mhat) {
  __shared__ double ws[256];
  const int h = blockIdx.y;
  const HeadDesc D = desc[h];
  int64_t p;
  if (polish) {
    p = D.t;
  } else {
    int64_t S0;
    const int Kc = cycle_keys(D, cycle, kR, &S0);
    if (Kc == 0) return;
    p = S0 + Kc;
  }
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const bool valid = i < D.n;
  const double *P = panel + D.panel_off;
  double acc = 0.0;
  // the weights pass through LDS 256 at a time
  for (int64_t a0 = 0; a0 < p; a0 += 256) {
    __syncthreads();
    if (a0 + threadIdx.x < p) ws[threadIdx.x] = w[D.t_off + a0 + threadIdx.x];
    __syncthreads();
    const int64_t cnt = p - a0 < 256 ? p - a0 : 256;
    if (valid)
      for (int64_t a = 0; a < cnt; ++a) acc = fma(P[(a0 + a) * D.n + i], ws[a], acc);
  }
  if (!valid) return;
  mhat[D.n_off + i] = acc;
  r[D.n_off + i] = m[D.n_off + i] - acc;
}

}  // namespace

hipError_t launch_sweep(const Dims &dm, const Buffers &b, int cycle, int kR, int gated, hipStream_t s) {
  hipLaunchKernelGGL(k_sweep, dim3(unsigned(dm.max_cblk), unsigned(dm.H)), dim3(256), 0, s, b.desc, b.phi16, b.r,
                     b.sel_slot, cycle, kR, gated ? b.exact : nullptr, b.cand_val, b.cand_idx, b.head_status);
  return hipGetLastError();
}

hipError_t launch_sweep_rc(const Dims &dm, const Buffers &b, int cycle, int kR, hipStream_t s) {
  dim3 grid(unsigned(dm.max_cblk), unsigned(dm.H));
#define AMC_RC_ARGS b.desc, b.Q, b.K, b.beta_in, dm.scale, b.shift, b.r, b.sel_slot, cycle, kR, b.cand_val, b.cand_idx, \
    b.head_status
  if (dm.d == 128) {
    if (dm.in_bf16) hipLaunchKernelGGL((k_sweep_rc<128, true>), grid, dim3(RC_THREADS), 0, s, AMC_RC_ARGS);
    else hipLaunchKernelGGL((k_sweep_rc<128, false>), grid, dim3(RC_THREADS), 0, s, AMC_RC_ARGS);
  } else {
    if (dm.in_bf16) hipLaunchKernelGGL((k_sweep_rc<64, true>), grid, dim3(RC_THREADS), 0, s, AMC_RC_ARGS);
    else hipLaunchKernelGGL((k_sweep_rc<64, false>), grid, dim3(RC_THREADS), 0, s, AMC_RC_ARGS);
  }
#undef AMC_RC_ARGS
  return hipGetLastError();
}

hipError_t launch_sweep_band(const Dims &dm, const Buffers &b, int cycle, int kR, hipStream_t s) {
  hipLaunchKernelGGL(k_sweep_band, dim3(unsigned(dm.max_cblk), unsigned(dm.H)), dim3(256), 0, s, b.desc, b.phi16,
                     b.r, b.sel_slot, cycle, kR, b.cand_val, b.cand_idx, b.cand_cnt, b.cand_lo, b.cand_lidx);
  return hipGetLastError();
}

hipError_t launch_band_merge(const Dims &dm, const Buffers &b, int cycle, int kR, hipStream_t s) {
  hipLaunchKernelGGL(k_band_merge, dim3(unsigned(dm.H)), dim3(256), 0, s, b.desc, cycle, kR, b.cand_val, b.cand_idx,
                     b.cand_cnt, b.cand_lo, b.cand_lidx, dm.band_cap, b.band_list, b.band_cnt, b.exact);
  return hipGetLastError();
}

hipError_t launch_rescore(const Dims &dm, const Buffers &b, int cycle, int kR, hipStream_t s) {
  dim3 grid(unsigned(dm.max_qblk), unsigned(dm.H));
#define AMC_RS_ARGS b.desc, b.Q, b.K, b.beta_in, dm.scale, b.shift, b.r, cycle, kR, b.band_list, b.band_cnt, b.exact, \
    dm.max_qblk, b.stage, b.part
  if (dm.d == 128) {
    if (dm.in_bf16) hipLaunchKernelGGL((k_rescore<128, true>), grid, dim3(256), 0, s, AMC_RS_ARGS);
    else hipLaunchKernelGGL((k_rescore<128, false>), grid, dim3(256), 0, s, AMC_RS_ARGS);
  } else {
    if (dm.in_bf16) hipLaunchKernelGGL((k_rescore<64, true>), grid, dim3(256), 0, s, AMC_RS_ARGS);
    else hipLaunchKernelGGL((k_rescore<64, false>), grid, dim3(256), 0, s, AMC_RS_ARGS);
  }
#undef AMC_RS_ARGS
  return hipGetLastError();
}

hipError_t launch_choose(const Dims &dm, const Buffers &b, int cycle, int kR, hipStream_t s) {
  // a few blocks per head share the copy of the picks' columns
  hipLaunchKernelGGL(k_choose, dim3(8, unsigned(dm.H)), dim3(256), 0, s, b.desc, cycle, kR, b.band_list, b.band_cnt,
                     b.exact, dm.max_qblk, b.part, b.stage, b.sel_slot, b.sel_list, b.panel, b.tr_pick,
                     b.tr_pick_score, b.tr_runner, b.head_status);
  return hipGetLastError();
}

hipError_t launch_merge(const Dims &dm, const Buffers &b, int cycle, int kR, int gated, hipStream_t s) {
  hipLaunchKernelGGL(k_merge, dim3(unsigned(dm.H)), dim3(256), 0, s, b.desc, cycle, kR, gated ? b.exact : nullptr,
                     b.cand_val, b.cand_idx, b.sel_slot, b.sel_list, b.tr_pick, b.tr_pick_score, b.tr_runner);
  return hipGetLastError();
}

hipError_t launch_panel(const Dims &dm, const Buffers &b, int cycle, int kR, int gated, hipStream_t s) {
  dim3 grid(unsigned((dm.max_n + 63) / 64), unsigned(dm.H));
#define AMC_PANEL_ARGS b.desc, b.Q, b.K, b.beta_in, dm.scale, b.shift, b.sel_list, cycle, kR, gated ? b.exact : nullptr, \
    b.panel
  if (dm.d == 128) {
    if (dm.in_bf16) hipLaunchKernelGGL((k_panel<128, true>), grid, dim3(256), 0, s, AMC_PANEL_ARGS);
    else hipLaunchKernelGGL((k_panel<128, false>), grid, dim3(256), 0, s, AMC_PANEL_ARGS);
  } else {
    if (dm.in_bf16) hipLaunchKernelGGL((k_panel<64, true>), grid, dim3(256), 0, s, AMC_PANEL_ARGS);
    else hipLaunchKernelGGL((k_panel<64, false>), grid, dim3(256), 0, s, AMC_PANEL_ARGS);
  }
#undef AMC_PANEL_ARGS
  return hipGetLastError();
}

hipError_t launch_gram(const Dims &dm, const Buffers &b, int cycle, int kR, int polish, hipStream_t s) {
  // rows [0, S0 + Kc] (the last is m), so up to max_t + 1; columns: up to kR new keys and r
  const int64_t rows = dm.max_t + 1;
  dim3 grid(unsigned((rows + 63) / 64), unsigned(polish ? 1 : (kR + 1 + 15) / 16), unsigned(dm.H));
  hipLaunchKernelGGL(k_gram, grid, dim3(256), 0, s, b.desc, b.panel, b.m, b.r, cycle, kR, polish, b.G, b.bvec, b.gA);
  return hipGetLastError();
}

hipError_t launch_resid(const Dims &dm, const Buffers &b, int cycle, int kR, int polish, hipStream_t s) {
  dim3 grid(unsigned((dm.max_n + 255) / 256), unsigned(dm.H));
  hipLaunchKernelGGL(k_resid, grid, dim3(256), 0, s, b.desc, b.panel, b.w, b.m, cycle, kR, polish, b.r, b.mhat);
  return hipGetLastError();
}

}  // namespace amc
