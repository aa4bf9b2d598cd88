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

#include <algorithm>

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

__device__ __forceinline__ int cycle_keys(const HeadDesc &D, int cycle, int kR, int64_t *S0) {
  const int64_t s0 = int64_t(cycle) * kR;
  *S0 = s0;
  if (s0 >= D.t) return 0;
  const int64_t left = D.t - s0;
  return int(left < kR ? left : kR);
}

// ---------------------------------------------------------------------------
// Stored Phi is two 16-bit planes of key columns (high and low halves of the
// float32 values, key k at k * ldN; queries from n to ldN are zero).  The
// sweeps read whole columns: a wave takes 8 keys at a time, 8 lanes per key,
// lane `sub` of a key reading queries 64 i + 8 sub .. 64 i + 8 sub + 7 (one
// 16-byte load per plane) for i = 0 .. ldN / 64 - 1, so each load
// instruction moves 8 full 128-byte lines.  r (or its float32 parts) is staged
// in LDS per block; the partial sums of a key meet across its 8 lanes.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 join_planes(u32x2 hv, u32x2 lv) {
  f32x4 x;
  x.x = __uint_as_float((hv.x << 16) | (lv.x & 0xffffu));
  x.y = __uint_as_float((hv.x & 0xffff0000u) | (lv.x >> 16));
  x.z = __uint_as_float((hv.y << 16) | (lv.y & 0xffffu));
  x.w = __uint_as_float((hv.y & 0xffff0000u) | (lv.y >> 16));
  return x;
}

// float64 v moved across lanes by a DPP pattern (CTRL) within rows of 16
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const int64_t b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, int(uint32_t(b)), CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, int(uint32_t(uint64_t(b) >> 32)), CTRL, 0xf, 0xf, false);
  return __longlong_as_double(int64_t((uint64_t(uint32_t(hi)) << 32) | uint32_t(lo)));
}

// sum over each aligned group of 8 lanes, in every lane of the group: swap
// neighbours, swap pairs (quad permutations), then each half of the group
// with the other (the half-row mirror pairs lane i with 7 - i)
__device__ __forceinline__ double sum8_lanes(double v) {
  v += dpp_f64<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp_f64<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp_f64<0x141>(v);  // row_half_mirror
  return v;
}

// ---------------------------------------------------------------------------
// exact sweep over the float32 Phi rebuilt from both planes, float64 sums:
// one block = 256 keys of one head (4 waves x 8 rounds of 8 keys).  gate:
// only the heads with gate[h] != 0.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_sweep(const HeadDesc *__restrict__ desc, const uint16_t *__restrict__ phi16,
                                               const double *__restrict__ r, const int32_t *__restrict__ sel_slot,
                                               int cycle, int kR, const int32_t *__restrict__ gate,
                                               double *__restrict__ cand_val,
                                               int32_t *__restrict__ cand_idx, int32_t *__restrict__ head_status,
                                               double *__restrict__ score_all) {
  __shared__ double s_r[kStoredMaxN];
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
  const int kq = lane >> 3, sub = lane & 7;
  for (int64_t q = tid; q < D.ldN; q += 256) s_r[q] = q < D.n ? r[D.n_off + q] : 0.0;
  __syncthreads();
  const uint16_t *hp0 = phi16 + 2 * D.phi_off;
  const uint16_t *lp0 = hp0 + D.ldT * D.ldN;
  const int nit = int(D.ldN >> 6);
  for (int round = 0; round < 8; ++round) {
    const int slot = 64 * wave + 8 * round + kq;
    const int64_t key = int64_t(blk) * kSweepCols + slot;  // < ldT: a stored (possibly zero) column
    const uint16_t *hp = hp0 + key * D.ldN + 8 * sub;
    const uint16_t *lp = lp0 + key * D.ldN + 8 * sub;
    double a[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    if (key < D.ldT) {
#pragma unroll 4
      for (int i = 0; i < nit; ++i) {
        const u32x4 hv = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(hp + 64 * i));
        const u32x4 lv = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(lp + 64 * i));
        const f32x4 x0 = join_planes(u32x2{hv.x, hv.y}, u32x2{lv.x, lv.y});
        const f32x4 x1 = join_planes(u32x2{hv.z, hv.w}, u32x2{lv.z, lv.w});
        const double *rr = s_r + 64 * i + 8 * sub;
        a[0] = fma(rr[0], double(x0.x), a[0]);
        a[1] = fma(rr[1], double(x0.y), a[1]);
        a[2] = fma(rr[2], double(x0.z), a[2]);
        a[3] = fma(rr[3], double(x0.w), a[3]);
        a[4] = fma(rr[4], double(x1.x), a[4]);
        a[5] = fma(rr[5], double(x1.y), a[5]);
        a[6] = fma(rr[6], double(x1.z), a[6]);
        a[7] = fma(rr[7], double(x1.w), a[7]);
      }
    }
    const double c = sum8_lanes(((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7])));
    if (sub == 0) sv[slot] = c;
  }
  __syncthreads();
  const int64_t col = int64_t(blk) * kSweepCols + tid;
  double c = sv[tid];
  int idx = int(col);
  __syncthreads();
  if (col >= D.T || sel_slot[D.k_off + col] != 0) {
    c = -INFINITY;
    idx = INT_MAX;
  } else if (!isfinite(c)) {
    if (head_status) atomicOr(head_status + h, int32_t(AMC_HS_NONFINITE));
    c = -DBL_MAX;  // still a valid, selectable key
  }
  if (score_all && col < D.T) score_all[D.k_off + col] = c;
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
    int32_t *__restrict__ cand_idx, int32_t *__restrict__ head_status, double *__restrict__ score_all) {
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
    if (score_all && col < Dh.T) score_all[Dh.k_off + col] = c;
    sv[tid] = c;
    si[tid] = idx;
  }
  __syncthreads();
  block_sort256(sv, si);
  if (tid <= Kc && tid < 256) {
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
// relative error of (terms per accumulator + 2) 2^-24 each), the float32
// rounding of Phi and of r, the float64 rescoring's own rounding, and an
// absolute term for values below float32's normal range.  A key's 8 lanes
// take 16 consecutive queries of every 128 each; a lane keeps 8 float32
// accumulators per sign (two of its 16 queries per block: ldN / 64 terms
// each), and the lanes meet in float64.
// The keys: every key on the first cycle (which also writes each key's
// high-plane sums over 128-query blocks, rounded down, for the pruning, and
// the 8-bit plane of the second pruning stage), else the cycle's survivor list
// (or every key when the list is off), in groups of 32 (4 waves of 8).  A
// block takes every gridDim.x-th group of its head's list: one group per block
// on the first cycle, after it a few blocks per head, each staging r once for
// all of its groups (the lists are short, and most of a grid sized for every
// key would find nothing to do).  Out, per listed key: its upper and lower
// bound (sw_up, sw_lo; -inf for a selected key) and the key (sw_key), at its
// place in the list.
// ---------------------------------------------------------------------------
constexpr int SB_KEYS = 32;  // keys per block of the bounded sweep

// ---------------------------------------------------------------------------
// 8-bit plane.  The grid g(c) = the float32 with bits Q8_BASE + c 2^20, c =
// 8..254: 2^-31 (1 + m/8) 2^e, three significand bits, from 2^-30 up to 1.75.
// The code of a value h of the high plane is the smallest c with g(c) > h,
// i.e. with g(c) >= next(h), the bfloat16 above h, but at least 8; since Phi <
// next(h) (the plane truncates the float32 Phi, which is within 2^-24 of
// Phi), g(c) bounds Phi from above.  From below, for a code not raised to 8,
// g(c - 1) <= h, so the float32 just under g(c - 1) is at most h (1 - 2^-24)
// <= Phi; two neighbours of the grid differ by at most 8/9 (1.0 against
// 1.125), so Phi >= (113/128) g(c); where the code was raised to 8, Phi >= 0 >
// (113/128) g(8) - 2^-30.  In bfloat16 bits hb: c = max(8, floor((hb -
// Q8_BASE / 2^16) / 16) + 1).  g(c) = 2^96 times the float32 with bits c 2^20
// (a normal number for c >= 8), so the sweep decodes a code with one shift
// and takes the 2^96 into its weights.  A value that would need code 255
// (h >= 1.75, which a shifted Phi never reaches) marks the head's plane
// unusable.
// ---------------------------------------------------------------------------
constexpr uint32_t Q8_BASE = 96u << 23;   // bits of 2^-31
constexpr int Q8_HB_OFF = (96 << 7) - 16;  // hb - this, over 16, rounded down, is the code
constexpr float Q8_KAPPA = 113.0f / 128.0f;  // Phi >= Q8_KAPPA g(c) for a code not raised to 8
constexpr int Q8_CMIN = 8;                    // smallest code (a normal float32 for bits c 2^20)

typedef short s16x2 __attribute__((ext_vector_type(2)));

// codes of the two bfloat16 values packed in w (low half first), one per
// 16-bit half; hmax keeps the largest raw value for the range check
__device__ __forceinline__ uint32_t q8_codes2(uint32_t w, s16x2 &hmax) {
  s16x2 v = __builtin_bit_cast(s16x2, w);
  hmax = hmax > v ? hmax : v;
  // (values below g(7), sign bit included, take code 8)
  const s16x2 off = {short(Q8_HB_OFF), short(Q8_HB_OFF)}, top = {254, 254};
  const s16x2 low = {short(Q8_HB_OFF + 16 * Q8_CMIN), short(Q8_HB_OFF + 16 * Q8_CMIN)};
  v = v > low ? v : low;
  s16x2 c = (v - off) >> short(4);
  c = c < top ? c : top;
  return __builtin_bit_cast(uint32_t, c);
}

typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

// 2^-96 g(c) for the code in byte B of w: the float32 with bits c 2^20, one
// SDWA shift of the selected byte (tw holds the shift count, 20)
template <int B>
__device__ __forceinline__ float q8_grid(uint32_t w, uint32_t tw) {
  uint32_t r;
  if constexpr (B == 0)
    asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0"
        : "=v"(r) : "v"(tw), "v"(w));
  else if constexpr (B == 1)
    asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1"
        : "=v"(r) : "v"(tw), "v"(w));
  else if constexpr (B == 2)
    asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2"
        : "=v"(r) : "v"(tw), "v"(w));
  else
    asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3"
        : "=v"(r) : "v"(tw), "v"(w));
  return __uint_as_float(r);
}

// eight codes of a 16-byte load of the high plane (queries in order), as 8 bytes
__device__ __forceinline__ u32x2v q8_pack8(const u32x4 &xv, s16x2 &hmax) {
  const uint32_t a = q8_codes2(xv.x, hmax), b = q8_codes2(xv.y, hmax);
  const uint32_t c = q8_codes2(xv.z, hmax), d = q8_codes2(xv.w, hmax);
  // bytes 0 and 2 of each code pair
  return u32x2v{__builtin_amdgcn_perm(b, a, 0x06040200u), __builtin_amdgcn_perm(d, c, 0x06040200u)};
}

template <bool FIRST>
__global__ __launch_bounds__(256) void k_sweep_band(const HeadDesc *__restrict__ desc,
                                                    const uint16_t *__restrict__ phi16, const float *__restrict__ rpn,
                                                    const double *__restrict__ rabs,
                                                    const int32_t *__restrict__ surv_list,
                                                    const int32_t *__restrict__ surv_cnt,
                                                    const int32_t *__restrict__ sel_slot, int cycle, int kR,
                                                    int64_t qb128, float *__restrict__ colsum,
                                                    uint8_t *__restrict__ q8, int32_t *__restrict__ q8_bad,
                                                    double *__restrict__ sw_up, double *__restrict__ sw_lo,
                                                    int32_t *__restrict__ sw_key) {
  extern __shared__ __attribute__((aligned(16))) float s_rpn[];  // (r+, r-) per query, ldN of them
  const int h = blockIdx.y;
  const HeadDesc D = desc[h];
  int64_t S0;
  const int Kc = cycle_keys(D, cycle, kR, &S0);
  if (Kc == 0) return;
  const int list = FIRST ? -1 : surv_cnt[h];
  const int64_t cnt = list < 0 ? D.T : list;
  if (int64_t(blockIdx.x) * SB_KEYS >= cnt) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kq = lane >> 3, sub = lane & 7;
  // (r+, r-) of query 128 i + 16 sb + 2 j + e at 16-byte slot 64 i + 8 j + sb,
  // half e: the 8 lanes of a key read 128 consecutive bytes
  for (int64_t q = tid; q < D.ldN; q += 256) {
    float2 v = make_float2(0.0f, 0.0f);
    if (q < D.n) v = *reinterpret_cast<const float2 *>(rpn + 2 * (D.n_off + q));
    const int64_t i = q >> 7, sb = (q >> 4) & 7, j = (q >> 1) & 7, e = q & 1;
    *reinterpret_cast<float2 *>(s_rpn + 4 * (64 * i + 8 * j + sb) + 2 * e) = v;
  }
  __syncthreads();
  const int nb = int(D.ldN >> 7);                   // full 128-query blocks
  const bool half = (D.ldN & 64) != 0 && sub < 4;  // this lane's part of a last 64-query block
  const double rs = rabs[h];
  const int64_t ldTp = (D.T + 63) / 64 * 64;        // keys per 128-query block of the sums
  // the block's keys: groups of SB_KEYS, gridDim.x apart in the list
  for (int64_t kb = blockIdx.x; kb * SB_KEYS < cnt; kb += gridDim.x) {
    const int64_t at = kb * SB_KEYS + 8 * wave + kq;
    int64_t key = -1;
    if (at < cnt) key = list < 0 ? at : int64_t(surv_list[D.kt_off + at]);
    // lane sub: queries 16 sub .. 16 sub + 15 of every 128 (two 16-byte loads)
    const uint16_t *hp = phi16 + 2 * D.phi_off + (key < 0 ? 0 : key) * D.ldN + 16 * sub;
    float P[8], N[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) P[e] = N[e] = 0.0f;
    auto step = [&](int b, const u32x4 &xa, const u32x4 &xb) __attribute__((always_inline)) {
      const f32x4 *ww = reinterpret_cast<const f32x4 *>(s_rpn) + 64 * b + sub;
      const uint32_t w[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const f32x4 pr = ww[8 * j];  // (r+, r-) of the lane's queries 2 j and 2 j + 1
        const float v0 = __uint_as_float(w[j] << 16);
        const float v1 = __uint_as_float(w[j] & 0xffff0000u);
        const int e = (2 * j) & 7;
        P[e] = fmaf(pr.x, v0, P[e]);
        N[e] = fmaf(pr.y, v0, N[e]);
        P[e + 1] = fmaf(pr.z, v1, P[e + 1]);
        N[e + 1] = fmaf(pr.w, v1, N[e + 1]);
      }
    };
    // FIRST: the high-plane sum of 128-query block b from this lane's 16 values
    // of it.  The float32 lane sums of 16 positive terms are within 2^-20 of
    // exact: scaled down by that much and rounded down, the stored sum is at
    // most the exact one and at least (1 - 2^-18.9) of it.
    auto hsum = [&](const u32x4 &a, const u32x4 &b) __attribute__((always_inline)) {
      float t = 0.0f;
      const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int c = 0; c < 8; ++c) t += __uint_as_float(w[c] << 16) + __uint_as_float(w[c] & 0xffff0000u);
      return t;
    };
    // FIRST with the 8-bit plane: the codes of the lane's 16 queries of a block
    // (128 consecutive bytes per key from its 8 lanes)
    s16x2 hmax = {0, 0};
    u32x4 *q8p = (FIRST && q8) ? reinterpret_cast<u32x4 *>(q8 + D.phi_off + (key < 0 ? 0 : key) * D.ldN + 16 * sub)
                               : nullptr;
    auto block = [&](int b, const u32x4 &xa, const u32x4 &xb) __attribute__((always_inline)) {
      step(b, xa, xb);
      if constexpr (FIRST) {
        const double bs = sum8_lanes(double(hsum(xa, xb)));
        if (sub == 0) colsum[D.kt_off * qb128 + b * ldTp + key] = __double2float_rd(bs * (1.0 - 0x1p-20));
        if (q8p) {
          const u32x2v ca = q8_pack8(xa, hmax), cb = q8_pack8(xb, hmax);
          q8p[8 * b] = u32x4{ca.x, ca.y, cb.x, cb.y};
        }
      }
    };
    if (key >= 0) {
      // sixteen 16-byte loads (eight blocks) in flight per lane; eight on the
      // first cycle, whose blocks also do the sums and the 8-bit codes
      constexpr int NBL = FIRST ? 4 : 8;
      int b = 0;
      for (; b + NBL <= nb; b += NBL) {
        u32x4 xv[2 * NBL];
#pragma unroll
        for (int u = 0; u < NBL; ++u) {
          xv[2 * u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(hp + 128 * (b + u)));
          xv[2 * u + 1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(hp + 128 * (b + u) + 8));
        }
        __builtin_amdgcn_sched_barrier(0);  // all of them issue before any is used
#pragma unroll
        for (int u = 0; u < NBL; ++u) block(b + u, xv[2 * u], xv[2 * u + 1]);
      }
      for (; b < nb; ++b)
        block(b, __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(hp + 128 * b)),
              __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(hp + 128 * b + 8)));
    }
    // a last 64-query block: lanes 0..3 hold its queries, the others add zeros
    if ((D.ldN & 64) != 0) {
      u32x4 xa = {0u, 0u, 0u, 0u}, xb = {0u, 0u, 0u, 0u};
      if (key >= 0 && half) {
        xa = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(hp + 128 * nb));
        xb = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(hp + 128 * nb + 8));
      }
      if constexpr (FIRST) {
        const double bs = sum8_lanes(double(hsum(xa, xb)));
        if (sub == 0 && key >= 0) colsum[D.kt_off * qb128 + nb * ldTp + key] = __double2float_rd(bs * (1.0 - 0x1p-20));
        if (q8p && key >= 0 && half) {
          const u32x2v ca = q8_pack8(xa, hmax), cb = q8_pack8(xb, hmax);
          q8p[8 * nb] = u32x4{ca.x, ca.y, cb.x, cb.y};
        }
      }
      if (key >= 0 && half) step(nb, xa, xb);
    }
    if (FIRST && q8p && key >= 0 &&
        (hmax.x >= short(Q8_HB_OFF + 16 * 255) || hmax.y >= short(Q8_HB_OFF + 16 * 255)))
      q8_bad[h] = 1;
    double Pd = 0.0, Nd = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      Pd += double(P[e]);
      Nd += double(N[e]);
    }
    Pd = sum8_lanes(Pd);
    Nd = sum8_lanes(Nd);
    if (sub == 0 && key >= 0) {
      const bool valid = key < D.T && sel_slot[D.k_off + key] == 0;
      const double crel = 2.0 * (double(D.ldN >> 6) + 16.0) * 0x1p-24 + 0x1p-22;
      const double slack = crel * (Pd - Nd) + (rs + double(D.n)) * 0x1p-120;
      const double c7 = 0x1.00001p-7;
      sw_up[D.kt_off + at] = valid ? (Pd + Nd) + c7 * Pd + slack : -INFINITY;
      sw_lo[D.kt_off + at] = valid ? (Pd + Nd) + c7 * Nd - slack : -INFINITY;
      sw_key[D.kt_off + at] = int(key);
    }
  }
}

// ---------------------------------------------------------------------------
// Second pruning stage, between k_prune and the bounded sweep: for each key of
// the survivor list an upper bound of r^T Phi[:, k] from the 8-bit plane,
//   U8_k = sum_{r_q > 0} r_q g(c_qk) + (113/128) sum_{r_q < 0} r_q g(c_qk)
//          + 2^-30 sum |r|
// (Phi <= g(c), Phi >= (113/128) g(c) less 2^-30 where the code was raised to
// 8), plus the float32 accumulation, rounding and underflow allowances of the
// bounded sweep (the product (113/128) r- is rounded to float32 once more).
// A code decodes with one SDWA shift of its byte to 2^-96 g(c), and the
// weights carry the factor 2^96 (exact), so the products are r g(c) and stay
// in float32's normal range.  Nothing is
// done where k_prune kept every key (its L is -inf) or the plane is unusable.
// Groups of 64 keys (8 waves of 8), 8 lanes per key, each lane 16 queries of
// every 128 (one 16-byte load), sixteen loads in flight; a block takes every
// gridDim.x-th group of its head's list.  The (r+, (113/128) r-) pairs sit in
// LDS lane-interleaved: pair j of lane sub's 16 queries of 128-query block i
// at 16-byte slot 64 i + 8 j + sub, so the 8 lanes of a key read 128
// consecutive bytes.  Out: sw_up and sw_key at the key's place in the list
// (-inf for a selected key).
// ---------------------------------------------------------------------------
constexpr int Q8_KEYS = 64;
constexpr int Q8_THREADS = 512;

__global__ __launch_bounds__(Q8_THREADS) void k_sweep_q8(const HeadDesc *__restrict__ desc,
                                                         const uint8_t *__restrict__ q8,
                                                         const float *__restrict__ rpn,
                                                         const double *__restrict__ rabs,
                                                         const double *__restrict__ prune_L,
                                                         const int32_t *__restrict__ q8_bad,
                                                         const int32_t *__restrict__ surv_list,
                                                         const int32_t *__restrict__ surv_cnt,
                                                         const int32_t *__restrict__ sel_slot, int cycle, int kR,
                                                         double *__restrict__ sw_up, int32_t *__restrict__ sw_key) {
  extern __shared__ __attribute__((aligned(16))) float s_w[];  // (r+, (113/128) r-) pairs, 2 per 16-byte slot
  const int h = blockIdx.y;
  const HeadDesc D = desc[h];
  int64_t S0;
  const int Kc = cycle_keys(D, cycle, kR, &S0);
  if (Kc == 0 || q8_bad[h] || prune_L[h] == -INFINITY) return;
  const int list = surv_cnt[h];
  const int64_t cnt = list < 0 ? D.T : list;
  if (int64_t(blockIdx.x) * Q8_KEYS >= cnt) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kq = lane >> 3, sub = lane & 7;
  // query q = 128 i + 16 sb + 2 j + e  ->  float2 at slot 64 i + 8 j + sb, half e
  for (int64_t q = tid; q < D.ldN; q += Q8_THREADS) {
    float2 v = make_float2(0.0f, 0.0f);
    if (q < D.n) v = *reinterpret_cast<const float2 *>(rpn + 2 * (D.n_off + q));
    v.y *= Q8_KAPPA;
    v.x *= 0x1p96f;
    v.y *= 0x1p96f;
    const int64_t i = q >> 7, sb = (q >> 4) & 7, j = (q >> 1) & 7, e = q & 1;
    *reinterpret_cast<float2 *>(s_w + 4 * (64 * i + 8 * j + sb) + 2 * e) = v;
  }
  __syncthreads();
  const int nit = int(D.ldN >> 7);                      // full 128-query steps
  const bool half = (D.ldN & 64) != 0 && 16 * sub < 64;  // this lane's part of a last 64-query step
  const double rs = rabs[h];
  const uint32_t twenty = 20;
  for (int64_t kb = blockIdx.x; kb * Q8_KEYS < cnt; kb += gridDim.x) {
    const int64_t at = kb * Q8_KEYS + 8 * wave + kq;
    int64_t key = -1;
    if (at < cnt) key = list < 0 ? at : int64_t(surv_list[D.kt_off + at]);
    const uint8_t *cp = q8 + D.phi_off + (key < 0 ? 0 : key) * D.ldN + 16 * sub;
    float P[8], N[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) P[e] = N[e] = 0.0f;
    auto step = [&](int i, const u32x4 &cv) __attribute__((always_inline)) {
      const f32x4 *ww = reinterpret_cast<const f32x4 *>(s_w) + 64 * i + sub;
      const uint32_t cw[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f32x4 w01 = ww[8 * (2 * c)], w23 = ww[8 * (2 * c + 1)];  // pairs of queries 4 c .. 4 c + 3
        const float g0 = q8_grid<0>(cw[c], twenty), g1 = q8_grid<1>(cw[c], twenty);
        const float g2 = q8_grid<2>(cw[c], twenty), g3 = q8_grid<3>(cw[c], twenty);
        const int e = (4 * c) & 7;
        P[e] = fmaf(w01.x, g0, P[e]);
        N[e] = fmaf(w01.y, g0, N[e]);
        P[e + 1] = fmaf(w01.z, g1, P[e + 1]);
        N[e + 1] = fmaf(w01.w, g1, N[e + 1]);
        P[e + 2] = fmaf(w23.x, g2, P[e + 2]);
        N[e + 2] = fmaf(w23.y, g2, N[e + 2]);
        P[e + 3] = fmaf(w23.z, g3, P[e + 3]);
        N[e + 3] = fmaf(w23.w, g3, N[e + 3]);
      }
    };
    if (key >= 0) {
      int i = 0;
      for (; i + 16 <= nit; i += 16) {
        u32x4 cv[16];
#pragma unroll
        for (int u = 0; u < 16; ++u)
          cv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(cp + 128 * (i + u)));
        __builtin_amdgcn_sched_barrier(0);  // all sixteen issue before any is used
#pragma unroll
        for (int u = 0; u < 16; ++u) step(i + u, cv[u]);
      }
      for (; i < nit; ++i) step(i, __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(cp + 128 * i)));
      if (half) step(nit, __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(cp + 128 * nit)));
    }
    double Pd = 0.0, Nd = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      Pd += double(P[e]);
      Nd += double(N[e]);
    }
    Pd = sum8_lanes(Pd);
    Nd = sum8_lanes(Nd);
    if (sub == 0 && key >= 0) {
      const bool valid = key < D.T && sel_slot[D.k_off + key] == 0;
      const double crel = 2.0 * (double(D.ldN >> 6) + 16.0) * 0x1p-24 + 0x1p-21;
      const double u = (Pd + Nd) + crel * (Pd - Nd) + rs * 0x1p-30 + (rs + double(D.n)) * 0x1p-120;
      sw_up[D.kt_off + at] = valid ? u : -INFINITY;
      sw_key[D.kt_off + at] = int(key);
    }
  }
}

// ---------------------------------------------------------------------------
// The keys the bounded sweep reads after the second stage: one block of 1024
// threads per head keeps, in list order, each listed key whose U8 reaches the
// threshold L of k_prune (a NaN bound keeps its key).  Where the stage did not
// run the list passes through unchanged.  Trace: keys read from the 8-bit
// plane and from the high plane this cycle.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_q8_compact(const HeadDesc *__restrict__ desc, int cycle, int kR,
                                                     const double *__restrict__ prune_L,
                                                     const int32_t *__restrict__ q8_bad,
                                                     const int32_t *__restrict__ surv_list,
                                                     const int32_t *__restrict__ surv_cnt,
                                                     const double *__restrict__ sw_up,
                                                     const int32_t *__restrict__ sw_key,
                                                     int32_t *__restrict__ surv2_list, int32_t *__restrict__ surv2_cnt,
                                                     int32_t *__restrict__ tr_swept, int32_t *__restrict__ tr_swept8) {
  __shared__ int s_wc[16];
  const int h = blockIdx.x;
  const HeadDesc D = desc[h];
  int64_t S0;
  const int Kc = cycle_keys(D, cycle, kR, &S0);
  if (Kc == 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sc = surv_cnt[h];
  const double L = prune_L[h];
  if (q8_bad[h] || L == -INFINITY) {
    for (int e = tid; e < sc; e += 1024) surv2_list[D.kt_off + e] = surv_list[D.kt_off + e];
    if (tid == 0) {
      surv2_cnt[h] = sc;
      if (tr_swept8) tr_swept8[D.cyc_off + cycle] = 0;
    }
    return;
  }
  const int64_t cnt = sc < 0 ? D.T : sc;
  int total = 0;
  for (int64_t e0 = 0; e0 < cnt; e0 += 1024) {
    const int64_t e = e0 + tid;
    int key = -1;
    if (e < cnt) {
      const double u = sw_up[D.kt_off + e];
      if (u != -INFINITY && !(u < L)) key = sw_key[D.kt_off + e];
    }
    const uint64_t m = __ballot(key >= 0);
    if (lane == 0) s_wc[wave] = __popcll(m);
    __syncthreads();
    int at = total;
    for (int w = 0; w < wave; ++w) at += s_wc[w];
    at += __popcll(m & ((uint64_t(1) << lane) - 1));
    if (key >= 0) surv2_list[D.kt_off + at] = key;
    for (int w = 0; w < 16; ++w) total += s_wc[w];
    __syncthreads();
  }
  if (tid == 0) {
    surv2_cnt[h] = total;
    if (tr_swept) tr_swept[D.cyc_off + cycle] = total;
    if (tr_swept8) tr_swept8[D.cyc_off + cycle] = int32_t(cnt);
  }
}

// ---------------------------------------------------------------------------
// Pruning for the bounded sweep, one block of 1024 threads per head.  With
// H_Bk the high-plane sum of key k over the 128-query block B (written by the
// first cycle's sweep, rounded down to within 2^-18 of the sum) and rmax_B the
// largest r_q in B,
//   r^T Phi[:, k] = sum_B sum_{q in B} r_q Phi_qk <= sum_B rmax_B M_Bk = U_k,
// M_Bk bounding sum_{q in B} Phi_qk from above where rmax_B >= 0 and from
// below where it is negative (H_Bk scaled by (1 + 2^-7)(1 + 2^-18), resp.
// by 1 - 2^-23: the plane truncates, float32 rounds), plus a float64 rounding
// allowance.  Each thread's best key by U over its share; the 64 best of
// those are scored from both planes (the float32 Phi, float64 sums) and bounded
// below by that score less the float32 rounding of Phi and the sum's own:
// L = the (Kc+1)-th best of those lower bounds is at most the (Kc+1)-th best
// score, so no key with U_k < L is among this cycle's top Kc+1 and the sweep
// skips it.
// Also writes r's float32 positive and negative parts and sum |r| for the
// sweep.  The first cycle (no sums yet), a non-finite r, Kc + 1 > 64 and
// heads longer than the list's LDS keep every key (surv_cnt = -1).
// ---------------------------------------------------------------------------
constexpr int PR_THREADS = 1024;
constexpr int PR_CAND = 64;
constexpr int PR_MAXT = 16384;  // keys whose U stays in LDS

__device__ void block_sort1024(double *v, int *ix) {
  const int tid = threadIdx.x;
  for (int k = 2; k <= 1024; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      const int p = tid ^ j;
      if (p > tid) {
        const double va = v[tid], vb = v[p];
        const int ia = ix[tid], ib = ix[p];
        if (better(va, ia, vb, ib) != ((tid & k) == 0)) {
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

__global__ __launch_bounds__(PR_THREADS) void k_prune(const HeadDesc *__restrict__ desc,
                                                      const double *__restrict__ r,
                                                      const int32_t *__restrict__ sel_slot,
                                                      const uint16_t *__restrict__ phi16,
                                                      const float *__restrict__ colsum, int64_t qb128, int cycle,
                                                      int kR, float *__restrict__ rpn, double *__restrict__ rabs,
                                                      int32_t *__restrict__ surv_list,
                                                      int32_t *__restrict__ surv_cnt, double *__restrict__ prune_L,
                                                      int32_t *__restrict__ tr_swept) {
  __shared__ double s_r[kStoredMaxN];
  __shared__ float s_u[PR_MAXT];
  __shared__ double s_wmax[kStoredMaxN / 64];
  __shared__ double s_rmax[kStoredMaxN / 128];
  __shared__ double s_cv[PR_THREADS];
  __shared__ int s_ci[PR_THREADS];
  __shared__ double s_part[PR_THREADS / 64];
  __shared__ double s_lo[PR_CAND];
  __shared__ int s_wc[PR_THREADS / 64];
  __shared__ double s_L;
  const int h = blockIdx.x;
  const HeadDesc D = desc[h];
  int64_t S0;
  const int Kc = cycle_keys(D, cycle, kR, &S0);
  if (Kc == 0) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // r's parts, sum |r|, and the largest r of every 64 queries
  double ra = 0.0;
  for (int64_t q0 = 0; q0 < D.ldN; q0 += PR_THREADS) {
    const int64_t q = q0 + tid;
    double rv = 0.0, rm = -INFINITY;
    if (q < D.n) {
      rv = r[D.n_off + q];
      rm = rv;
      *reinterpret_cast<float2 *>(rpn + 2 * (D.n_off + q)) = make_float2(float(fmax(rv, 0.0)), float(fmin(rv, 0.0)));
    }
    if (q < D.ldN) s_r[q] = rv;
    ra += fabs(rv);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) rm = fmax(rm, __shfl_xor(rm, off));
    if (lane == 0 && q < D.ldN) s_wmax[q >> 6] = rm;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ra += __shfl_xor(ra, off);
  if (lane == 0) s_part[wave] = ra;
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;
    for (int w = 0; w < PR_THREADS / 64; ++w) t += s_part[w];
    rabs[h] = t;
    s_L = t;
  }
  const int nb = int((D.n + 127) >> 7);
  if (tid < nb) s_rmax[tid] = fmax(s_wmax[2 * tid], 2 * tid + 1 < (D.ldN >> 6) ? s_wmax[2 * tid + 1] : -INFINITY);
  __syncthreads();
  const bool keep_all = cycle == 0 || !isfinite(s_L) || Kc + 1 > PR_CAND || D.T > PR_MAXT;
  if (keep_all) {
    if (tid == 0) {
      surv_cnt[h] = -1;
      if (prune_L) prune_L[h] = -INFINITY;
      if (tr_swept) tr_swept[D.cyc_off + cycle] = int32_t(D.T);
    }
    return;
  }
  // U for every key (-inf for selected keys), each thread's best
  const double kup = (1.0 + 0x1p-7) * (1.0 + 0x1p-18) + 0x1p-40;  // the plane truncates; the sums round down
  const double kdn = 1.0 - 0x1p-23;
  double bv = -INFINITY;
  int bi = INT_MAX;
  for (int64_t k = tid; k < D.T; k += PR_THREADS) {
    double u = -INFINITY;
    if (sel_slot[D.k_off + k] == 0) {
      const float *cs = colsum + D.kt_off * qb128 + k;
      const int64_t ldTp = (D.T + 63) / 64 * 64;
      double s = 0.0, a = 0.0;
      for (int b = 0; b < nb; ++b) {
        const double rm = s_rmax[b];
        const double c = double(cs[b * ldTp]);
        const double t = rm * (rm >= 0.0 ? c * kup : c * kdn);
        s += t;
        a += fabs(t);
      }
      u = s + a * double(nb + 2) * 0x1p-50;
      if (better(u, int(k), bv, bi)) {
        bv = u;
        bi = int(k);
      }
    }
    if (u != u) u = INFINITY;  // a NaN bound keeps the key
    s_u[k] = __double2float_ru(u);  // rounded up: the stored value bounds u
  }
  s_cv[tid] = bv;
  s_ci[tid] = bi;
  __syncthreads();
  block_sort1024(s_cv, s_ci);
  // lower bounds of the PR_CAND best candidates (4 per wave) from the float32 Phi
  const uint16_t *hp0 = phi16 + 2 * D.phi_off;
  const uint16_t *lp0 = hp0 + D.ldT * D.ldN;
  for (int cnd = wave; cnd < PR_CAND; cnd += PR_THREADS / 64) {
    const int key = s_ci[cnd];
    double lo = -INFINITY;
    if (key != INT_MAX) {
      const uint16_t *hp = hp0 + int64_t(key) * D.ldN;
      const uint16_t *lp = lp0 + int64_t(key) * D.ldN;
      double sc = 0.0, ab = 0.0;
      auto part = [&](int64_t q, const u32x4 &hv, const u32x4 &lv) __attribute__((always_inline)) {
        const f32x4 x0 = join_planes(u32x2{hv.x, hv.y}, u32x2{lv.x, lv.y});
        const f32x4 x1 = join_planes(u32x2{hv.z, hv.w}, u32x2{lv.z, lv.w});
        const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double t = s_r[q + e] * double(xs[e]);
          sc += t;
          ab += fabs(t);
        }
      };
      // eight 512-query steps of both planes in flight at once
      int64_t q = 8 * lane;
      for (; q + 7 * 512 < D.ldN; q += 8 * 512) {
        u32x4 hv[8], lv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          hv[u] = *reinterpret_cast<const u32x4 *>(hp + q + 512 * u);
          lv[u] = *reinterpret_cast<const u32x4 *>(lp + q + 512 * u);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) part(q + 512 * u, hv[u], lv[u]);
      }
      for (; q < D.ldN; q += 512)
        part(q, *reinterpret_cast<const u32x4 *>(hp + q), *reinterpret_cast<const u32x4 *>(lp + q));
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        sc += __shfl_xor(sc, off);
        ab += __shfl_xor(ab, off);
      }
      // |Phi - x| <= 2^-24 (1 + 2^-23) x, float64 products and sums within n 2^-52 of ab
      lo = sc - ab * (0x1p-24 + 0x1p-46 + double(D.ldN) * 0x1p-52) - (s_L + double(D.n)) * 0x1p-120;
      if (!isfinite(lo)) lo = -INFINITY;
    }
    if (lane == 0) s_lo[cnd] = lo;
  }
  __syncthreads();
  if (wave == 0) {
    // L: the (Kc+1)-th best lower bound (ranks by value, then candidate slot)
    const double v = s_lo[lane];
    int rank = 0;
    for (int j = 0; j < PR_CAND; ++j) {
      const double o = s_lo[j];
      rank += (o > v || (o == v && j < lane)) ? 1 : 0;
    }
    if (rank == Kc) s_L = v;
  }
  __syncthreads();
  const double L = s_L;
  // survivors: unselected keys with U >= L, in key order
  int total = 0;
  for (int64_t k0 = 0; k0 < D.T; k0 += PR_THREADS) {
    const int64_t k = k0 + tid;
    const bool take = k < D.T && double(s_u[k]) >= L;
    const uint64_t m = __ballot(take);
    if (lane == 0) s_wc[wave] = __popcll(m);
    __syncthreads();
    int at = total;
    for (int w = 0; w < wave; ++w) at += s_wc[w];
    at += __popcll(m & ((uint64_t(1) << lane) - 1));
    if (take) surv_list[D.kt_off + at] = int(k);
    for (int w = 0; w < PR_THREADS / 64; ++w) total += s_wc[w];
    __syncthreads();
  }
  if (tid == 0) {
    surv_cnt[h] = total;
    if (prune_L) prune_L[h] = L;
    if (tr_swept) tr_swept[D.cyc_off + cycle] = total;
  }
}

// ---------------------------------------------------------------------------
// band merge: one block of 1024 threads per head.  L = the (Kc+1)-th best
// lower bound over the swept keys, found by radix selection on the bounds'
// order-preserving 64-bit images (8 passes of 8 bits); the band is every key
// whose upper bound reaches L, in list order.  It holds the true top Kc+1:
// each of those scores at least L, and its upper bound at least its score.
// exact[h] = 1 when the band overflows band_cap (<= kBandCap; lower only to
// exercise the exact path), holds fewer than Kc keys, or a bound of an
// unselected key is not finite: the head takes the float32 sweep this cycle.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t order_key(double v) {
  const uint64_t b = __double_as_longlong(v);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

__global__ __launch_bounds__(1024) void k_band_merge(const HeadDesc *__restrict__ desc, int cycle, int kR,
                                                     const double *__restrict__ sw_up,
                                                     const double *__restrict__ sw_lo,
                                                     const int32_t *__restrict__ sw_key,
                                                     const int32_t *__restrict__ surv_cnt, int band_cap,
                                                     int32_t *__restrict__ band_list, int32_t *__restrict__ band_cnt,
                                                     int32_t *__restrict__ exact) {
  __shared__ int hist[256];
  __shared__ int s_wc[16];
  __shared__ uint64_t s_prefix;
  __shared__ int s_need;
  const int h = blockIdx.x;
  const HeadDesc D = desc[h];
  int64_t S0;
  const int Kc = cycle_keys(D, cycle, kR, &S0);
  if (Kc == 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sc = surv_cnt[h];
  const int64_t cnt = sc < 0 ? D.T : sc;
  const double *up = sw_up + D.kt_off;
  const double *lo = sw_lo + D.kt_off;
  int bad = 0;
  for (int64_t e = tid; e < cnt; e += 1024)
    bad |= (lo[e] != -INFINITY || up[e] != -INFINITY) && !(isfinite(up[e]) && isfinite(lo[e]));
  if (__syncthreads_or(bad)) {
    if (tid == 0) {
      band_cnt[h] = 0;
      exact[h] = 1;
    }
    return;
  }
  // radix selection of the (Kc+1)-th largest order key among the lower bounds
  if (tid == 0) {
    s_prefix = 0;
    s_need = Kc + 1;
  }
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    const uint64_t prefix = s_prefix;
    const uint64_t pmask = pass == 0 ? 0ull : (~0ull << (shift + 8));
    for (int64_t e = tid; e < cnt; e += 1024) {
      const uint64_t k = order_key(lo[e]);
      if ((k & pmask) == prefix) atomicAdd(&hist[int((k >> shift) & 255u)], 1);
    }
    __syncthreads();
    if (tid == 0) {
      int need = s_need, d = 255;
      for (; d > 0; --d) {
        if (hist[d] >= need) break;
        need -= hist[d];
      }
      s_need = need;
      s_prefix = prefix | (uint64_t(d) << shift);
    }
    __syncthreads();
  }
  // (with fewer than Kc + 1 keys the selection runs off the bottom: L = -inf,
  // the band is every unselected key)
  const uint64_t kL = s_prefix;
  double L = __longlong_as_double(int64_t((kL >> 63) ? (kL & 0x7fffffffffffffffull) : ~kL));
  if (L != L) L = -INFINITY;
  int total = 0;
  int32_t *out = band_list + int64_t(h) * kBandCap;
  for (int64_t e0 = 0; e0 < cnt; e0 += 1024) {
    const int64_t e = e0 + tid;
    const bool take = e < cnt && up[e] != -INFINITY && up[e] >= L;
    const uint64_t m = __ballot(take);
    if (lane == 0) s_wc[wave] = __popcll(m);
    __syncthreads();
    int at = total;
    for (int w = 0; w < wave; ++w) at += s_wc[w];
    at += __popcll(m & ((uint64_t(1) << lane) - 1));
    if (take && at < kBandCap) out[at] = sw_key[D.kt_off + e];
    for (int w = 0; w < 16; ++w) total += s_wc[w];
    __syncthreads();
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
                                               int kR, int polish, double *__restrict__ r, double *__restrict__ mhat,
                                               double *__restrict__ rpart) {
  static_assert(kResidRows == 256, "one query per thread");
  __shared__ double ws[256];
  __shared__ double red[2][4];
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
  double rv = 0.0, mv = 0.0;
  if (valid) {
    const double mi = m[D.n_off + i];
    rv = mi - acc;
    mv = mi;
    mhat[D.n_off + i] = acc;
    r[D.n_off + i] = rv;
  }
  // the block's sums of r^2 and m^2 (the relative residual the exact-refit
  // gate reads), in a fixed order
  double s0 = rv * rv, s1 = mv * mv;
  for (int o = 32; o > 0; o >>= 1) {
    s0 += __shfl_xor(s0, o);
    s1 += __shfl_xor(s1, o);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    red[0][wave] = s0;
    red[1][wave] = s1;
  }
  __syncthreads();
  if (threadIdx.x == 0 && rpart) {
    const int64_t at = (int64_t(h) * gridDim.x + blockIdx.x) * 2;
    rpart[at] = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
    rpart[at + 1] = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
  }
}

// AM-Highest: 1 / m into the m-hat buffer (unused until the first residual),
// which the sweep then takes as its r: r^T Phi[:, j] is key j's attention
// summed over the queries.
__global__ __launch_bounds__(256) void k_recip(const HeadDesc *__restrict__ desc, const double *__restrict__ m,
                                               double *__restrict__ r) {
  const HeadDesc D = desc[blockIdx.y];
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= D.n) return;
  const double mi = m[D.n_off + i];
  r[D.n_off + i] = mi > 0.0 ? 1.0 / mi : 0.0;
}

// AM-Highest: each head's t largest scores (ties to the lower key) become
// its picks, in ascending key order: radix selection of the t-th largest
// order key (8 passes of 8 bits), then one pass that takes every key above it
// and the first keys equal to it.  The trace gets the picks, their scores and
// the best score left out.
__global__ __launch_bounds__(1024) void k_topt(const HeadDesc *__restrict__ desc,
                                               const double *__restrict__ score_all,
                                               int32_t *__restrict__ sel_slot, int32_t *__restrict__ sel_list,
                                               int32_t *__restrict__ tr_pick, double *__restrict__ tr_pick_score,
                                               double *__restrict__ tr_runner) {
  __shared__ int hist[256];
  __shared__ int s_wt[16], s_we[16];
  __shared__ double s_wmax[16];
  __shared__ uint64_t s_prefix;
  __shared__ int s_need;
  const int h = blockIdx.x;
  const HeadDesc D = desc[h];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t T = D.T;
  const double *sc = score_all + D.k_off;
  if (tid == 0) {
    s_prefix = 0;
    s_need = int(D.t);
  }
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    const uint64_t prefix = s_prefix;
    const uint64_t pmask = pass == 0 ? 0ull : (~0ull << (shift + 8));
    for (int64_t e = tid; e < T; e += 1024) {
      const uint64_t k = order_key(sc[e]);
      if ((k & pmask) == prefix) atomicAdd(&hist[int((k >> shift) & 255u)], 1);
    }
    __syncthreads();
    if (tid == 0) {
      int need = s_need, dg = 255;
      for (; dg > 0; --dg) {
        if (hist[dg] >= need) break;
        need -= hist[dg];
      }
      s_need = need;
      s_prefix = prefix | (uint64_t(dg) << shift);
    }
    __syncthreads();
  }
  const uint64_t kL = s_prefix;
  const int need = s_need;  // keys equal to the t-th largest that are taken
  int taken = 0, eq_seen = 0;
  double runner = -INFINITY;
  for (int64_t e0 = 0; e0 < T; e0 += 1024) {
    const int64_t e = e0 + tid;
    const bool valid = e < T;
    const double v = valid ? sc[e] : -INFINITY;
    const uint64_t k = valid ? order_key(v) : 0ull;
    const bool gt = valid && k > kL, eq = valid && k == kL;
    const uint64_t me = __ballot(eq);
    if (lane == 0) s_we[wave] = __popcll(me);
    __syncthreads();
    int eq_rank = eq_seen;
    for (int w = 0; w < wave; ++w) eq_rank += s_we[w];
    eq_rank += __popcll(me & ((uint64_t(1) << lane) - 1));
    const bool take = gt || (eq && eq_rank < need);
    const uint64_t mt = __ballot(take);
    if (lane == 0) s_wt[wave] = __popcll(mt);
    double best = (valid && !take) ? v : -INFINITY;
    for (int o = 32; o > 0; o >>= 1) best = fmax(best, __shfl_xor(best, o));
    if (lane == 0) s_wmax[wave] = best;
    __syncthreads();
    int at = taken;
    for (int w = 0; w < wave; ++w) at += s_wt[w];
    at += __popcll(mt & ((uint64_t(1) << lane) - 1));
    if (take && at < D.t) {
      sel_list[D.t_off + at] = int32_t(e);
      sel_slot[D.k_off + e] = at + 1;
      if (tr_pick) tr_pick[D.t_off + at] = int32_t(e);
      if (tr_pick_score) tr_pick_score[D.t_off + at] = v;
    }
    for (int w = 0; w < 16; ++w) {
      taken += s_wt[w];
      eq_seen += s_we[w];
      runner = fmax(runner, s_wmax[w]);
    }
    __syncthreads();
  }
  if (tid == 0 && tr_runner) tr_runner[D.cyc_off] = runner;
}

// Trace: the relative mass residual ||r|| / ||m|| of each head after the
// cycle's refit (the last cycle's entry after the polish refits), from
// k_resid's per-block sums in a fixed order.
__global__ __launch_bounds__(64) void k_relres(const HeadDesc *__restrict__ desc, int cycle, int kR, int polish,
                                               int nrb, const double *__restrict__ rpart,
                                               double *__restrict__ tr_relres) {
  const int h = blockIdx.x;
  const HeadDesc D = desc[h];
  int64_t cyc;
  if (polish) {
    cyc = (D.t + kR - 1) / kR - 1;
  } else {
    int64_t S0;
    if (cycle_keys(D, cycle, kR, &S0) == 0) return;
    cyc = cycle;
  }
  double r2 = 0.0, m2 = 0.0;
  for (int k = threadIdx.x; k < nrb; k += 64) {
    r2 += rpart[(int64_t(h) * nrb + k) * 2];
    m2 += rpart[(int64_t(h) * nrb + k) * 2 + 1];
  }
  for (int o = 32; o > 0; o >>= 1) {
    r2 += __shfl_xor(r2, o);
    m2 += __shfl_xor(m2, o);
  }
  if (threadIdx.x == 0) tr_relres[D.cyc_off + cyc] = m2 > 0.0 ? sqrt(r2 / m2) : 0.0;
}

}  // namespace

hipError_t launch_recip(const Dims &dm, const Buffers &b, hipStream_t s) {
  hipLaunchKernelGGL(k_recip, dim3(unsigned((dm.max_n + 255) / 256), unsigned(dm.H)), dim3(256), 0, s, b.desc, b.m,
                     b.mhat);
  return hipGetLastError();
}

hipError_t launch_topt(const Dims &dm, const Buffers &b, hipStream_t s) {
  if (!b.score_all) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_topt, dim3(unsigned(dm.H)), dim3(1024), 0, s, b.desc, b.score_all, b.sel_slot, b.sel_list,
                     b.tr_pick, b.tr_pick_score, b.tr_runner);
  return hipGetLastError();
}

hipError_t launch_relres(const Dims &dm, const Buffers &b, int cycle, int kR, int polish, hipStream_t s) {
  if (!b.tr_relres || !b.rpart) return hipSuccess;
  hipLaunchKernelGGL(k_relres, dim3(unsigned(dm.H)), dim3(64), 0, s, b.desc, cycle, kR, polish, int(dm.nrb), b.rpart,
                     b.tr_relres);
  return hipGetLastError();
}

hipError_t launch_sweep(const Dims &dm, const Buffers &b, int cycle, int kR, int gated, hipStream_t s) {
  hipLaunchKernelGGL(k_sweep, dim3(unsigned(dm.max_cblk), unsigned(dm.H)), dim3(256), 0, s, b.desc, b.phi16, b.r,
                     b.sel_slot, cycle, kR, gated ? b.exact : nullptr, b.cand_val, b.cand_idx, b.head_status,
                     b.score_all);
  return hipGetLastError();
}

hipError_t launch_sweep_rc(const Dims &dm, const Buffers &b, int cycle, int kR, hipStream_t s) {
  dim3 grid(unsigned(dm.max_cblk), unsigned(dm.H));
#define AMC_RC_ARGS b.desc, b.Q, b.K, b.beta_in, dm.scale, b.shift, b.r, b.sel_slot, cycle, kR, b.cand_val, b.cand_idx, \
    b.head_status, b.score_all
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

// Blocks per head of the bounded sweep after the first cycle and of the
// 8-bit stage: each loops over its share of the head's list.
constexpr int SB_BLOCKS_Q8 = 4;   // the list after both pruning stages (about 1% of the keys)
constexpr int SB_BLOCKS = 16;     // the list after the first stage alone
constexpr int Q8_BLOCKS = 16;

hipError_t launch_sweep_band(const Dims &dm, const Buffers &b, int cycle, int kR, hipStream_t s) {
  const int64_t all = (dm.max_T + SB_KEYS - 1) / SB_KEYS;
  const int64_t bph = cycle == 0 ? all : std::min<int64_t>(all, b.q8 ? SB_BLOCKS_Q8 : SB_BLOCKS);
  const dim3 grid(unsigned(bph), unsigned(dm.H));
  const size_t lds = size_t((dm.max_n + 127) / 128 * 128) * 8;
#define AMC_SB_ARGS b.desc, b.phi16, b.rpn, b.rabs, b.surv_list, b.surv_cnt, b.sel_slot, cycle, kR, dm.qb128, b.colsum, \
    b.q8, b.q8_bad, b.sw_up, b.sw_lo, b.sw_key
  if (cycle == 0) hipLaunchKernelGGL(k_sweep_band<true>, grid, dim3(256), lds, s, AMC_SB_ARGS);
  else hipLaunchKernelGGL(k_sweep_band<false>, grid, dim3(256), lds, s, AMC_SB_ARGS);
#undef AMC_SB_ARGS
  return hipGetLastError();
}

hipError_t launch_prune(const Dims &dm, const Buffers &b, int cycle, int kR, hipStream_t s) {
  hipLaunchKernelGGL(k_prune, dim3(unsigned(dm.H)), dim3(PR_THREADS), 0, s, b.desc, b.r, b.sel_slot, b.phi16, b.colsum,
                     dm.qb128, cycle, kR, b.rpn, b.rabs, b.surv_list, b.surv_cnt, b.prune_L, b.tr_swept);
  return hipGetLastError();
}

hipError_t launch_sweep_q8(const Dims &dm, const Buffers &b, int cycle, int kR, hipStream_t s) {
  const dim3 grid(unsigned(std::min<int64_t>((dm.max_T + Q8_KEYS - 1) / Q8_KEYS, Q8_BLOCKS)), unsigned(dm.H));
  const size_t lds = size_t((dm.max_n + 127) / 128 * 128) * 8;
  hipLaunchKernelGGL(k_sweep_q8, grid, dim3(Q8_THREADS), lds, s, b.desc, b.q8, b.rpn, b.rabs, b.prune_L, b.q8_bad,
                     b.surv_list, b.surv_cnt, b.sel_slot, cycle, kR, b.sw_up, b.sw_key);
  return hipGetLastError();
}

hipError_t launch_q8_compact(const Dims &dm, const Buffers &b, int cycle, int kR, hipStream_t s) {
  hipLaunchKernelGGL(k_q8_compact, dim3(unsigned(dm.H)), dim3(1024), 0, s, b.desc, cycle, kR, b.prune_L, b.q8_bad,
                     b.surv_list, b.surv_cnt, b.sw_up, b.sw_key, b.surv2_list, b.surv2_cnt, b.tr_swept, b.tr_swept8);
  return hipGetLastError();
}

hipError_t launch_band_merge(const Dims &dm, const Buffers &b, int cycle, int kR, hipStream_t s) {
  hipLaunchKernelGGL(k_band_merge, dim3(unsigned(dm.H)), dim3(1024), 0, s, b.desc, cycle, kR, b.sw_up, b.sw_lo,
                     b.sw_key, b.surv_cnt, dm.band_cap, b.band_list, b.band_cnt, b.exact);
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
  dim3 grid(unsigned(dm.nrb), unsigned(dm.H));
  hipLaunchKernelGGL(k_resid, grid, dim3(256), 0, s, b.desc, b.panel, b.w, b.m, cycle, kR, polish, b.r, b.mhat,
                     b.rpart);
  return hipGetLastError();
}

}  // namespace amc
