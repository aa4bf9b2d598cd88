// Stage 1 kernels: the per-head logit shift, and the mass features
// Phi = exp(l - s), the target mass m = Phi 1 and the attention output
// Y = Phi V / m (zhichai.net deep-dive, section 1.6; xinfinite.net article,
// section 2, step 3).
//
// The fit side of the method (m, and later the Gram system and residual) is
// conditioned like cond(Phi_S^T Phi_S) ~ 1e9, so the logits that feed m are
// float64 dot products of the exact bf16/fp32 inputs: for bf16 rows, exact
// integer products on the int8 MFMA units (the rows written as base-256
// digits) joined in float64; otherwise v_mfma_f64_16x16x4f64.  Phi is
// rounded to float32 only for storage, where
// the memory-bound correlation sweeps read it.  Stored for the selection, each
// float32 value is split into its high and low 16 bits, kept in two planes:
// the high plane alone is Phi truncated to bfloat16 (what the bounded sweep
// reads), both together give the float32 value back exactly.  The shift only
// needs to keep exp() in range, so it comes from a cheap bf16 MFMA pass.
#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>

#include "amc_internal.h"

namespace amc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t u16) { return __uint_as_float(u16 << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// 8 consecutive elements of an input row as 8 bf16 bit patterns.
template <bool BF16>
__device__ __forceinline__ uint4 load8_bf16(const void *base, int64_t off) {
  if constexpr (BF16) {
    return *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(base) + off);
  } else {
    const float4 a = *reinterpret_cast<const float4 *>(static_cast<const float *>(base) + off);
    const float4 b = *reinterpret_cast<const float4 *>(static_cast<const float *>(base) + off + 4);
    uint4 r;
    r.x = f32_to_bf16_bits(a.x) | (f32_to_bf16_bits(a.y) << 16);
    r.y = f32_to_bf16_bits(a.z) | (f32_to_bf16_bits(a.w) << 16);
    r.z = f32_to_bf16_bits(b.x) | (f32_to_bf16_bits(b.y) << 16);
    r.w = f32_to_bf16_bits(b.z) | (f32_to_bf16_bits(b.w) << 16);
    return r;
  }
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

struct WordChunk {
  uint64_t w[384];
};

__global__ void k_put_words(uint64_t *dst, int count, WordChunk c) {
  const int i = threadIdx.x + blockIdx.x * blockDim.x;
  if (i < count) dst[i] = c.w[i];
}

__global__ void k_fill_i32(int32_t *p, int64_t count, int32_t v) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < count; i += int64_t(gridDim.x) * blockDim.x)
    p[i] = v;
}

// ---------------------------------------------------------------------------
// logit maximum: one partial per (head, 128 queries), bf16 MFMA 16x16x32.
// Blocks map to heads XCD by XCD when xcd_map is set (H a multiple of 8), so
// that the blocks of one head read its keys through one L2.
// ---------------------------------------------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(256) void k_shift(const HeadDesc *__restrict__ desc, int H, int nsb, int xcd_map,
                                               const void *__restrict__ Q, const void *__restrict__ K,
                                               const float *__restrict__ beta_in, float scale,
                                               float *__restrict__ shift_part) {
  constexpr int KC = D / 32;
  constexpr int KSTR = D + 8;  // bf16 elements per LDS row (16-byte pad)
  __shared__ __attribute__((aligned(16))) uint16_t ks[64 * KSTR];
  __shared__ float red[4];
  int h, blk;
  {
    const int b = blockIdx.x;
    if (xcd_map) {
      const int x = b & 7, slot = b >> 3;
      h = x + 8 * (slot / nsb);
      blk = slot % nsb;
    } else {
      h = b / nsb;
      blk = b % nsb;
    }
  }
  if (h >= H) return;
  const HeadDesc Dh = desc[h];
  if (blk >= Dh.n_sblk) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  const int64_t qb = int64_t(blk) * kShiftRows + wave * 32;

  uint4 qf[2][KC];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int64_t row = qb + rb * 16 + c16;
#pragma unroll
    for (int c = 0; c < KC; ++c)
      qf[rb][c] = row < Dh.n ? load8_bf16<BF16>(Q, (Dh.q_off + row) * D + 32 * c + 8 * g) : make_uint4(0, 0, 0, 0);
  }
  float mx = -INFINITY;
  // Without a bias and with a positive scale the largest logit is the scale
  // times the largest dot product (rounding is monotonic), so tiles whose rows
  // and keys all exist keep the raw maximum, one v_max per value.
  float mxr = -INFINITY;
  const bool raw_ok = beta_in == nullptr && scale > 0.0f && qb + 32 <= Dh.n;
  // the next 64-key tile is loaded into registers while the current one is
  // multiplied
  constexpr int PER = 64 * D / 8 / 256;  // 16-byte pieces of a tile per thread
  uint4 pre[PER];
  auto fetch = [&](int64_t k0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int gi = tid + 256 * u, key = gi / (D / 8), c8 = gi % (D / 8);
      pre[u] = (k0 + key < Dh.T) ? load8_bf16<BF16>(K, (Dh.k_off + k0 + key) * D + 8 * c8) : make_uint4(0, 0, 0, 0);
    }
  };
  fetch(0);
  for (int64_t k0 = 0; k0 < Dh.T; k0 += 64) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int gi = tid + 256 * u, key = gi / (D / 8), c8 = gi % (D / 8);
      *reinterpret_cast<uint4 *>(&ks[key * KSTR + 8 * c8]) = pre[u];
    }
    __syncthreads();
    if (k0 + 64 < Dh.T) fetch(k0 + 64);
    if (raw_ok && k0 + 64 <= Dh.T) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        uint4 kf[KC];
#pragma unroll
        for (int c = 0; c < KC; ++c) kf[c] = *reinterpret_cast<const uint4 *>(&ks[(kb * 16 + c16) * KSTR + 32 * c + 8 * g]);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < KC; ++c)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qf[rb][c]), as_bf16x8(kf[c]), acc, 0, 0, 0);
          mxr = fmaxf(mxr, fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3])));
        }
      }
      continue;
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      uint4 kf[KC];
#pragma unroll
      for (int c = 0; c < KC; ++c) kf[c] = *reinterpret_cast<const uint4 *>(&ks[(kb * 16 + c16) * KSTR + 32 * c + 8 * g]);
      const int64_t key = k0 + kb * 16 + c16;
      const float bias = (key < Dh.T && beta_in) ? beta_in[Dh.k_off + key] : 0.0f;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < KC; ++c)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qf[rb][c]), as_bf16x8(kf[c]), acc, 0, 0, 0);
        if (key < Dh.T) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int64_t q = qb + rb * 16 + 4 * g + e;
            if (q < Dh.n) mx = fmaxf(mx, fmaf(scale, acc[e], bias));
          }
        }
      }
    }
  }
  if (mxr != -INFINITY) mx = fmaxf(mx, scale * mxr);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  if (tid == 0) shift_part[Dh.sblk_off + blk] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// ---------------------------------------------------------------------------
// mass features: float64 MFMA logits (S^T = K Q^T), fused exp / row sum /
// Phi store and Phi V on MFMA.  One block = 64 queries, 4 waves of 16.
// STORE: 0 = Phi not stored, 1 = float32 rows [n][ldT] at phi + phi_off,
// 2 = the two 16-bit planes at phi16 + 2 phi_off (ldT a multiple of 8).
// ---------------------------------------------------------------------------
template <typename T>
struct In;
template <>
struct In<uint16_t> {
  __device__ static float f(uint16_t v) { return bf16_bits_to_f32(v); }
};
template <>
struct In<float> {
  __device__ static float f(float v) { return v; }
};

// v_mfma_f64_16x16x4f64 leaves output row i in lane group i % 4, element
// i / 4 (rows interleaved across the lane groups).  With S^T = K Q^T the rows
// are keys, so lane group g, element e of key block kb holds this key:
__device__ __forceinline__ int phi_key(int kb, int g, int e) { return kb * 16 + g + 4 * e; }
// The stored planes keep each 64-key tile in a lane-friendly order: key
// 16 kb + g + 4 e at position 32 (kb / 2) + 8 g + 4 (kb % 2) + e.  The 16
// values a lane holds for one query are then two runs of 8 positions, and the
// four lanes of a query write 64 contiguous bytes of a plane per store.
__device__ __forceinline__ int store_pos(int kb, int g, int e) { return 32 * (kb >> 1) + 8 * g + 4 * (kb & 1) + e; }
// Stored planes are key columns: the high and low 16 bits of the float32 Phi
// of key k and query q at k * ldN + q of the head's high and low plane.  A
// lane's 16 values of one tile (keys k0 + 16 kb + g + 4 e, query q) leave as
// 16-bit stores; the 16 lanes of one g write 32 contiguous bytes of a column.
// Queries from n to ldN get zeros (the caller passes x = 0 for them).
__device__ __forceinline__ void store_planes(uint16_t *hp, uint16_t *lp, int64_t ldN, int64_t k0, int g, int64_t q,
                                             const float (&x)[4][4]) {
  const uint32_t lane_off = uint32_t((int64_t(g) * ldN + q) * 2);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t col = (k0 + 16 * kb + 4 * e) * ldN;
      const uint32_t u = __float_as_uint(x[kb][e]);
      *reinterpret_cast<uint16_t *>(reinterpret_cast<char *>(hp + col) + lane_off) = uint16_t(u >> 16);
      *reinterpret_cast<uint16_t *>(reinterpret_cast<char *>(lp + col) + lane_off) = uint16_t(u & 0xffffu);
    }
}

// The Phi V product consumes those values as its A operand at k-step (kb, e)
// (A[query][k = g]); its B operand B[k = g][dim] is then V[phi_key(kb, g, e)][dim],
// a row of the V tile, read directly.

template <int D, bool BF16, int STORE>
__global__ __launch_bounds__(256) void k_phi(const HeadDesc *__restrict__ desc, const void *__restrict__ Qv,
                                             const void *__restrict__ Kv, const void *__restrict__ Vv,
                                             const float *__restrict__ beta_in, double scale,
                                             const float *__restrict__ shift_part, double *__restrict__ shift_out,
                                             double *__restrict__ tr_shift, float *__restrict__ phi,
                                             uint16_t *__restrict__ phi16,
                                             double *__restrict__ m_out, double *__restrict__ r_out,
                                             float *__restrict__ Y_out, int32_t *__restrict__ head_status) {
  using E = typename std::conditional<BF16, uint16_t, float>::type;
  constexpr int KSTR = D + 16 / int(sizeof(E));  // elements per K / V row in LDS (16-byte pad)
  constexpr int NU = D / 16;
  constexpr int VEC = 16 / int(sizeof(E));         // elements per 16-byte access
  __shared__ __attribute__((aligned(16))) E ks[64 * KSTR];
  __shared__ __attribute__((aligned(16))) E vs[64 * KSTR];
  constexpr int PSTR = 64 + 4;  // floats per staged Phi row
  __shared__ __attribute__((aligned(16))) float ps[4][16 * PSTR];  // per wave: 16 queries x 64 keys
  __shared__ float sbias[64];
  __shared__ double s_shift;
  const E *Q = static_cast<const E *>(Qv);
  const E *K = static_cast<const E *>(Kv);
  const E *V = static_cast<const E *>(Vv);

  const int h = blockIdx.y;
  const HeadDesc Dh = desc[h];
  const int blk = blockIdx.x;
  if (int64_t(blk) * kPhiRows >= Dh.n) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, g = lane >> 4;

  if (tid < 64) {
    float v = -INFINITY;
    for (int64_t i = tid; i < Dh.n_sblk; i += 64) v = fmaxf(v, shift_part[Dh.sblk_off + i]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    if (tid == 0) s_shift = double(v);
  }
  __syncthreads();
  const double s = s_shift;
  if (blk == 0 && tid == 0) {
    shift_out[h] = s;
    if (tr_shift) tr_shift[h] = s;
  }

  const int64_t q0 = int64_t(blk) * kPhiRows + wave * 16;
  const int64_t q = q0 + c16;  // this lane's query in the logit tile
  const bool qvalid = q < Dh.n;
  float qf[D / 4];
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v)
      qf[4 * u + v] = qvalid ? In<E>::f(Q[(Dh.q_off + q) * D + 16 * u + 4 * g + v]) : 0.0f;

  f32x4 uacc[NU];
#pragma unroll
  for (int i = 0; i < NU; ++i) uacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  double msum = 0.0;

  for (int64_t k0 = 0; k0 < Dh.T; k0 += kPhiKeys) {
    __syncthreads();
    // K and V tiles [64][D], zero beyond T, 16 bytes per access
    for (int gi = tid; gi < 64 * D / VEC; gi += 256) {
      const int key = gi / (D / VEC), cv = gi % (D / VEC);
      const bool ok = k0 + key < Dh.T;
      const int64_t src = (Dh.k_off + k0 + key) * D + VEC * cv;
      uint4 kq = make_uint4(0, 0, 0, 0), vq = make_uint4(0, 0, 0, 0);
      if (ok) {
        kq = *reinterpret_cast<const uint4 *>(K + src);
        vq = *reinterpret_cast<const uint4 *>(V + src);
      }
      *reinterpret_cast<uint4 *>(&ks[key * KSTR + VEC * cv]) = kq;
      *reinterpret_cast<uint4 *>(&vs[key * KSTR + VEC * cv]) = vq;
    }
    if (tid < 64) sbias[tid] = (k0 + tid < Dh.T && beta_in) ? beta_in[Dh.k_off + k0 + tid] : 0.0f;
    __syncthreads();

    float pf[4][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const E *kp = &ks[(kb * 16 + c16) * KSTR + 16 * u + 4 * g];
#pragma unroll
        for (int v = 0; v < 4; ++v)
          acc = __builtin_amdgcn_mfma_f64_16x16x4f64(double(In<E>::f(kp[v])), double(qf[4 * u + v]), acc, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kl = phi_key(kb, g, e);
        double p = 0.0;
        if (k0 + kl < Dh.T) p = exp(scale * acc[e] + double(sbias[kl]) - s);
        msum += p;
        pf[kb][e] = float(p);
        if constexpr (STORE == 1) ps[wave][c16 * PSTR + kl] = pf[kb][e];
        if constexpr (STORE == 2) ps[wave][c16 * PSTR + kl] = qvalid ? pf[kb][e] : 0.0f;
      }
    }
    if constexpr (STORE == 1) {
      // the wave's 16 x 64 Phi tile leaves as 16-byte row segments (ldT is a
      // multiple of 4, so a segment that starts below ldT ends within the row)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int row = (lane >> 4) + 4 * it, col = 4 * (lane & 15);
        const int64_t qr = q0 + row;
        if (qr < Dh.n && k0 + col < Dh.ldT) {
          const f32x4 v = *reinterpret_cast<const f32x4 *>(&ps[wave][row * PSTR + col]);
          __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(phi + Dh.phi_off + qr * Dh.ldT + k0 + col));
        }
      }
    } else if constexpr (STORE == 2) {
      // lane l takes key k0 + l: the wave's 16 queries of its column leave as
      // 32 contiguous bytes of each plane (ldN is a multiple of 64, so the
      // wave's 16 queries lie all below it or all above)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (q0 < Dh.ldN) {
        uint16_t *hp = phi16 + 2 * Dh.phi_off + (k0 + lane) * Dh.ldN + q0;
        uint16_t *lp = hp + Dh.ldT * Dh.ldN;
        uint32_t hw[8], lw[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t u0 = __float_as_uint(ps[wave][(2 * i) * PSTR + lane]);
          const uint32_t u1 = __float_as_uint(ps[wave][(2 * i + 1) * PSTR + lane]);
          hw[i] = (u0 >> 16) | (u1 & 0xffff0000u);
          lw[i] = (u0 & 0xffffu) | (u1 << 16);
        }
        *reinterpret_cast<u32x4 *>(hp) = u32x4{hw[0], hw[1], hw[2], hw[3]};
        *reinterpret_cast<u32x4 *>(hp + 8) = u32x4{hw[4], hw[5], hw[6], hw[7]};
        *reinterpret_cast<u32x4 *>(lp) = u32x4{lw[0], lw[1], lw[2], lw[3]};
        *reinterpret_cast<u32x4 *>(lp + 8) = u32x4{lw[4], lw[5], lw[6], lw[7]};
      }
    }
    if constexpr (BF16) {
      // U += Phi V on bf16 MFMA (16x16x32): Phi = hi + mid + lo exactly in
      // three bf16 terms (24 significant bits, float32's), V is exact bf16,
      // products are exact in float32 and accumulate in float32.  Reduction
      // index k = 8 g + 4 j + e of chunk c is key phi_key(2 c + j, g, e).
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        uint32_t w[3][4];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int e2 = 0; e2 < 2; ++e2) {
            uint32_t t[3][2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              const float x = pf[2 * c + j][2 * e2 + h2];
              const uint32_t hi = f32_to_bf16_bits(x);
              const float r1 = x - bf16_bits_to_f32(hi);
              const uint32_t mi = f32_to_bf16_bits(r1);
              const uint32_t lo = f32_to_bf16_bits(r1 - bf16_bits_to_f32(mi));
              t[0][h2] = hi;
              t[1][h2] = mi;
              t[2][h2] = lo;
            }
#pragma unroll
            for (int q = 0; q < 3; ++q) w[q][2 * j + e2] = t[q][0] | (t[q][1] << 16);
          }
#pragma unroll
        for (int db = 0; db < NU; ++db) {
          uint32_t bv[4];
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e2 = 0; e2 < 2; ++e2) {
              const uint32_t v0 = vs[phi_key(2 * c + j, g, 2 * e2) * KSTR + db * 16 + c16];
              const uint32_t v1 = vs[phi_key(2 * c + j, g, 2 * e2 + 1) * KSTR + db * 16 + c16];
              bv[2 * j + e2] = v0 | (v1 << 16);
            }
          const bf16x8 b = as_bf16x8(make_uint4(bv[0], bv[1], bv[2], bv[3]));
#pragma unroll
          for (int q = 2; q >= 0; --q)
            uacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(make_uint4(w[q][0], w[q][1], w[q][2], w[q][3])),
                                                               b, uacc[db], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int db = 0; db < NU; ++db) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            uacc[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                pf[kb][e], In<E>::f(vs[phi_key(kb, g, e) * KSTR + db * 16 + c16]), uacc[db], 0, 0, 0);
        }
      }
    }
  }

  // m for query q0 + c16: partial sums sit in the four lanes c16, c16+16, c16+32, c16+48
  msum += __shfl_xor(msum, 16);
  msum += __shfl_xor(msum, 32);
  bool bad = false;
  if (g == 0 && qvalid) {
    m_out[Dh.n_off + q] = msum;
    if (r_out) r_out[Dh.n_off + q] = msum;
    bad |= !isfinite(msum);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const double mq = __shfl(msum, 4 * g + e);
    const int64_t qy = q0 + 4 * g + e;
    if (qy < Dh.n) {
#pragma unroll
      for (int db = 0; db < NU; ++db) {
        const float y = float(double(uacc[db][e]) / mq);
        bad |= !isfinite(y);
        Y_out[(Dh.n_off + qy) * D + db * 16 + c16] = y;
      }
    }
  }
  if (bad && head_status) atomicOr(head_status + h, int32_t(AMC_HS_NONFINITE));
}

// ---------------------------------------------------------------------------
// value tiles for the bf16 mass-feature kernels: per head and 64-key tile, V
// transposed to [d][72] with the keys in the order the Phi V product reduces
// them: position 32 c + 8 g + 4 j + e holds key 32 c + 16 j + g + 4 e (keys
// past T are zero), positions 64..71 zero.  Each row is thus the nine 16-byte
// slots the kernels stage in LDS (eight and a pad that spreads the reads over
// the banks), and a tile reaches LDS as one contiguous copy.  One block = one
// tile.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k_vt(const HeadDesc *__restrict__ desc, const uint16_t *__restrict__ V,
                                            uint16_t *__restrict__ vt) {
  constexpr int VSTR = D + 8;  // bf16 per staged row (16-byte pad)
  __shared__ __attribute__((aligned(16))) uint16_t vs[64 * VSTR];
  const int h = blockIdx.y;
  const HeadDesc Dh = desc[h];
  const int tile = blockIdx.x;
  const int64_t k0 = int64_t(tile) * 64;
  if (k0 >= Dh.T) return;
  const int tid = threadIdx.x;
  for (int gi = tid; gi < 64 * D / 8; gi += 256) {
    const int key = gi / (D / 8), c = gi % (D / 8);
    u32x4 w = {0u, 0u, 0u, 0u};
    if (k0 + key < Dh.T) w = *reinterpret_cast<const u32x4 *>(V + (Dh.k_off + k0 + key) * D + 8 * c);
    *reinterpret_cast<u32x4 *>(&vs[key * VSTR + 8 * c]) = w;
  }
  __syncthreads();
  uint16_t *out = vt + Dh.vt_off + int64_t(tile) * D * 72;
  for (int gi = tid; gi < D * 9; gi += 256) {
    const int dim = gi / 9, c8 = gi % 9;
    if (c8 == 8) {
      *reinterpret_cast<u32x4 *>(out + dim * 72 + 64) = u32x4{0u, 0u, 0u, 0u};
      continue;
    }
    uint32_t w[4];
#pragma unroll
    for (int t2 = 0; t2 < 4; ++t2) {
      uint32_t pair[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int pos = 8 * c8 + 2 * t2 + h2;
        const int c = pos >> 5, g = (pos >> 3) & 3, j = (pos >> 2) & 1, e = pos & 3;
        pair[h2] = vs[(32 * c + 16 * j + g + 4 * e) * VSTR + dim];
      }
      w[t2] = pair[0] | (pair[1] << 16);
    }
    *reinterpret_cast<u32x4 *>(out + dim * 72 + 8 * c8) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// ---------------------------------------------------------------------------
// mass features for bf16 inputs, tiled for the MFMA pipes: one block = 128
// queries in 8 waves of 16 (two waves per SIMD).  The 64-key tiles of K and of
// the transposed V reach LDS by asynchronous global-to-LDS copies, double
// buffered: tile t + 1 is in flight while tile t computes.  Per tile and wave:
//   logits  S^T = K Q^T on v_mfma_f64_16x16x4f64 (keys as rows, four 16-key
//           blocks as four accumulation chains), head dims 32 a + 8 g + b at
//           k-step 8 a + b, so a lane's K operands for one a are one 16-byte
//           read (K rows padded by one 16-byte slot: conflict-free reads);
//   Phi     float64 exp, row sums for m, the two 16-bit planes written from
//           registers (each lane's 16 values are 16 consecutive positions);
//   Phi V   v_mfma_f32_16x16x32_bf16 with Phi = hi + mid + lo exactly (three
//           bf16 terms, split by truncation), V operands one 16-byte read.
// STORE: 0 = Phi not stored (every sweep recomputes it), 2 = stored planes.
// Blocks map to heads XCD by XCD when xcd_map is set (H a multiple of 8):
// the blocks of one head share one L2.  gate (nullable): only the heads with
// gate[h] != 0.
// ---------------------------------------------------------------------------
constexpr int P16_WAVES = kPhi16Rows / 16;

template <int D, int STORE>
__device__ __forceinline__ void phi16_block(
    int h, int qb, const HeadDesc *__restrict__ desc, const uint16_t *__restrict__ Q,
    const uint16_t *__restrict__ K, const uint16_t *__restrict__ vt, const float *__restrict__ beta_in,
    double scale, const float *__restrict__ shift_part, double *__restrict__ shift_out,
    double *__restrict__ tr_shift, uint16_t *__restrict__ phi16, double *__restrict__ m_out,
    double *__restrict__ r_out, float *__restrict__ Y_out, int32_t *__restrict__ head_status) {
  constexpr int KCH = D / 8;        // 16-byte chunks per K row
  constexpr int NS = D / 4;         // k-steps of the logit MFMA
  constexpr int NA = D / 32;        // 16-byte K reads per key block
  constexpr int NU = D / 16;        // 16-dim output blocks of Phi V
  constexpr int KROW = KCH + 1;         // 16-byte slots per K row in LDS (one of padding)
  constexpr int KSLOT = 64 * KROW;      // slots per K tile
  constexpr int VSLOT = D * 9;          // slots per V tile: D rows of 8 chunks and a pad
  constexpr int KWORDS = KSLOT * 4;     // uint32 per K tile
  constexpr int VWORDS = VSLOT * 4;     // uint32 per V tile
  // both K buffers in one array and both V buffers in another, so that every
  // operand read is one base register plus an immediate offset
  __shared__ __attribute__((aligned(16))) uint32_t lk_all[2 * KWORDS];
  __shared__ __attribute__((aligned(16))) uint32_t lv_all[2 * VWORDS];
  __shared__ __attribute__((aligned(16))) float sb[2][64];
  uint32_t *const lk0 = lk_all, *const lk1 = lk_all + KWORDS;
  uint32_t *const lv0 = lv_all, *const lv1 = lv_all + VWORDS;
  __shared__ double s_shift;

  const HeadDesc Dh = desc[h];
  const int64_t q0 = int64_t(qb) * kPhi16Rows;
  if (q0 >= Dh.n) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, g = lane >> 4;

  if (tid < 64) {
    float v = -INFINITY;
    for (int64_t i = tid; i < Dh.n_sblk; i += 64) v = fmaxf(v, shift_part[Dh.sblk_off + i]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    if (tid == 0) s_shift = double(v);
  }

  // B operand of the logits: query q, head dims 32 a + 8 g + b at k-step 8 a + b
  const int64_t qw = q0 + 16 * wave;
  const int64_t q = qw + c16;
  const bool qvalid = q < Dh.n;
  // (kept as bf16 pairs; each becomes a float64 operand where it is used)
  u32x4 qraw[NA];
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    qraw[a] = *reinterpret_cast<const u32x4 *>(Q + (Dh.q_off + (qvalid ? q : Dh.n - 1)) * D + 32 * a + 8 * g);
    if (!qvalid) qraw[a] = u32x4{0u, 0u, 0u, 0u};
  }

  const int64_t T = Dh.T;
  const int ntiles = int((T + 63) / 64);
  // Asynchronous copies of tile `tile` into one buffer set: each copy fills
  // 64 consecutive 16-byte slots (lane i the i-th); the copies are dealt to
  // the waves in turn.  K rows are KROW slots (chunk m of key k at slot
  // k KROW + m; the padding slot takes a duplicate of the row's first chunk),
  // V rows (dims) 9 slots, copied as they lie in the value tiles.  The
  // biases take one 4-byte copy (wave 0), slot i holding the key stored at
  // position i (store_pos), so that a lane's 16 biases are two runs of 8.
  // Sources are a per-head base plus a 32-bit byte offset.
  const char *kbase = reinterpret_cast<const char *>(K + Dh.k_off * D);
  const char *vbase = reinterpret_cast<const char *>(vt + Dh.vt_off);
  const char *bbase = beta_in ? reinterpret_cast<const char *>(beta_in + Dh.k_off) : nullptr;
  auto issue = [&](int tile, uint32_t *lk, uint32_t *lv, float *lb) {
    const int k0 = tile * 64;
#pragma unroll
    for (int inst = wave; inst < KSLOT / 64; inst += P16_WAVES) {
      const int slot = inst * 64 + lane;
      const int key = slot / KROW, m = slot % KROW;
      const int row = k0 + key < T ? k0 + key : int(T) - 1;
      const uint32_t off = uint32_t(row * D + 8 * (m < KCH ? m : 0)) * 2u;
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)(kbase + off),
                                       (void __attribute__((address_space(3))) *)(lk + inst * 256), 16, 0, 0);
    }
#pragma unroll
    for (int inst = wave; inst < VSLOT / 64; inst += P16_WAVES) {
      const uint32_t off = uint32_t(tile * (VSLOT * 16) + inst * 1024 + lane * 16);
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)(vbase + off),
                                       (void __attribute__((address_space(3))) *)(lv + inst * 256), 16, 0, 0);
    }
    if (bbase && wave == 0) {
      const int key = k0 + 16 * (2 * (lane >> 5) + ((lane >> 2) & 1)) + ((lane >> 3) & 3) + 4 * (lane & 3);
      const uint32_t off = uint32_t(key < T ? key : int(T) - 1) * 4u;
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)(bbase + off),
                                       (void __attribute__((address_space(3))) *)lb, 4, 0, 0);
    }
  };

  f32x4 uacc[NU];
#pragma unroll
  for (int i = 0; i < NU; ++i) uacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  double msum = 0.0;

  // One tile from the buffer set (lk, lv, lb).  The copies of the next tile
  // (into the other set) go out first; this wave waits for them once, after
  // its exps, and the barrier that closes the tile publishes them.
  auto compute = [&](int tile, const uint32_t *lk, const uint32_t *lv, const float *lb, bool next,
                     uint32_t *nk, uint32_t *nv, float *nb, double s) {
    const int64_t k0 = int64_t(tile) * 64;
    if (next) issue(tile + 1, nk, nv, nb);
    // this lane's first K slot and V slot; every operand below is a constant
    // number of slots past them
    const u32x4 *kl4 = reinterpret_cast<const u32x4 *>(lk) + (c16 * KROW + g);
    const u32x4 *vl4 = reinterpret_cast<const u32x4 *>(lv) + (c16 * 9 + g);
    f64x4 acc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) acc[kb] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int a = 0; a < NA; ++a) {
      u32x4 kw[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        kw[kb] = kl4[kb * 16 * KROW + 4 * a];
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const uint32_t qw2 = qraw[a][b >> 1];
        const double qv = double(__uint_as_float((b & 1) ? (qw2 & 0xffff0000u) : (qw2 << 16)));
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const uint32_t wd = kw[kb][b >> 1];
          const double kv = double(__uint_as_float((b & 1) ? (wd & 0xffff0000u) : (wd << 16)));
          acc[kb] = __builtin_amdgcn_mfma_f64_16x16x4f64(kv, qv, acc[kb], 0, 0, 0);
        }
      }
    }
    f32x4 bz[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      bz[kb] = bbase ? *reinterpret_cast<const f32x4 *>(lb + store_pos(kb, g, 0)) : f32x4{0.f, 0.f, 0.f, 0.f};
    // Phi for keys 16 kb + g + 4 e and query q; x = float32 Phi
    float x[4][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kl = phi_key(kb, g, e);
        double p = 0.0;
        if (k0 + kl < T) p = exp(scale * acc[kb][e] + double(bz[kb][e]) - s);
        msum += p;
        x[kb][e] = float(p);
      }
    // the next tile's copies have landed
    __builtin_amdgcn_s_waitcnt(0);
    if constexpr (STORE == 2) {
      if (q < Dh.ldN) {
        uint16_t *hp = phi16 + 2 * Dh.phi_off;
        float xs[4][4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e) xs[kb][e] = qvalid ? x[kb][e] : 0.0f;
        store_planes(hp, hp + Dh.ldT * Dh.ldN, Dh.ldN, k0, g, q, xs);
      }
    }
    // Phi V: reduction index k = 8 g + 4 j + e of chunk c is key phi_key(2 c + j, g, e)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      uint32_t w[3][4];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
          uint32_t t[3][2];
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const float v = x[2 * c + j][2 * e2 + h2];
            const float hi = __uint_as_float(__float_as_uint(v) & 0xffff0000u);
            const float r1 = v - hi;
            const float mi = __uint_as_float(__float_as_uint(r1) & 0xffff0000u);
            const float lo = r1 - mi;
            t[0][h2] = __float_as_uint(hi);
            t[1][h2] = __float_as_uint(mi);
            t[2][h2] = __float_as_uint(lo);
          }
#pragma unroll
          for (int qq = 0; qq < 3; ++qq) w[qq][2 * j + e2] = (t[qq][0] >> 16) | (t[qq][1] & 0xffff0000u);
        }
#pragma unroll
      for (int db = 0; db < NU; ++db) {
        const u32x4 vv = vl4[db * 16 * 9 + 4 * c];
        const bf16x8 bv = __builtin_bit_cast(bf16x8, vv);
#pragma unroll
        for (int qq = 2; qq >= 0; --qq)
          uacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, u32x4{w[qq][0], w[qq][1], w[qq][2], w[qq][3]}), bv, uacc[db], 0, 0, 0);
      }
    }
  };

  // prologue: tile 0 into buffer set 0
  issue(0, lk0, lv0, sb[0]);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const double s = s_shift;
  if (qb == 0 && tid == 0) {
    shift_out[h] = s;
    if (tr_shift) tr_shift[h] = s;
  }
  for (int tile = 0; tile < ntiles; tile += 2) {
    // even tiles from buffer set 0, odd tiles from set 1
    compute(tile, lk0, lv0, sb[0], tile + 1 < ntiles, lk1, lv1, sb[1], s);
    __syncthreads();
    if (tile + 1 >= ntiles) break;
    compute(tile + 1, lk1, lv1, sb[1], tile + 2 < ntiles, lk0, lv0, sb[0], s);
    __syncthreads();
  }

  // m for query q: partial sums sit in the four lanes c16, c16+16, c16+32, c16+48
  msum += __shfl_xor(msum, 16);
  msum += __shfl_xor(msum, 32);
  bool bad = false;
  if (g == 0 && qvalid) {
    m_out[Dh.n_off + q] = msum;
    if (r_out) r_out[Dh.n_off + q] = msum;
    bad |= !isfinite(msum);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const double mq = __shfl(msum, 4 * g + e);
    const int64_t qy = qw + 4 * g + e;
    if (qy < Dh.n) {
#pragma unroll
      for (int db = 0; db < NU; ++db) {
        const float y = float(double(uacc[db][e]) / mq);
        bad |= !isfinite(y);
        Y_out[(Dh.n_off + qy) * D + db * 16 + c16] = y;
      }
    }
  }
  if (bad && head_status) atomicOr(head_status + h, int32_t(AMC_HS_NONFINITE));
}

// One launch of the float64 kernel: with `list` null, block b takes head and
// query block from b (XCD by XCD when xcd_map is set); else the blocks walk
// the (head, query block) pairs of the *list_cnt heads in `list` (the heads
// the int8 kernel leaves to it), so that the launch costs next to nothing
// when the list is empty.
template <int D, int STORE>
__global__ __launch_bounds__(kPhi16Rows * 4) void k_phi16(
    const HeadDesc *__restrict__ desc, int H, int nqb, int xcd_map, const uint16_t *__restrict__ Q,
    const uint16_t *__restrict__ K, const uint16_t *__restrict__ vt, const float *__restrict__ beta_in,
    double scale, const float *__restrict__ shift_part, double *__restrict__ shift_out,
    double *__restrict__ tr_shift, uint16_t *__restrict__ phi16, double *__restrict__ m_out,
    double *__restrict__ r_out, float *__restrict__ Y_out, int32_t *__restrict__ head_status,
    const int32_t *__restrict__ list, const int32_t *__restrict__ list_cnt) {
#define AMC_P16_BODY desc, Q, K, vt, beta_in, scale, shift_part, shift_out, tr_shift, phi16, m_out, r_out, Y_out, head_status
  if (list) {
    const int items = *list_cnt * nqb;
    for (int it = blockIdx.x; it < items; it += gridDim.x) {
      phi16_block<D, STORE>(list[it / nqb], it % nqb, AMC_P16_BODY);
      __syncthreads();
    }
    return;
  }
  const int b = blockIdx.x;
  int h, qb;
  if (xcd_map) {
    const int x = b & 7, slot = b >> 3;
    h = x + 8 * (slot / nqb);
    qb = slot % nqb;
  } else {
    h = b / nqb;
    qb = b % nqb;
  }
  if (h >= H) return;
  phi16_block<D, STORE>(h, qb, AMC_P16_BODY);
#undef AMC_P16_BODY
}

// The heads with flag[h] != 0, in order, and their number (one block).
__global__ __launch_bounds__(256) void k_list_flags(const int32_t *__restrict__ flag, int H, int32_t *__restrict__ list,
                                                    int32_t *__restrict__ cnt) {
  __shared__ int s_wc[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int total = 0;
  for (int h0 = 0; h0 < H; h0 += 256) {
    const bool take = h0 + tid < H && flag[h0 + tid] != 0;
    const uint64_t m = __ballot(take);
    if (lane == 0) s_wc[wave] = __popcll(m);
    __syncthreads();
    int at = total;
    for (int w = 0; w < wave; ++w) at += s_wc[w];
    at += __popcll(m & ((uint64_t(1) << lane) - 1));
    if (take) list[at] = h0 + tid;
    total += s_wc[0] + s_wc[1] + s_wc[2] + s_wc[3];
    __syncthreads();
  }
  if (tid == 0) *cnt = total;
}

constexpr int kDigits = 5;
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef double f64x2 __attribute__((ext_vector_type(2)));

// 2^(j/64) for j = 0..63, each rounded to the nearest float64.
__constant__ double kExp2Tab64[64] = {
    1.0, 1.0108892860517005, 1.0218971486541166, 1.0330248790212284,
    1.0442737824274138, 1.0556451783605572, 1.0671404006768237, 1.0787607977571199,
    1.0905077326652577, 1.102382583307841, 1.1143867425958924, 1.1265216186082418,
    1.1387886347566916, 1.1511892299529827, 1.1637248587775775, 1.1763969916502812,
    1.189207115002721, 1.202156731452703, 1.215247359980469, 1.22848053610687,
    1.241857812073484, 1.255380757024691, 1.2690509571917332, 1.2828700160787783,
    1.2968395546510096, 1.3109612115247644, 1.3252366431597413, 1.339667524053303,
    1.3542555469368927, 1.3690024229745905, 1.383909881963832, 1.3989796725383112,
    1.4142135623730951, 1.42961333839197, 1.4451808069770467, 1.460917794180647,
    1.4768261459394993, 1.4929077282912648, 1.5091644275934228, 1.5255981507445384,
    1.5422108254079407, 1.559004400237837, 1.5759808451078865, 1.593142151342267,
    1.6104903319492543, 1.6280274218573478, 1.645755478153965, 1.6636765803267364,
    1.681792830507429, 1.7001063537185235, 1.718619298122478, 1.7373338352737062,
    1.7562521603732995, 1.7753764925265212, 1.7947090750031072, 1.8142521755003989,
    1.8340080864093424, 1.8539791250833855, 1.8741676341103, 1.8945759815869656,
    1.9152065613971474, 1.9360617934922943, 1.9571441241754002, 1.978456026387951};

// exp(x) in float64 after the table-driven reduction of P. T. P. Tang (ACM
// TOMS 15(2), 1989) with 64 table entries: x = (64 m + j) ln2/64 + r with
// |r| <= ln2/128, exp(x) = 2^m 2^(j/64) exp(r), and exp(r) from its Taylor
// polynomial of degree 4 (truncation below 4e-14 relative).  N = 64 m + j is
// rounded by one fused multiply-add with 1.5 2^52, whose low word then holds
// N; ln2/64 enters in one part, which moves r by at most |N| 2^-60 (below
// 4e-15 for x >= -40).  x is first raised to -746, so -inf and anything below
// give 0; a NaN x would give 0 too, so callers never pass one (heads whose
// bias is NaN or +inf take the float64 kernel).
// tab: the 64 values of kExp2Tab64.
__device__ __forceinline__ double exp_t64(double x, const double *tab) {
  x = __builtin_fmax(x, -746.0);
  const double kd = __builtin_fma(x, 92.33248261689366, 6755399441055744.0);  // 64/ln2, 1.5 2^52
  const int k = int(uint32_t(__builtin_bit_cast(uint64_t, kd)));
  const double N = kd - 6755399441055744.0;
  const double r = __builtin_fma(N, -0.010830424696249145, x);  // ln2/64
  double q = __builtin_fma(r, 1.0 / 24.0, 1.0 / 6.0);
  q = __builtin_fma(q, r, 0.5);
  q = __builtin_fma(q, r, 1.0);
  const double t = tab[k & 63];
  return __builtin_amdgcn_ldexp(__builtin_fma(t * r, q, t), k >> 6);
}

// ---------------------------------------------------------------------------
// Exact integer form of bf16 rows for the int8 logit kernel.  Per row of Q or
// K, E is the largest binary exponent of its nonzero entries; each entry x
// becomes the integer N = x 2^(37 - E) (|N| < 2^38), stored as five balanced
// base-256 digits d_0..d_4 in [-128, 127] with N = sum_s d_s 256^s.  x lies on
// this grid when its last significand bit is worth at least 2^(E - 37): for a
// normal bf16, when its exponent is at least E - 30.  A head with an entry
// off the grid, a non-finite entry, or a bias - shift that is NaN or +inf
// gets f64_heads[h] = 1 and takes the float64 logit kernel.
// Layouts: a Q row r: digit s of dims 8 j .. 8 j + 7 at qdig[5 D r + D s + 8 j],
// 4 E + z at qexp[r] (rows numbered as in Q), z the row's low digits that are
// zero in all its entries, counted up to 2.  K rows run over the head's keys
// padded to whole 64-key tiles (rows past T all zero), 5 D + 16 bytes each
// (the five digit rows, then 16 bytes that only keep the rows of a tile
// spread over the LDS banks once staged), from row kt_off.  Per tile, 1 KiB
// of ktab: the float64 bias - shift of each key (-inf past T), then its int32
// E, both in stored-key order (position store_pos of the key), then at byte
// 768 z of each 16-key block (its smallest row z).  One block = 256 / (D / 8)
// rows, a head's n query rows first (to a whole block), then its padded key
// rows.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k_digits(const HeadDesc *__restrict__ desc, const uint16_t *__restrict__ Q,
                                                const uint16_t *__restrict__ K, const float *__restrict__ beta_in,
                                                const float *__restrict__ shift_part, int8_t *__restrict__ qdig,
                                                int32_t *__restrict__ qexp, int8_t *__restrict__ kdig,
                                                uint8_t *__restrict__ ktab, int32_t *__restrict__ f64_heads) {
  constexpr int TPR = D / 8;      // threads per row, 8 entries each
  constexpr int RPB = 256 / TPR;  // rows per block
  constexpr int KROWB = kDigits * D + 16;
  __shared__ float s_shift;
  __shared__ int s_zmin[2];
  const int h = blockIdx.y;
  const HeadDesc Dh = desc[h];
  const int tid = threadIdx.x, j = tid % TPR;
  const int64_t Tp = (Dh.T + 63) / 64 * 64;
  const int64_t nR = (Dh.n + RPB - 1) / RPB * RPB;  // key rows start on a block boundary
  const int64_t r0 = int64_t(blockIdx.x) * RPB;
  if (r0 >= nR + Tp) return;
  const bool kblock = r0 >= nR;
  if (kblock) {  // the block holds key rows: the head's shift
    if (tid < 2) s_zmin[tid] = 2;
    if (tid < 64) {
      float v = -INFINITY;
      for (int64_t i = tid; i < Dh.n_sblk; i += 64) v = fmaxf(v, shift_part[Dh.sblk_off + i]);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
      if (tid == 0) s_shift = v;
    }
    __syncthreads();
  }
  const int64_t r = r0 + tid / TPR;
  const bool isq = !kblock;
  const bool active = isq ? r < Dh.n : r < nR + Tp;
  const int64_t key = r - nR;
  const bool live = active && (isq || key < Dh.T);  // a row with data (not tile padding)
  u32x4 w = {0u, 0u, 0u, 0u};
  if (live) w = *reinterpret_cast<const u32x4 *>((isq ? Q + (Dh.q_off + r) * D : K + (Dh.k_off + key) * D) + 8 * j);
  // x = M 2^P with M a signed integer (0 for zero)
  int32_t M[8], P[8];
  int emax = -100000, pmin = 100000;
  int bad = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t b = (w[i >> 1] >> (16 * (i & 1))) & 0xffffu;
    const uint32_t ef = (b >> 7) & 0xffu, mt = b & 0x7fu;
    int m = 0, p = 0;
    if (ef == 0xffu) {
      bad = 1;
    } else if (ef == 0u) {
      m = int(mt);  // zero or subnormal: mt 2^-133
      p = -133;
    } else {
      m = int(mt | 0x80u);  // (128 + mt) 2^(ef - 134)
      p = int(ef) - 134;
    }
    if (m != 0) {
      emax = max(emax, p + 31 - __clz(m));
      pmin = min(pmin, p);
    }
    M[i] = (b & 0x8000u) ? -m : m;
    P[i] = p;
  }
#pragma unroll
  for (int off = TPR / 2; off >= 1; off >>= 1) {
    emax = max(emax, __shfl_xor(emax, off));
    pmin = min(pmin, __shfl_xor(pmin, off));
    bad |= __shfl_xor(bad, off);
  }
  const int E = emax == -100000 ? 0 : emax;
  if (pmin < E - 37) bad = 1;
  // low digits that are zero in every entry of the row (N a multiple of
  // 2^(pmin + 37 - E)), counted up to 2
  const int z = pmin == 100000 ? 2 : min(2, (pmin + 37 - E) >> 3);
  uint32_t dg[kDigits][2];
#pragma unroll
  for (int sd = 0; sd < kDigits; ++sd) dg[sd][0] = dg[sd][1] = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int64_t N = (bad || M[i] == 0) ? 0 : int64_t(M[i]) * (int64_t(1) << (P[i] + 37 - E));
#pragma unroll
    for (int sd = 0; sd < kDigits; ++sd) {
      const int32_t dd = int32_t(int8_t(uint8_t(uint64_t(N) & 0xffu)));
      N = (N - dd) >> 8;
      dg[sd][i >> 2] |= (uint32_t(dd) & 0xffu) << (8 * (i & 3));
    }
  }
  if (active) {
    int8_t *out = isq ? qdig + (Dh.q_off + r) * (kDigits * D) : kdig + (Dh.kt_off + key) * KROWB;
#pragma unroll
    for (int sd = 0; sd < kDigits; ++sd) *reinterpret_cast<u32x2 *>(out + sd * D + 8 * j) = u32x2{dg[sd][0], dg[sd][1]};
    if (j == 0) {
      if (isq) {
        qexp[Dh.q_off + r] = E * 4 + z;
      } else {
        const int kk = int(key & 63);
        const int pos = store_pos(kk >> 4, kk & 3, (kk >> 2) & 3);
        uint8_t *tb = ktab + ((Dh.kt_off + key) >> 6) * 1024;
        double bms = -INFINITY;
        if (key < Dh.T) {
          bms = (beta_in ? double(beta_in[Dh.k_off + key]) : 0.0) - double(s_shift);
          // a NaN or +inf bias (or shift) is the float64 kernel's to report
          if (!(bms < INFINITY)) bad = 1;
        }
        reinterpret_cast<double *>(tb)[pos] = bms;
        reinterpret_cast<int32_t *>(tb + 512)[pos] = E;
        atomicMin(&s_zmin[(tid / TPR) >> 4], z);
      }
      if (bad) atomicOr(f64_heads + h, 1);
    }
  }
  if (kblock) {
    // per 16-key block: the low digits zero in all its keys
    __syncthreads();
    if (tid < RPB / 16) {
      const int64_t k16 = r0 - nR + 16 * tid;
      if (k16 < Tp)
        reinterpret_cast<int32_t *>(ktab + ((Dh.kt_off + k16) >> 6) * 1024 + 768)[(k16 & 63) >> 4] = s_zmin[tid];
    }
  }
}

// ---------------------------------------------------------------------------
// Mass features for bf16 inputs with the logits on the int8 matrix units:
// blocks, Phi planes and Phi V as in k_phi16.  With the rows in digit form
// (k_digits), the logit of query q and key k is
//   2^(E_q + E_k - 74) sum_c C_c 256^c,  C_c = sum over digit pairs s + t = c
//   of the int32 dot products of Q digit s and K digit t,
// each product on v_mfma_i32_16x16x64_i8 (exact: |C_c| < 2^24).
//
// Joining the classes.  Digits 0..3 are at most 128 in size and digit 4 at
// most 64, so with Q digits from 1 up (a wave's zq >= 1) the pairs
//   P1 = C_3 + 256 C_4,  P2 = C_5 + 256 C_6,  P3 = C_7 + 256 C_8
// stay below 2^31 (the largest, P1 with zq = 1, below 1.9e9), and the logit
// in units of class 3 is P1 + 2^16 P2 + 2^32 P3 (+ C_2 / 256 when zq = 1):
// three or four int32 -> float64 conversions and fused multiply-adds, the
// first exact and the last rounded once, as the float64 MFMA gives the dot
// product to within a few roundings.  Waves with zq = 0 (an entry more than
// 22 binades below its row's largest) join the classes one by one.  K digit
// 0 is zero in almost every 16-key block (zk >= 1); a block with zk = 0 takes
// its digit-0 products in a branch, which folds the lowest class (below the
// join's) into the key's bias term.  The power of two, the logit scale, the
// bias and the shift enter in one fused multiply-add.
//
// Schedule.  Per 64-key tile three contiguous asynchronous copies stage the K
// digit rows (KROW slots per key), the value tile and the key table (bias -
// shift, -inf past T, so padding keys give 0 with no test; row exponents; zk
// per block).  MFMA row 4 g + e is fed key g + 4 e of its 16-key block, so the
// outputs land where the float64 kernel has them.  The four 16-key blocks run
// as a two-stage pipeline: the class products of block kb on the matrix units
// next to the join and exp of block kb - 1 on the vector units (two class
// accumulator sets), then Phi V of keys 0..31 next to block 3, and of keys
// 32..63 last.  Heads with f64_heads[h] != 0 return at once (the float64
// kernel takes them).
// ---------------------------------------------------------------------------
template <int D, int STORE>
__global__ __launch_bounds__(kPhi16Rows * 4) void k_phi8(
    const HeadDesc *__restrict__ desc, int H, int nqb, int xcd_map, const int8_t *__restrict__ qdig,
    const int32_t *__restrict__ qexp, const int8_t *__restrict__ kdig, const uint8_t *__restrict__ ktab,
    const int32_t *__restrict__ f64_heads, const uint16_t *__restrict__ vt, double scale,
    const float *__restrict__ shift_part, double *__restrict__ shift_out, double *__restrict__ tr_shift,
    uint16_t *__restrict__ phi16, double *__restrict__ m_out, double *__restrict__ r_out, float *__restrict__ Y_out,
    int32_t *__restrict__ head_status) {
  constexpr int NCH = D / 64;             // 64-dim k-steps of the int8 MFMA
  constexpr int DSL = kDigits * D / 16;   // 16-byte slots of one key's digits
  constexpr int KROW = DSL + 1;           // slots per key row (one of padding)
  constexpr int KSLOT = 64 * KROW;        // slots per K tile
  constexpr int VSLOT = D * 9;            // slots per V tile
  constexpr int NU = D / 16;              // 16-dim output blocks of Phi V
  constexpr int KWORDS = KSLOT * 4;
  constexpr int VWORDS = VSLOT * 4;
  constexpr int NC = 2 * kDigits - 1;     // digit-pair classes s + t
  static_assert(KSLOT % 64 == 0 && VSLOT % 64 == 0, "whole copies");
  __shared__ __attribute__((aligned(16))) uint32_t lk_all[2 * KWORDS];
  __shared__ __attribute__((aligned(16))) uint32_t lv_all[2 * VWORDS];
  __shared__ __attribute__((aligned(16))) uint32_t lt_all[2 * 256];  // key tables
  __shared__ double s_tab[64];
  // STORE == 2: each wave's Phi of a tile, [64 keys][16 queries], turned into
  // key rows for 16-byte stores of the two planes
  __shared__ __attribute__((aligned(16))) uint32_t lx_all[STORE == 2 ? P16_WAVES * 1024 : 1];
  uint32_t *const lk0 = lk_all, *const lk1 = lk_all + KWORDS;
  uint32_t *const lv0 = lv_all, *const lv1 = lv_all + VWORDS;
  uint32_t *const lt0 = lt_all, *const lt1 = lt_all + 256;
  __shared__ double s_shift;

  int h, qb;
  {
    const int b = blockIdx.x;
    if (xcd_map) {
      const int x = b & 7, slot = b >> 3;
      h = x + 8 * (slot / nqb);
      qb = slot % nqb;
    } else {
      h = b / nqb;
      qb = b % nqb;
    }
  }
  if (h >= H) return;
  if (f64_heads[h] != 0) return;
  const HeadDesc Dh = desc[h];
  const int64_t q0 = int64_t(qb) * kPhi16Rows;
  if (q0 >= Dh.n) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, g = lane >> 4;

  if (tid < 64) {
    float v = -INFINITY;
    for (int64_t i = tid; i < Dh.n_sblk; i += 64) v = fmaxf(v, shift_part[Dh.sblk_off + i]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    if (tid == 0) s_shift = double(v);
  } else if (tid < 128) {
    s_tab[tid - 64] = kExp2Tab64[tid - 64];
  }

  // B operand: query q, digit s, dims 64 c + 16 g + (0..15) at k-step c
  const int64_t qw = q0 + 16 * wave;
  const int64_t q = qw + c16;
  const bool qvalid = q < Dh.n;
  const bool wfull = qw + 16 <= Dh.n;  // no padding query in the wave
  const int64_t qrow = Dh.q_off + (qvalid ? q : Dh.n - 1);
  const int8_t *qsrc = qdig + qrow * (kDigits * D) + 16 * g;
  // scale of class 3: 2^(E_q - 74 + 24), times 2^(E_k) per key, an exact
  // power-of-two rescaling
  const int qx = qexp[qrow];
  const double qs3 = ldexp(scale, (qx >> 2) - 50);
  // low Q digits zero in all 16 queries of the wave (0, 1 or 2: most waves
  // have every entry within 14 binades of its row's largest, two)
  int zq = qvalid ? (qx & 3) : 2;
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) zq = min(zq, __shfl_xor(zq, off));
  zq = __builtin_amdgcn_readfirstlane(zq);

  const int ntiles = int((Dh.T + 63) / 64);
  // Copies of tile `tile`: K digit rows, value tile and key table, each lying
  // contiguously in global memory as it lies in LDS; copy i of a kind moves
  // bytes 1024 i .. 1024 i + 1023 (lane l the 16 at 16 l), dealt to the waves
  // in turn.
  const char *kbase = reinterpret_cast<const char *>(kdig + Dh.kt_off * (kDigits * D + 16));
  const char *vbase = reinterpret_cast<const char *>(vt + Dh.vt_off);
  const char *tbase = reinterpret_cast<const char *>(ktab + (Dh.kt_off >> 6) * 1024);
  auto issue = [&](int tile, uint32_t *lk, uint32_t *lv, uint32_t *lt) __attribute__((always_inline)) {
#pragma unroll
    for (int inst = wave; inst < KSLOT / 64; inst += P16_WAVES) {
      const uint32_t off = uint32_t(tile * (KSLOT * 16) + inst * 1024 + lane * 16);
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)(kbase + off),
                                       (void __attribute__((address_space(3))) *)(lk + inst * 256), 16, 0, 0);
    }
#pragma unroll
    for (int inst = wave; inst < VSLOT / 64; inst += P16_WAVES) {
      const uint32_t off = uint32_t(tile * (VSLOT * 16) + inst * 1024 + lane * 16);
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)(vbase + off),
                                       (void __attribute__((address_space(3))) *)(lv + inst * 256), 16, 0, 0);
    }
    if (wave == P16_WAVES - 1) {
      const uint32_t off = uint32_t(tile * 1024 + lane * 16);
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)(tbase + off),
                                       (void __attribute__((address_space(3))) *)lt, 16, 0, 0);
    }
  };

  f32x4 uacc[NU];
#pragma unroll
  for (int i = 0; i < NU; ++i) uacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  double msum = 0.0;
  // MFMA row c16 of a 16-key block is fed key (c16 >> 2) + 4 (c16 & 3)
  const int krow = (c16 >> 2) + 4 * (c16 & 3);

  // Phi V of the 32 keys 32 c .. 32 c + 31 (blocks 2 c and 2 c + 1): each
  // float32 Phi as three bf16 parts (high, middle, low: exact), all three
  // against the bf16 values
  auto phiv = [&](const float (&x)[4][4], const u32x4 *vl4, int c) __attribute__((always_inline)) {
    uint32_t w[3][4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) {
        uint32_t t[3][2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const float v = x[2 * c + j][2 * e2 + h2];
          const float hi = __uint_as_float(__float_as_uint(v) & 0xffff0000u);
          const float r1 = v - hi;
          const float mi = __uint_as_float(__float_as_uint(r1) & 0xffff0000u);
          const float lo = r1 - mi;
          t[0][h2] = __float_as_uint(v);
          t[1][h2] = __float_as_uint(r1);
          t[2][h2] = __float_as_uint(lo);
        }
        // the high halves of v, r1 and lo are the three parts
#pragma unroll
        for (int qq = 0; qq < 3; ++qq) w[qq][2 * j + e2] = __builtin_amdgcn_perm(t[qq][1], t[qq][0], 0x07060302u);
      }
#pragma unroll
    for (int db = 0; db < NU; ++db) {
      const u32x4 vv = vl4[db * 16 * 9 + 4 * c];
      const bf16x8 bv = __builtin_bit_cast(bf16x8, vv);
#pragma unroll
      for (int qq = 2; qq >= 0; --qq)
        uacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, u32x4{w[qq][0], w[qq][1], w[qq][2], w[qq][3]}), bv, uacc[db], 0, 0, 0);
    }
  };

  // ZQ: Q digits below ZQ are zero for the whole wave and skipped.
  auto compute = [&](auto zq_c, const u32x4 (&qd)[kDigits][NCH], int tile, const uint32_t *lk, const uint32_t *lv,
                     const uint32_t *lt, bool next, uint32_t *nk, uint32_t *nv, uint32_t *nt)
      __attribute__((always_inline)) {
    constexpr int ZQ = decltype(zq_c)::value;
    const int64_t k0 = int64_t(tile) * 64;
    if (next) issue(tile + 1, nk, nv, nt);
    const u32x4 *kl4 = reinterpret_cast<const u32x4 *>(lk) + (krow * KROW + g);
    const u32x4 *vl4 = reinterpret_cast<const u32x4 *>(lv) + (c16 * 9 + g);
    const double *tbm = reinterpret_cast<const double *>(lt);
    const int32_t *tke = reinterpret_cast<const int32_t *>(lt) + 128;
    const i32x4 zk4 = *reinterpret_cast<const i32x4 *>(reinterpret_cast<const int32_t *>(lt) + 192);
    float x[4][4];
    i32x4 acc[2][NC];
    double bms[2][4];
    int32_t kex[2][4];
#pragma unroll
    for (int kb = 0; kb <= 4; ++kb) {
      const int cur = kb & 1, prv = cur ^ 1;
      if (kb < 4) {
        const int pos = store_pos(kb, g, 0);
        const f64x2 bm0 = *reinterpret_cast<const f64x2 *>(tbm + pos);
        const f64x2 bm1 = *reinterpret_cast<const f64x2 *>(tbm + pos + 2);
        const i32x4 ke = *reinterpret_cast<const i32x4 *>(tke + pos);
        bms[cur][0] = bm0[0];
        bms[cur][1] = bm0[1];
        bms[cur][2] = bm1[0];
        bms[cur][3] = bm1[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) kex[cur][e] = ke[e];
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[cur][c] = i32x4{0, 0, 0, 0};
        // class products of K digits 1..4
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
#pragma unroll
          for (int t = 1; t < kDigits; ++t) {
            const u32x4 kd = kl4[kb * 16 * KROW + t * (D / 16) + 4 * c];
#pragma unroll
            for (int sd = ZQ; sd < kDigits; ++sd)
              acc[cur][sd + t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, kd),
                                                                      __builtin_bit_cast(i32x4, qd[sd][c]),
                                                                      acc[cur][sd + t], 0, 0, 0);
          }
        }
      }
      if (kb > 0) {
        // join and exp of block kb - 1
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          double v;
          if constexpr (ZQ >= 1) {
            const int32_t p1 = acc[prv][3][e] + (acc[prv][4][e] << 8);
            const int32_t p2 = acc[prv][5][e] + (acc[prv][6][e] << 8);
            const int32_t p3 = acc[prv][7][e] + (acc[prv][8][e] << 8);
            v = fma(double(p2), 65536.0, double(p1));
            v = fma(double(p3), 4294967296.0, v);
            if constexpr (ZQ == 1) v = fma(double(acc[prv][2][e]), 0.00390625, v);
          } else {
            v = double(acc[prv][1][e]) * 1.52587890625e-05;  // 2^-16
            double w = 0.00390625;
#pragma unroll
            for (int c = 2; c < NC; ++c) {
              v = fma(double(acc[prv][c][e]), w, v);
              w *= 256.0;
            }
          }
          const double p = exp_t64(fma(v, ldexp(qs3, kex[prv][e]), bms[prv][e]), s_tab);
          msum += p;
          x[kb - 1][e] = float(p);
        }
      }
      if (kb == 3) phiv(x, vl4, 0);
      if (kb < 4) {
        const int zk = __builtin_amdgcn_readfirstlane(zk4[kb]);
        if (zk == 0) {
          // K digit 0 is live in this block: its products, the lowest class
          // (s = ZQ, t = 0) folded into the bias term
          i32x4 low = {0, 0, 0, 0};
#pragma unroll
          for (int c = 0; c < NCH; ++c) {
            const u32x4 kd = kl4[kb * 16 * KROW + 4 * c];
            low = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, kd),
                                                       __builtin_bit_cast(i32x4, qd[ZQ][c]), low, 0, 0, 0);
#pragma unroll
            for (int sd = ZQ + 1; sd < kDigits; ++sd)
              acc[cur][sd] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, kd),
                                                                  __builtin_bit_cast(i32x4, qd[sd][c]), acc[cur][sd],
                                                                  0, 0, 0);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e)
            bms[cur][e] = fma(double(low[e]), ldexp(qs3, kex[cur][e] - 8 * (3 - ZQ)), bms[cur][e]);
        }
      }
    }
    phiv(x, vl4, 1);
    // the next tile's copies have landed
    __builtin_amdgcn_s_waitcnt(0);
    if constexpr (STORE == 2) {
      if (qw < Dh.ldN) {
        if (!wfull) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e) x[kb][e] = qvalid ? x[kb][e] : 0.0f;
        }
        // lane (c16, g) puts its values at [key][c16] of the wave's block; then
        // lane l takes (key, 8 queries) items l and l + 64 and writes the high
        // and the low halves of the 8 values as one 16-byte store each (the
        // wave's own LDS writes land before its reads)
        uint32_t *lx = lx_all + wave * 1024;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e) lx[(16 * kb + g + 4 * e) * 16 + c16] = __float_as_uint(x[kb][e]);
        uint16_t *hp = phi16 + 2 * Dh.phi_off;
        uint16_t *lp = hp + Dh.ldT * Dh.ldN;
#pragma unroll
        for (int it = 0; it < 2; ++it) {
          const int item = lane + 64 * it, key = item >> 1, hf = item & 1;
          const u32x4 a = *reinterpret_cast<const u32x4 *>(lx + key * 16 + 8 * hf);
          const u32x4 b = *reinterpret_cast<const u32x4 *>(lx + key * 16 + 8 * hf + 4);
          const u32x4 hv = {__builtin_amdgcn_perm(a.y, a.x, 0x07060302u), __builtin_amdgcn_perm(a.w, a.z, 0x07060302u),
                            __builtin_amdgcn_perm(b.y, b.x, 0x07060302u), __builtin_amdgcn_perm(b.w, b.z, 0x07060302u)};
          const u32x4 lv = {__builtin_amdgcn_perm(a.y, a.x, 0x05040100u), __builtin_amdgcn_perm(a.w, a.z, 0x05040100u),
                            __builtin_amdgcn_perm(b.y, b.x, 0x05040100u), __builtin_amdgcn_perm(b.w, b.z, 0x05040100u)};
          const int64_t at = (k0 + key) * Dh.ldN + qw + 8 * hf;
          *reinterpret_cast<u32x4 *>(hp + at) = hv;
          *reinterpret_cast<u32x4 *>(lp + at) = lv;
        }
      }
    }
  };

  issue(0, lk0, lv0, lt0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (qb == 0 && tid == 0) {
    shift_out[h] = s_shift;
    if (tr_shift) tr_shift[h] = s_shift;
  }
  // waves of one block may take different variants; every path meets the
  // same barriers
  auto run = [&](auto zq_c) __attribute__((always_inline)) {
    constexpr int ZQ = decltype(zq_c)::value;
    u32x4 qd[kDigits][NCH];
#pragma unroll
    for (int sd = 0; sd < kDigits; ++sd)
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        qd[sd][c] = u32x4{0u, 0u, 0u, 0u};
        if (sd >= ZQ && qvalid) qd[sd][c] = *reinterpret_cast<const u32x4 *>(qsrc + sd * D + 64 * c);
      }
    for (int tile = 0; tile < ntiles; tile += 2) {
      compute(zq_c, qd, tile, lk0, lv0, lt0, tile + 1 < ntiles, lk1, lv1, lt1);
      __syncthreads();
      if (tile + 1 >= ntiles) break;
      compute(zq_c, qd, tile + 1, lk1, lv1, lt1, tile + 2 < ntiles, lk0, lv0, lt0);
      __syncthreads();
    }
  };
  if (zq >= 2) run(std::integral_constant<int, 2>{});
  else if (zq == 1) run(std::integral_constant<int, 1>{});
  else run(std::integral_constant<int, 0>{});

  msum += __shfl_xor(msum, 16);
  msum += __shfl_xor(msum, 32);
  bool bad = false;
  if (g == 0 && qvalid) {
    m_out[Dh.n_off + q] = msum;
    if (r_out) r_out[Dh.n_off + q] = msum;
    bad |= !isfinite(msum);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const double mq = __shfl(msum, 4 * g + e);
    const int64_t qy = qw + 4 * g + e;
    if (qy < Dh.n) {
#pragma unroll
      for (int db = 0; db < NU; ++db) {
        const float y = float(double(uacc[db][e]) / mq);
        bad |= !isfinite(y);
        Y_out[(Dh.n_off + qy) * D + db * 16 + c16] = y;
      }
    }
  }
  if (bad && head_status) atomicOr(head_status + h, int32_t(AMC_HS_NONFINITE));
}

}  // namespace

hipError_t launch_copy_words(uint64_t *dst, const uint64_t *src, int64_t count, hipStream_t s) {
  for (int64_t base = 0; base < count; base += 384) {
    WordChunk c;
    const int n = int(count - base < 384 ? count - base : 384);
    for (int i = 0; i < n; ++i) c.w[i] = src[base + i];
    hipLaunchKernelGGL(k_put_words, dim3(2), dim3(256), 0, s, dst + base, n, c);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_fill_i32(int32_t *p, int64_t count, int32_t value, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  int64_t blocks = (count + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_fill_i32, dim3(unsigned(blocks)), dim3(256), 0, s, p, count, value);
  return hipGetLastError();
}

hipError_t launch_shift(const Dims &dm, const Buffers &b, hipStream_t s) {
  const int nsb = int(dm.max_sblk);
  const int xcd_map = (dm.H % 8 == 0) ? 1 : 0;
  dim3 grid(unsigned(nsb * dm.H));
  const float sc = float(dm.scale);
#define AMC_SHIFT_ARGS b.desc, dm.H, nsb, xcd_map, b.Q, b.K, b.beta_in, sc, b.shift_part
  if (dm.d == 128) {
    if (dm.in_bf16) hipLaunchKernelGGL((k_shift<128, true>), grid, dim3(256), 0, s, AMC_SHIFT_ARGS);
    else hipLaunchKernelGGL((k_shift<128, false>), grid, dim3(256), 0, s, AMC_SHIFT_ARGS);
  } else {
    if (dm.in_bf16) hipLaunchKernelGGL((k_shift<64, true>), grid, dim3(256), 0, s, AMC_SHIFT_ARGS);
    else hipLaunchKernelGGL((k_shift<64, false>), grid, dim3(256), 0, s, AMC_SHIFT_ARGS);
  }
#undef AMC_SHIFT_ARGS
  return hipGetLastError();
}

template <int STORE>
static void launch_phi_store(const Dims &dm, const Buffers &b, hipStream_t s) {
  dim3 grid(unsigned((dm.max_n + kPhiRows - 1) / kPhiRows), unsigned(dm.H));
#define AMC_PHI_ARGS b.desc, b.Q, b.K, b.V, b.beta_in, dm.scale, b.shift_part, b.shift, b.tr_shift, b.phi, b.phi16, \
    b.m, b.r, b.Y, b.head_status
  if (dm.d == 128) {
    if (dm.in_bf16)
      hipLaunchKernelGGL((k_phi<128, true, STORE>), grid, dim3(256), 0, s, AMC_PHI_ARGS);
    else
      hipLaunchKernelGGL((k_phi<128, false, STORE>), grid, dim3(256), 0, s, AMC_PHI_ARGS);
  } else {
    if (dm.in_bf16)
      hipLaunchKernelGGL((k_phi<64, true, STORE>), grid, dim3(256), 0, s, AMC_PHI_ARGS);
    else
      hipLaunchKernelGGL((k_phi<64, false, STORE>), grid, dim3(256), 0, s, AMC_PHI_ARGS);
  }
#undef AMC_PHI_ARGS
}

template <int STORE>
static void launch_phi8(const Dims &dm, const Buffers &b, hipStream_t s) {
  const int nqb = int((dm.max_n + kPhi16Rows - 1) / kPhi16Rows);
  const int xcd_map = (dm.H % 8 == 0) ? 1 : 0;
  dim3 grid(unsigned(nqb * dm.H));
#define AMC_PHI8_ARGS b.desc, dm.H, nqb, xcd_map, b.qdig, b.qexp, b.kdig, b.ktab, b.f64_heads, b.vt, dm.scale, \
    b.shift_part, b.shift, b.tr_shift, b.phi16, b.m, b.r, b.Y, b.head_status
  if (dm.d == 128)
    hipLaunchKernelGGL((k_phi8<128, STORE>), grid, dim3(kPhi16Rows * 4), 0, s, AMC_PHI8_ARGS);
  else
    hipLaunchKernelGGL((k_phi8<64, STORE>), grid, dim3(kPhi16Rows * 4), 0, s, AMC_PHI8_ARGS);
#undef AMC_PHI8_ARGS
}

template <int STORE>
static void launch_phi16(const Dims &dm, const Buffers &b, const int32_t *list, const int32_t *list_cnt,
                         hipStream_t s) {
  const int nqb = int((dm.max_n + kPhi16Rows - 1) / kPhi16Rows);
  const int xcd_map = (dm.H % 8 == 0) ? 1 : 0;
  dim3 grid(unsigned(list ? 256 : nqb * dm.H));
  const uint16_t *Q = static_cast<const uint16_t *>(b.Q);
  const uint16_t *K = static_cast<const uint16_t *>(b.K);
#define AMC_PHI16_ARGS b.desc, dm.H, nqb, xcd_map, Q, K, b.vt, b.beta_in, dm.scale, b.shift_part, b.shift, b.tr_shift, \
    b.phi16, b.m, b.r, b.Y, b.head_status, list, list_cnt
  if (dm.d == 128)
    hipLaunchKernelGGL((k_phi16<128, STORE>), grid, dim3(kPhi16Rows * 4), 0, s, AMC_PHI16_ARGS);
  else
    hipLaunchKernelGGL((k_phi16<64, STORE>), grid, dim3(kPhi16Rows * 4), 0, s, AMC_PHI16_ARGS);
#undef AMC_PHI16_ARGS
}

// The two 16-bit planes of a head's stored Phi ([ldT keys][ldN queries]: the
// high and the low halves of the float32 bits) to the caller's dense float32
// Phi ([n][T] rows from out_off), one 64 x 64 tile per block through LDS (reads
// along queries, writes along keys).
__global__ __launch_bounds__(256) void k_planes_to_phi(const HeadDesc *__restrict__ desc,
                                                       const uint16_t *__restrict__ phi16, float *__restrict__ phi) {
  __shared__ float tile[64][65];
  const HeadDesc D = desc[blockIdx.y];
  const int64_t ntq = (D.n + 63) / 64, ntk = (D.T + 63) / 64;
  if (int64_t(blockIdx.x) >= ntq * ntk) return;
  const int64_t q0 = (blockIdx.x % ntq) * 64, k0 = (blockIdx.x / ntq) * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const uint16_t *hp = phi16 + 2 * D.phi_off;
  const uint16_t *lp = hp + D.ldT * D.ldN;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int kl = ty + 4 * i;
    const int64_t at = (k0 + kl) * D.ldN + q0 + tx;  // inside the padded planes
    tile[kl][tx] = __uint_as_float((uint32_t(hp[at]) << 16) | lp[at]);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int ql = ty + 4 * i;
    const int64_t q = q0 + ql, k = k0 + tx;
    if (q < D.n && k < D.T) phi[D.out_off + q * D.T + k] = tile[tx][ql];
  }
}

hipError_t launch_planes_to_phi(const Dims &dm, const Buffers &b, hipStream_t s) {
  if (!b.phi16 || !b.phi) return hipErrorInvalidValue;
  const int64_t tiles = ((dm.max_n + 63) / 64) * ((dm.max_T + 63) / 64);
  hipLaunchKernelGGL(k_planes_to_phi, dim3(unsigned(tiles), unsigned(dm.H)), dim3(256), 0, s, b.desc, b.phi16, b.phi);
  return hipGetLastError();
}

hipError_t launch_vt(const Dims &dm, const Buffers &b, hipStream_t s) {
  if (!b.vt || !dm.in_bf16) return hipErrorInvalidValue;
  dim3 grid(unsigned((dm.max_T + 63) / 64), unsigned(dm.H));
  const uint16_t *V = static_cast<const uint16_t *>(b.V);
  if (dm.d == 128) hipLaunchKernelGGL((k_vt<128>), grid, dim3(256), 0, s, b.desc, V, b.vt);
  else hipLaunchKernelGGL((k_vt<64>), grid, dim3(256), 0, s, b.desc, V, b.vt);
  return hipGetLastError();
}

hipError_t launch_digits(const Dims &dm, const Buffers &b, hipStream_t s) {
  if (!b.qdig || !dm.in_bf16) return hipErrorInvalidValue;
  hipError_t e = launch_fill_i32(b.f64_heads, dm.H, 0, s);
  if (e != hipSuccess) return e;
  constexpr int kRowsPerBlock128 = 256 / 16, kRowsPerBlock64 = 256 / 8;
  const int64_t rows = dm.max_n + 32 + (dm.max_T + 63) / 64 * 64;  // queries to a whole block, then keys
  const uint16_t *Q = static_cast<const uint16_t *>(b.Q);
  const uint16_t *K = static_cast<const uint16_t *>(b.K);
#define AMC_DIGITS_ARGS b.desc, Q, K, b.beta_in, b.shift_part, b.qdig, b.qexp, b.kdig, b.ktab, b.f64_heads
  if (dm.d == 128)
    hipLaunchKernelGGL(k_digits<128>, dim3(unsigned((rows + kRowsPerBlock128 - 1) / kRowsPerBlock128), unsigned(dm.H)),
                       dim3(256), 0, s, AMC_DIGITS_ARGS);
  else
    hipLaunchKernelGGL(k_digits<64>, dim3(unsigned((rows + kRowsPerBlock64 - 1) / kRowsPerBlock64), unsigned(dm.H)),
                       dim3(256), 0, s, AMC_DIGITS_ARGS);
#undef AMC_DIGITS_ARGS
  // the heads off the digit grid, listed for the float64 kernel
  hipLaunchKernelGGL(k_list_flags, dim3(1), dim3(256), 0, s, b.f64_heads, dm.H, b.f64_list, b.f64_cnt);
  return hipGetLastError();
}

hipError_t launch_phi(const Dims &dm, const Buffers &b, int store, hipStream_t s) {
  if (store == 1 && !b.phi) return hipErrorInvalidValue;
  if (store == 2 && !b.phi16) return hipErrorInvalidValue;
  if (dm.in_bf16 && b.vt && store != 1) {
    // int8 logits (after launch_digits) for the heads on the digit grid, else
    // the float64-MFMA kernel for every head
    if (b.qdig) {
      if (store == 2) launch_phi8<2>(dm, b, s);
      else launch_phi8<0>(dm, b, s);
    } else {
      if (store == 2) launch_phi16<2>(dm, b, nullptr, nullptr, s);
      else launch_phi16<0>(dm, b, nullptr, nullptr, s);
    }
    return hipGetLastError();
  }
  if (store == 1) launch_phi_store<1>(dm, b, s);
  else if (store == 2) launch_phi_store<2>(dm, b, s);
  else launch_phi_store<0>(dm, b, s);
  return hipGetLastError();
}

hipError_t launch_phi_fallback(const Dims &dm, const Buffers &b, int store, hipStream_t s) {
  if (!b.qdig || !dm.in_bf16 || !b.vt || store == 1) return hipErrorInvalidValue;
  if (store == 2) launch_phi16<2>(dm, b, b.f64_list, b.f64_cnt, s);
  else launch_phi16<0>(dm, b, b.f64_list, b.f64_cnt, s);
  return hipGetLastError();
}

}  // namespace amc
