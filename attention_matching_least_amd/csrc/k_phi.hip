// Stage 1 kernels: the per-head logit shift, and the mass features
// Phi = exp(l - s), the target mass m = Phi 1 and the attention output
// Y = Phi V / m (zhichai.net deep-dive, section 1.6; xinfinite.net article,
// section 2, step 3).
//
// The fit side of the method (m, and later the Gram system and residual) is
// conditioned like cond(Phi_S^T Phi_S) ~ 1e9, so the logits that feed m are
// computed in float64 on the MFMA units (v_mfma_f64_16x16x4f64) from the
// exact bf16/fp32 inputs; Phi is rounded to float32 only for storage, where
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
// logit maximum: one partial per (head, 128 queries), bf16 MFMA 16x16x32
// ---------------------------------------------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(256) void k_shift(const HeadDesc *__restrict__ desc, const void *__restrict__ Q,
                                               const void *__restrict__ K, const float *__restrict__ beta_in,
                                               float scale, float *__restrict__ shift_part) {
  constexpr int KC = D / 32;
  constexpr int KSTR = D + 8;  // bf16 elements per LDS row (16-byte pad)
  __shared__ __attribute__((aligned(16))) uint16_t ks[64 * KSTR];
  __shared__ float red[4];
  const HeadDesc Dh = desc[blockIdx.y];
  const int blk = blockIdx.x;
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
  for (int64_t k0 = 0; k0 < Dh.T; k0 += 64) {
    __syncthreads();
    for (int gi = tid; gi < 64 * D / 8; gi += 256) {
      const int key = gi / (D / 8), c8 = gi % (D / 8);
      const uint4 v = (k0 + key < Dh.T) ? load8_bf16<BF16>(K, (Dh.k_off + k0 + key) * D + 8 * c8) : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4 *>(&ks[key * KSTR + 8 * c8]) = v;
    }
    __syncthreads();
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
        if constexpr (STORE != 0) ps[wave][c16 * PSTR + kl] = pf[kb][e];
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
      // 8 keys of one row per lane: their high halves leave as one 16-byte
      // segment of the high plane, their low halves as one of the low plane
      // (ldT is a multiple of 8, so a segment that starts below ldT ends
      // within the row)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      uint16_t *hp = phi16 + 2 * Dh.phi_off;
      uint16_t *lp = hp + Dh.n * Dh.ldT;
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int row = (lane >> 3) + 8 * it, col = 8 * (lane & 7);
        const int64_t qr = q0 + row;
        if (qr < Dh.n && k0 + col < Dh.ldT) {
          const f32x4 a = *reinterpret_cast<const f32x4 *>(&ps[wave][row * PSTR + col]);
          const f32x4 c = *reinterpret_cast<const f32x4 *>(&ps[wave][row * PSTR + col + 4]);
          const uint32_t u[8] = {__float_as_uint(a.x), __float_as_uint(a.y), __float_as_uint(a.z),
                                 __float_as_uint(a.w), __float_as_uint(c.x), __float_as_uint(c.y),
                                 __float_as_uint(c.z), __float_as_uint(c.w)};
          u32x4 hv, lv;
          hv.x = (u[0] >> 16) | (u[1] & 0xffff0000u);
          hv.y = (u[2] >> 16) | (u[3] & 0xffff0000u);
          hv.z = (u[4] >> 16) | (u[5] & 0xffff0000u);
          hv.w = (u[6] >> 16) | (u[7] & 0xffff0000u);
          lv.x = (u[0] & 0xffffu) | (u[1] << 16);
          lv.y = (u[2] & 0xffffu) | (u[3] << 16);
          lv.z = (u[4] & 0xffffu) | (u[5] << 16);
          lv.w = (u[6] & 0xffffu) | (u[7] << 16);
          const int64_t at = qr * Dh.ldT + k0 + col;
          __builtin_nontemporal_store(hv, reinterpret_cast<u32x4 *>(hp + at));
          __builtin_nontemporal_store(lv, reinterpret_cast<u32x4 *>(lp + at));
        }
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
  dim3 grid(unsigned(dm.max_sblk), unsigned(dm.H));
  const float sc = float(dm.scale);
  if (dm.d == 128) {
    if (dm.in_bf16)
      hipLaunchKernelGGL((k_shift<128, true>), grid, dim3(256), 0, s, b.desc, b.Q, b.K, b.beta_in, sc, b.shift_part);
    else
      hipLaunchKernelGGL((k_shift<128, false>), grid, dim3(256), 0, s, b.desc, b.Q, b.K, b.beta_in, sc, b.shift_part);
  } else {
    if (dm.in_bf16)
      hipLaunchKernelGGL((k_shift<64, true>), grid, dim3(256), 0, s, b.desc, b.Q, b.K, b.beta_in, sc, b.shift_part);
    else
      hipLaunchKernelGGL((k_shift<64, false>), grid, dim3(256), 0, s, b.desc, b.Q, b.K, b.beta_in, sc, b.shift_part);
  }
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

hipError_t launch_phi(const Dims &dm, const Buffers &b, int store, hipStream_t s) {
  if (store == 1 && !b.phi) return hipErrorInvalidValue;
  if (store == 2 && !b.phi16) return hipErrorInvalidValue;
  if (store == 1) launch_phi_store<1>(dm, b, s);
  else if (store == 2) launch_phi_store<2>(dm, b, s);
  else launch_phi_store<0>(dm, b, s);
  return hipGetLastError();
}

}  // namespace amc
