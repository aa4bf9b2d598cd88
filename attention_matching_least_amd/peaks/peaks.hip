// Throughput probe for the roofline denominators on the machine at hand: the
// MFMA instructions the library uses, float64 vector FMA, and an HBM read
// stream.  Each kernel runs twice; the second run is reported.  Prints one
// JSON object.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

typedef double d4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef int i4 __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                         \
  do {                                                                   \
    hipError_t e_ = (x);                                                 \
    if (e_ != hipSuccess) {                                              \
      std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));       \
      std::exit(1);                                                      \
    }                                                                    \
  } while (0)

// Four independent accumulation chains per wave, operands in registers.
__global__ __launch_bounds__(256) void p_f64_16x16x4(double *o, int iters) {
  d4 a0 = {0, 0, 0, 0}, a1 = a0, a2 = a0, a3 = a0;
  const double x = threadIdx.x * 1e-3, y = 1.0 + x;
  for (int i = 0; i < iters; ++i) {
    a0 = __builtin_amdgcn_mfma_f64_16x16x4f64(x, y, a0, 0, 0, 0);
    a1 = __builtin_amdgcn_mfma_f64_16x16x4f64(y, x, a1, 0, 0, 0);
    a2 = __builtin_amdgcn_mfma_f64_16x16x4f64(x, x, a2, 0, 0, 0);
    a3 = __builtin_amdgcn_mfma_f64_16x16x4f64(y, y, a3, 0, 0, 0);
  }
  o[blockIdx.x * blockDim.x + threadIdx.x] = a0[0] + a1[1] + a2[2] + a3[3];
}

__global__ __launch_bounds__(256) void p_f64_4x4x4(double *o, int iters) {
  double a0 = 0, a1 = 0, a2 = 0, a3 = 0;
  const double x = threadIdx.x * 1e-3, y = 1.0 + x;
  for (int i = 0; i < iters; ++i) {
    a0 = __builtin_amdgcn_mfma_f64_4x4x4f64(x, y, a0, 0, 0, 0);
    a1 = __builtin_amdgcn_mfma_f64_4x4x4f64(y, x, a1, 0, 0, 0);
    a2 = __builtin_amdgcn_mfma_f64_4x4x4f64(x, x, a2, 0, 0, 0);
    a3 = __builtin_amdgcn_mfma_f64_4x4x4f64(y, y, a3, 0, 0, 0);
  }
  o[blockIdx.x * blockDim.x + threadIdx.x] = a0 + a1 + a2 + a3;
}

__global__ __launch_bounds__(256) void p_f32_16x16x4(double *o, int iters) {
  f4 a0 = {0, 0, 0, 0}, a1 = a0, a2 = a0, a3 = a0;
  const float x = threadIdx.x * 1e-3f, y = 1.0f + x;
  for (int i = 0; i < iters; ++i) {
    a0 = __builtin_amdgcn_mfma_f32_16x16x4f32(x, y, a0, 0, 0, 0);
    a1 = __builtin_amdgcn_mfma_f32_16x16x4f32(y, x, a1, 0, 0, 0);
    a2 = __builtin_amdgcn_mfma_f32_16x16x4f32(x, x, a2, 0, 0, 0);
    a3 = __builtin_amdgcn_mfma_f32_16x16x4f32(y, y, a3, 0, 0, 0);
  }
  o[blockIdx.x * blockDim.x + threadIdx.x] = a0[0] + a1[1] + a2[2] + a3[3];
}

__global__ __launch_bounds__(256) void p_bf16_16x16x32(double *o, int iters) {
  f4 a0 = {0, 0, 0, 0}, a1 = a0, a2 = a0, a3 = a0;
  bf8 x, y;
  for (int i = 0; i < 8; ++i) {
    x[i] = (__bf16)(threadIdx.x * 1e-3f + i);
    y[i] = (__bf16)(1.0f + i);
  }
  for (int i = 0; i < iters; ++i) {
    a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, a0, 0, 0, 0);
    a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(y, x, a1, 0, 0, 0);
    a2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, x, a2, 0, 0, 0);
    a3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(y, y, a3, 0, 0, 0);
  }
  o[blockIdx.x * blockDim.x + threadIdx.x] = a0[0] + a1[1] + a2[2] + a3[3];
}

// eight accumulation chains (the int8 MFMA needs more in flight than the others)
__global__ __launch_bounds__(256) void p_i8_16x16x64(double *o, int iters) {
  i4 a[8];
  for (int c = 0; c < 8; ++c) a[c] = i4{c, 0, 0, 0};
  const i4 x = {int(threadIdx.x), 3, 5, 7}, y = {1, int(threadIdx.x) * 3, 9, 11};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < 8; ++c) a[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8((c & 1) ? x : y, (c & 2) ? y : x, a[c], 0, 0, 0);
  }
  double t = 0.0;
  for (int c = 0; c < 8; ++c) t += double(a[c][c & 3]);
  o[blockIdx.x * blockDim.x + threadIdx.x] = t;
}

__global__ __launch_bounds__(256) void p_f64_fma(double *o, int iters) {
  double a0 = 0, a1 = 0, a2 = 0, a3 = 0;
  const double x = threadIdx.x * 1e-3, y = 1.0 + x;
  for (int i = 0; i < iters; ++i) {
    a0 = fma(x, y, a0);
    a1 = fma(y, x, a1);
    a2 = fma(x, x, a2);
    a3 = fma(y, y, a3);
  }
  o[blockIdx.x * blockDim.x + threadIdx.x] = a0 + a1 + a2 + a3;
}

// Reads n float4 (n a multiple of 8 x the grid) with non-temporal loads, eight
// in flight per thread; one partial sum per thread.
__global__ __launch_bounds__(256) void p_read(const f4 *__restrict__ in, int64_t n, float *__restrict__ o) {
  f4 acc = {0, 0, 0, 0};
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i + 7 * stride < n; i += 8 * stride) {
    f4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(in + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u];
  }
  o[int64_t(blockIdx.x) * blockDim.x + threadIdx.x] = acc[0] + acc[1] + acc[2] + acc[3];
}

template <typename K>
static double time_ms(K kernel, dim3 grid, double *o, int iters) {
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  float ms = 0.0f;
  for (int rep = 0; rep < 2; ++rep) {
    CHECK(hipEventRecord(e0));
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, 0, o, iters);
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    CHECK(hipEventElapsedTime(&ms, e0, e1));
  }
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  return ms;
}

int main() {
  const int blocks = 2048, iters = 512;
  double *o = nullptr;
  CHECK(hipMalloc(&o, sizeof(double) * blocks * 256));
  // flops per instruction (per wave), times 4 chains, 4 waves per block
  const double waves_x_chains = double(blocks) * 4 * 4 * iters;
  const double t0 = time_ms(p_f64_16x16x4, dim3(blocks), o, iters);
  const double t1 = time_ms(p_f64_4x4x4, dim3(blocks), o, iters);
  const double t2 = time_ms(p_f32_16x16x4, dim3(blocks), o, iters);
  const double t3 = time_ms(p_bf16_16x16x32, dim3(blocks), o, iters);
  const double t4 = time_ms(p_f64_fma, dim3(blocks), o, iters * 64);
  const double t5 = time_ms(p_i8_16x16x64, dim3(blocks), o, iters);
  const double tf = 1e9;  // (flop / ms) -> TFLOP/s
  const double f64_16 = waves_x_chains * (16 * 16 * 4 * 2) / t0 / tf;
  const double f64_4 = waves_x_chains * (4 * 4 * 4 * 2 * 4) / t1 / tf;  // four 4x4 blocks per instruction
  const double f32_16 = waves_x_chains * (16 * 16 * 4 * 2) / t2 / tf;
  const double bf16 = waves_x_chains * (16 * 16 * 32 * 2) / t3 / tf;
  const double fma64 = waves_x_chains * 64 * (64 * 2) / t4 / tf;
  const double i8 = 2.0 * waves_x_chains * (16 * 16 * 64 * 2) / t5 / tf;  // eight chains
  // HBM read stream over 8 GiB
  const int64_t nbytes = int64_t(8) << 30;
  f4 *buf = nullptr;
  float *part = nullptr;
  CHECK(hipMalloc(&buf, nbytes));
  CHECK(hipMemset(buf, 0, nbytes));
  const int rblocks = 4096;
  CHECK(hipMalloc(&part, sizeof(float) * rblocks * 256));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  float rms = 0.0f;
  for (int rep = 0; rep < 3; ++rep) {
    CHECK(hipEventRecord(e0));
    hipLaunchKernelGGL(p_read, dim3(rblocks), dim3(256), 0, 0, buf, nbytes / 16, part);
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    CHECK(hipEventElapsedTime(&rms, e0, e1));
  }
  const double read_gbs = double(nbytes) / (rms * 1e-3) / 1e9;
  std::printf(
      "{\"mfma_f64_16x16x4_tflops\": %.1f, \"mfma_f64_4x4x4_tflops\": %.1f, \"mfma_f32_16x16x4_tflops\": %.1f, "
      "\"mfma_bf16_16x16x32_tflops\": %.1f, \"mfma_i8_16x16x64_tops\": %.1f, \"vector_f64_fma_tflops\": %.1f, "
      "\"hbm_read_gbs\": %.0f}\n",
      f64_16, f64_4, f32_16, bf16, i8, fma64, read_gbs);
  CHECK(hipFree(buf));
  CHECK(hipFree(part));
  CHECK(hipFree(o));
  return 0;
}
