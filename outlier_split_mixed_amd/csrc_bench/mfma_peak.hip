// mfma_peak.hip -- matrix-unit rate micro-benchmark (measurement only, not
// part of the path or its C ABI).  Every wave runs the dual GEMM's register
// pattern without memory traffic: 8 A and 4 B operand fragments, 32
// independent accumulators, one MFMA per (A, B) pair per round; two waves
// per SIMD (512-thread blocks, one per CU).  The rate is taken from HIP
// events around the launch.
//
// The sustained rate of the 6-/4-bit unit depends on the operand bits (the
// chip's power and clock management): a low-entropy pattern runs at nearly
// the published rate, random bits well below it.  So the operands come in two
// kinds:
//   data 0: a pattern of byte values 0..3 (the upper bound of the unit);
//   data 1: drawn like the workload's (per-field values of an approximately
//     normal variable g): FP6 = int4 code c = clamp(rint(1.75 g), -7, 7) as
//     the E2M3 subnormal c/8; FP4 = the E2M1 code nearest 2|g| with g's
//     sign; int8 = 16 c; bf16 = g rounded to bf16.  1.75 g is the code of a
//     normal value under a per-row absmax of about 4 standard deviations.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
constexpr int kTM = 8, kTN = 4;

__device__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}
// Irwin-Hall sum of four uniform bytes, centred and scaled to unit variance.
__device__ float approx_normal(uint32_t h) {
  const float s = (float)(h & 255u) + (float)((h >> 8) & 255u) + (float)((h >> 16) & 255u) + (float)(h >> 24);
  return (s - 510.0f) * (1.0f / 147.8f);
}
__device__ int int4_code(float g) {
  int c = (int)rintf(1.75f * g);
  return c > 7 ? 7 : (c < -7 ? -7 : c);
}
__device__ uint32_t e2m1_code(float g) {
  const float a = fabsf(2.0f * g);
  const float grid[8] = {0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f};
  uint32_t best = 0;
  for (uint32_t k = 1; k < 8; ++k)
    if (fabsf(a - grid[k]) < fabsf(a - grid[best])) best = k;
  return (g < 0.f && best ? 8u : 0u) | best;
}

// One operand fragment (eight registers; FP6 uses six, the others four).
template <int KIND, int DATA>
__device__ v8i fragment(int lane, int f) {
  v8i r;
  if constexpr (DATA == 0) {
#pragma unroll
    for (int q = 0; q < 8; ++q) r[q] = (int)(0x01010101u * (uint32_t)((lane * (f + 1) + q) & 3));
    return r;
  }
  const uint32_t seed = (uint32_t)(((blockIdx.x * 512u + threadIdx.x) * 16u + (uint32_t)f) * 64u);
  uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if constexpr (KIND == 0) {  // 32 six-bit fields over six registers
    for (int k = 0; k < 32; ++k) {
      const int c = int4_code(approx_normal(mix32(seed + (uint32_t)k)));
      const uint32_t v = (c < 0 ? 32u : 0u) | (uint32_t)(c < 0 ? -c : c);
      const int bit = 6 * k, d = bit >> 5, sh = bit & 31;
      w[d] |= v << sh;
      if (sh > 26) w[d + 1] |= v >> (32 - sh);
    }
  } else if constexpr (KIND == 1) {  // 32 four-bit fields over four registers
    for (int k = 0; k < 32; ++k) w[k >> 3] |= e2m1_code(approx_normal(mix32(seed + (uint32_t)k))) << (4 * (k & 7));
  } else if constexpr (KIND == 2) {  // 16 int8 values
    for (int k = 0; k < 16; ++k) {
      const int c = int4_code(approx_normal(mix32(seed + (uint32_t)k)));
      w[k >> 2] |= ((uint32_t)(16 * c) & 0xFFu) << (8 * (k & 3));
    }
  } else {  // 8 bf16 values
    for (int k = 0; k < 8; ++k) {
      const __bf16 b = (__bf16)approx_normal(mix32(seed + (uint32_t)k));
      w[k >> 1] |= (uint32_t)__builtin_bit_cast(uint16_t, b) << (16 * (k & 1));
    }
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) r[q] = (int)w[q];
  return r;
}

__device__ __forceinline__ v4i lo4(v8i a) { return v4i{a[0], a[1], a[2], a[3]}; }

// KIND: 0 FP6 (E2M3 x E2M3, 16x16x128), 1 FP4 (E2M1 x E2M1, 16x16x128),
// 2 int8 (16x16x64), 3 bf16 (16x16x32)
template <int KIND, int DATA>
__global__ __launch_bounds__(512, 2) void k_mfma_rate(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  v8i A[kTM], B[kTN];
#pragma unroll
  for (int i = 0; i < kTM; ++i) A[i] = fragment<KIND, DATA>(lane, i);
#pragma unroll
  for (int j = 0; j < kTN; ++j) B[j] = fragment<KIND, DATA>(lane, kTM + j);
  v4f acc[kTM][kTN];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j) {
        if constexpr (KIND == 0)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[i], B[j], acc[i][j], 2, 2, 0, 0, 0, 0);
        else if constexpr (KIND == 1)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[i], B[j], acc[i][j], 4, 4, 0, 0, 0, 0);
        else if constexpr (KIND == 2)
          acc[i][j] = __builtin_bit_cast(
              v4f, __builtin_amdgcn_mfma_i32_16x16x64_i8(lo4(A[i]), lo4(B[j]), __builtin_bit_cast(v4i, acc[i][j]),
                                                          0, 0, 0));
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, lo4(A[i])),
                                                              __builtin_bit_cast(v8bf, lo4(B[j])), acc[i][j], 0, 0, 0);
      }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j) s += acc[i][j][0] + acc[i][j][3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;  // keeps the accumulators live
}

template <int KIND, int DATA>
hipError_t run(int blocks, int iters, float* out, hipStream_t st) {
  hipLaunchKernelGGL((k_mfma_rate<KIND, DATA>), dim3((unsigned)blocks), dim3(512), 0, st, iters, out);
  return hipGetLastError();
}

}  // namespace

// Matrix-unit rate of one instruction kind (0 FP6, 1 FP4, 2 int8, 3 bf16) on
// operands of kind `data` (0 pattern, 1 workload-shaped), in TOP/s: blocks x
// 512 threads, iters x 32 instructions per wave, one warm-up launch, then the
// median of `reps` timed launches.  Returns 0, or a HIP error code (-1 for a
// bad argument).
extern "C" int sqfb_mfma_rate(int kind, int data, int blocks, int iters, int reps, double* tops) {
  if (kind < 0 || kind > 3 || data < 0 || data > 1 || blocks <= 0 || iters <= 0 || reps <= 0 || reps > 64 ||
      !tops)
    return -1;
  float* out = nullptr;
  hipError_t e = hipMalloc(&out, (size_t)blocks * 512 * sizeof(float));
  if (e != hipSuccess) return (int)e;
  hipStream_t st = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if ((e = hipStreamCreate(&st)) != hipSuccess || (e = hipEventCreate(&e0)) != hipSuccess ||
      (e = hipEventCreate(&e1)) != hipSuccess) {
    (void)hipFree(out);
    return (int)e;
  }
  auto launch = [&]() {
    switch (kind * 2 + data) {
      case 0: return run<0, 0>(blocks, iters, out, st);
      case 1: return run<0, 1>(blocks, iters, out, st);
      case 2: return run<1, 0>(blocks, iters, out, st);
      case 3: return run<1, 1>(blocks, iters, out, st);
      case 4: return run<2, 0>(blocks, iters, out, st);
      case 5: return run<2, 1>(blocks, iters, out, st);
      case 6: return run<3, 0>(blocks, iters, out, st);
      default: return run<3, 1>(blocks, iters, out, st);
    }
  };
  // operations per instruction: 2 * 16 * 16 * K
  const double k = kind <= 1 ? 128.0 : (kind == 2 ? 64.0 : 32.0);
  const double ops = 2.0 * 16 * 16 * k * (kTM * kTN) * (double)iters * (double)blocks * 8.0;
  float ms[64];
  e = launch();
  for (int r = 0; r < reps && e == hipSuccess; ++r) {
    if ((e = hipEventRecord(e0, st)) != hipSuccess || (e = launch()) != hipSuccess ||
        (e = hipEventRecord(e1, st)) != hipSuccess || (e = hipEventSynchronize(e1)) != hipSuccess)
      break;
    e = hipEventElapsedTime(&ms[r], e0, e1);
  }
  if (e == hipSuccess) {
    for (int i = 1; i < reps; ++i)  // insertion sort, then the median
      for (int j = i; j > 0 && ms[j] < ms[j - 1]; --j) {
        const float t = ms[j];
        ms[j] = ms[j - 1];
        ms[j - 1] = t;
      }
    *tops = ops / (ms[reps / 2] * 1e-3) / 1e12;
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  (void)hipStreamDestroy(st);
  (void)hipFree(out);
  return (int)e;
}
