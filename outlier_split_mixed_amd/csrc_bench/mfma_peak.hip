// mfma_peak.hip -- matrix-unit rate micro-benchmark (measurement only, not
// part of the path or its C ABI): every wave runs eight independent
// accumulation chains of one MFMA instruction on register operands, two
// waves per SIMD (512-thread blocks, one per CU) as in the dual GEMM, and
// the rate is taken from HIP events around the launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kChains = 8;

// KIND: 0 FP6 (E2M3 x E2M3, 16x16x128), 1 FP4 (E2M1 x E2M1, 16x16x128),
// 2 int8 (16x16x64), 3 bf16 (16x16x32)
template <int KIND>
__global__ __launch_bounds__(512, 2) void k_mfma_rate(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  v8i a8, b8;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    a8[q] = (int)(0x01010101u * (uint32_t)((lane + q) & 3));
    b8[q] = (int)(0x01010101u * (uint32_t)((lane * 3 + q) & 3));
  }
  v4f accf[kChains];
  v4i acci[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) {
    accf[c] = v4f{0.f, 0.f, 0.f, 0.f};
    acci[c] = v4i{0, 0, 0, 0};
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
      if constexpr (KIND == 0)
        accf[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, accf[c], 2, 2, 0, 0, 0, 0);
      else if constexpr (KIND == 1)
        accf[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, accf[c], 4, 4, 0, 0, 0, 0);
      else if constexpr (KIND == 2)
        acci[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(v4i{a8[0], a8[1], a8[2], a8[3]},
                                                         v4i{b8[0], b8[1], b8[2], b8[3]}, acci[c], 0, 0, 0);
      else
        accf[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(v8bf, v4i{a8[0], a8[1], a8[2], a8[3]}),
            __builtin_bit_cast(v8bf, v4i{b8[0], b8[1], b8[2], b8[3]}), accf[c], 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += accf[c][0] + accf[c][3] + (float)acci[c][0] + (float)acci[c][3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;  // keeps the chains live
}

template <int KIND>
hipError_t run(int blocks, int iters, float* out, hipStream_t st) {
  hipLaunchKernelGGL(k_mfma_rate<KIND>, dim3((unsigned)blocks), dim3(512), 0, st, iters, out);
  return hipGetLastError();
}

}  // namespace

// Matrix-unit rate of one instruction kind (0 FP6, 1 FP4, 2 int8, 3 bf16),
// in TOP/s: blocks x 512 threads, iters x 8 instructions per wave, one
// warm-up launch, then the median of `reps` timed launches.  Returns 0, or a
// HIP error code.
extern "C" int sqfb_mfma_rate(int kind, int blocks, int iters, int reps, double* tops) {
  if (kind < 0 || kind > 3 || blocks <= 0 || iters <= 0 || reps <= 0 || reps > 64 || !tops) return -1;
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
    switch (kind) {
      case 0: return run<0>(blocks, iters, out, st);
      case 1: return run<1>(blocks, iters, out, st);
      case 2: return run<2>(blocks, iters, out, st);
      default: return run<3>(blocks, iters, out, st);
    }
  };
  // operations per instruction: 2 * 16 * 16 * K
  const double k = kind <= 1 ? 128.0 : (kind == 2 ? 64.0 : 32.0);
  const double ops = 2.0 * 16 * 16 * k * kChains * (double)iters * (double)blocks * 8.0;
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
        const float t = ms[j]; ms[j] = ms[j - 1]; ms[j - 1] = t;
      }
    *tops = ops / (ms[reps / 2] * 1e-3) / 1e12;
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  (void)hipStreamDestroy(st);
  (void)hipFree(out);
  return (int)e;
}
