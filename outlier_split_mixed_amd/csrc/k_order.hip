// k_order.hip -- the channel order that turns the split into a slice.
//
// SQ-format article, section 九: weight columns are reordered by the
// importance mask.  Reordering the channel axis that connects two layers --
// the producer's output channels (its weight columns, and a norm's gamma)
// and the consumer's input channels (its weight rows) -- leaves every product
// unchanged; in slot order (the low channels in slot order, then the outlier
// channels in branch order) the consumer's split is a slice: low slots are
// the first k_low channels, the branch the last k_out.
#include "sqf_device.h"
#include "sqf_launch.h"

namespace sqf {

// One block: k_out = the largest branch slot + 1, then position
// p(c) = map[c] (low) or k - k_out + t (outlier slot t), perm[p(c)] = c, and
// the slice map p -> p (p < k_low) or -(p - k_low + 1).
__global__ __launch_bounds__(1024) void k_slot_order(const int32_t* __restrict__ map, int64_t k,
                                                     int32_t* __restrict__ perm,
                                                     int32_t* __restrict__ slice_map) {
  __shared__ int32_t wmax[16];
  int32_t mx = 0;
  for (int64_t c = threadIdx.x; c < k; c += 1024) mx = max(mx, -map[c]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = max(mx, __shfl_xor(mx, off, kWave));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = mx;
  __syncthreads();
  int32_t k_out = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) k_out = max(k_out, wmax[w]);
  const int64_t k_low = k - k_out;
  for (int64_t c = threadIdx.x; c < k; c += 1024) {
    const int32_t s = map[c];
    const int64_t pos = s >= 0 ? (int64_t)s : k_low + (-(int64_t)s - 1);
    perm[pos] = (int32_t)c;
    slice_map[c] = c < k_low ? (int32_t)c : (int32_t)(-(c - k_low + 1));
  }
}

// dst[r][p] = src[r][perm[p]] (axis 1) or dst[p][j] = src[perm[p]][j]
// (axis 0); one thread per output element, consecutive threads along a dst
// row (coalesced stores; axis 0 also reads whole rows).
__global__ __launch_bounds__(256) void k_permute(const float* __restrict__ src, int64_t rows,
                                                 int64_t cols, int64_t ld_src,
                                                 const int32_t* __restrict__ perm, int axis,
                                                 float* __restrict__ dst, int64_t ld_dst) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t r = blockIdx.y;
  if (j >= cols) return;
  for (int64_t rr = r; rr < rows; rr += gridDim.y) {
    const float v = axis == 1 ? src[rr * ld_src + perm[j]] : src[(int64_t)perm[rr] * ld_src + j];
    dst[rr * ld_dst + j] = v;
  }
}

hipError_t launch_slot_order(const int32_t* map, int64_t k, int32_t* perm, int32_t* slice_map,
                             hipStream_t s) {
  hipLaunchKernelGGL(k_slot_order, dim3(1), dim3(1024), 0, s, map, k, perm, slice_map);
  return hipGetLastError();
}

hipError_t launch_permute(const float* src, int64_t rows, int64_t cols, int64_t ld_src,
                          const int32_t* perm, int axis, float* dst, int64_t ld_dst, hipStream_t s) {
  const int64_t gx = (cols + 255) / 256;
  const int64_t gy = rows < 4096 ? rows : 4096;
  if (gx <= 0 || gy <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_permute, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, s, src, rows, cols,
                     ld_src, perm, axis, dst, ld_dst);
  return hipGetLastError();
}

}  // namespace sqf
