// k_select.hip -- offline outlier-channel choice on the GPU.
//
// Follows the static activation strategy of the SQ-format article (sections
// 二 and 五: per-channel mean activation from a calibration set, weighted by
// the channel's contribution through the weights, fixed offline so inference
// needs no top-k) and OSC's offline outlier-channel identification (abstract).
//
//   score[c] = (sum_m |x[m,c]| / m_cal) * sqrt(sum_j W[c,j]^2)
//   hdiag[c] = (float) sum_m x[m,c]^2
// Both sums are fp64 and taken sequentially in index order (one thread owns
// one channel), so the scores are reproducible bit for bit.  Squares of fp32
// values are exact in fp64, so a fused multiply-add gives the same sum.
// Ranking: score descending, lower channel first on ties.
#include "sqf_device.h"
#include "sqf_launch.h"

namespace sqf {

// Pass 1: per-channel sum |x| (into score[] as a temporary) and sum x^2.
__global__ __launch_bounds__(256) void k_colstats_x(const float* __restrict__ x, int64_t m_cal,
                                                    int64_t k, double* __restrict__ score,
                                                    float* __restrict__ hdiag) {
  int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= k) return;
  double sa = 0.0, s2 = 0.0;
  for (int64_t m = 0; m < m_cal; ++m) {
    double v = (double)x[m * k + c];
    sa += fabs(v);
    s2 += v * v;
  }
  score[c] = sa;
  if (hdiag) hdiag[c] = (float)s2;
}

// Pass 2: sum_j W[c,j]^2 for 64 channels per block, streamed through LDS so the
// global reads stay coalesced while each channel's sum stays sequential.
// Then score[c] = (score[c] / m_cal) * sqrt(sum).
__global__ __launch_bounds__(256) void k_wnorm_score(const float* __restrict__ w, int64_t k,
                                                     int64_t n, int64_t m_cal,
                                                     double* __restrict__ score) {
  __shared__ float tile[64][65];
  const int64_t c0 = (int64_t)blockIdx.x * 64;
  const int tid = threadIdx.x;
  double acc = 0.0;
  for (int64_t j0 = 0; j0 < n; j0 += 64) {
    // 256 threads load 64 rows x 64 columns: thread -> (row = tid/4 + 64*i?, ...)
    for (int e = tid; e < 64 * 64; e += 256) {
      int r = e >> 6, col = e & 63;
      int64_t c = c0 + r, j = j0 + col;
      tile[r][col] = (c < k && j < n) ? w[c * n + j] : 0.0f;
    }
    __syncthreads();
    if (tid < 64) {
      int64_t jmax = n - j0 < 64 ? n - j0 : 64;
      for (int col = 0; col < jmax; ++col) {
        double v = (double)tile[tid][col];
        acc += v * v;
      }
    }
    __syncthreads();
  }
  if (tid < 64 && c0 + tid < k) {
    int64_t c = c0 + tid;
    double mean_abs = score[c] / (double)m_cal;
    score[c] = mean_abs * sqrt(acc);
  }
}

// Pass 3: rank[c] = #{c' : s[c'] > s[c] or (s[c'] == s[c] and c' < c)};
// flag[c] = rank < k_out.  Scores are streamed through LDS in chunks.
__global__ __launch_bounds__(256) void k_rank(const double* __restrict__ score, int64_t k,
                                              int64_t k_out, int32_t* __restrict__ flag) {
  __shared__ double chunk[1024];
  int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  double s = c < k ? score[c] : 0.0;
  int64_t rank = 0;
  for (int64_t base = 0; base < k; base += 1024) {
    for (int e = threadIdx.x; e < 1024; e += 256) chunk[e] = base + e < k ? score[base + e] : 0.0;
    __syncthreads();
    int64_t lim = k - base < 1024 ? k - base : 1024;
    for (int e = 0; e < lim; ++e) {
      double t = chunk[e];
      rank += (t > s) || (t == s && base + e < c);
    }
    __syncthreads();
  }
  if (c < k) flag[c] = rank < k_out ? 1 : 0;
}

// Pass 4 (one block): turn outlier flags into idx (ascending) and the
// channel map with an exclusive scan over the channels.
__global__ __launch_bounds__(1024) void k_flags_to_map(int32_t* __restrict__ map, int64_t k,
                                                       int32_t* __restrict__ idx) {
  __shared__ int wave_tot[16];
  __shared__ int carry;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int64_t base = 0; base < k; base += 1024) {
    int64_t c = base + tid;
    int f = c < k ? map[c] : 0;
    int inc = wave_inclusive_scan(f);
    if (lane == 63) wave_tot[wv] = inc;
    __syncthreads();
    int before = carry;
    for (int i = 0; i < wv; ++i) before += wave_tot[i];
    int t = before + inc - f;  // outliers before channel c
    if (c < k) {
      if (f) {
        map[c] = -(t + 1);
        idx[t] = (int32_t)c;
      } else {
        map[c] = (int32_t)(c - t);
      }
    }
    __syncthreads();
    if (tid == 1023) carry = before + inc;
    __syncthreads();
  }
}

hipError_t launch_select(const float* x_cal, int64_t m_cal, int64_t k, const float* w, int64_t n,
                         int64_t k_out, int32_t* idx, int32_t* map, double* score, float* hdiag,
                         hipStream_t s) {
  int64_t nb = (k + 255) / 256;
  hipLaunchKernelGGL(k_colstats_x, dim3((unsigned)nb), dim3(256), 0, s, x_cal, m_cal, k, score,
                     hdiag);
  hipLaunchKernelGGL(k_wnorm_score, dim3((unsigned)((k + 63) / 64)), dim3(256), 0, s, w, k, n,
                     m_cal, score);
  hipLaunchKernelGGL(k_rank, dim3((unsigned)nb), dim3(256), 0, s, score, k, k_out, map);
  hipLaunchKernelGGL(k_flags_to_map, dim3(1), dim3(1024), 0, s, map, k, idx);
  return hipGetLastError();
}

}  // namespace sqf
