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

// Pass 1: per-channel sum |x| (into score[] as a temporary) and sum x^2; also
// clears the channel's rank counter (map[c]) for pass 3.  One thread per
// channel with 64-thread blocks (spread over the CUs); the rows are read 16 at
// a time so that many loads are in flight while each sum stays sequential.
__global__ __launch_bounds__(64) void k_colstats_x(const float* __restrict__ x, int64_t m_cal,
                                                   int64_t k, double* __restrict__ score,
                                                   float* __restrict__ hdiag,
                                                   int32_t* __restrict__ rank) {
  int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= k) return;
  double sa = 0.0, s2 = 0.0;
  int64_t m = 0;
  for (; m + 16 <= m_cal; m += 16) {
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = x[(m + u) * k + c];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const double d = (double)v[u];
      sa += fabs(d);
      s2 += d * d;
    }
  }
  for (; m < m_cal; ++m) {
    const double d = (double)x[m * k + c];
    sa += fabs(d);
    s2 += d * d;
  }
  score[c] = sa;
  if (hdiag) hdiag[c] = (float)s2;
  rank[c] = 0;
}

// Pass 2: sum_j W[c,j]^2 for 32 channels (rows of W) per block, then
// score[c] = (score[c] / m_cal) * sqrt(sum).  The block streams stages of
// 32 rows x 512 columns: all 256 threads load a stage with coalesced 16-byte
// reads into registers, store it to one of two LDS buffers, and start loading
// the next stage while lanes 0..31 of wave 0 add their channel's squares
// column by column (one sequential fp64 chain per channel).
constexpr int kWsCh = 32, kWsCols = 512, kWsLd = kWsCols + 4;  // 16-byte rows
constexpr size_t kWsSmem = 2 * kWsCh * kWsLd * sizeof(float);

__global__ __launch_bounds__(256) void k_wnorm_score(const float* __restrict__ w, int64_t k,
                                                     int64_t n, int64_t m_cal,
                                                     double* __restrict__ score) {
  extern __shared__ float tile[];  // [2][kWsCh][kWsLd]
  const int64_t c0 = (int64_t)blockIdx.x * kWsCh;
  const int tid = threadIdx.x;
  // loader: float4 f = tid + 256 i of a stage is row (tid >> 7) + 2 i, columns
  // 4 (tid & 127) .. +3; a wave reads 1 KiB of one row
  const int lrow = tid >> 7, lcol = (tid & 127) * 4;
  const bool vec = (n & 3) == 0 && (((uintptr_t)w) & 15) == 0;
  float4 r[16];
  auto load = [&](int64_t j0) {
    const int64_t j = j0 + lcol;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t c = c0 + lrow + 2 * i;
      float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (c < k) {
        const float* src = w + c * n + j;
        if (vec && j + 3 < n) {
          v = *(const float4*)src;
        } else {
          if (j < n) v.x = src[0];
          if (j + 1 < n) v.y = src[1];
          if (j + 2 < n) v.z = src[2];
          if (j + 3 < n) v.w = src[3];
        }
      }
      r[i] = v;
    }
  };
  double acc = 0.0;
  const int64_t stages = (n + kWsCols - 1) / kWsCols;
  load(0);
  for (int64_t st = 0; st < stages; ++st) {
    float* buf = tile + (st & 1) * kWsCh * kWsLd;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      *(float4*)(buf + (lrow + 2 * i) * kWsLd + lcol) = r[i];
    }
    __syncthreads();
    if (st + 1 < stages) load((st + 1) * kWsCols);
    if (tid < kWsCh) {
      const int64_t rem = n - st * kWsCols;
      const int jmax = rem < kWsCols ? (int)rem : kWsCols;
      const float* row = buf + tid * kWsLd;
      int col = 0;
      for (; col + 16 <= jmax; col += 16) {  // 16 LDS values ahead of the chain
        float4 q[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) q[u] = *(const float4*)(row + col + 4 * u);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          acc += (double)q[u].x * (double)q[u].x;
          acc += (double)q[u].y * (double)q[u].y;
          acc += (double)q[u].z * (double)q[u].z;
          acc += (double)q[u].w * (double)q[u].w;
        }
      }
      for (; col < jmax; ++col) {
        const double v = (double)row[col];
        acc += v * v;
      }
    }
  }
  if (tid < kWsCh && c0 + tid < k) {
    const int64_t c = c0 + tid;
    const double mean_abs = score[c] / (double)m_cal;
    score[c] = mean_abs * sqrt(acc);
  }
}

// Pass 3: rank[c] = #{c' : s[c'] > s[c] or (s[c'] == s[c] and c' < c)}.
// Block (x, y) compares 256 channels with the kRankSlice scores of slice y
// (staged in LDS) and adds its count to rank[c]; the counts are integers, so
// their order does not matter.
constexpr int kRankSlice = 1024;

__global__ __launch_bounds__(256) void k_rank(const double* __restrict__ score, int64_t k,
                                              int32_t* __restrict__ rank) {
  __shared__ double chunk[kRankSlice];
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t base = (int64_t)blockIdx.y * kRankSlice;
  for (int e = threadIdx.x; e < kRankSlice; e += 256) chunk[e] = base + e < k ? score[base + e] : 0.0;
  __syncthreads();
  if (c >= k) return;
  const double s = score[c];
  const int lim = k - base < kRankSlice ? (int)(k - base) : kRankSlice;
  // channels base + e < c win ties, the others need a strictly larger score
  const int64_t split = c - base < 0 ? 0 : (c - base > lim ? lim : c - base);
  int cnt = 0;
  int e = 0;
#pragma unroll 8
  for (; e < (int)split; ++e) cnt += chunk[e] >= s;
#pragma unroll 8
  for (; e < lim; ++e) cnt += chunk[e] > s;
  if (cnt) atomicAdd(&rank[c], cnt);
}

// Pass 4 (one block): channel c is an outlier when rank[c] < k_out (rank is
// held in map[]); an exclusive scan over the flags gives idx (ascending) and
// the channel map.
__global__ __launch_bounds__(1024) void k_flags_to_map(int32_t* __restrict__ map, int64_t k,
                                                       int64_t k_out, int32_t* __restrict__ idx) {
  __shared__ int wave_tot[16];
  __shared__ int carry;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int64_t base = 0; base < k; base += 1024) {
    int64_t c = base + tid;
    int f = c < k ? (map[c] < k_out ? 1 : 0) : 0;
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
  hipError_t e = hipFuncSetAttribute((const void*)k_wnorm_score,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kWsSmem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_colstats_x, dim3((unsigned)((k + 63) / 64)), dim3(64), 0, s, x_cal, m_cal,
                     k, score, hdiag, map);
  hipLaunchKernelGGL(k_wnorm_score, dim3((unsigned)((k + kWsCh - 1) / kWsCh)), dim3(256), kWsSmem,
                     s, w, k, n, m_cal, score);
  hipLaunchKernelGGL(k_rank, dim3((unsigned)((k + 255) / 256), (unsigned)((k + kRankSlice - 1) / kRankSlice)),
                     dim3(256), 0, s, score, k, map);
  hipLaunchKernelGGL(k_flags_to_map, dim3(1), dim3(1024), 0, s, map, k, k_out, idx);
  return hipGetLastError();
}

}  // namespace sqf
