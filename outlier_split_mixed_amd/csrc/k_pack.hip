// k_pack.hip -- offline weight conversion on the GPU.
//
// Channel-split format (OSC abstract: low-precision 4-bit GEMM over the
// ordinary channels, high-precision branch over the outlier channels): for
// every output channel n, the weights of the low channels in slot order are
// quantised per output channel to int4 and packed; the outlier channels'
// weights form the branch row (bf16 / E4M3 / int8).
//
// Weight-side SQ-format (SQ-format article, section 九: dense low-precision
// codes in which the unused code of symmetric quantisation marks the
// high-precision positions, a sparse high-precision part, positions chosen
// per bank as the top fraction by a weight x Hessian-diagonal score; section
// 三: the marked positions are served by a separate gather): the bank is one
// output row; the nnz low slots with the largest w^2 * hdiag (fp64; ties to
// the lower slot) get nibble 0x8 and keep an int8 value with its own scale;
// the other slots are int4 with an absmax taken over them only.
#include "sqf_device.h"
#include "sqf_launch.h"

namespace sqf {

// One thread per output channel; reads of W[c][n] are coalesced across the
// wave, map[c] is wave-uniform.  Two passes over the column: absmax, codes.
template <int BR>
__global__ __launch_bounds__(256) void k_pack_osc(PackArgs p) {
  const int64_t g = blockIdx.y;
  const int64_t nn = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (nn >= p.n) return;
  const float* w = p.w + g * p.k * p.n;
  const int32_t* map = p.map + g * p.k;
  uint8_t* wl = p.w_low + (g * p.n + nn) * p.ldk;
  constexpr int ESZ = BR == kBF16 ? 2 : 1;
  uint8_t* wo = p.w_out ? p.w_out + (g * p.n + nn) * p.ldo * ESZ : nullptr;

  float alo = 0.0f, ahi = 0.0f;
  for (int64_t c = 0; c < p.k; ++c) {
    float a = fabsf(w[c * p.n + nn]);
    if (map[c] >= 0) alo = fmaxf(alo, a); else ahi = fmaxf(ahi, a);
  }
  const float inv = quant_inv(alo, 7.0f);
  p.s_w[g * p.n + nn] = quant_scale(alo, 7.0f);
  const float qhi = BR == kFP8 ? 448.0f : 127.0f;
  const float inv_hi = BR == kBF16 ? 0.0f : quant_inv(ahi, qhi);
  if (BR != kBF16 && p.s_wo) p.s_wo[g * p.n + nn] = quant_scale(ahi, qhi);

  uint32_t buf[4] = {0, 0, 0, 0};
  int cnt = 0;
  int64_t grp = 0;
  for (int64_t c = 0; c < p.k; ++c) {
    const int32_t s = map[c];
    const float v = w[c * p.n + nn];
    if (s >= 0) {
      uint32_t nib = (uint32_t)quant_code(v, inv, 7.0f) & 0xFu;
      buf[cnt >> 3] |= nib << ((cnt & 7) * 4);
      if (++cnt == 32) {
        *(uint4*)(wl + grp * 16) = make_uint4(buf[0], buf[1], buf[2], buf[3]);
        buf[0] = buf[1] = buf[2] = buf[3] = 0;
        cnt = 0;
        ++grp;
      }
    } else {
      const int t = -s - 1;
      if constexpr (BR == kBF16) ((uint16_t*)wo)[t] = (uint16_t)bf16_rne(v);
      else if constexpr (BR == kFP8) wo[t] = (uint8_t)e4m3_rne_sat(v * inv_hi);
      else wo[t] = (uint8_t)quant_code(v, inv_hi, 127.0f);
    }
  }
  for (; grp < p.ldk / 16; ++grp) {  // flush the partial group, then zero padding
    *(uint4*)(wl + grp * 16) = make_uint4(buf[0], buf[1], buf[2], buf[3]);
    buf[0] = buf[1] = buf[2] = buf[3] = 0;
  }
  for (int64_t t = p.k_out * ESZ; t < p.ldo * ESZ; ++t) wo[t] = 0;
}

// Block-wide helpers for the weight-side kernel (256 threads).
__device__ __forceinline__ int block_sum_i(int v, int* scratch) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  v = wave_sum_i(v);
  __syncthreads();
  if (lane == 0) scratch[wv] = v;
  __syncthreads();
  int t = scratch[0] + scratch[1] + scratch[2] + scratch[3];
  return t;
}
__device__ __forceinline__ float block_max_f(float v, float* scratch) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  v = wave_max(v);
  __syncthreads();
  if (lane == 0) scratch[wv] = v;
  __syncthreads();
  return fmaxf(fmaxf(scratch[0], scratch[1]), fmaxf(scratch[2], scratch[3]));
}
// Exclusive prefix of v over the block in thread order; returns it.
__device__ __forceinline__ int block_excl_scan(int v, int* scratch) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int inc = wave_inclusive_scan(v);
  __syncthreads();
  if (lane == 63) scratch[wv] = inc;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < wv; ++i) before += scratch[i];
  return before + inc - v;
}

// One block (256 threads) per output channel.  Thread t owns the contiguous
// slot range [t*per, (t+1)*per) so block scans give slot order directly.
__global__ __launch_bounds__(256) void k_pack_sq(PackArgs p) {
  extern __shared__ uint8_t sm[];
  __shared__ int iscr[8];
  __shared__ float fscr[8];
  const int64_t nn = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t kl = p.k_low;
  float* vals = (float*)sm;                   // [k_low]
  float* hd = vals + kl;                      // [k_low]
  float* ov = hd + kl;                        // [k_out]
  uint8_t* keep = (uint8_t*)(ov + p.k_out);   // [k_low]

  for (int64_t c = tid; c < p.k; c += 256) {
    const int32_t s = p.map[c];
    const float v = p.w[c * p.n + nn];
    if (s >= 0) {
      vals[s] = v;
      hd[s] = p.hdiag[c];
    } else {
      ov[-s - 1] = v;
    }
  }
  __syncthreads();
  const int64_t per = (kl + 255) / 256;
  const int64_t j0 = tid * per, j1 = j0 + per < kl ? j0 + per : kl;
  auto keybits = [&](int64_t j) -> uint64_t {
    double wv = (double)vals[j];
    double key = wv * wv * (double)hd[j];  // >= 0: bit pattern is monotone
    return (uint64_t)__double_as_longlong(key);
  };
  // threshold T = nnz-th largest key (bitwise binary search over the keys)
  uint64_t T = 0;
  if (p.nnz > 0) {
    for (int bit = 63; bit >= 0; --bit) {
      uint64_t cand = T | (1ull << bit);
      int cnt = 0;
      for (int64_t j = j0; j < j1; ++j) cnt += keybits(j) >= cand;
      if (block_sum_i(cnt, iscr) >= p.nnz) T = cand;
    }
  }
  // keep = key > T, plus the lowest-slot keys equal to T until nnz are kept
  int gt = 0, eq = 0;
  if (p.nnz > 0)
    for (int64_t j = j0; j < j1; ++j) {
      uint64_t kb = keybits(j);
      gt += kb > T;
      eq += kb == T;
    }
  const int n_gt = block_sum_i(gt, iscr);
  int eq_before = block_excl_scan(eq, iscr);
  const int need = (int)p.nnz - n_gt;
  float a8 = 0.0f, a4 = 0.0f;
  for (int64_t j = j0; j < j1; ++j) {
    uint8_t kp = 0;
    if (p.nnz > 0) {
      uint64_t kb = keybits(j);
      if (kb > T) kp = 1;
      else if (kb == T) kp = (eq_before++ < need) ? 1 : 0;
    }
    keep[j] = kp;
    if (kp) a8 = fmaxf(a8, fabsf(vals[j])); else a4 = fmaxf(a4, fabsf(vals[j]));
  }
  a8 = block_max_f(a8, fscr);
  a4 = block_max_f(a4, fscr);
  const float inv8 = quant_inv(a8, 127.0f), inv4 = quant_inv(a4, 7.0f);
  if (tid == 0) {
    p.s_w8[nn] = quant_scale(a8, 127.0f);
    p.s_w[nn] = quant_scale(a4, 7.0f);
  }
  // int8 values in ascending slot order
  int kc = 0;
  for (int64_t j = j0; j < j1; ++j) kc += keep[j];
  int pos = block_excl_scan(kc, iscr);
  for (int64_t j = j0; j < j1; ++j)
    if (keep[j]) p.sq_val[nn * p.nnz + pos++] = (int8_t)quant_code(vals[j], inv8, 127.0f);
  __syncthreads();
  // packed row: 16-byte groups of 32 slots
  uint8_t* wl = p.w_low + nn * p.ldk;
  for (int64_t q = tid; q < p.ldk / 16; q += 256) {
    uint32_t ow[4] = {0, 0, 0, 0};
    for (int e = 0; e < 32; ++e) {
      int64_t j = q * 32 + e;
      uint32_t nib = 0;
      if (j < kl) nib = keep[j] ? 0x8u : ((uint32_t)quant_code(vals[j], inv4, 7.0f) & 0xFu);
      ow[e >> 3] |= nib << ((e & 7) * 4);
    }
    *(uint4*)(wl + q * 16) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
  }
  // marked-slot count before each 256-slot tile
  const int64_t ntiles = p.ldk / 128;
  for (int64_t t = tid; t <= ntiles; t += 256) {
    int cnt = 0;
    int64_t lim = t * 256 < kl ? t * 256 : kl;
    for (int64_t j = 0; j < lim; ++j) cnt += keep[j];
    p.tile_off[nn * (ntiles + 1) + t] = cnt;
  }
  // int8 branch over the outlier channels
  float ao = 0.0f;
  for (int64_t t = tid; t < p.k_out; t += 256) ao = fmaxf(ao, fabsf(ov[t]));
  ao = block_max_f(ao, fscr);
  const float invo = quant_inv(ao, 127.0f);
  if (tid == 0 && p.s_wo) p.s_wo[nn] = quant_scale(ao, 127.0f);
  for (int64_t t = tid; t < p.ldo; t += 256)
    p.w_out[nn * p.ldo + t] = t < p.k_out ? (uint8_t)quant_code(ov[t], invo, 127.0f) : 0;
}

hipError_t launch_pack(const PackArgs& a, int branch, int groups, hipStream_t s) {
  if (a.nnz > 0) {
    size_t lds = (size_t)a.k_low * 9 + (size_t)a.k_out * 4 + 16;
    if (lds > 65536) {
      hipError_t e = hipFuncSetAttribute((const void*)k_pack_sq,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_pack_sq, dim3((unsigned)a.n), dim3(256), lds, s, a);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((a.n + 255) / 256), (unsigned)groups);
  if (branch == kBF16) hipLaunchKernelGGL(k_pack_osc<kBF16>, grid, dim3(256), 0, s, a);
  else if (branch == kFP8) hipLaunchKernelGGL(k_pack_osc<kFP8>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_pack_osc<kI8>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace sqf
