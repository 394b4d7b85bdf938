// k_act.hip -- online per-token quantisation and outlier extraction.
//
// One pass over each activation row: the per-token absmax over the low
// channels, int4 (or int8) codes for those channels compacted into slot order
// and packed, and the outlier channels gathered into the compact dense branch
// row.  This is OSC's structured sub-tensor extraction (abstract: the
// scattered outlier channels are coalesced online into one dense tensor) and
// the per-token low-precision activation path of both pages.
//
// Memory plan (HBM-bound kernel): each row is read once with 16-byte loads per
// lane (8 channels), the channel map comes from L2 (the same [k] array for
// every row) and is kept in registers while a block walks several rows.
// Codes are scattered into an LDS staging row by slot, then read back in slot
// order and written with 16-byte stores, so every HBM write is coalesced.
// The absmax is a wave max over shuffles followed by a cross-wave max in LDS.
#include "sqf_device.h"
#include "sqf_launch.h"

namespace sqf {

template <int XT, int LOW, int BR, bool GROUPED, int NT, int CPT>
__global__ __launch_bounds__(NT) void k_act_split(ActArgs p) {
  extern __shared__ uint8_t sm[];
  // LDS: [pad_lo] code bytes | [ldo * esz] branch codes | reduction scratch
  constexpr int ESZ = BR == kBF16 ? 2 : 1;
  constexpr int NW = NT / 64;
  uint8_t* codes = sm;
  uint8_t* bcodes = sm + p.pad_lo;
  float* red = (float*)(sm + ((p.pad_lo + p.ldo * ESZ + 15) & ~(int64_t)15));
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const float qlow = LOW == kI4X2 ? 7.0f : 127.0f;
  const float qhi = BR == kFP8 ? 448.0f : 127.0f;

  // padding slots are never written by the scatter below: zero them once
  for (int64_t j = p.k_low + tid; j < p.pad_lo; j += NT) codes[j] = 0;
  for (int64_t t = p.k_out * ESZ + tid; t < p.ldo * ESZ; t += NT) bcodes[t] = 0;

  int32_t mreg[CPT][8];
  int cached_group = -1;

  for (int64_t m = blockIdx.x; m < p.m; m += gridDim.x) {
    int g = 0;
    if constexpr (GROUPED) {
      int lo = 0, hi = p.groups;  // largest g with row_off[g] <= m
      while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (p.row_off[mid] <= m) lo = mid; else hi = mid;
      }
      g = lo;
    }
    if (g != cached_group) {
      const int32_t* mp = p.map + (int64_t)g * p.k;
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        int64_t c8 = ((int64_t)tid + (int64_t)i * NT) * 8;
        if (c8 < p.k) {
          int4 u0 = *(const int4*)(mp + c8);
          int4 u1 = *(const int4*)(mp + c8 + 4);
          mreg[i][0] = u0.x; mreg[i][1] = u0.y; mreg[i][2] = u0.z; mreg[i][3] = u0.w;
          mreg[i][4] = u1.x; mreg[i][5] = u1.y; mreg[i][6] = u1.z; mreg[i][7] = u1.w;
        }
      }
      cached_group = g;
    }
    // ---- load the row (16 B per lane per chunk) ----
    float v[CPT][8];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      int64_t c8 = ((int64_t)tid + (int64_t)i * NT) * 8;
      if (c8 < p.k) {
        if constexpr (XT == kBF16) {
          uint4 u = *(const uint4*)((const uint16_t*)p.x + m * p.ldx + c8);
          uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[i][2 * e] = __uint_as_float(w4[e] << 16);
            v[i][2 * e + 1] = __uint_as_float(w4[e] & 0xFFFF0000u);
          }
        } else {
          const float* xr = (const float*)p.x + m * p.ldx + c8;
          float4 a = *(const float4*)xr, b = *(const float4*)(xr + 4);
          v[i][0] = a.x; v[i][1] = a.y; v[i][2] = a.z; v[i][3] = a.w;
          v[i][4] = b.x; v[i][5] = b.y; v[i][6] = b.z; v[i][7] = b.w;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[i][e] = 0.0f;
      }
    }
    // ---- absmax over low (and outlier) channels ----
    float alo = 0.0f, ahi = 0.0f;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      int64_t c8 = ((int64_t)tid + (int64_t)i * NT) * 8;
      if (c8 < p.k) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float t = fabsf(v[i][e]);
          if (mreg[i][e] >= 0) alo = fmaxf(alo, t); else ahi = fmaxf(ahi, t);
        }
      }
    }
    alo = wave_max(alo);
    if constexpr (BR != kBF16) ahi = wave_max(ahi);
    if (lane == 0) {
      red[wv] = alo;
      red[NW + wv] = ahi;
    }
    __syncthreads();
    alo = red[0];
    ahi = red[NW];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      alo = fmaxf(alo, red[w]);
      ahi = fmaxf(ahi, red[NW + w]);
    }
    const float inv_lo = quant_inv(alo, qlow);
    const float inv_hi = BR == kBF16 ? 0.0f : quant_inv(ahi, qhi);
    if (tid == 0) {
      p.s_x[m] = quant_scale(alo, qlow);
      if constexpr (BR != kBF16) p.s_xo[m] = quant_scale(ahi, qhi);
    }
    // ---- codes -> LDS staging row ----
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      int64_t c8 = ((int64_t)tid + (int64_t)i * NT) * 8;
      if (c8 < p.k) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          int32_t s = mreg[i][e];
          if (s >= 0) {
            codes[s] = (uint8_t)quant_code(v[i][e], inv_lo, qlow);
          } else {
            int t = -s - 1;
            if constexpr (BR == kBF16) {
              ((uint16_t*)bcodes)[t] = (uint16_t)bf16_rne(v[i][e]);
            } else if constexpr (BR == kFP8) {
              bcodes[t] = (uint8_t)e4m3_rne_sat(v[i][e] * inv_hi);
            } else {
              bcodes[t] = (uint8_t)quant_code(v[i][e], inv_hi, qhi);
            }
          }
        }
      }
    }
    __syncthreads();
    // ---- LDS -> packed HBM rows, 16-byte stores ----
    const int64_t ngrp = p.ldk / 16;
    uint8_t* xl = p.x_low + m * p.ldk;
    for (int64_t q = tid; q < ngrp; q += NT) {
      uint4 o;
      if constexpr (LOW == kI4X2) {
        const uint32_t* src = (const uint32_t*)(codes + q * 32);
        uint32_t ow[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          uint32_t t0 = src[2 * h] & 0x0F0F0F0Fu, t1 = src[2 * h + 1] & 0x0F0F0F0Fu;
          uint32_t s0 = t0 | (t0 >> 4), s1 = t1 | (t1 >> 4);
          uint32_t p0 = (s0 & 0xFFu) | ((s0 >> 8) & 0xFF00u);
          uint32_t p1 = (s1 & 0xFFu) | ((s1 >> 8) & 0xFF00u);
          ow[h] = p0 | (p1 << 16);
        }
        o = make_uint4(ow[0], ow[1], ow[2], ow[3]);
      } else {
        o = *(const uint4*)(codes + q * 16);
      }
      *(uint4*)(xl + q * 16) = o;
    }
    const int64_t ogrp = p.ldo * ESZ / 16;
    uint8_t* xo = p.x_out + m * p.ldo * ESZ;
    for (int64_t q = tid; q < ogrp; q += NT) *(uint4*)(xo + q * 16) = *(const uint4*)(bcodes + q * 16);
    __syncthreads();
  }
}

template <int XT, int LOW, int BR, bool GROUPED, int NT, int CPT>
static hipError_t launch_one(const ActArgs& a, int64_t grid, size_t lds, hipStream_t s) {
  auto kern = k_act_split<XT, LOW, BR, GROUPED, NT, CPT>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NT), lds, s, a);
  return hipGetLastError();
}

template <int XT, int LOW, int BR, bool GROUPED>
static hipError_t launch_shape(const ActArgs& a, int64_t grid, size_t lds, hipStream_t s) {
  const int64_t chunks = a.k / 8;
  if (chunks <= 256) return launch_one<XT, LOW, BR, GROUPED, 256, 1>(a, grid, lds, s);
  if (chunks <= 512) return launch_one<XT, LOW, BR, GROUPED, 256, 2>(a, grid, lds, s);
  if (chunks <= 1024) return launch_one<XT, LOW, BR, GROUPED, 256, 4>(a, grid, lds, s);
  if (chunks <= 2048) return launch_one<XT, LOW, BR, GROUPED, 512, 4>(a, grid, lds, s);
  if (chunks <= 4096) return launch_one<XT, LOW, BR, GROUPED, 1024, 4>(a, grid, lds, s);
  return launch_one<XT, LOW, BR, GROUPED, 1024, 8>(a, grid, lds, s);
}

template <int XT, int LOW, bool GROUPED>
static hipError_t launch_br(const ActArgs& a, int br, int64_t grid, size_t lds, hipStream_t s) {
  if (br == kBF16) return launch_shape<XT, LOW, kBF16, GROUPED>(a, grid, lds, s);
  if (br == kFP8) return launch_shape<XT, LOW, kFP8, GROUPED>(a, grid, lds, s);
  return launch_shape<XT, LOW, kI8, GROUPED>(a, grid, lds, s);
}

hipError_t launch_act_split(const ActArgs& a, int x_dtype, int low, int branch, bool grouped,
                            hipStream_t s) {
  const int esz = branch == kBF16 ? 2 : 1;
  size_t lds = (size_t)((a.pad_lo + a.ldo * esz + 15) & ~(int64_t)15) + 2 * 16 * sizeof(float);
  int64_t grid = a.m < 2048 ? a.m : 2048;
  if (grid <= 0) return hipSuccess;
  if (x_dtype == kBF16) {
    if (low == kI4X2)
      return grouped ? launch_br<kBF16, kI4X2, true>(a, branch, grid, lds, s)
                     : launch_br<kBF16, kI4X2, false>(a, branch, grid, lds, s);
    return grouped ? launch_br<kBF16, kI8, true>(a, branch, grid, lds, s)
                   : launch_br<kBF16, kI8, false>(a, branch, grid, lds, s);
  }
  if (low == kI4X2)
    return grouped ? launch_br<kF32, kI4X2, true>(a, branch, grid, lds, s)
                   : launch_br<kF32, kI4X2, false>(a, branch, grid, lds, s);
  return grouped ? launch_br<kF32, kI8, true>(a, branch, grid, lds, s)
                 : launch_br<kF32, kI8, false>(a, branch, grid, lds, s);
}

}  // namespace sqf
