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
// lane (8 channels); the next row is loaded while the current one is
// processed.  The channel map is read once per block and condensed to one
// word per 8-channel chunk.  Codes are scattered into an LDS staging row by
// slot, then read back in slot order and written with 16-byte stores, so every
// HBM write is coalesced.  The absmax is a wave max over shuffles followed by
// a cross-wave max in LDS; block barriers wait for LDS traffic only.
#include <cstdlib>

#include "sqf_device.h"
#include "sqf_launch.h"

namespace sqf {

// Barrier for LDS hand-offs only: waits for this wave's LDS operations, then
// s_barrier.  Unlike __syncthreads() it does not wait for outstanding global
// loads, so the next row's prefetch stays in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt untouched
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int XT, int LOW, int BR, bool GROUPED, int NT, int CPT>
__global__ __launch_bounds__(NT) void k_act_split(ActArgs p) {
  extern __shared__ uint8_t sm[];
  constexpr int ESZ = BR == kBF16 ? 2 : 1;
  constexpr int NW = NT / 64;
  constexpr int OPT = 4;  // outlier channels gathered per thread per pass
  // LDS: [pad_lo + 16] code bytes (the last 16 are a dump slot written by
  // outlier lanes) | [k_out] int32 outlier channel list | reduction scratch
  uint8_t* codes = sm;
  const int dump_lo = (int)p.pad_lo;
  int32_t* oidx = (int32_t*)(sm + p.pad_lo + 16);
  float* red = (float*)(sm + p.pad_lo + 16 + ((p.k_out * 4 + 15) & ~(int64_t)15));
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const float qlow = LOW == kI4X2 ? 7.0f : 127.0f;
  const float qhi = BR == kFP8 ? 448.0f : 127.0f;
  const int k_out = (int)p.k_out;

  // padding slots are never written by the scatter below: zero them once
  for (int64_t j = p.k_low + tid; j < p.pad_lo; j += NT) codes[j] = 0;

  // One word per 8-channel chunk: (low slots before the chunk) << 8 | mask of
  // the chunk's outlier channels.  The outlier channel list goes to LDS.
  uint32_t cw[CPT];
  auto load_map = [&](int g) {
    const int32_t* mp = p.map + (int64_t)g * p.k;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int64_t c8 = ((int64_t)tid + (int64_t)i * NT) * 8;
      cw[i] = 0;
      if (c8 < p.k) {
        const int4 u0 = *(const int4*)(mp + c8);
        const int4 u1 = *(const int4*)(mp + c8 + 4);
        const int m8[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
        uint32_t mask = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          mask |= (m8[e] < 0 ? 1u : 0u) << e;
          if (m8[e] < 0) oidx[-m8[e] - 1] = (int32_t)(c8 + e);
        }
        const int64_t before = m8[0] >= 0 ? m8[0] : c8 - (-m8[0] - 1);
        cw[i] = ((uint32_t)before << 8) | mask;
      }
    }
  };
  // one map for every row: load it once, outside the row loop (a load inside
  // the loop would make every iteration wait for all outstanding loads)
  int cached_group = -1;
  if constexpr (!GROUPED) load_map(0);

  // raw row words: 4 per chunk for bf16, 8 for fp32; the next row's words are
  // loaded while the current row is processed
  constexpr int WPC = XT == kBF16 ? 4 : 8;
  typedef uint32_t v4u __attribute__((ext_vector_type(4)));
  auto load_raw = [&](int64_t row, uint32_t (&r)[CPT][WPC]) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int64_t c8 = ((int64_t)tid + (int64_t)i * NT) * 8;
      if (c8 < p.k) {
        const v4u* src = XT == kBF16 ? (const v4u*)((const uint16_t*)p.x + row * p.ldx + c8)
                                     : (const v4u*)((const float*)p.x + row * p.ldx + c8);
#pragma unroll
        for (int h = 0; h < WPC / 4; ++h) {
          const v4u u = src[h];
          r[i][4 * h] = u[0]; r[i][4 * h + 1] = u[1]; r[i][4 * h + 2] = u[2]; r[i][4 * h + 3] = u[3];
        }
      } else {
#pragma unroll
        for (int w = 0; w < WPC; ++w) r[i][w] = 0;
      }
    }
  };
  auto val = [&](const uint32_t (&r)[CPT][WPC], int i, int e) -> float {
    if constexpr (XT == kBF16) {
      const uint32_t w = r[i][e >> 1];
      return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
    } else {
      return __uint_as_float(r[i][e]);
    }
  };
  auto xval = [&](int64_t row, int c) -> float {
    if constexpr (XT == kBF16) return __uint_as_float((uint32_t)((const uint16_t*)p.x)[row * p.ldx + c] << 16);
    else return ((const float*)p.x)[row * p.ldx + c];
  };
  uint32_t raw[CPT][WPC], nxt[CPT][WPC];
  if (blockIdx.x < p.m) load_raw(blockIdx.x, raw);
  lds_barrier();  // outlier list and padding in place

  for (int64_t m = blockIdx.x; m < p.m; m += gridDim.x) {
    if constexpr (GROUPED) {
      int lo = 0, hi = p.groups;  // largest g with row_off[g] <= m
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.row_off[mid] <= m) lo = mid; else hi = mid;
      }
      if (lo != cached_group) {
        lds_barrier();  // nobody still reads the previous group's outlier list
        load_map(lo);
        cached_group = lo;
        lds_barrier();
      }
    }
    // ---- outlier channels: gathered from the row (cache-resident).  Issued
    // before the next-row prefetch: loads retire in order, so waiting for
    // these does not wait for the prefetch. ----
    float ov[OPT];
#pragma unroll
    for (int u = 0; u < OPT; ++u) {
      const int t = tid + u * NT;
      ov[u] = t < k_out ? xval(m, oidx[t]) : 0.0f;
    }
    if (m + gridDim.x < p.m) load_raw(m + gridDim.x, nxt);
    // Register pressure: the chunk words are constant across rows and the
    // decoded values are needed twice; without these opaque redefinitions the
    // compiler keeps every derived value live across the whole loop.
#pragma unroll
    for (int i = 0; i < CPT; ++i) asm volatile("" : "+v"(cw[i]));
    // ---- absmax over the low channels (and the outlier channels) ----
    float alo = 0.0f, ahi = 0.0f;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float t = fabsf(val(raw, i, e));
        alo = fmaxf(alo, ((cw[i] >> e) & 1u) ? 0.0f : t);
      }
    }
    if constexpr (BR != kBF16) {
#pragma unroll
      for (int u = 0; u < OPT; ++u) ahi = fmaxf(ahi, fabsf(ov[u]));
      for (int t = OPT * NT + tid; t < k_out; t += NT) ahi = fmaxf(ahi, fabsf(xval(m, oidx[t])));
    }
    alo = wave_max(alo);
    if constexpr (BR != kBF16) ahi = wave_max(ahi);
    if (lane == 0) {
      red[wv] = alo;
      red[NW + wv] = ahi;
    }
    lds_barrier();
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
    // ---- branch row: coalesced direct stores, zero padding up to ldo ----
    uint8_t* xo = p.x_out + m * p.ldo * ESZ;
#pragma unroll
    for (int u = 0; u < OPT; ++u) {
      const int t = tid + u * NT;
      if (t < k_out) {
        if constexpr (BR == kBF16) ((uint16_t*)xo)[t] = (uint16_t)bf16_rne(ov[u]);
        else if constexpr (BR == kFP8) xo[t] = (uint8_t)e4m3_rne_sat(ov[u] * inv_hi);
        else xo[t] = (uint8_t)quant_code(ov[u], inv_hi, qhi);
      }
    }
    for (int t = OPT * NT + tid; t < k_out; t += NT) {  // outliers beyond the registers
      const float x = xval(m, oidx[t]);
      if constexpr (BR == kBF16) ((uint16_t*)xo)[t] = (uint16_t)bf16_rne(x);
      else if constexpr (BR == kFP8) xo[t] = (uint8_t)e4m3_rne_sat(x * inv_hi);
      else xo[t] = (uint8_t)quant_code(x, inv_hi, qhi);
    }
    for (int64_t t = k_out + tid; t < p.ldo; t += NT) {
      if constexpr (BR == kBF16) ((uint16_t*)xo)[t] = 0;
      else xo[t] = 0;
    }
#pragma unroll
    for (int i = 0; i < CPT; ++i)
#pragma unroll
      for (int w = 0; w < WPC; ++w) asm volatile("" : "+v"(raw[i][w]));
    // ---- low codes -> LDS staging row (outlier lanes write a dump slot) ----
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int64_t c8 = ((int64_t)tid + (int64_t)i * NT) * 8;
      if (c8 < p.k) {
        int slot = (int)(cw[i] >> 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const bool out = (cw[i] >> e) & 1u;
          codes[out ? dump_lo : slot] = (uint8_t)quant_code(val(raw, i, e), inv_lo, qlow);
          slot += out ? 0 : 1;
        }
      }
    }
    lds_barrier();
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
    lds_barrier();
#pragma unroll
    for (int i = 0; i < CPT; ++i)
#pragma unroll
      for (int w = 0; w < WPC; ++w) raw[i][w] = nxt[i][w];
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
  size_t lds = (size_t)(a.pad_lo + 16 + ((a.k_out * 4 + 15) & ~(int64_t)15)) + 2 * 16 * sizeof(float);
  // rows per block: SQF_ACT_GRID overrides the grid size (tuning aid)
  const char* env = getenv("SQF_ACT_GRID");
  const int64_t cap = env ? atoll(env) : 1024;
  int64_t grid = a.m < cap ? a.m : cap;
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
