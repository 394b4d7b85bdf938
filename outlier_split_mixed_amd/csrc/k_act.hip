// k_act.hip -- online per-token quantisation and outlier extraction.
//
// One pass over each activation row: the per-token absmax over the low
// channels, int4 (or int8) codes for those channels compacted into slot order
// and packed, and the outlier channels gathered into the compact dense branch
// row.  This is OSC's structured sub-tensor extraction (abstract: the
// scattered outlier channels are coalesced online into one dense tensor) and
// the per-token low-precision activation path of both pages.
//
// Memory plan (HBM-bound kernel): a block owns a row at a time; each lane
// reads 16 bytes (8 channels, one "chunk") per load and the next row is loaded
// while the current one is processed.  The channel map is static, so it is
// condensed once per block into per-chunk constants: the number of low slots
// before the chunk, the chunk's outlier mask, the absmax mask and two byte-
// permute selectors that drop the chunk's outlier codes.
//
// Arithmetic per chunk:
//   absmax   |x| of bf16 data is compared as 15-bit integers, two channels per
//            packed u16 max (integer order equals float order for |x|);
//   codes    y = fl(x * inv) + 1.5 * 2^23 rounds fl(x * inv) to the nearest
//            integer, ties to even (the addition's own rounding), and leaves
//            that integer in the low mantissa bits: the low byte of y's bit
//            pattern is the two's complement code.  |fl(x * inv)| <= Q(1+2^-23)
//            because the absmax covers every low channel, so no clamp is
//            needed;
//   packing  the code bytes are compacted with byte permutes, nibble-packed
//            in registers and OR-ed (two LDS atomics per chunk) into a zeroed
//            LDS image of the packed row at the chunk's slot offset.
// The image is read back with 16-byte loads, stored coalesced to HBM and
// re-zeroed.  Two images and two reduction slots alternate between rows, so
// a row needs two barriers (absmax, image complete); the barriers wait for
// LDS traffic only, never for the next row's loads.
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

// v_perm_b32: byte j of the result is byte sel.byte[j] of the pool {hi, lo}
// (0..3 = lo's bytes, 4..7 = hi's bytes, 0x0C = zero).
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

constexpr float kRoundMagic = 12582912.0f;  // 1.5 * 2^23

// Bytes of the image row beyond ldk that the OR of a chunk's upper part may
// touch (always with zero data at the very end of the row).
constexpr int kImgSlack = 16;

template <int XT, int LOW, int BR, bool GROUPED, int NT, int CPT>
__global__ __launch_bounds__(NT) void k_act_split(ActArgs p) {
  extern __shared__ uint8_t sm[];
  constexpr int ESZ = BR == kBF16 ? 2 : 1;
  constexpr int NW = NT / 64;
  constexpr int OPT = 4;  // outlier channels gathered per thread per pass
  constexpr int WPC = XT == kBF16 ? 4 : 8;  // raw words per 8-channel chunk
  const int64_t ldk = p.ldk;
  const int img_bytes = (int)ldk + kImgSlack;  // a multiple of 16
  // LDS: image[2][ldk + slack] | outlier channel list int32[k_out] |
  // reduction slots float[2][2 * NW]
  uint8_t* img0 = sm;
  int32_t* oidx = (int32_t*)(sm + 2 * img_bytes);
  float* red = (float*)(sm + 2 * img_bytes + ((p.k_out * 4 + 15) & ~(int64_t)15));
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const float qlow = LOW == kI4X2 ? 7.0f : 127.0f;
  const float qhi = BR == kFP8 ? 448.0f : 127.0f;
  const int k_out = (int)p.k_out;

  // both images start zeroed
  for (int j = tid * 16; j < 2 * img_bytes; j += NT * 16) *(uint4*)(img0 + j) = make_uint4(0, 0, 0, 0);

  // Per-chunk constants (chunk i of this thread = channels 8*(tid + i*NT) ..+7):
  //   cw   (low slots before the chunk) << 8 | outlier mask (bit e = channel e)
  //   am   absmax masks: 0x7FFF per low channel's bf16 half, 0 for outliers
  //   sel  byte-permute selectors taking the low channels' code bytes, in
  //        order, to bytes 0.. of the compacted pair (zero beyond them)
  uint32_t cw[CPT], sel0[CPT], sel1[CPT], am[CPT][XT == kBF16 ? 4 : 1];
  auto load_map = [&](int g) {
    const int32_t* mp = p.map + (int64_t)g * p.k;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int64_t c8 = ((int64_t)tid + (int64_t)i * NT) * 8;
      uint32_t mask = 0xFFu, before = 0;
      if (c8 < p.k) {
        const int4 u0 = *(const int4*)(mp + c8);
        const int4 u1 = *(const int4*)(mp + c8 + 4);
        const int m8[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
        mask = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          mask |= (m8[e] < 0 ? 1u : 0u) << e;
          if (m8[e] < 0) oidx[-m8[e] - 1] = (int32_t)(c8 + e);
        }
        before = (uint32_t)(m8[0] >= 0 ? m8[0] : c8 - (-m8[0] - 1));
      }
      cw[i] = (before << 8) | mask;
      uint64_t sel = 0x0C0C0C0C0C0C0C0Cull;
      int j = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (!((mask >> e) & 1u)) {
          sel = (sel & ~(0xFFull << (8 * j))) | ((uint64_t)e << (8 * j));
          ++j;
        }
      }
      sel0[i] = (uint32_t)sel;
      sel1[i] = (uint32_t)(sel >> 32);
      if constexpr (XT == kBF16) {
#pragma unroll
        for (int d = 0; d < 4; ++d)
          am[i][d] = (((mask >> (2 * d)) & 1u) ? 0u : 0x7FFFu) |
                     (((mask >> (2 * d + 1)) & 1u) ? 0u : 0x7FFF0000u);
      } else {
        am[i][0] = mask;
      }
    }
  };
  // one map for every row: load it once, outside the row loop (a load inside
  // the loop would make every iteration wait for all outstanding loads)
  int cached_group = -1;
  if constexpr (!GROUPED) load_map(0);

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
  // fp32 value of channel e of chunk i
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
  // Rows of a block: a strided set (one map for all rows), or, for expert
  // groups, a contiguous run, so that the group (and its map) rarely changes
  // between consecutive rows of a block.
  int64_t m_first = blockIdx.x, m_stop = p.m, m_step = gridDim.x;
  int g_cur = 0;      // group of the current row (expert groups)
  int64_t g_end = 0;  // first row after it
  if constexpr (GROUPED) {
    const int64_t per = (p.m + gridDim.x - 1) / gridDim.x;
    m_first = (int64_t)blockIdx.x * per;
    m_stop = m_first + per < p.m ? m_first + per : p.m;
    m_step = 1;
    // largest g with row_off[g] <= m_first, once per block
    int lo = 0, hi = p.groups;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.row_off[mid] <= m_first) lo = mid; else hi = mid;
    }
    g_cur = lo;
    g_end = p.row_off[lo + 1];
  }
  // rows in flight ahead of the current one: enough bytes per thread to hide
  // HBM latency when a row is only a few chunks per thread
  constexpr int PF = CPT >= 4 ? 1 : 4 / CPT;
  // ring of PF + 1 row buffers; the row loop below is unrolled PF + 1 times so
  // that every buffer index is static (no register moves, which would wait
  // for the loads still in flight)
  uint32_t ring[PF + 1][CPT][WPC];
#pragma unroll
  for (int f = 0; f < PF; ++f)
    if (m_first + f * m_step < m_stop) load_raw(m_first + f * m_step, ring[f]);
  lds_barrier();  // outlier list and zeroed images in place

  // the group of row m (expert groups): the map and outlier list follow it
  auto enter_row = [&](int64_t m) {
    if constexpr (GROUPED) {
      // rows of a block are contiguous: advance to the group holding m
      while (m >= g_end) {
        ++g_cur;
        g_end = p.row_off[g_cur + 1];
      }
      if (g_cur != cached_group) {
        lds_barrier();  // nobody still reads the previous group's outlier list
        load_map(g_cur);
        cached_group = g_cur;
        lds_barrier();
      }
    }
  };
  // outlier channels of row m, gathered from the row (cache-resident).  The
  // row loop issues these before the next-row prefetch: loads retire in
  // order, so waiting for them does not wait for the prefetch.
  auto gather = [&](int64_t m, float (&ov)[OPT]) {
#pragma unroll
    for (int u = 0; u < OPT; ++u) {
      const int t = tid + u * NT;
      ov[u] = t < k_out ? xval(m, oidx[t]) : 0.0f;
    }
  };
  auto row_body = [&](int64_t m, int it, uint32_t (&raw)[CPT][WPC], const float (&ov)[OPT]) {
    const int buf = it & 1;
    uint8_t* img = img0 + buf * img_bytes;
    float* rd = red + buf * 2 * NW;
    // Register pressure: the per-chunk constants are row-invariant and the
    // raw words are read twice; without these opaque redefinitions the
    // compiler keeps every derived value live across the whole loop.
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      asm volatile("" : "+v"(cw[i]), "+v"(sel0[i]), "+v"(sel1[i]));
#pragma unroll
      for (int d = 0; d < (XT == kBF16 ? 4 : 1); ++d) asm volatile("" : "+v"(am[i][d]));
    }
    // ---- absmax over the low channels (and the outlier channels) ----
    float alo, ahi = 0.0f;
    if constexpr (XT == kBF16) {
      typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
      u16x2 mx = {0, 0};
#pragma unroll
      for (int i = 0; i < CPT; ++i)
#pragma unroll
        for (int d = 0; d < 4; ++d)
          mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, raw[i][d] & am[i][d]));
      alo = __uint_as_float((uint32_t)(mx[0] > mx[1] ? mx[0] : mx[1]) << 16);
    } else {
      uint32_t mx = 0;
#pragma unroll
      for (int i = 0; i < CPT; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t t = ((am[i][0] >> e) & 1u) ? 0u : (raw[i][e] & 0x7FFFFFFFu);
          mx = mx > t ? mx : t;
        }
      alo = __uint_as_float(mx);
    }
    if constexpr (BR != kBF16) {
#pragma unroll
      for (int u = 0; u < OPT; ++u) ahi = fmaxf(ahi, fabsf(ov[u]));
      for (int t = OPT * NT + tid; t < k_out; t += NT) ahi = fmaxf(ahi, fabsf(xval(m, oidx[t])));
    }
    alo = wave_max(alo);
    if constexpr (BR != kBF16) ahi = wave_max(ahi);
    if (lane == 0) {
      rd[wv] = alo;
      rd[NW + wv] = ahi;
    }
    lds_barrier();  // (A) partial maxima in place
    alo = rd[0];
    ahi = rd[NW];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      alo = fmaxf(alo, rd[w]);
      ahi = fmaxf(ahi, rd[NW + w]);
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
    // ---- low codes: compacted, packed and OR-ed into the image row ----
    uint32_t* im = (uint32_t*)img;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int64_t c8 = ((int64_t)tid + (int64_t)i * NT) * 8;
      if (c8 < p.k) {
        // code byte e = low byte of fl(fl(x_e * inv) + 1.5*2^23); the product
        // must be rounded on its own (a fused multiply-add would round the
        // exact product instead and differ at ties)
        uint32_t y[8];
        {
#pragma clang fp contract(off)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float prod = val(raw, i, e) * inv_lo;
            y[e] = __float_as_uint(prod + kRoundMagic);
          }
        }
        const uint32_t d0 = perm(y[1], y[0], 0x0C0C0400u) | (perm(y[3], y[2], 0x0C0C0400u) << 16);
        const uint32_t d1 = perm(y[5], y[4], 0x0C0C0400u) | (perm(y[7], y[6], 0x0C0C0400u) << 16);
        // the low channels' codes, in order, then zero bytes
        const uint32_t q0 = perm(d1, d0, sel0[i]), q1 = perm(d1, d0, sel1[i]);
        const uint32_t before = cw[i] >> 8;
        if constexpr (LOW == kI4X2) {
          const uint32_t t0 = q0 & 0x0F0F0F0Fu, t1 = q1 & 0x0F0F0F0Fu;
          const uint32_t u0 = t0 | (t0 >> 4), u1 = t1 | (t1 >> 4);
          const uint32_t w = perm(u1, u0, 0x06040200u);  // 8 nibbles, slot order
          const uint64_t v = (uint64_t)w << (4 * (before & 7u));
          atomicOr(im + (before >> 3), (uint32_t)v);
          atomicOr(im + (before >> 3) + 1, (uint32_t)(v >> 32));
        } else {
          const uint32_t sh = 8 * (before & 3u);
          const uint64_t lo = (uint64_t)q0 << sh;
          const uint64_t hi = (uint64_t)q1 << sh;
          atomicOr(im + (before >> 2), (uint32_t)lo);
          atomicOr(im + (before >> 2) + 1, (uint32_t)(lo >> 32) | (uint32_t)hi);
          atomicOr(im + (before >> 2) + 2, (uint32_t)(hi >> 32));
        }
      }
    }
    lds_barrier();  // (B) the image row is complete
    // ---- image -> packed HBM row (16-byte stores), then re-zero it ----
    uint8_t* xl = p.x_low + m * ldk;
    for (int64_t q = tid; q < ldk / 16; q += NT) {
      *(uint4*)(xl + q * 16) = *(const uint4*)(img + q * 16);
      *(uint4*)(img + q * 16) = make_uint4(0, 0, 0, 0);
    }
    if (tid == 0) *(uint4*)(img + ldk) = make_uint4(0, 0, 0, 0);  // slack
  };

  int it = 0;
  for (int64_t m = m_first; m < m_stop;) {
#pragma unroll
    for (int u = 0; u <= PF; ++u) {
      if (m >= m_stop) break;
      enter_row(m);
      float ov[OPT];
      gather(m, ov);
      // refill the buffer the previous row used with the row PF ahead
      if (m + PF * m_step < m_stop) load_raw(m + PF * m_step, ring[(u + PF) % (PF + 1)]);
      row_body(m, it, ring[u], ov);
      m += m_step;
      ++it;
    }
  }
}

template <int XT, int LOW, int BR, bool GROUPED, int NT, int CPT>
static hipError_t launch_one(const ActArgs& a, int64_t cap, size_t lds, hipStream_t s) {
  auto kern = k_act_split<XT, LOW, BR, GROUPED, NT, CPT>;
  // about 16 waves per CU over the 256 CUs (32 single-wave blocks); each
  // block walks a set of rows, so the per-block setup (the channel map) is
  // amortised
  int64_t grid = NT == 64 ? (int64_t)256 * 32 : (int64_t)256 * 16 * 64 / NT;
  if (cap > 0) grid = cap;
  if (grid > a.m) grid = a.m;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NT), lds, s, a);
  return hipGetLastError();
}

template <int XT, int LOW, int BR, bool GROUPED>
static hipError_t launch_shape(const ActArgs& a, int64_t cap, size_t lds, hipStream_t s) {
  const int64_t chunks = a.k / 8;
  // rows of up to 2048 channels: one wave per block, so that the per-row
  // reduction and image hand-off need no cross-wave barrier wait and many
  // more rows are in flight per CU
  if (chunks <= 64) return launch_one<XT, LOW, BR, GROUPED, 64, 1>(a, cap, lds, s);
  if (chunks <= 128) return launch_one<XT, LOW, BR, GROUPED, 64, 2>(a, cap, lds, s);
  if (chunks <= 256) return launch_one<XT, LOW, BR, GROUPED, 64, 4>(a, cap, lds, s);
  if (chunks <= 512) return launch_one<XT, LOW, BR, GROUPED, 256, 2>(a, cap, lds, s);
  if (chunks <= 1024) return launch_one<XT, LOW, BR, GROUPED, 512, 2>(a, cap, lds, s);
  if (chunks <= 2048) return launch_one<XT, LOW, BR, GROUPED, 512, 4>(a, cap, lds, s);
  if (chunks <= 4096) return launch_one<XT, LOW, BR, GROUPED, 1024, 4>(a, cap, lds, s);
  return launch_one<XT, LOW, BR, GROUPED, 1024, 8>(a, cap, lds, s);
}

template <int XT, int LOW, bool GROUPED>
static hipError_t launch_br(const ActArgs& a, int br, int64_t cap, size_t lds, hipStream_t s) {
  if (br == kBF16) return launch_shape<XT, LOW, kBF16, GROUPED>(a, cap, lds, s);
  if (br == kFP8) return launch_shape<XT, LOW, kFP8, GROUPED>(a, cap, lds, s);
  return launch_shape<XT, LOW, kI8, GROUPED>(a, cap, lds, s);
}

size_t act_split_lds_bytes(int64_t ldk, int64_t k_out) {
  return (size_t)(2 * (ldk + kImgSlack) + ((k_out * 4 + 15) & ~(int64_t)15) + 2 * 2 * 16 * sizeof(float));
}

hipError_t launch_act_split(const ActArgs& a, int x_dtype, int low, int branch, bool grouped,
                            hipStream_t s) {
  const size_t lds = act_split_lds_bytes(a.ldk, a.k_out);
  // SQF_ACT_GRID overrides the number of blocks (tuning aid)
  const char* env = getenv("SQF_ACT_GRID");
  const int64_t cap = env ? atoll(env) : 0;
  if (a.m <= 0) return hipSuccess;
  if (x_dtype == kBF16) {
    if (low == kI4X2)
      return grouped ? launch_br<kBF16, kI4X2, true>(a, branch, cap, lds, s)
                     : launch_br<kBF16, kI4X2, false>(a, branch, cap, lds, s);
    return grouped ? launch_br<kBF16, kI8, true>(a, branch, cap, lds, s)
                   : launch_br<kBF16, kI8, false>(a, branch, cap, lds, s);
  }
  if (low == kI4X2)
    return grouped ? launch_br<kF32, kI4X2, true>(a, branch, cap, lds, s)
                   : launch_br<kF32, kI4X2, false>(a, branch, cap, lds, s);
  return grouped ? launch_br<kF32, kI8, true>(a, branch, cap, lds, s)
                 : launch_br<kF32, kI8, false>(a, branch, cap, lds, s);
}

}  // namespace sqf
