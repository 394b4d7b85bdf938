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

// Channel-split packer.  A block of 1024 threads (16 waves) owns 64 output
// channels: lane l of every wave works on column n0 + l, so each wave-wide
// load of one weight row W[c][n0 .. n0+63] is 256 contiguous bytes.  Pass 1:
// the waves split the K rows (wave w takes rows w, w+16, ...) for the low and
// outlier absmax of their columns, combined across waves through LDS.  Pass 2
// walks the slot space in chunks of kPackChunk slots: the block scatters the
// map into an LDS slot -> channel list for the chunk, then each wave packs
// 32-slot groups (one 16-byte store per lane) from the listed rows.  The
// branch rows are packed the same way, 16 bytes per lane per store.  Every
// code is a function of its own value and its column's absmax alone, so the
// result is the same as a sequential walk over the column.
constexpr int kPackCols = 64;
constexpr int kPackWaves = 16;
constexpr int kPackChunk = 8192;

// LOWF: kI4X2 (packed nibbles, [n][ldk]), kI4E2M3 (the same codes in 6-bit
// E2M3 fields, K-blocked [pad/128][rows_pad/16][4][16][24]; one weight set)
// or kMXFP4 (OSC abstract: the low path on 4-bit micro-scaling hardware,
// read as OCP MXFP4: each 32-slot group of a row is one block with its own
// E8M0 scale and E2M1 codes, K-blocked [pad/128][rows_pad/16][4][16][16],
// scales [pad/128][rows_pad/64][4][16][4]; one weight set).
template <int BR, int LOWF>
__global__ __launch_bounds__(1024) void k_pack_osc(PackArgs p) {
  __shared__ int32_t list[kPackChunk];
  __shared__ float red[2][kPackWaves][kPackCols];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t g = blockIdx.y;
  const int64_t nn = (int64_t)blockIdx.x * kPackCols + lane;
  const bool live = nn < p.n;
  const float* w = p.w + g * p.k * p.n + (live ? nn : 0);
  const int32_t* map = p.map + g * p.k;
  constexpr int ESZ = BR == kBF16 ? 2 : 1;

  // pass 1: absmax over the low and the outlier channels of the column
  float alo = 0.0f, ahi = 0.0f;
  {
    int64_t c = wv;
    for (; c + 7 * kPackWaves < p.k; c += 8 * kPackWaves) {
      float v[8];
      int32_t m[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        m[u] = map[c + u * kPackWaves];
        v[u] = fabsf(w[(c + u * kPackWaves) * p.n]);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (m[u] >= 0) alo = fmaxf(alo, v[u]); else ahi = fmaxf(ahi, v[u]);
      }
    }
    for (; c < p.k; c += kPackWaves) {
      const float v = fabsf(w[c * p.n]);
      if (map[c] >= 0) alo = fmaxf(alo, v); else ahi = fmaxf(ahi, v);
    }
  }
  red[0][wv][lane] = alo;
  red[1][wv][lane] = ahi;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPackWaves; ++i) {
    alo = fmaxf(alo, red[0][i][lane]);
    ahi = fmaxf(ahi, red[1][i][lane]);
  }
  const float inv = quant_inv(alo, 7.0f);
  const float qhi = BR == kFP8 ? 448.0f : 127.0f;
  const float inv_hi = BR == kBF16 ? 0.0f : quant_inv(ahi, qhi);
  if (wv == 0 && live) {
    if (LOWF != kMXFP4) p.s_w[g * p.n + nn] = quant_scale(alo, 7.0f);
    if (BR != kBF16 && p.s_wo) p.s_wo[g * p.n + nn] = quant_scale(ahi, qhi);
  }

  // slot -> channel list for slots [s0, s0 + kPackChunk) of one kind (low:
  // map value s, outlier: map value -(t+1)); unlisted slots read as value 0
  auto build_list = [&](int64_t s0, bool low) {
    __syncthreads();  // the previous chunk's readers are done
    for (int i = threadIdx.x; i < kPackChunk; i += 1024) list[i] = -1;
    __syncthreads();
    const int64_t lim = low ? p.k_low : p.k_out;
    for (int64_t c = threadIdx.x; c < p.k; c += 1024) {
      const int32_t m = map[c];
      const int64_t s = low ? (int64_t)m : -(int64_t)m - 1;
      if (s >= s0 && s < s0 + kPackChunk && s < lim) list[s - s0] = (int32_t)c;
    }
    __syncthreads();
  };

  // pass 2a: int4 codes, 32 slots per 16-byte group (24 bytes of 6-bit
  // fields), zero past k_low
  uint8_t* wl = p.w_low + (g * p.n + nn) * p.ldk;
  const int64_t slots = LOWF == kI4E2M3 ? p.ldk / 3 * 4 : p.ldk * 2;
  for (int64_t s0 = 0; s0 < slots; s0 += kPackChunk) {
    const int64_t s1 = s0 + kPackChunk < slots ? s0 + kPackChunk : slots;
    if (s0 < p.k_low) build_list(s0, true);
    for (int64_t q = s0 / 32 + wv; q < s1 / 32; q += kPackWaves) {
      uint32_t ow[4] = {0, 0, 0, 0};
      uint32_t sbyte = 0;  // MXFP4 scale (an all-zero block: 0)
      if (q * 32 < p.k_low) {
        float v[32];
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          const int32_t c = list[q * 32 - s0 + e];  // -1 past k_low (cleared)
          v[e] = c >= 0 ? w[(int64_t)c * p.n] : 0.0f;
        }
        if constexpr (LOWF == kMXFP4) {
          uint32_t amax = 0;
#pragma unroll
          for (int e = 0; e < 32; ++e) {
            const uint32_t a = __float_as_uint(v[e]) & 0x7FFFFFFFu;
            amax = a > amax ? a : amax;
          }
          sbyte = mx_scale_byte(amax);
          const float f = mx_inv_scale(sbyte);
#pragma unroll
          for (int e = 0; e < 32; ++e) ow[e >> 3] |= e2m1_code(v[e], f) << ((e & 7) * 4);
        } else {
#pragma unroll
          for (int e = 0; e < 32; ++e)
            ow[e >> 3] |= ((uint32_t)quant_code(v[e], inv, 7.0f) & 0xFu) << ((e & 7) * 4);
        }
      }
      if constexpr (LOWF == kMXFP4) {
        if (live) {
          // K block q/4, 16-row group nn/16, slot group q%4, row nn%16; the
          // scale byte with the 64-row group's other three fragments
          *(uint4*)(p.w_low + ((((q >> 2) * (p.rows_pad / 16) + nn / 16) * 4 + (q & 3)) * 16 + (nn & 15)) * 16) =
              make_uint4(ow[0], ow[1], ow[2], ow[3]);
          p.s_wb[((((q >> 2) * (p.rows_pad / 64) + nn / 64) * 4 + (q & 3)) * 16 + (nn & 15)) * 4 +
                 ((nn >> 4) & 3)] = (uint8_t)sbyte;
        }
      } else if constexpr (LOWF == kI4E2M3) {
        // nibbles -> one code per byte -> 6-bit fields, 24 bits per 4 codes
        uint32_t f[8];
#pragma unroll
        for (int h = 0; h < 8; ++h) {
          const uint32_t nib = ow[h >> 1] >> (16 * (h & 1));  // 4 codes, 4 bits each
          // sign-extend each nibble into its own byte
          const uint32_t b = (nib & 0xFu) | ((nib & 0xF0u) << 4) | ((nib & 0xF00u) << 8) |
                             ((nib & 0xF000u) << 12);
          const uint32_t sx = ((b & 0x08080808u) >> 3) * 0xF0u;
          f[h] = e2m3_fields4(b | sx);
        }
        // 8 x 24 bits -> 6 dwords (fields of slot e at bits 6e .. 6e+5)
        const uint32_t d0 = f[0] | (f[1] << 24), d1 = (f[1] >> 8) | (f[2] << 16),
                       d2 = (f[2] >> 16) | (f[3] << 8), d3 = f[4] | (f[5] << 24),
                       d4 = (f[5] >> 8) | (f[6] << 16), d5 = (f[6] >> 16) | (f[7] << 8);
        if (live) {
          // K block q/4, row pair nn/32, slot group q%4: bytes 0..15 to the
          // head KiB (nn/16)%2 at 16*lane, bytes 16..23 to the tail KiB at
          // 16*lane + 8*((nn/16)%2), lane = 16*(q%4) + nn%16
          const int64_t lane = (q & 3) * 16 + (nn & 15), h = (nn >> 4) & 1;
          uint8_t* base = p.w_low + ((q >> 2) * (p.rows_pad / 32) + nn / 32) * 3072;
          *(uint4*)(base + h * 1024 + lane * 16) = make_uint4(d0, d1, d2, d3);
          *(v2u*)(base + 2048 + lane * 16 + h * 8) = v2u{d4, d5};
        }
      } else {
        if (live) *(uint4*)(wl + q * 16) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
      }
    }
  }

  // pass 2b: branch codes, 16 bytes per store, zero past k_out
  if (p.w_out == nullptr || p.ldo == 0) return;
  constexpr int PER = 16 / ESZ;  // elements per 16-byte store
  uint8_t* wo = p.w_out + (g * p.n + nn) * p.ldo * ESZ;
  for (int64_t s0 = 0; s0 < p.ldo; s0 += kPackChunk) {
    const int64_t s1 = s0 + kPackChunk < p.ldo ? s0 + kPackChunk : p.ldo;
    if (s0 < p.k_out) build_list(s0, false);
    for (int64_t q = s0 / PER + wv; q < s1 / PER; q += kPackWaves) {
      uint32_t ow[4] = {0, 0, 0, 0};
      if (q * PER < p.k_out) {
        float v[PER];
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          const int32_t c = list[q * PER - s0 + e];
          v[e] = c >= 0 ? w[(int64_t)c * p.n] : 0.0f;
        }
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          uint32_t code;
          if constexpr (BR == kBF16) code = bf16_rne(v[e]);
          else if constexpr (BR == kFP8) code = e4m3_rne_sat(v[e] * inv_hi);
          else code = (uint32_t)quant_code(v[e], inv_hi, 127.0f) & 0xFFu;
          ow[e / (4 / ESZ)] |= code << ((e % (4 / ESZ)) * 8 * ESZ);
        }
      }
      if (live) *(uint4*)(wo + q * 16) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
    }
  }
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
// A block reads one column of W (one 4-byte value per row); consecutive
// blocks run on different XCDs (block b on XCD b mod 8), so XCD x is given the
// contiguous column range [x*per_x, (x+1)*per_x): its concurrently running
// blocks then share the 128-byte lines of W in their XCD's L2.
//
// Banks (SQ-format article, section 九: the top fraction inside each bank;
// section 七: equal work per bank): with p.bank > 0 the row is cut into banks
// of p.bank consecutive slots and each keeps its nnz / banks largest keys.
// Every slot then counts the keys of its bank that rank above it (larger,
// or equal at a lower slot) and is kept when fewer than that many do; a
// wave's 64 slots share a bank, so its reads of the bank are broadcasts.
//
// FP (SQ-format article, section 八: FP8 high-precision part, FP4 low part):
// the same marks; the kept values become E4M3 codes of v * 448/a8 and the
// other slots E2M1 codes of v * 6/a4 (0x8, E2M1 -0, is never produced by
// the encoder and stays the mark); the branch is E4M3 with its own scale.
template <bool FP>
__global__ __launch_bounds__(256) void k_pack_sq(PackArgs p) {
  extern __shared__ uint8_t sm[];
  __shared__ int iscr[8];
  __shared__ float fscr[8];
  __shared__ int hist[256];
  __shared__ int sel[2];
  const int64_t per_x = gridDim.x >> 3;  // the grid is a multiple of 8
  const int64_t nn = (int64_t)(blockIdx.x & 7) * per_x + (blockIdx.x >> 3);
  if (nn >= p.n) return;
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
  // threshold T = nnz-th largest key (0 when there are fewer keys): radix
  // select over the 64-bit patterns, 8 bits per pass from the top.  Each pass
  // histograms the next byte of the keys that match the bytes chosen so far,
  // then takes the largest byte d whose keys at or above it still cover the
  // `need` keys not yet accounted for above the matching range.
  const int64_t bank = p.bank > 0 && p.bank < kl ? p.bank : 0;
  uint64_t T = 0;
  if (p.nnz > 0 && bank == 0) {
    uint64_t mask = 0;
    int need = (int)p.nnz;
    for (int shift = 56; shift >= 0; shift -= 8) {
      hist[tid] = 0;
      __syncthreads();
      for (int64_t j = j0; j < j1; ++j) {
        const uint64_t kb = keybits(j);
        if ((kb & mask) == T) atomicAdd(&hist[(kb >> shift) & 255], 1);
      }
      __syncthreads();
      if (tid < 64) {  // wave 0: lane l holds bins 4l .. 4l+3
        const int h0 = hist[4 * tid], h1 = hist[4 * tid + 1], h2 = hist[4 * tid + 2],
                  h3 = hist[4 * tid + 3];
        const int s_l = h0 + h1 + h2 + h3;
        const int incl = wave_inclusive_scan(s_l);
        const int above = __shfl(incl, 63, 64) - incl;  // keys in the bins of lanes > l
        const int s3 = above + h3, s2 = s3 + h2, s1 = s2 + h1, s0 = s1 + h0;
        int d = -1, cover = 0, hd_d = 0;
        if (s3 >= need) { d = 4 * tid + 3; cover = s3; hd_d = h3; }
        else if (s2 >= need) { d = 4 * tid + 2; cover = s2; hd_d = h2; }
        else if (s1 >= need) { d = 4 * tid + 1; cover = s1; hd_d = h1; }
        else if (s0 >= need) { d = 4 * tid; cover = s0; hd_d = h0; }
        int best = d;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) best = max(best, __shfl_xor(best, off, 64));
        if (best < 0) {
          if (tid == 0) { sel[0] = 0; sel[1] = need; }
        } else if (d == best) {
          sel[0] = best;
          sel[1] = need - (cover - hd_d);  // keys above byte d are already in
        }
      }
      __syncthreads();
      T |= (uint64_t)sel[0] << shift;
      need = sel[1];
      mask |= 255ull << shift;
    }
  }
  if (bank == 0) {
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
    for (int64_t j = j0; j < j1; ++j) {
      uint8_t kp = 0;
      if (p.nnz > 0) {
        uint64_t kb = keybits(j);
        if (kb > T) kp = 1;
        else if (kb == T) kp = (eq_before++ < need) ? 1 : 0;
      }
      keep[j] = kp;
    }
  } else {
    const int per_bank = (int)(p.nnz / (kl / bank));
    for (int64_t j = tid; j < kl; j += 256) {
      const int64_t b0 = j / bank * bank;
      const uint64_t kj = keybits(j);
      int above = 0;
      for (int64_t i = b0; i < b0 + bank; ++i) {
        const uint64_t ki = keybits(i);
        above += (ki > kj) || (ki == kj && i < j);
      }
      keep[j] = above < per_bank ? 1 : 0;
    }
    __syncthreads();
  }
  float a8 = 0.0f, a4 = 0.0f;
  for (int64_t j = j0; j < j1; ++j) {
    if (keep[j]) a8 = fmaxf(a8, fabsf(vals[j])); else a4 = fmaxf(a4, fabsf(vals[j]));
  }
  a8 = block_max_f(a8, fscr);
  a4 = block_max_f(a4, fscr);
  constexpr float Q8 = FP ? 448.0f : 127.0f, Q4 = FP ? 6.0f : 7.0f;
  const float inv8 = quant_inv(a8, Q8), inv4 = quant_inv(a4, Q4);
  if (tid == 0) {
    p.s_w8[nn] = quant_scale(a8, Q8);
    p.s_w[nn] = quant_scale(a4, Q4);
  }
  // int8 values in ascending slot order
  int kc = 0;
  for (int64_t j = j0; j < j1; ++j) kc += keep[j];
  int pos = block_excl_scan(kc, iscr);
  for (int64_t j = j0; j < j1; ++j)
    if (keep[j])
      p.sq_val[nn * p.nnz + pos++] =
          FP ? (int8_t)e4m3_rne_sat(vals[j] * inv8) : (int8_t)quant_code(vals[j], inv8, 127.0f);
  // packed row: 16-byte groups of 32 slots
  uint8_t* wl = p.w_low + nn * p.ldk;
  for (int64_t q = tid; q < p.ldk / 16; q += 256) {
    uint32_t ow[4] = {0, 0, 0, 0};
    for (int e = 0; e < 32; ++e) {
      int64_t j = q * 32 + e;
      uint32_t nib = 0;
      if (j < kl)
        nib = keep[j] ? 0x8u
                      : (FP ? e2m1_code(vals[j], inv4) : ((uint32_t)quant_code(vals[j], inv4, 7.0f) & 0xFu));
      ow[e >> 3] |= nib << ((e & 7) * 4);
    }
    *(uint4*)(wl + q * 16) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
  }
  // int8 (FP: E4M3) branch over the outlier channels
  float ao = 0.0f;
  for (int64_t t = tid; t < p.k_out; t += 256) ao = fmaxf(ao, fabsf(ov[t]));
  ao = block_max_f(ao, fscr);
  const float invo = quant_inv(ao, Q8);
  if (tid == 0 && p.s_wo) p.s_wo[nn] = quant_scale(ao, Q8);
  for (int64_t t = tid; t < p.ldo; t += 256)
    p.w_out[nn * p.ldo + t] =
        t < p.k_out ? (FP ? (uint8_t)e4m3_rne_sat(ov[t] * invo) : (uint8_t)quant_code(ov[t], invo, 127.0f))
                    : 0;
}

hipError_t launch_pack(const PackArgs& a, int branch, int low, int groups, hipStream_t s) {
  if (a.nnz > 0) {
    // integer form (int4 + int8) or floating-point form (E2M1 + E4M3)
    const bool fp = low == kFP4E2M1;
    if (fp != (branch == kFP8)) return hipErrorInvalidValue;
    const void* kern = fp ? (const void*)k_pack_sq<true> : (const void*)k_pack_sq<false>;
    size_t lds = (size_t)a.k_low * 9 + (size_t)a.k_out * 4 + 16;
    if (lds > 65536) {
      hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    const dim3 grid((unsigned)((a.n + 7) / 8 * 8));
    if (fp)
      hipLaunchKernelGGL(k_pack_sq<true>, grid, dim3(256), lds, s, a);
    else
      hipLaunchKernelGGL(k_pack_sq<false>, grid, dim3(256), lds, s, a);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((a.n + kPackCols - 1) / kPackCols), (unsigned)groups);
  dim3 block(kPackCols * kPackWaves);
  if (low == kI4E2M3) {
    if (branch != kBF16 || groups != 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_pack_osc<kBF16, kI4E2M3>), grid, block, 0, s, a);
  } else if (low == kMXFP4) {
    if (branch != kBF16 || groups != 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_pack_osc<kBF16, kMXFP4>), grid, block, 0, s, a);
  } else if (branch == kBF16) {
    hipLaunchKernelGGL((k_pack_osc<kBF16, kI4X2>), grid, block, 0, s, a);
  } else if (branch == kFP8) {
    hipLaunchKernelGGL((k_pack_osc<kFP8, kI4X2>), grid, block, 0, s, a);
  } else {
    hipLaunchKernelGGL((k_pack_osc<kI8, kI4X2>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace sqf
