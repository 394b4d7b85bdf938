// sqf_device.h -- device helpers shared by the gfx950 kernels of libsqf.
//
// Number-format conversions are written from the formats' definitions:
//   bf16: the top 16 bits of an fp32 pattern, rounded to nearest-even.
//   E4M3 (OCP): 1 sign, 4 exponent bits with bias 7, 3 mantissa bits, largest
//   finite 448, no infinities.  A value is rounded by scaling it with the
//   power-of-two quantum of its binade and rounding half to even.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sqf {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Status codes mirrored from the public header (kept in sync by the host code).
enum : int { kBF16 = 1, kFP8 = 2, kI8 = 3, kI4X2 = 4, kI4E2M3 = 5, kMXFP4 = 6, kFP4E2M1 = 7, kF32 = 0 };

// Four int4 codes, one per byte (two's complement, |c| <= 7), as four 6-bit
// OCP E2M3 fields holding c/8 (the subnormal: sign << 5 | |c|), packed into
// the low 24 bits: code i at bits 6i .. 6i+5.
__device__ __forceinline__ uint32_t e2m3_fields4(uint32_t q) {
  const uint32_t s = q & 0x80808080u;           // sign bits
  const uint32_t neg = (s >> 7) * 0xFFu;         // 0xFF in each negative byte
  const uint32_t mag = (q ^ neg) + (neg & 0x01010101u);  // |c| per byte (no carries: |c| <= 7)
  const uint32_t f = mag | (s >> 2);             // sign to bit 5
  const uint32_t t = (f & 0x003F003Fu) | ((f & 0x3F003F00u) >> 2);  // 12-bit pairs
  return (t & 0xFFFu) | ((t >> 4) & 0xFFF000u);
}

__device__ __forceinline__ uint32_t f32_bits(float f) { return __float_as_uint(f); }

// OCP MXFP4.  E8M0 scale byte of a 32-value block from its max |v| (fp32
// bits): X = floor(log2 max) - 2 (2 = exponent of the largest E2M1 value, 6),
// clamped at -127; the byte is X + 127 = max(biased exponent - 2, 0) (a zero
// or subnormal max gives 0).
__device__ __forceinline__ uint32_t mx_scale_byte(uint32_t amax_bits) {
  const int e = (int)(amax_bits >> 23) - 2;
  return (uint32_t)(e > 0 ? e : 0);
}
// 2^-X for scale byte b (b <= 252: a normal float, exact scaling)
__device__ __forceinline__ float mx_inv_scale(uint32_t b) { return __uint_as_float((254u - b) << 23); }
// E2M1 code (sign bit 3) of v * inv: the nearest of 0, 0.5, 1, 1.5, 2, 3, 4,
// 6 with ties to the even code, saturating at 6.  The code is the count of
// midpoints below |t|; at a midpoint the even neighbour wins (down at 0.25,
// 1.25, 2.5, 5; up at 0.75, 1.75, 3.5).  A zero code has no sign.
__device__ __forceinline__ uint32_t e2m1_code(float v, float inv) {
  const float t = fabsf(v) * inv;
  uint32_t c = (uint32_t)(t > 0.25f) + (uint32_t)(t >= 0.75f) + (uint32_t)(t > 1.25f) +
               (uint32_t)(t >= 1.75f) + (uint32_t)(t > 2.5f) + (uint32_t)(t >= 3.5f) + (uint32_t)(t > 5.0f);
  if (c != 0u && v < 0.0f) c |= 8u;
  return c;
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  uint32_t lsb = (b >> 16) & 1u;
  return (b + 0x7FFFu + lsb) >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> OCP E4M3 byte, nearest-even, saturating to +-448.  A value that
// rounds to zero gives +0 (0x00) whatever its sign.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float v) {
  float a = fabsf(v);
  uint32_t code;
  if (a >= 464.0f) {
    code = 0x7E;  // beyond the midpoint to the (absent) next value: saturate
  } else {
    int e = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;  // binade of a (a > 0)
    if (a < 0.015625f) {  // below 2^-6: subnormal quantum 2^-9
      code = (uint32_t)rintf(a * 512.0f);  // 0..8; 8 encodes 2^-6 exactly
    } else {
      // quantum 2^(e-3); q in [8, 16]; q == 16 carries into the next binade
      float q = rintf(a * __uint_as_float((uint32_t)(127 + 3 - e) << 23));
      code = (uint32_t)((e + 7) << 3) + ((uint32_t)q - 8u);
    }
    if (code > 0x7E) code = 0x7E;
  }
  if (code != 0 && v < 0.0f) code |= 0x80u;
  return code;
}

// Wave-wide max of a non-negative float (order independent, exact).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Inclusive prefix sum across the wave (Hillis-Steele over shuffles).
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int t = __shfl_up(v, off, kWave);
    if (lane >= off) v += t;
  }
  return v;
}

// Symmetric quantisation helpers: inv = q / a (IEEE fp32 division), code =
// clamp(rint(v * inv), -q, q).  a == 0 -> inv = 0 -> every code 0.
__device__ __forceinline__ float quant_inv(float a, float q) { return a == 0.0f ? 0.0f : q / a; }
__device__ __forceinline__ float quant_scale(float a, float q) { return a == 0.0f ? 0.0f : a / q; }
__device__ __forceinline__ int quant_code(float v, float inv, float q) {
  float r = rintf(v * inv);
  r = fminf(fmaxf(r, -q), q);
  return (int)r;
}


// ---------------------------------------------------------------------------
// Global -> LDS DMA and the waits around it (the GEMM kernels' operand rings).

// 16-byte chunk swizzle of a 2 KiB block of 16 rows x 128 bytes, stored as
// two halves of 8 rows: chunk C of row r of half h sits at chunk C ^ swz(h, r).
// The 16 rows x one chunk of an MFMA operand read then hit 16 distinct 16-byte
// bank groups (and any 8 consecutive lanes distinct ones).
__host__ __device__ constexpr int pair_swz(int h, int r) { return r ^ (2 * h); }

// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt bits [3:0] and [15:14]; expcnt and
// lgkmcnt left at their maximum, i.e. not waited on).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// One 16-byte-per-lane global -> LDS DMA (global_load_lds_dwordx4): lane l's
// 16 bytes land at LDS byte address lds + 16*l.  Written as a two-instruction
// asm block rather than the compiler builtin because the builtin is a FLAT
// instruction that also counts as an LDS access, and while one is outstanding
// the compiler's wait insertion can only wait for every LDS read at once
// (lgkmcnt(0)); the ring keeps DMAs outstanding across the whole K loop.  The
// block has no register outputs; completion is tracked by the explicit vmcnt
// waits of the ring (wait_vmcnt), and the "memory" clobber keeps the compiler
// from moving LDS accesses across it.
__device__ __forceinline__ void dma_16B(const uint8_t* base, uint32_t voff, uint32_t lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds);
  // base: wave-uniform 64-bit address (SGPR pair); voff: per-lane byte offset.
  // M0 holds the LDS base; one wait state separates its write from the DMA.
  asm volatile(
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(base), "{m0}"(m0v)
      : "memory");
}

// Byte address of a __shared__ object inside the workgroup's LDS.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Workgroup barrier that does not drain outstanding loads.  __syncthreads()
// carries a workgroup fence, and the fence makes the compiler wait for every
// outstanding LDS-DMA load (they count as LDS writes), which would cap the
// ring at one stage in flight.  Here the caller has already waited for the
// stage it needs (vmcnt) and for its own LDS reads (lgkmcnt), and the empty
// asm statements keep the compiler from moving LDS accesses across the
// barrier.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}


}  // namespace sqf
