// k_sq.hip -- dual GEMM for the weight-side SQ-format.
//
// SQ-format article, section 三: the dense low-precision weight tensor keeps
// its layout and is consumed by the ordinary matrix units, while positions
// carrying the reserved mark are served from a sparse high-precision part by
// a gather unit; section 九 defines the format (dense codes, sparse values,
// mask) and the reserved code.  Here:
//   acc_low[m,n] = sum_j qx[m,j] * qw[n,j]          (marked slots count 0)
//   acc_sp [m,n] = sum_i qx[m,pos_i(n)] * v8[n,i]   (i-th marked slot of row n)
//   acc_o  [m,n] = sum_t xo[m,t] * wo[n,t]          (int8 outlier-channel branch)
//   y = s_x*(s_w4*acc_low + s_w8*acc_sp) + s_xo*s_wo*acc_o
//
// gfx950 mapping.  The "gather unit" is the decode of each K stage of W into
// LDS, done once per block: a 128-slot stage of a W row becomes
//   * an int4 low tile with the marks cleared to 0 (SWAR: a nibble is the
//     mark iff its top bit is set and its low three bits are zero), widened
//     to int8 at MFMA time with the x16 trick (w << 4 & 0xF0.. and
//     w & 0xF0..), which puts a group of 8 slots in the order 0,2,4,6,1,3,5,7;
//   * an int8 tile holding the row's sparse values at their marked slots
//     (zero elsewhere), in that same slot order.  Only the marked slots (1/8)
//     are written: a lane walks the marks of its 64 slots with find-first-set
//     and copies each value from the row's value window, which was fetched
//     into LDS with the stage (the row's running value index is carried from
//     stage to stage, so the window is known before the stage is decoded).
// The int8 activations are written to LDS with the same slot permutation, so
// both tiles feed v_mfma_i32_16x16x64_i8 with one A fragment.  The low
// accumulator carries the x16 factor (|acc| <= 16*127*7*k_low < 2^31 for the
// k_low the host accepts); it is removed exactly in the epilogue.  Global
// loads of stage s+1 are issued right after stage s is in LDS, so their
// latency hides behind stage s's MFMAs; two blocks share a CU.
#include "sqf_device.h"
#include "sqf_launch.h"

namespace sqf {

namespace {

// LDS barrier that does not wait for outstanding global loads.
__device__ __forceinline__ void lds_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// byte position, inside a lane's 16-byte MFMA operand, of slot k (0..15) in
// the widened order 0,2,4,6,1,3,5,7 | 8,10,12,14,9,11,13,15
__device__ __forceinline__ int perm_pos(int k) {
  return (k & 8) + ((k & 1) ? 4 + ((k & 7) >> 1) : ((k & 7) >> 1));
}

}  // namespace

template <bool DEBUG>
__global__ __launch_bounds__(256, 2) void k_sq_gemm(SqArgs p) {
  constexpr int BM = 128, BN = 128, TM = 4, TN = 4;
  // stage = 128 low slots: A 128 B / row, W 64 B / row
  __shared__ uint4 sA[BM * 8];            // [rb][f][lane] x 16 B (permuted slot order)
  __shared__ uint2 sL[BN * 8];            // [rb][f][lane] x 8 B (clean int4)
  __shared__ uint4 sS[BN * 8];            // [rb][f][lane] x 16 B (values at marks)
  __shared__ __attribute__((aligned(16))) uint8_t sV[BN * 64 + 16];  // value windows (+ read slack)
  __shared__ uint2 sSel[256];  // expand selectors per 8-slot mark mask

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t tiles_m = (p.m + BM - 1) / BM;
  const int64_t tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
  if (tn * BN >= p.n) return;
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int nst = (int)(p.ldkw / 64);  // 128-slot stages (ldkw is a multiple of 128)

  // this thread's share of a stage: row r (of A and of W), half h = K64 chunk
  const int r = tid >> 1, h = tid & 1;
  const int64_t ga = (m0 + r < p.m ? m0 + r : p.m - 1);
  const int64_t gn = (n0 + r < p.n ? n0 + r : p.n - 1);
  const uint8_t* arow = p.x_low + ga * p.ldkx + h * 64;
  const uint8_t* wrow = p.w_low + gn * p.ldkw + h * 32;
  const int8_t* vrow = p.sq_val + gn * p.nnz;
  const int64_t vtotal = p.n * p.nnz;  // bytes in the value buffer
  // byte offset of the buffer start past the previous 16-byte boundary
  const int vmis = (int)((uintptr_t)p.sq_val & 15);
  const int rb = r >> 4, rr = r & 15;

  // Expand selectors: for the mark mask m of an 8-slot group, byte p of the
  // group's operand bytes (slot order 0,2,4,6,1,3,5,7) takes value number
  // rank(slot) (a byte of the pool {hi, lo} of the group's values) if the
  // slot is marked, else zero (selector 0x0C).
  {
    const int m = tid;  // 256 threads, 256 masks
    uint32_t sel[2] = {0, 0};
#pragma unroll
    for (int pp = 0; pp < 8; ++pp) {
      const int sl = pp < 4 ? 2 * pp : 2 * (pp - 4) + 1;
      const uint32_t b = ((m >> sl) & 1) ? (uint32_t)__builtin_popcount(m & ((1 << sl) - 1)) : 0x0Cu;
      sel[pp >> 2] |= b << (8 * (pp & 3));
    }
    sSel[m] = make_uint2(sel[0], sel[1]);
    if (tid < 4) ((uint32_t*)(sV + BN * 64))[tid] = 0;
    lds_sync();
  }

  // prefetched global data of one stage
  uint4 ra[4], rw[2], rv[2];
  int vi = 0;         // row r's value index at the current stage
  int win_valid = 0;  // bytes of the fetched window that lie inside the buffer
  int64_t win_lo = 0; // buffer offset of the window's first byte (may be < 0)
  auto fetch = [&](int s) {
#pragma unroll
    for (int q = 0; q < 4; ++q) ra[q] = *(const uint4*)(arow + s * 128 + q * 16);
#pragma unroll
    for (int q = 0; q < 2; ++q) rw[q] = *(const uint4*)(wrow + s * 64 + q * 16);
    // value window [win_lo, win_lo + 64) (16-byte aligned addresses) holding
    // row r's values from vi on; this lane brings its half (32 bytes)
    const int64_t a0 = gn * p.nnz + vi;
    win_lo = ((a0 + vmis) & ~(int64_t)15) - vmis;
    // whole 16-byte blocks inside the buffer (the rest is read byte by byte)
    const int64_t room = vtotal - win_lo;
    win_valid = room > 0 ? (int)(room < 64 ? room : 64) & ~15 : 0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int off = h * 32 + q * 16;
      rv[q] = (off + 16 <= win_valid && win_lo + off >= 0)
                  ? *(const uint4*)(p.sq_val + win_lo + off) : make_uint4(0, 0, 0, 0);
    }
  };

  v4i acc[TM][TN], acs[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = acs[i][j] = v4i{0, 0, 0, 0};

  if (nst > 0) fetch(0);
  for (int s = 0; s < nst; ++s) {
    // ---- A: 64 bytes (chunk h of row r) in the widened slot order ----
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint4 u = ra[g];
      sA[(rb * 2 + h) * 64 + g * 16 + rr] =
          make_uint4(perm(u.y, u.x, 0x06040200u), perm(u.y, u.x, 0x07050301u),
                     perm(u.w, u.z, 0x06040200u), perm(u.w, u.z, 0x07050301u));
    }
    // ---- value window of row r ----
    *(uint4*)(sV + r * 64 + h * 32) = rv[0];
    *(uint4*)(sV + r * 64 + h * 32 + 16) = rv[1];
    // ---- W: 64 slots (chunk h of row r): clean low tile, marks ----
    uint32_t wd[8], mk[8];
    int cnt = 0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t d4[4] = {rw[q].x, rw[q].y, rw[q].z, rw[q].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t x = d4[e];
        const uint32_t nz = ((x & 0x77777777u) + 0x77777777u) & 0x88888888u;
        const uint32_t m8 = x & 0x88888888u & ~nz;  // bit 3 of each marked nibble
        mk[q * 4 + e] = m8;
        wd[q * 4 + e] = x & ~((m8 - (m8 >> 3)) | m8);
        cnt += __builtin_popcount(m8);
      }
    }
#pragma unroll
    for (int g = 0; g < 4; ++g)
      sL[(rb * 2 + h) * 64 + g * 16 + rr] = make_uint2(wd[2 * g], wd[2 * g + 1]);
    uint4* srow = sS + (rb * 2 + h) * 64 + rr;  // this lane's sparse-tile bytes
    // marks of the first half of the row precede this lane's (partner lane ^ 1)
    const int cnt_other = __shfl_xor(cnt, 1, 64);
    const int v0 = vi + (h ? cnt_other : 0);         // value index of this lane's first mark
    const int wo0 = (int)(gn * p.nnz + v0 - win_lo);  // its offset in the value window
    // ---- sparse tile: every 8-slot group expanded from its values at once ----
    {
      const uint32_t* vw = (const uint32_t*)sV;
      int pre = 0;
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        // byte offset of the group's first value; past the row's window the
        // bytes are not used (those lanes take the path below), so the read
        // only has to stay inside the array
        const int off = min(r * 64 + wo0 + pre, r * 64 + 64);
        const uint32_t d0 = vw[off >> 2], d1 = vw[(off >> 2) + 1], d2 = vw[(off >> 2) + 2];
        const uint32_t lo = __builtin_amdgcn_alignbyte(d1, d0, off & 3);
        const uint32_t hi = __builtin_amdgcn_alignbyte(d2, d1, off & 3);
        uint32_t x = mk[d] >> 3;  // mark bits at 4i -> bit i
        x = (x | (x >> 3)) & 0x03030303u;
        x = (x | (x >> 6)) & 0x000F000Fu;
        x = (x | (x >> 12)) & 0xFFu;
        const uint2 sl = sSel[x];
        *(uint2*)((uint8_t*)(srow + (d >> 1) * 16) + (d & 1) * 8) = make_uint2(perm(hi, lo, sl.x), perm(hi, lo, sl.y));
        pre += __builtin_popcount(mk[d]);
      }
    }
    // rare: values beyond the window (or more marks than values) -> one by one
    if (wo0 + cnt > win_valid || v0 + cnt > p.nnz) {
      int j = 0;
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        uint32_t m8 = mk[d];
        while (m8) {
          const int k = d * 8 + (__builtin_ctz(m8) >> 2);
          m8 &= m8 - 1;
          const int8_t v = v0 + j >= p.nnz ? (int8_t)0 : vrow[v0 + j];
          ((uint8_t*)(srow + (k >> 4) * 16))[perm_pos(k & 15)] = (uint8_t)v;
          ++j;
        }
      }
    }
    vi += cnt + cnt_other;
    lds_sync();
    // ---- next stage's global data (its latency hides behind the MFMAs) ----
    if (s + 1 < nst) fetch(s + 1);
    // ---- MFMAs: two K64 chunks ----
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      v4i a[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i) a[i] = __builtin_bit_cast(v4i, sA[((wm * TM + i) * 2 + f) * 64 + lane]);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int idx = ((wn * TN + j) * 2 + f) * 64 + lane;
        const uint2 x = sL[idx];
        const v4i bl = v4i{(int)((x.x << 4) & 0xF0F0F0F0u), (int)(x.x & 0xF0F0F0F0u),
                           (int)((x.y << 4) & 0xF0F0F0F0u), (int)(x.y & 0xF0F0F0F0u)};
        const v4i bs = __builtin_bit_cast(v4i, sS[idx]);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], bl, acc[i][j], 0, 0, 0);
          acs[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], bs, acs[i][j], 0, 0, 0);
        }
      }
    }
    lds_sync();
  }

  // ---- low + masked parts -> fp32 partial (the low accumulator is x16) ----
  // (the fp32 partial reuses the low accumulator's registers)
  const int lr = (lane >> 4) * 4, lc = lane & 15;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = m0 + wm * 64 + i * 16 + lr + q, col = n0 + wn * 64 + j * 16 + lc;
        const int64_t rc = row < p.m ? row : p.m - 1, cc = col < p.n ? col : p.n - 1;
        const int32_t lo = acc[i][j][q] >> 4;
        if (DEBUG && row < p.m && col < p.n) {
          p.dbg_low[row * p.n + col] = lo;
          p.dbg_sp[row * p.n + col] = acs[i][j][q];
        }
        acc[i][j][q] = __float_as_int(p.s_x[rc] * (p.s_w4[cc] * (float)lo + p.s_w8[cc] * (float)acs[i][j][q]));
        acs[i][j][q] = 0;
      }

  // ---- int8 branch (outlier channels), 128 bytes per row per stage ----
  for (int s = 0; s < p.s_out; ++s) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      sA[(rb * 2 + h) * 64 + q * 16 + rr] = *(const uint4*)(p.x_out + ga * p.ldo + s * 128 + h * 64 + q * 16);
      sS[(rb * 2 + h) * 64 + q * 16 + rr] = *(const uint4*)(p.w_out + gn * p.ldo + s * 128 + h * 64 + q * 16);
    }
    __syncthreads();
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      v4i b[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) b[j] = __builtin_bit_cast(v4i, sS[((wn * TN + j) * 2 + f) * 64 + lane]);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const v4i a = __builtin_bit_cast(v4i, sA[((wm * TM + i) * 2 + f) * 64 + lane]);
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acs[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b[j], acs[i][j], 0, 0, 0);
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = m0 + wm * 64 + i * 16 + lr + q, col = n0 + wn * 64 + j * 16 + lc;
        if (row >= p.m || col >= p.n) continue;
        if (DEBUG) p.dbg_o[row * p.n + col] = acs[i][j][q];
        float v = __int_as_float(acc[i][j][q]);
        if (p.s_out > 0) v += (p.s_xo[row] * p.s_wo[col]) * (float)acs[i][j][q];
        p.y[row * p.ldy + col] = v;
      }
}

hipError_t launch_sq_gemm(const SqArgs& a, bool debug, hipStream_t s) {
  int64_t blocks = ((a.m + 127) / 128) * ((a.n + 127) / 128);
  if (blocks <= 0) return hipSuccess;
  if (debug) hipLaunchKernelGGL(k_sq_gemm<true>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_sq_gemm<false>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace sqf
