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
// Activations are int8 per token.  The "gather unit" is realised while a
// stage of W is staged into LDS: each packed 16-byte piece of a row is
// decoded into an int8 low tile (marks -> 0) and a dense int8 tile holding the
// row's sparse values at their marked slots (0 elsewhere).  The index of a
// marked slot's value is the row's mark count before the stage (precomputed
// per 256-slot tile) plus the count before it inside the stage, found with a
// shuffle scan across the 8 lanes that share the row.  Both tiles then feed
// v_mfma_i32_16x16x64_i8 with the same A fragment.
#include "sqf_device.h"
#include "sqf_launch.h"

namespace sqf {

__device__ __forceinline__ int lds_frag_idx(int r, int f, int g) {
  return ((r >> 4) * 4 + f) * 64 + g * 16 + (r & 15);
}

template <bool DEBUG>
__global__ __launch_bounds__(256) void k_sq_gemm(SqArgs p) {
  constexpr int BM = 128, BN = 128, TM = 4, TN = 4;
  __shared__ uint4 sA[BM * 16];
  __shared__ uint4 sL[BN * 16];
  __shared__ uint4 sS[BN * 16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t tiles_n = (p.n + BN - 1) / BN;
  const int64_t tm = blockIdx.x % ((p.m + BM - 1) / BM), tn = blockIdx.x / ((p.m + BM - 1) / BM);
  if (tn >= tiles_n) return;
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int64_t ntile1 = p.ldkw / 128 + 1;

  v4i acc[TM][TN], acs[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = acs[i][j] = v4i{0, 0, 0, 0};

  for (int s = 0; s < p.s_low; ++s) {
    // A: 128 rows x 256 bytes, fragment order (4 K64 chunks per stage)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int e = tid + i * 256, r = e >> 4, pc = e & 15;
      int64_t gr = m0 + r < p.m ? m0 + r : p.m - 1;
      sA[lds_frag_idx(r, pc >> 2, pc & 3)] = *(const uint4*)(p.x_low + gr * p.ldkx + s * 256 + pc * 16);
    }
    // W: 128 rows x 128 packed bytes -> low tile + sparse tile
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int e = tid + i * 256, r = e >> 3, pc = e & 7;
      int64_t gn = n0 + r < p.n ? n0 + r : p.n - 1;
      uint4 q = *(const uint4*)(p.w_low + gn * p.ldkw + s * 128 + pc * 16);
      uint32_t qw[4] = {q.x, q.y, q.z, q.w};
      int marks = 0;
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int b = 0; b < 8; ++b) marks += ((qw[h] >> (4 * b)) & 0xF) == 0x8;
      int incl = marks;  // inclusive scan across the 8 lanes of this row
#pragma unroll
      for (int off = 1; off < 8; off <<= 1) {
        int t = __shfl_up(incl, off, 8);
        if ((lane & 7) >= off) incl += t;
      }
      int vi = p.tile_off[gn * ntile1 + s] + incl - marks;
      const int8_t* vals = p.sq_val + gn * p.nnz;
      uint32_t lo[8], sp[8];
#pragma unroll
      for (int h = 0; h < 8; ++h) lo[h] = sp[h] = 0;
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          uint32_t nib = (qw[h] >> (4 * b)) & 0xF;
          int slot = h * 8 + b;  // 0..31 inside the piece
          uint32_t lb, sb = 0;
          if (nib == 0x8) {
            lb = 0;
            sb = vi < p.nnz ? (uint8_t)vals[vi] : 0u;  // marks beyond nnz: malformed input
            ++vi;
          } else {
            lb = (uint8_t)(int8_t)((int)(nib << 28) >> 28);
          }
          lo[slot >> 2] |= lb << ((slot & 3) * 8);
          sp[slot >> 2] |= sb << ((slot & 3) * 8);
        }
      // slots 32*pc .. +31 of the stage: K64 chunk f = pc/2, byte groups g, g+1
      int f = pc >> 1, g = (pc & 1) * 2;
      sL[lds_frag_idx(r, f, g)] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
      sL[lds_frag_idx(r, f, g + 1)] = make_uint4(lo[4], lo[5], lo[6], lo[7]);
      sS[lds_frag_idx(r, f, g)] = make_uint4(sp[0], sp[1], sp[2], sp[3]);
      sS[lds_frag_idx(r, f, g + 1)] = make_uint4(sp[4], sp[5], sp[6], sp[7]);
    }
    __syncthreads();
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      v4i bl[TN], bs[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        bl[j] = __builtin_bit_cast(v4i, sL[(((wn * TN + j) * 4) + f) * 64 + lane]);
        bs[j] = __builtin_bit_cast(v4i, sS[(((wn * TN + j) * 4) + f) * 64 + lane]);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        v4i a = __builtin_bit_cast(v4i, sA[(((wm * TM + i) * 4) + f) * 64 + lane]);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bl[j], acc[i][j], 0, 0, 0);
          acs[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bs[j], acs[i][j], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }

  const int lr = (lane >> 4) * 4, lc = lane & 15;
  float part[TM][TN][4];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int64_t row = m0 + wm * 64 + i * 16 + lr + r, col = n0 + wn * 64 + j * 16 + lc;
        int64_t rc = row < p.m ? row : p.m - 1, cc = col < p.n ? col : p.n - 1;
        if (DEBUG && row < p.m && col < p.n) {
          p.dbg_low[row * p.n + col] = acc[i][j][r];
          p.dbg_sp[row * p.n + col] = acs[i][j][r];
        }
        part[i][j][r] = p.s_x[rc] * (p.s_w4[cc] * (float)acc[i][j][r] + p.s_w8[cc] * (float)acs[i][j][r]);
        acs[i][j][r] = 0;
      }

  // int8 branch (outlier channels), 128 bytes per row per stage
  for (int s = 0; s < p.s_out; ++s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int e = tid + i * 256, r = e >> 3, pc = e & 7;
      int64_t gr = m0 + r < p.m ? m0 + r : p.m - 1;
      sA[lds_frag_idx(r, pc >> 2, pc & 3)] = *(const uint4*)(p.x_out + gr * p.ldo + s * 128 + pc * 16);
      int64_t gn = n0 + r < p.n ? n0 + r : p.n - 1;
      sL[lds_frag_idx(r, pc >> 2, pc & 3)] = *(const uint4*)(p.w_out + gn * p.ldo + s * 128 + pc * 16);
    }
    __syncthreads();
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      v4i b[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) b[j] = __builtin_bit_cast(v4i, sL[(((wn * TN + j) * 4) + f) * 64 + lane]);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        v4i a = __builtin_bit_cast(v4i, sA[(((wm * TM + i) * 4) + f) * 64 + lane]);
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
      for (int r = 0; r < 4; ++r) {
        int64_t row = m0 + wm * 64 + i * 16 + lr + r, col = n0 + wn * 64 + j * 16 + lc;
        if (row >= p.m || col >= p.n) continue;
        if (DEBUG) p.dbg_o[row * p.n + col] = acs[i][j][r];
        float v = part[i][j][r];
        if (p.s_out > 0) v += (p.s_xo[row] * p.s_wo[col]) * (float)acs[i][j][r];
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
