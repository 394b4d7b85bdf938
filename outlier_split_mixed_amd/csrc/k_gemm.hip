// k_gemm.hip -- the fused dual-path GEMM for gfx950 (channel-split format).
//
//   y[m,n] = s_x[m]*s_w[n]*sum_j qx[m,j]*qw[n,j]  +  branch[m,n]
//   branch = sum_t xo[m,t]*wo[n,t]                       (bf16, unscaled)
//          | s_xo[m]*s_wo[n]*sum_t xo[m,t]*wo[n,t]       (E4M3)
// This is the dual-path computation of OSC (abstract and method framework:
// a 4-bit GEMM over the ordinary channels, a high-precision GEMM over the
// compact outlier sub-tensor, results summed) and the two parallel paths
// with result fusion of the SQ-format article (section 三).
//
// gfx950 mapping.  CDNA4 has no int4 matrix instruction, so the low path runs
// on v_mfma_i32_16x16x64_i8.  Packed int4 stays packed in HBM and LDS (half
// the bytes of int8) and is widened in registers right before the MFMA:
//   byte = (w << 4) & 0xF0F0F0F0   -> 16 * (low nibble, sign-extended)
//   byte =  w       & 0xF0F0F0F0   -> 16 * (high nibble, sign-extended)
// Both operands carry the factor 16, so the int32 sum is exactly 256 times
// the true sum (|true sum| <= 49 * k_low, checked on the host to fit).  The
// K order inside one MFMA is irrelevant as long as A and B use the same
// lane/byte layout, which they do.  After the low K loop the accumulators are
// turned into fp32 in place (times s_x*s_w/256, exact power-of-two scaling),
// and the bf16 branch (v_mfma_f32_16x16x32_bf16) accumulates on top of them;
// an E4M3 branch (v_mfma_f32_16x16x32_fp8_fp8) uses a second accumulator set
// because it carries its own scales.
//
// Tiles.  A block computes BM x BN outputs with WGM x WGN waves; each wave a
// (TM*16) x (TN*16) sub-tile.  One K stage is 128 bytes of every row (256
// int4 slots, or 64 bf16, or 128 E4M3).  LDS holds each stage in "fragment
// order": the 16 bytes lane l feeds to the MFMA for a 16-row block are
// stored at index (rowblock*2 + f)*64 + l, so every ds_read_b128 of a wave is
// one contiguous, conflict-free 1 KiB read.  Stages are double buffered with
// register prefetch.  The block -> tile map is XCD-aware: consecutive
// hardware block ids go to different XCDs, so they are remapped to give every
// XCD a contiguous run of logical tiles, then rastered in groups of GROUP_M
// tile rows to share operand panels in each XCD's L2.
#include "sqf_device.h"
#include "sqf_launch.h"

namespace sqf {

__device__ __forceinline__ void unpack_i4x32(const uint4 q, v4i& lo, v4i& hi) {
  lo[0] = (int)((q.x << 4) & 0xF0F0F0F0u);
  lo[1] = (int)(q.x & 0xF0F0F0F0u);
  lo[2] = (int)((q.y << 4) & 0xF0F0F0F0u);
  lo[3] = (int)(q.y & 0xF0F0F0F0u);
  hi[0] = (int)((q.z << 4) & 0xF0F0F0F0u);
  hi[1] = (int)(q.z & 0xF0F0F0F0u);
  hi[2] = (int)((q.w << 4) & 0xF0F0F0F0u);
  hi[3] = (int)(q.w & 0xF0F0F0F0u);
}

template <int BM, int BN, int NT>
struct StageLoader {
  static constexpr int PIECES = (BM + BN) * 8;  // 16-byte pieces per stage
  static constexpr int L = PIECES / NT;
  static_assert(PIECES % NT == 0, "pieces must divide evenly");
  static_assert((BM * 8) % NT == 0, "A/B split must fall on a load boundary");
  static constexpr int LA = BM * 8 / NT;
  uint32_t off[L];   // byte offset of the piece inside its operand (stage 0)
  int lds_idx[L];    // fragment-order LDS index (uint4 units)

  __device__ __forceinline__ void init(int tid, int64_t a_row0, int64_t a_rows_end, int64_t b_row0,
                                       int64_t b_rows_end, int64_t ld) {
#pragma unroll
    for (int i = 0; i < L; ++i) {
      int e = tid + i * NT;
      int r = e >> 3, p = e & 7;
      int64_t grow;
      int rr;
      if (i < LA) {
        rr = r;
        grow = a_row0 + rr;
        if (grow > a_rows_end - 1) grow = a_rows_end - 1;
      } else {
        rr = r - BM;
        grow = b_row0 + rr;
        if (grow > b_rows_end - 1) grow = b_rows_end - 1;
      }
      off[i] = (uint32_t)(grow * ld + p * 16);
      lds_idx[i] = (i < LA ? 0 : BM * 8) + (((rr >> 4) * 2 + (p >> 2)) * 64 + (p & 3) * 16 + (rr & 15));
    }
  }
  __device__ __forceinline__ void load(uint4 (&buf)[L], const uint8_t* a, const uint8_t* b,
                                       uint32_t stage_off) const {
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const uint8_t* base = i < LA ? a : b;
      buf[i] = *(const uint4*)(base + off[i] + stage_off);
    }
  }
  __device__ __forceinline__ void store(const uint4 (&buf)[L], uint4* lds) const {
#pragma unroll
    for (int i = 0; i < L; ++i) lds[lds_idx[i]] = buf[i];
  }
};

template <int BM, int BN, int WGM, int WGN, int BR, bool GROUPED, bool DEBUG, int GROUP_M>
__global__ __launch_bounds__(WGM* WGN * 64) void k_dual_gemm(GemmArgs p) {
  constexpr int NT = WGM * WGN * 64;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TM = WM / 16, TN = WN / 16;
  static_assert(TM >= 1 && TN >= 1, "wave tile too small");
  __shared__ uint4 smem[2][(BM + BN) * 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int64_t tiles_n = (p.n + BN - 1) / BN;

  // ---- block -> tile (XCD-aware) ----
  int64_t lid = blockIdx.x;
  {
    const int64_t nb = gridDim.x;
    if ((nb & 7) == 0) lid = (lid & 7) * (nb >> 3) + (lid >> 3);
  }
  int64_t m_begin = 0, m_end = p.m, tm, tn;
  const uint8_t* w_low = p.w_low;
  const uint8_t* w_out = p.w_out;
  const float* s_w = p.s_w;
  const float* s_wo = p.s_wo;
  if constexpr (GROUPED) {
    // walk the groups: group g owns ceil(rows_g / BM) * tiles_n tiles
    int64_t base = 0;
    int g = 0;
    for (; g < p.groups; ++g) {
      int64_t r0 = p.row_off[g], r1 = p.row_off[g + 1];
      int64_t t = ((r1 - r0 + BM - 1) / BM) * tiles_n;
      if (lid < base + t) {
        m_begin = r0;
        m_end = r1;
        break;
      }
      base += t;
    }
    if (g == p.groups) return;
    int64_t local = lid - base;
    int64_t tiles_m = (m_end - m_begin + BM - 1) / BM;
    tm = local % tiles_m;
    tn = local / tiles_m;
    w_low += g * p.w_stride_low;
    w_out += g * p.w_stride_out;
    s_w += g * p.w_stride_s;
    if (s_wo) s_wo += g * p.w_stride_s;
  } else {
    const int64_t tiles_m = (p.m + BM - 1) / BM;
    const int64_t per_group = (int64_t)GROUP_M * tiles_n;
    int64_t grp = lid / per_group;
    int64_t first_m = grp * GROUP_M;
    int64_t gsz = tiles_m - first_m < GROUP_M ? tiles_m - first_m : GROUP_M;
    int64_t in = lid % per_group;
    tm = first_m + in % gsz;
    tn = in / gsz;
    if (tm >= tiles_m || tn >= tiles_n) return;
  }
  const int64_t m0 = m_begin + tm * BM;
  const int64_t n0 = tn * BN;

  StageLoader<BM, BN, NT> ld;
  uint4 pre[StageLoader<BM, BN, NT>::L];

  v4i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  // ---------------- low path: int4 x int4 on int8 MFMA ----------------
  if (p.s_low > 0) {
    ld.init(tid, m0, m_end, n0, p.n, p.ldk);
    ld.load(pre, p.x_low, w_low, 0);
    ld.store(pre, smem[0]);
    __syncthreads();
    for (int s = 0; s < p.s_low; ++s) {
      const int b = s & 1;
      if (s + 1 < p.s_low) ld.load(pre, p.x_low, w_low, (uint32_t)(s + 1) * 128u);
      const uint4* As = smem[b];
      const uint4* Bs = smem[b] + BM * 8;
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        v4i b0[TN], b1[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) unpack_i4x32(Bs[((wn * TN + j) * 2 + f) * 64 + lane], b0[j], b1[j]);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          v4i a0, a1;
          unpack_i4x32(As[((wm * TM + i) * 2 + f) * 64 + lane], a0, a1);
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0[j], acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1[j], acc[i][j], 0, 0, 0);
          }
        }
      }
      if (s + 1 < p.s_low) ld.store(pre, smem[b ^ 1]);
      __syncthreads();
    }
  }

  // ---------------- epilogue part 1: exact int32 -> scaled fp32 ----------------
  const int lr = (lane >> 4) * 4;  // first of the 4 rows this lane holds in a 16x16 tile
  const int lc = lane & 15;
  int64_t rows[TM][4];
  int64_t cols[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) rows[i][r] = m0 + wm * WM + i * 16 + lr + r;
#pragma unroll
  for (int j = 0; j < TN; ++j) cols[j] = n0 + wn * WN + j * 16 + lc;

  float swv[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) swv[j] = s_w[cols[j] < p.n ? cols[j] : p.n - 1];

  v4f c[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    float sxv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sxv[r] = p.s_x[rows[i][r] < m_end ? rows[i][r] : m_end - 1];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (DEBUG) {
          if (rows[i][r] < m_end && cols[j] < p.n)
            p.acc_dbg[rows[i][r] * p.n + cols[j]] = acc[i][j][r] >> 8;
        }
        c[i][j][r] = (float)acc[i][j][r] * (sxv[r] * swv[j] * 0.00390625f);
      }
    }
  }

  // ---------------- branch: outlier sub-tensor GEMM ----------------
  v4f c2[TM][TN];
  if constexpr (BR == kFP8) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) c2[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  if (p.s_out > 0) {
    ld.init(tid, m0, m_end, n0, p.n, p.ldo_b);
    ld.load(pre, p.x_out, w_out, 0);
    ld.store(pre, smem[0]);
    __syncthreads();
    for (int s = 0; s < p.s_out; ++s) {
      const int b = s & 1;
      if (s + 1 < p.s_out) ld.load(pre, p.x_out, w_out, (uint32_t)(s + 1) * 128u);
      const uint4* As = smem[b];
      const uint4* Bs = smem[b] + BM * 8;
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        uint4 bq[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) bq[j] = Bs[((wn * TN + j) * 2 + f) * 64 + lane];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          uint4 aq = As[((wm * TM + i) * 2 + f) * 64 + lane];
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            if constexpr (BR == kBF16) {
              c[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, aq),
                                                                __builtin_bit_cast(v8bf, bq[j]),
                                                                c[i][j], 0, 0, 0);
            } else {
              long a_lo = (long)(((uint64_t)aq.y << 32) | aq.x);
              long a_hi = (long)(((uint64_t)aq.w << 32) | aq.z);
              long b_lo = (long)(((uint64_t)bq[j].y << 32) | bq[j].x);
              long b_hi = (long)(((uint64_t)bq[j].w << 32) | bq[j].z);
              c2[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a_lo, b_lo, c2[i][j], 0, 0, 0);
              c2[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a_hi, b_hi, c2[i][j], 0, 0, 0);
            }
          }
        }
      }
      if (s + 1 < p.s_out) ld.store(pre, smem[b ^ 1]);
      __syncthreads();
    }
  }

  // ---------------- epilogue part 2: fuse and store ----------------
  float swo[TN];
  if constexpr (BR == kFP8) {
#pragma unroll
    for (int j = 0; j < TN; ++j) swo[j] = s_wo[cols[j] < p.n ? cols[j] : p.n - 1];
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = rows[i][r];
      if (row >= m_end) continue;
      float sxo = 0.f;
      if constexpr (BR == kFP8) sxo = p.s_xo[row];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if (cols[j] >= p.n) continue;
        float v = c[i][j][r];
        if constexpr (BR == kFP8) v += (sxo * swo[j]) * c2[i][j][r];
        p.y[row * p.ldy + cols[j]] = v;
      }
    }
  }
}

// ------------------------------------------------------------------ launch
template <int BM, int BN, int WGM, int WGN, int BR, bool GROUPED, bool DEBUG>
static hipError_t launch_cfg(const GemmArgs& a, hipStream_t s) {
  int64_t tiles_n = (a.n + BN - 1) / BN;
  int64_t blocks;
  if (GROUPED)
    blocks = ((a.m + BM - 1) / BM + a.groups) * tiles_n;
  else
    blocks = ((a.m + BM - 1) / BM) * tiles_n;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_dual_gemm<BM, BN, WGM, WGN, BR, GROUPED, DEBUG, 8>), dim3((unsigned)blocks),
                     dim3(WGM * WGN * 64), 0, s, a);
  return hipGetLastError();
}

template <int BR, bool GROUPED, bool DEBUG>
static hipError_t launch_br(const GemmArgs& a, int cfg, hipStream_t s) {
  // an E4M3 branch keeps a second accumulator set: no 256x256 tile for it
  if (BR == kFP8 && cfg == 0) cfg = 1;
  switch (cfg) {
    case 0:
      if constexpr (BR != kFP8) return launch_cfg<256, 256, 2, 4, BR, GROUPED, DEBUG>(a, s);
      [[fallthrough]];
    case 1:
      return launch_cfg<128, 128, 2, 2, BR, GROUPED, DEBUG>(a, s);
    default:
      return launch_cfg<64, 64, 2, 2, BR, GROUPED, DEBUG>(a, s);
  }
}

// cfg: 0 = 256x256 (8 waves), 1 = 128x128 (4 waves), 2 = 64x64 (4 waves).
hipError_t launch_dual_gemm(const GemmArgs& a, int branch, bool grouped, bool debug, int cfg,
                            hipStream_t s) {
  if (branch == kFP8) {
    if (grouped) return debug ? launch_br<kFP8, true, true>(a, cfg, s) : launch_br<kFP8, true, false>(a, cfg, s);
    return debug ? launch_br<kFP8, false, true>(a, cfg, s) : launch_br<kFP8, false, false>(a, cfg, s);
  }
  if (grouped) return debug ? launch_br<kBF16, true, true>(a, cfg, s) : launch_br<kBF16, true, false>(a, cfg, s);
  return debug ? launch_br<kBF16, false, true>(a, cfg, s) : launch_br<kBF16, false, false>(a, cfg, s);
}

}  // namespace sqf
