// k_gemm6.hip -- the fused dual-path GEMM on gfx950's 6-bit matrix unit.
//
//   y[m,n] = s_x[m]*s_w[n]*sum_j qx[m,j]*qw[n,j]  +  sum_t xo[m,t]*wo[n,t]
// The dual-path computation of OSC (abstract and method framework: a 4-bit
// GEMM over the ordinary channels, a 16-bit GEMM over the compact outlier
// sub-tensor, results summed) with the same int4 codes and the same bf16
// branch as the channel-split kernel; only the storage of the int4 codes and
// the matrix instruction differ.
//
// Arithmetic.  Every int4 code c in [-7, 7] is held in a 6-bit OCP E2M3
// field as the subnormal c/8, so v_mfma_f32_16x16x128_f8f6f4 (FP6 operands,
// unit block scales) forms sum c_x*c_w/64 for 128 slots per instruction, at
// twice the int8 instruction's rate and with no unpacking.  Each product is
// a multiple of 2^-6 and every partial sum stays below 2^18 in magnitude
// (|sum| <= 49 * k_low / 64, the host keeps k_low below 2^24 / 49), so the
// fp32 accumulation is exact in any order: the accumulator times 64 is the
// int32 sum of the int4 path, bit for bit.
//
// Layout.  Both low operands are K-blocked and stored in the matrix unit's
// lane order: for K block kb (128 slots) and 16-row group rg, 1536 bytes
// hold slot group g (32 slots, 24 bytes) of row r at (g*16 + r%16)*24, which
// is exactly lane 16g + r%16's share of one 16 x 128 FP6 operand.  A 256-row
// panel of one K block is one contiguous 24 KiB run (moved by the stage's
// DMAs as whole cache lines), and each lane's fragment read is 24 bytes at
// 24*lane: consecutive lanes, consecutive banks.  (A plain row pitch of 96
// bytes put rows r, r+4, r+8, r+12 on the same banks: 73% of the LDS cycles
// were bank conflicts.)  The rows are padded to a multiple of 256, so a
// panel never leaves its block.
//
// Tiles.  A block computes 256 x 256 outputs with 8 waves (2 x 4), each
// wave 128 x 64 (8 x 4 fragments of 16 x 16, 128 accumulator registers), two
// waves per SIMD.  K runs as one stream of stages through a ring of three
// 48 KiB LDS slots: low stages (128 slots: A panel 24 KiB, B panel 24 KiB),
// then branch stages (32 bf16 channels: 16 KiB + 16 KiB, rows 64 bytes with
// their 16-byte chunks XOR-swizzled by row so the MFMA operand reads hit
// distinct banks).  At the top of stage t every wave waits for its own DMAs
// of stage t, crosses one barrier, and issues stage t+2 into the slot stage
// t-1 used.  Blocks are mapped XCD-aware (each XCD a contiguous run of tiles,
// rastered in groups of 8 tile rows).
#include "sqf_device.h"
#include "sqf_launch.h"

namespace sqf {

namespace {

constexpr int kBM = 256, kBN = 256;
constexpr int kWGM = 2, kWGN = 4, kNW = kWGM * kWGN;
constexpr int kTM = kBM / kWGM / 16, kTN = kBN / kWGN / 16;  // 8 x 4 fragments
constexpr int kSlot = 48 * 1024;                               // bytes per ring slot
constexpr int kRing = 3;
constexpr int kLowRowB = 96;                                   // bytes per row per low stage
constexpr int kBrRowB = 64;                                    // bytes per row per branch stage
constexpr int kLowDmaPerWave = (kBM + kBN) * kLowRowB / 1024 / kNW;  // 6
constexpr int kBrDmaPerWave = (kBM + kBN) * kBrRowB / 1024 / kNW;    // 4
constexpr int kGroupM = 8;

typedef int v8i __attribute__((ext_vector_type(8)));

// Three 8-byte LDS reads -> the 6 registers of one FP6 operand (32 fields of
// lane l: row l%16 of the fragment, slots 32*(l/16) .. +31 of the stage,
// stored at byte 24*l of the fragment's 1536 bytes).
__device__ __forceinline__ v8i ld_fp6(const uint8_t* p) {
  const v2u a = *(const v2u*)p, b = *(const v2u*)(p + 8), c = *(const v2u*)(p + 16);
  return v8i{(int)a.x, (int)a.y, (int)b.x, (int)b.y, (int)c.x, (int)c.y, 0, 0};
}

// s_waitcnt vmcnt for a wave-uniform count of DMAs still allowed in flight.
__device__ __forceinline__ void wait_dmas(int n) {
  if (n >= kLowDmaPerWave) wait_vmcnt<kLowDmaPerWave>();
  else if (n >= kBrDmaPerWave) wait_vmcnt<kBrDmaPerWave>();
  else wait_vmcnt<0>();
}

}  // namespace

template <bool DEBUG, bool YB>
__global__ __launch_bounds__(kNW * 64, 2) void k_gemm6(Gemm6Args p) {
  static_assert(!(DEBUG && YB), "the accumulator dump comes with fp32 Y");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kRing * kSlot];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kWGN, wn = wave % kWGN;
  const int64_t tiles_m = (p.m + kBM - 1) / kBM, tiles_n = (p.n + kBN - 1) / kBN;

  // ---- block -> tile (XCD-aware, grouped raster) ----
  int64_t lid = blockIdx.x;
  {
    const int64_t nb = gridDim.x;
    if ((nb & 7) == 0) lid = (lid & 7) * (nb >> 3) + (lid >> 3);
  }
  const int64_t per_group = (int64_t)kGroupM * tiles_n;
  const int64_t first_m = (lid / per_group) * kGroupM;
  const int64_t gsz = tiles_m - first_m < kGroupM ? tiles_m - first_m : kGroupM;
  const int64_t in = lid % per_group;
  const int64_t tm = first_m + in % gsz, tn = in / gsz;
  if (tm >= tiles_m || tn >= tiles_n) return;
  const int64_t m0 = tm * kBM, n0 = tn * kBN;

  const int S = p.s_low, SB = p.s_br, ST = S + SB;
  const uint32_t smem_lds = lds_offset(smem);

  // DMA of stage t into ring slot t % 3.  Low stage: the A panel (rows
  // m0..m0+255 of K block t) and the B panel are contiguous 24 KiB runs;
  // instruction q of 48 moves bytes q*1024 .. +1023 of the pair of panels.
  // Branch stage: row-major bf16 rows; instruction q of 32 covers 16 rows x
  // 4 chunks of 16 bytes, lane l -> row q*16 + l/4 (clamped to the last
  // real row), chunk (l%4) ^ ((row/4)%4) of the stage's 64 bytes.
  const int br_r = lane >> 2, br_c = lane & 3;
  auto issue = [&](int t) {
    const uint32_t slot = smem_lds + (uint32_t)((t % kRing) * kSlot);
    if (t < S) {
      const uint8_t* a = p.x6 + ((int64_t)t * p.x_rows + m0) * kLowRowB;
      const uint8_t* b = p.w6 + ((int64_t)t * p.w_rows + n0) * kLowRowB;
#pragma unroll
      for (int i = 0; i < kLowDmaPerWave; ++i) {
        const int q = wave * kLowDmaPerWave + i;  // wave-uniform
        const bool is_a = q < kBM * kLowRowB / 1024;
        const int ql = is_a ? q : q - kBM * kLowRowB / 1024;
        dma_16B(is_a ? a : b, (uint32_t)(ql * 1024 + lane * 16),
                slot + (uint32_t)(q * 1024));
      }
    } else {
      const uint32_t kb = (uint32_t)(t - S) * kBrRowB;
#pragma unroll
      for (int i = 0; i < kBrDmaPerWave; ++i) {
        const int q = wave * kBrDmaPerWave + i;
        const bool is_a = q < kBM * kBrRowB / 1024;
        const int ql = is_a ? q : q - kBM * kBrRowB / 1024;
        const int r = ql * 16 + br_r;
        int64_t row = (is_a ? m0 : n0) + r;
        const int64_t lim = (is_a ? p.m : p.n) - 1;
        if (row > lim) row = lim;
        const uint32_t voff = (uint32_t)(row * p.ldo_b) + kb + 16u * (uint32_t)(br_c ^ ((r >> 2) & 3));
        dma_16B(is_a ? p.x_out : p.w_out, voff, slot + (uint32_t)(q * 1024));
      }
    }
  };
  // DMAs per wave of stage t (0 past the end)
  auto dmas_of = [&](int t) { return t >= ST ? 0 : (t < S ? kLowDmaPerWave : kBrDmaPerWave); };

  // The epilogue's arguments are read with scalar loads; landing them before
  // the loop keeps the LDS read counter waits of the loop in order.
  {
    const float* y_ = p.y;
    const float* sx_ = p.s_x;
    const float* sw_ = p.s_w;
    int32_t* dbg_ = p.acc_dbg;
    const int64_t ldy_ = p.ldy, n_ = p.n;
    asm volatile("" ::"s"(y_), "s"(sx_), "s"(sw_), "s"(dbg_), "s"(ldy_), "s"(n_));
  }

  v4f acc[kTM][kTN];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // this lane's byte offsets inside a low stage's panels: fragment (16 rows)
  // f of a panel is bytes f*1536 .. +1535, lane l's share at 24*l
  const int fr = lane & 15, fg = lane >> 4;
  constexpr int kFragB = 16 * kLowRowB;  // 1536
  const uint32_t a_off = (uint32_t)(wm * kTM * kFragB + lane * 24);
  const uint32_t b_off = (uint32_t)(kBM * kLowRowB + wn * kTN * kFragB + lane * 24);

  issue(0);
  if (ST > 1) issue(1);

  // ---------------- low path: int4 codes on the 6-bit matrix unit ----------------
  for (int t = 0; t < S; ++t) {
    wait_dmas(dmas_of(t + 1));
    __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's LDS reads are done
    stage_barrier();
    if (t + 2 < ST) issue(t + 2);
    const uint8_t* sl = smem + (t % kRing) * kSlot;
    v8i B[kTN];
#pragma unroll
    for (int j = 0; j < kTN; ++j) B[j] = ld_fp6(sl + b_off + j * kFragB);
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      const v8i A = ld_fp6(sl + a_off + i * kFragB);
      // Wave priority: the two waves of a SIMD cross the same barrier and
      // reach their MFMA runs together; raising it after the first fragment
      // and dropping it before the last lets one issue back to back while
      // the other reads LDS.
      if (i == 1) __builtin_amdgcn_s_setprio(1);
      if (i == kTM - 1) __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int j = 0; j < kTN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B[j], acc[i][j], 2, 2, 0, 0,
                                                                      0, 0);
    }
  }

  // ---------------- exact sums -> scaled fp32 ----------------
  // Lane l holds rows 4*(l/16)+r (r < 4) and column l%16 of each fragment.
  const int row0 = (int)m0 + wm * kTM * 16 + (lane >> 4) * 4;
  const int col0 = (int)n0 + wn * kTN * 16 + (lane & 15);
  const int mrows = (int)p.m, ncols = (int)p.n;
#pragma unroll
  for (int j = 0; j < kTN; ++j) {
    const int col = col0 + j * 16;
    const float sw = p.s_w[col < ncols ? col : ncols - 1] * 64.0f;
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + i * 16 + r;
        if constexpr (DEBUG) {
          if (row < mrows && col < ncols)
            p.acc_dbg[(int64_t)row * p.n + col] = (int32_t)(acc[i][j][r] * 64.0f);
        }
        acc[i][j][r] *= p.s_x[row < mrows ? row : mrows - 1] * sw;
      }
  }

  // ---------------- branch: bf16 outlier sub-tensor GEMM ----------------
  // Lane l reads row l%16 of a fragment, chunk l/16 of the stage's 4.
  const int bc = fg;
  auto br_off = [&](int r) { return (uint32_t)(r * kBrRowB + 16 * (bc ^ ((r >> 2) & 3))); };
  for (int t = S; t < ST; ++t) {
    wait_dmas(dmas_of(t + 1));
    __builtin_amdgcn_s_waitcnt(0xC07F);
    stage_barrier();
    if (t + 2 < ST) issue(t + 2);
    const uint8_t* sl = smem + (t % kRing) * kSlot;
    v4i B[kTN];
#pragma unroll
    for (int j = 0; j < kTN; ++j)
      B[j] = *(const v4i*)(sl + kBM * kBrRowB + br_off(wn * kTN * 16 + j * 16 + fr));
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      const v4i A = *(const v4i*)(sl + br_off(wm * kTM * 16 + i * 16 + fr));
#pragma unroll
      for (int j = 0; j < kTN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(v8bf, A), __builtin_bit_cast(v8bf, B[j]), acc[i][j], 0, 0, 0);
    }
  }

  // ---------------- store ----------------
  const int wrow0 = (int)m0 + wm * kTM * 16, wcol0 = (int)n0 + wn * kTN * 16;
  constexpr int WN = kTN * 16, LDW = WN + 4;
  const bool whole = wrow0 + kTM * 16 <= mrows && wcol0 + WN <= ncols && (p.ldy & 3) == 0 &&
                     (((uintptr_t)p.y) & (YB ? 7 : 15)) == 0;
  // every wave is past its last LDS read of the ring (and no DMA is in
  // flight: the last stage waited for all of them)
  __builtin_amdgcn_s_waitcnt(0xC07F);
  stage_barrier();
  float* y = p.y;
  uint16_t* yb = (uint16_t*)p.y;
  if (whole) {
    // Each 16-row slice of the wave tile goes through this wave's part of
    // the (now idle) ring and leaves as 16-byte non-temporal stores of
    // whole row segments.
    static_assert(kNW * 16 * LDW * 4 <= kSlot, "staging fits one ring slot");
    float* stg = (float*)smem + wave * (16 * LDW);
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
#pragma unroll
      for (int j = 0; j < kTN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) stg[((lane >> 4) * 4 + r) * LDW + j * 16 + (lane & 15)] = acc[i][j][r];
#pragma unroll
      for (int k = 0; k < WN / 16; ++k) {
        const int idx = k * 64 + lane, rr = idx / (WN / 4), c4 = idx % (WN / 4);
        const v4f v = *(const v4f*)(stg + rr * LDW + 4 * c4);
        const int64_t o = (int64_t)(wrow0 + i * 16 + rr) * p.ldy + wcol0 + 4 * c4;
        if constexpr (YB) {
          const v2u h = v2u{__builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{v.x, v.y}, v2bf)),
                            __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{v.z, v.w}, v2bf))};
          __builtin_nontemporal_store(h, (v2u*)(yb + o));
        } else {
          __builtin_nontemporal_store(v, (v4f*)(y + o));
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + i * 16 + r;
        if (row >= mrows) continue;
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
          const int col = col0 + j * 16;
          if (col >= ncols) continue;
          const float v = acc[i][j][r];
          if constexpr (YB)
            __builtin_nontemporal_store(__builtin_bit_cast(uint16_t, (__bf16)v),
                                        yb + (int64_t)row * p.ldy + col);
          else
            __builtin_nontemporal_store(v, y + (int64_t)row * p.ldy + col);
        }
      }
  }
}

hipError_t launch_gemm6(const Gemm6Args& a, bool debug, bool ybf16, hipStream_t s) {
  if (debug && ybf16) return hipErrorInvalidValue;
  const int64_t blocks = ((a.m + kBM - 1) / kBM) * ((a.n + kBN - 1) / kBN);
  if (blocks <= 0) return hipSuccess;
  if (debug)
    hipLaunchKernelGGL((k_gemm6<true, false>), dim3((unsigned)blocks), dim3(kNW * 64), 0, s, a);
  else if (ybf16)
    hipLaunchKernelGGL((k_gemm6<false, true>), dim3((unsigned)blocks), dim3(kNW * 64), 0, s, a);
  else
    hipLaunchKernelGGL((k_gemm6<false, false>), dim3((unsigned)blocks), dim3(kNW * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace sqf
