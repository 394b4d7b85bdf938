// k_gemm6.hip -- the fused dual-path GEMM on gfx950's 6-/4-bit matrix unit
// (v_mfma_scale_f32_16x16x128_f8f6f4), in two forms sharing one pipeline:
//
// int4 codes in E2M3 fields (FP6 operands):
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
// MXFP4 (FP4 operands; OSC abstract: the low path on 4-bit micro-scaling
// hardware, read as OCP MXFP4):
//   y[m,n] = sum_j 2^Xx(m,j/32) e2m1(cx[m,j]) * 2^Xw(n,j/32) e2m1(cw[n,j])
//            + sum_t xo[m,t]*wo[n,t]
// Lane l of a 16 x 128 operand holds the 32 slots of one block, so the
// block's E8M0 scale is that lane's scale operand: the matrix unit applies
// both block scales to every product; sums are fp32 (not exact).  The scale
// bytes of four 16-row fragments (rows r, r+16, r+32, r+48 of a 64-row
// group) share one dword per lane and the instruction's opsel picks the
// fragment's byte.
//
// Layout.  Both low operands are K-blocked and stored in the matrix unit's
// lane order.  For K block kb (128 slots), slot group g (32 slots, 24 bytes
// of fields) of row r belongs to lane 16g + r%16 of the 16 x 128 FP6 operand
// of its 16-row group.  Rows go in pairs of 16-row groups (rows 32p ..
// 32p+31, 3 KiB per K block): the first KiB holds bytes 0..15 of every lane
// of the first group, the second KiB those of the second group, the third
// KiB bytes 16..23 of both (lane l at 16l: the first group's 8, then the
// second's).  Each lane's 24 bytes of two fragments are then three
// conflict-free 16-byte reads; 8-byte reads moved ~40% fewer bytes per
// clock and made the LDS the limit (and a plain 96-byte row pitch put rows
// r, r+4, r+8, r+12 on the same banks: 73% of the LDS cycles were bank
// conflicts).  A 256-row panel of one K block is one contiguous 24 KiB run,
// moved by the stage's DMAs as whole cache lines; rows are padded to a
// multiple of 256, so a panel never leaves its block.
//
// (MXFP4: 16 bytes per lane, 1 KiB per 16-row fragment, 16 KiB per panel;
// the scales of a panel's K block are one contiguous KiB.)
//
// Tiles.  A block computes 256 x 256 outputs with 8 waves (2 x 4), each
// wave 128 x 64 (8 x 4 fragments of 16 x 16, 128 accumulator registers), two
// waves per SIMD.  K runs as one stream of stages through a ring of LDS
// slots (three of 48 KiB for E2M3, four of 34 KiB for MXFP4): low stages
// (128 slots: A panel, B panel, MXFP4 also their scales), then branch stages (32 bf16 channels: 16 KiB + 16 KiB, rows 64 bytes with
// their 16-byte chunks XOR-swizzled by row so the MFMA operand reads hit
// distinct banks).  The two waves of a SIMD take turns: while one multiplies
// a stage from registers, the other reads its next stage's fragments from
// LDS and issues a later stage's DMAs (two phases per stage, each ended by a
// workgroup barrier; the schedule is spelled out at the loop).  Blocks are
// mapped XCD-aware (each XCD a contiguous run of tiles, rastered in groups of
// 8 tile rows).
#include "sqf_device.h"
#include "sqf_launch.h"

namespace sqf {

typedef int v6i __attribute__((ext_vector_type(6)));

// The FP6 overload of the scaled f8f6f4 MFMA: an FP6 operand is six
// registers (the clang builtin only takes the eight-register FP8 tuple, which
// would hold two dead registers per fragment).
__device__ v4f mfma_fp6(v6i a, v6i b, v4f c, int cbsz, int blgp, int opsel_a, int scale_a, int opsel_b,
                        int scale_b) __asm("llvm.amdgcn.mfma.scale.f32.16x16x128.f8f6f4.v6i32.v6i32");

namespace {

constexpr int kBM = 256, kBN = 256;
constexpr int kWGM = 2, kWGN = 4, kNW = kWGM * kWGN;
constexpr int kTM = kBM / kWGM / 16, kTN = kBN / kWGN / 16;  // 8 x 4 fragments
constexpr int kBrRowB = 64;                                    // bytes per row per branch stage
constexpr int kBrDmaPerWave = (kBM + kBN) * kBrRowB / 1024 / kNW;  // 4
constexpr int kGroupM = 8;
constexpr int kStageWN = kTN * 16, kLDW = kStageWN + 4;         // epilogue staging (floats)
constexpr int kStageBytes = kNW * 16 * kLDW * 4;                // 34816

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f_a4 __attribute__((ext_vector_type(4), aligned(4)));  // s_x is only float-aligned

// Per low-format constants.
template <int LF>
struct LowFmt;
template <>
struct LowFmt<kI4E2M3> {
  static constexpr int kRowB = 96;                           // bytes per row per low stage
  static constexpr int kPanelB = kBM * kRowB;                // 24 KiB
  static constexpr int kDma = (kBM + kBN) * kRowB / 1024 / kNW;  // 6 per wave
  static constexpr int kScaleB = 0;
  static constexpr int kSlot = 48 * 1024;
  static constexpr int kRing = 3;
  static constexpr int kType = 2;  // FP6 E2M3 operands
};
template <>
struct LowFmt<kMXFP4> {
  static constexpr int kRowB = 64;
  static constexpr int kPanelB = kBM * kRowB;                // 16 KiB
  static constexpr int kDma = (kBM + kBN) * kRowB / 1024 / kNW;  // 4 per wave (+1 scale DMA on waves 0, 1)
  static constexpr int kScaleB = 1024;                       // E8M0 bytes per panel per K block
  static constexpr int kSlot = 34 * 1024;
  static constexpr int kRing = 4;
  static constexpr int kType = 4;  // FP4 E2M1 operands
};

// Operand fragments of lane l (32 fields: row l%16 of the fragment, slots
// 32*(l/16) .. +31 of the stage).  E2M1: one 16-byte read into 4 registers
// (the rest of the tuple unused).  E2M3: fragments come in pairs (rows
// 32p .. 32p+31); three 16-byte reads -- the two fragments' heads (bytes
// 0..15 of each lane's 24) and their interleaved tails (bytes 16..23) --
// fill 6 registers of each.  (ds_read_b128 moves about 1.6x the bytes per
// clock of ds_read_b64 here, and 24-byte reads as b64 x 3 made the LDS the
// limit of the stage.)
__device__ __forceinline__ v8i ld_fp4(const uint8_t* p) {
  const v4i a = *(const v4i*)p;
  return __builtin_shufflevector(a, a, 0, 1, 2, 3, -1, -1, -1, -1);
}
__device__ __forceinline__ void ld_fp6_pair(const uint8_t* pair, int lane, v6i& f0, v6i& f1) {
  const v4i h0 = *(const v4i*)(pair + lane * 16);
  const v4i h1 = *(const v4i*)(pair + 1024 + lane * 16);
  const v4i t = *(const v4i*)(pair + 2048 + lane * 16);
  f0 = __builtin_shufflevector(h0, t, 0, 1, 2, 3, 4, 5);
  f1 = __builtin_shufflevector(h1, t, 0, 1, 2, 3, 6, 7);
}

// s_waitcnt vmcnt for a wave-uniform count n of DMAs still allowed in
// flight, rounded down to one of the counts a wave can have outstanding.
template <int LF>
__device__ __forceinline__ void wait_dmas(int n) {
  if constexpr (LF == kI4E2M3) {
    if (n >= 6) wait_vmcnt<6>();
    else if (n >= 4) wait_vmcnt<4>();
    else wait_vmcnt<0>();
  } else {
    if (n >= 10) wait_vmcnt<10>();
    else if (n >= 9) wait_vmcnt<9>();
    else if (n >= 8) wait_vmcnt<8>();
    else if (n >= 5) wait_vmcnt<5>();
    else if (n >= 4) wait_vmcnt<4>();
    else wait_vmcnt<0>();
  }
}

// FP4 x FP4 with per-lane E8M0 scales; OA / OB pick the byte of the scale
// dwords (the builtin takes them as constants: the switch folds once the
// fragment loops are unrolled).
template <int OA, int OB>
__device__ __forceinline__ v4f mfma_fp4(v8i a, v8i b, v4f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 4, OA, sa, OB, sb);
}
__device__ __forceinline__ v4f mfma_fp4_sel(int oa, int ob, v8i a, v8i b, v4f c, int sa, int sb) {
  switch (oa * 4 + ob) {
    case 0: return mfma_fp4<0, 0>(a, b, c, sa, sb);
    case 1: return mfma_fp4<0, 1>(a, b, c, sa, sb);
    case 2: return mfma_fp4<0, 2>(a, b, c, sa, sb);
    case 3: return mfma_fp4<0, 3>(a, b, c, sa, sb);
    case 4: return mfma_fp4<1, 0>(a, b, c, sa, sb);
    case 5: return mfma_fp4<1, 1>(a, b, c, sa, sb);
    case 6: return mfma_fp4<1, 2>(a, b, c, sa, sb);
    case 7: return mfma_fp4<1, 3>(a, b, c, sa, sb);
    case 8: return mfma_fp4<2, 0>(a, b, c, sa, sb);
    case 9: return mfma_fp4<2, 1>(a, b, c, sa, sb);
    case 10: return mfma_fp4<2, 2>(a, b, c, sa, sb);
    case 11: return mfma_fp4<2, 3>(a, b, c, sa, sb);
    case 12: return mfma_fp4<3, 0>(a, b, c, sa, sb);
    case 13: return mfma_fp4<3, 1>(a, b, c, sa, sb);
    case 14: return mfma_fp4<3, 2>(a, b, c, sa, sb);
    default: return mfma_fp4<3, 3>(a, b, c, sa, sb);
  }
}

}  // namespace

template <int LF, bool DEBUG, bool YB>
__global__ __launch_bounds__(kNW * 64, 2) void k_gemm6(Gemm6Args p) {
  using F = LowFmt<LF>;
  static_assert(!(DEBUG && YB), "the accumulator dump comes with fp32 Y");
  static_assert(!(DEBUG && LF == kMXFP4), "MXFP4 sums are not integers");
  static_assert(2 * F::kPanelB + 2 * F::kScaleB <= F::kSlot && kBM * kBrRowB * 2 <= F::kSlot,
                "a stage fits its slot");
  static_assert(kStageBytes <= F::kSlot, "the epilogue staging fits one ring slot");
  constexpr int kRing = F::kRing;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kRing * F::kSlot];

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

  // DMA of stage t into ring slot t % kRing.  Low stage: the A panel (rows
  // m0..m0+255 of K block t) and the B panel are contiguous runs; instruction
  // q moves bytes q*1024 .. +1023 of the pair.  MXFP4: waves 0 and 1 also
  // move the A and B panels' scale KiB (after the panels in the slot).
  // Branch stage: row-major bf16 rows; instruction q of 32 covers 16 rows x
  // 4 chunks of 16 bytes, lane l -> row q*16 + l/4 (clamped to the last
  // real row), chunk (l%4) ^ ((row/4)%4) of the stage's 64 bytes.
  const int br_r = lane >> 2, br_c = lane & 3;
  auto issue = [&](int t) {
    const uint32_t slot = smem_lds + (uint32_t)((t % kRing) * F::kSlot);
    if (t < S) {
      const uint8_t* a = p.x6 + ((int64_t)t * p.x_rows + m0) * F::kRowB;
      const uint8_t* b = p.w6 + ((int64_t)t * p.w_rows + n0) * F::kRowB;
      constexpr int kPanelDma = F::kPanelB / 1024;
#pragma unroll
      for (int i = 0; i < F::kDma; ++i) {
        const int q = wave * F::kDma + i;  // wave-uniform
        const bool is_a = q < kPanelDma;
        const int ql = is_a ? q : q - kPanelDma;
        dma_16B(is_a ? a : b, (uint32_t)(ql * 1024 + lane * 16), slot + (uint32_t)(q * 1024));
      }
      if constexpr (F::kScaleB > 0) {
        if (wave < 2) {
          const uint8_t* sc = wave == 0 ? p.x_sc + ((int64_t)t * p.x_rows + m0) * 4
                                        : p.w_sc + ((int64_t)t * p.w_rows + n0) * 4;
          dma_16B(sc, (uint32_t)(lane * 16), slot + (uint32_t)(2 * F::kPanelB + wave * 1024));
        }
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
  // DMAs this wave issues for stage t (0 past the end)
  const int low_dmas = F::kDma + ((F::kScaleB > 0 && wave < 2) ? 1 : 0);
  auto dmas_of = [&](int t) { return t >= ST ? 0 : (t < S ? low_dmas : kBrDmaPerWave); };
  // DMAs allowed in flight at the top of stage t: those of the stages after it
  auto ahead = [&](int t) {
    int n = 0;
#pragma unroll
    for (int d = 1; d < kRing - 1; ++d) n += dmas_of(t + d);
    return n;
  };

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

  // the wave's fragments inside a low stage's panels: fragment (16 rows) f of
  // a panel is bytes f*16*kRowB .. +16*kRowB-1 (E2M3: fragment pairs of 3 KiB)
  const int fr = lane & 15, fg = lane >> 4;
  constexpr int kFragB = 16 * F::kRowB;
  const uint32_t a_off = (uint32_t)(wm * kTM * kFragB);
  const uint32_t b_off = (uint32_t)(F::kPanelB + wn * kTN * kFragB);
  // MXFP4 scale dwords: 64-row group h of the panel, lane l at 4*l
  const uint32_t as_off = (uint32_t)(2 * F::kPanelB + wm * 2 * 256 + 4 * lane);
  const uint32_t bs_off = (uint32_t)(2 * F::kPanelB + 1024 + wn * 256 + 4 * lane);

  // Two wave groups with one wave of every SIMD in each: waves 0-3 and 4-7
  // (a workgroup's waves go to the SIMDs round-robin; read back from HW_ID
  // on this chip).  Every stage is a load phase (the stage's fragments from
  // LDS into registers, then this wave's DMAs of stage t+kRing-1) and a
  // multiply phase (the stage's MFMAs from registers only), each ended by a
  // workgroup barrier.  Group 1 runs one phase behind group 0, so on every
  // SIMD one wave multiplies while the other loads.  Stage t is read in
  // phases 2t (group 0) and 2t+1 (group 1), so its slot is free from phase
  // 2t+2 on, where the load phase of stage t+1 refills it (with stage
  // t+kRing).  At the end of phase 2t+1 (group 0 after multiplying, group 1
  // after loading) every wave waits for its own DMAs of stage t+1, so the
  // barrier there hands group 0 a landed stage in phase 2t+2.
  const int grp = wave >> 2;
#pragma unroll
  for (int d = 0; d < kRing - 1; ++d)
    if (d < ST) issue(d);
  wait_dmas<LF>(ahead(0));
  stage_barrier();
  if (grp == 1) stage_barrier();

  // End of a load phase: the fragments are in registers (and, for group 1,
  // the slot is free).  The multiply phase runs at raised wave priority, so
  // when both waves of a SIMD can issue, the MFMA goes first.
  auto load_end = [&](int t) {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    if (grp == 1) wait_dmas<LF>(ahead(t + 1));
    __builtin_amdgcn_sched_barrier(0);
    stage_barrier();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
  };
  auto mul_end = [&](int t) {
    __builtin_amdgcn_s_setprio(0);
    if (grp == 0) wait_dmas<LF>(ahead(t + 1));
    __builtin_amdgcn_sched_barrier(0);
    stage_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---------------- low path on the 6-/4-bit matrix unit ----------------
  for (int t = 0; t < S; ++t) {
    const uint8_t* sl = smem + (t % kRing) * F::kSlot;
    // E2M3 fragments are six registers, FP4 ones four (of an eight-register tuple)
    typedef typename std::conditional<LF == kI4E2M3, v6i, v8i>::type frag_t;
    frag_t A[kTM], B[kTN];
    int sa0 = 0, sa1 = 0, sb = 0;
    if constexpr (LF == kI4E2M3) {
#pragma unroll
      for (int j = 0; j < kTN; j += 2) ld_fp6_pair(sl + b_off + j * kFragB, lane, B[j], B[j + 1]);
#pragma unroll
      for (int i = 0; i < kTM; i += 2) ld_fp6_pair(sl + a_off + i * kFragB, lane, A[i], A[i + 1]);
    } else {
#pragma unroll
      for (int j = 0; j < kTN; ++j) B[j] = ld_fp4(sl + b_off + j * kFragB + lane * 16);
#pragma unroll
      for (int i = 0; i < kTM; ++i) A[i] = ld_fp4(sl + a_off + i * kFragB + lane * 16);
      sa0 = *(const int*)(sl + as_off);
      sa1 = *(const int*)(sl + as_off + 256);
      sb = *(const int*)(sl + bs_off);
    }
    if (t + kRing - 1 < ST) issue(t + kRing - 1);
    load_end(t);
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j) {
        if constexpr (LF == kI4E2M3) {
          acc[i][j] = mfma_fp6(A[i], B[j], acc[i][j], 2, 2, 0, 0, 0, 0);
        } else {
          // opsel picks the fragment's byte of the scale dwords
          acc[i][j] = mfma_fp4_sel(i & 3, j & 3, A[i], B[j], acc[i][j], i < 4 ? sa0 : sa1, sb);
        }
      }
    mul_end(t);
  }

  const int mrows = (int)p.m, ncols = (int)p.n;
  if constexpr (LF == kI4E2M3) {
    // ---------------- exact sums -> scaled fp32 ----------------
    // Lane l holds rows 4*(l/16)+r (r < 4) and column l%16 of each fragment:
    // one 16-byte read of s_x per fragment row (clamped reads at the edge).
    // The indices are derived from an opaque copy of the lane id so that
    // they die here instead of living through the branch loop.
    int ls = lane;
    asm volatile("" : "+v"(ls));
    const int srow0 = (int)m0 + wm * kTM * 16 + (ls >> 4) * 4;
    const int scol0 = (int)n0 + wn * kTN * 16 + (ls & 15);
    float sw[kTN];
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
      const int col = scol0 + j * 16;
      sw[j] = p.s_w[col < ncols ? col : ncols - 1] * 64.0f;
    }
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      const int row = srow0 + i * 16;
      v4f sx;
      if (row + 3 < mrows) {
        sx = *(const v4f_a4*)(p.s_x + row);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) sx[r] = p.s_x[row + r < mrows ? row + r : mrows - 1];
      }
#pragma unroll
      for (int j = 0; j < kTN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (DEBUG) {
            const int col = scol0 + j * 16;
            if (row + r < mrows && col < ncols)
              p.acc_dbg[(int64_t)(row + r) * p.n + col] = (int32_t)(acc[i][j][r] * 64.0f);
          }
          acc[i][j][r] *= sx[r] * sw[j];
        }
    }
  }

  // ---------------- branch: bf16 outlier sub-tensor GEMM ----------------
  // Lane l reads row l%16 of a fragment, chunk l/16 of the stage's 4.
  const int bc = fg;
  auto br_off = [&](int r) { return (uint32_t)(r * kBrRowB + 16 * (bc ^ ((r >> 2) & 3))); };
  for (int t = S; t < ST; ++t) {
    const uint8_t* sl = smem + (t % kRing) * F::kSlot;
    v4i A[kTM], B[kTN];
#pragma unroll
    for (int j = 0; j < kTN; ++j)
      B[j] = *(const v4i*)(sl + kBM * kBrRowB + br_off(wn * kTN * 16 + j * 16 + fr));
#pragma unroll
    for (int i = 0; i < kTM; ++i) A[i] = *(const v4i*)(sl + br_off(wm * kTM * 16 + i * 16 + fr));
    if (t + kRing - 1 < ST) issue(t + kRing - 1);
    load_end(t);
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(v8bf, A[i]), __builtin_bit_cast(v8bf, B[j]), acc[i][j], 0, 0, 0);
    mul_end(t);
  }
  if (grp == 0) stage_barrier();
  // ---------------- store ----------------
  // Lane l holds rows 4*(l/16)+r (r < 4) and column l%16 of each fragment.
  const int row0 = (int)m0 + wm * kTM * 16 + (lane >> 4) * 4;
  const int col0 = (int)n0 + wn * kTN * 16 + (lane & 15);
  const int wrow0 = (int)m0 + wm * kTM * 16, wcol0 = (int)n0 + wn * kTN * 16;
  constexpr int WN = kStageWN, LDW = kLDW;
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

hipError_t launch_gemm6(const Gemm6Args& a, int low, bool debug, bool ybf16, hipStream_t s) {
  if (debug && ybf16) return hipErrorInvalidValue;
  if (low != kI4E2M3 && low != kMXFP4) return hipErrorInvalidValue;
  if (low == kMXFP4 && debug) return hipErrorInvalidValue;
  const int64_t blocks = ((a.m + kBM - 1) / kBM) * ((a.n + kBN - 1) / kBN);
  if (blocks <= 0) return hipSuccess;
  const dim3 grid((unsigned)blocks), block(kNW * 64);
  if (low == kMXFP4) {
    if (ybf16)
      hipLaunchKernelGGL((k_gemm6<kMXFP4, false, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((k_gemm6<kMXFP4, false, false>), grid, block, 0, s, a);
  } else if (debug) {
    hipLaunchKernelGGL((k_gemm6<kI4E2M3, true, false>), grid, block, 0, s, a);
  } else if (ybf16) {
    hipLaunchKernelGGL((k_gemm6<kI4E2M3, false, true>), grid, block, 0, s, a);
  } else {
    hipLaunchKernelGGL((k_gemm6<kI4E2M3, false, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace sqf
