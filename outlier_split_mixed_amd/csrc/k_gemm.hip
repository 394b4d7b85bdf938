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
// (TM*16) x (TN*16) sub-tile.  K advances in 64-byte steps of every operand
// row (128 int4 slots, 32 bf16 or 64 E4M3), and operands move from global
// memory to LDS in pairs of steps: one global_load_lds_dwordx4 brings 8 full
// 128-byte row segments, so every request it makes is a whole cache line
// (16 half lines per instruction cost markedly more).  LDS holds two pair
// buffers; the 16-byte chunks of each row are XOR-swizzled on the way in, so
// that the ds_read_b128 that feeds an MFMA operand (16 rows x one chunk)
// touches distinct banks.  The block -> tile map is XCD-aware: consecutive
// hardware block ids go to different XCDs, so they are remapped to give every
// XCD a contiguous run of logical tiles, then rastered in groups of GROUP_M
// tile rows to share operand panels in each XCD's L2.
#include "sqf_device.h"
#include "sqf_launch.h"

namespace sqf {

// Direct global -> LDS loader for one pair of K steps.  A pair buffer holds
// (BM + BN) / 16 row blocks of 2 KiB: 16 rows x 128 bytes (two steps of 64).
// Half h of block rb (rows rb*16 + 8h .. +7) is filled by one DMA: lane l
// brings row 8h + l/8, chunk (l%8) ^ swz(h, l/8) of the 128 bytes, and lands
// at byte 16*l of that half (LDS offset rb*2048 + h*1024 + 16*l).  Reading it
// back: chunk C of row R sits at (R/8)*1024 + (R%8)*128 + 16*(C ^ swz(R/8, R%8)).
// swz(h, r) = r ^ 2h makes the 16 rows x one chunk of an MFMA operand read
// hit 16 distinct 16-byte bank groups (and any 8 consecutive lanes distinct
// ones).  Each wave owns PW consecutive halves (A rows first, then B rows).

template <int BM, int BN, int NW>
struct DmaLoader {
  static constexpr int HALVES = (BM + BN) / 8;  // DMAs per pair buffer
  static constexpr int PW = HALVES / NW;
  static constexpr int AH = BM / 8;  // halves holding A rows
  static_assert(HALVES % NW == 0, "DMAs must split evenly over waves");
  uint32_t off[PW];
  int q0;

  __device__ __forceinline__ void init(int wave, int lane, int64_t a_row0, int64_t a_end,
                                       int64_t b_row0, int64_t b_end, int64_t ld) {
    q0 = wave * PW;
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const int q = q0 + i;  // wave-uniform: A rows if q < AH
      const bool is_a = q < AH;
      const int ql = is_a ? q : q - AH;  // half index within the operand
      const int rl = lane >> 3;
      int64_t grow = (is_a ? a_row0 : b_row0) + ql * 8 + rl;
      const int64_t lim = (is_a ? a_end : b_end) - 1;
      if (grow > lim) grow = lim;
      off[i] = (uint32_t)(grow * ld + ((lane & 7) ^ pair_swz(ql & 1, rl)) * 16);
    }
  }
};
// OCC: blocks meant to share a CU (sets the register budget so that
// OCC * WGM * WGN waves fit: 2 waves per SIMD either way).
// YB: Y is written as bf16 (round to nearest even of the fused fp32 value).
template <int BM, int BN, int WGM, int WGN, int OCC, int BR, bool GROUPED, bool DEBUG, int GROUP_M,
          bool YB>
__global__ __launch_bounds__(WGM* WGN * 64, (WGM * WGN * OCC + 3) / 4) void k_dual_gemm(GemmArgs p) {
  constexpr int NW = WGM * WGN;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int PAIR = (BM + BN) * 128;  // bytes per pair buffer
  constexpr int PW = DmaLoader<BM, BN, NW>::PW;
  static_assert(TM >= 1 && TN >= 1, "wave tile too small");
  static_assert(2 * PAIR * OCC <= 160 * 1024, "LDS budget");
  static_assert(!(DEBUG && YB), "the accumulator dump comes with fp32 Y");
  __shared__ __attribute__((aligned(2048))) uint8_t smem[2 * PAIR];

  const int tid = threadIdx.x, lane = tid & 63;
  // wave index, provably uniform (operand bases and LDS addresses stay scalar)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int64_t tiles_n = (p.n + BN - 1) / BN;

  // ---- block -> tile (XCD-aware) ----
  int64_t lid = blockIdx.x;
  if constexpr (!GROUPED) {
    const int64_t nb = gridDim.x;
    if ((nb & 7) == 0) lid = (lid & 7) * (nb >> 3) + (lid >> 3);
  }
  int64_t m_begin = 0, m_end = p.m, tm, tn;
  const uint8_t* w_low = p.w_low;
  const uint8_t* w_out = p.w_out;
  const float* s_w = p.s_w;
  const float* s_wo = p.s_wo;
  if constexpr (GROUPED) {
    // Group g owns ceil(rows_g / BM) * tiles_n tiles, in group order.  The
    // block finds the group of its tile cooperatively: each thread counts the
    // tiles of one group, a block-wide prefix sum turns the counts into tile
    // ranges, and the thread whose range holds the tile publishes it.
    __shared__ int64_t s_part[NW];
    __shared__ int64_t s_found[2];  // group, first tile of the group
    if (tid == 0) s_found[0] = -1;
    // The grid is an upper bound on the tile count, so the XCD remap runs over
    // the real count T: XCD x (hardware blocks x, x + 8, ...) takes the
    // logical tiles [x * ceil(T/8), (x + 1) * ceil(T/8)).
    {
      int64_t cnt = 0;
      for (int g = tid; g < p.groups; g += NW * 64)
        cnt += ((p.row_off[g + 1] - p.row_off[g] + BM - 1) / BM) * tiles_n;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
      if (lane == 0) s_part[wave] = cnt;
      __syncthreads();
      int64_t total = 0;
      for (int w = 0; w < NW; ++w) total += s_part[w];
      __syncthreads();
      const int64_t per = (total + 7) >> 3;
      const int64_t j = lid >> 3;
      lid = (lid & 7) * per + j;
      if (j >= per || lid >= total) return;
    }
    int64_t carry = 0;
    for (int g0 = 0; g0 < p.groups; g0 += NW * 64) {
      const int g = g0 + tid;
      int64_t cnt = 0;
      if (g < p.groups) cnt = ((p.row_off[g + 1] - p.row_off[g] + BM - 1) / BM) * tiles_n;
      int64_t incl = cnt;  // inclusive prefix within the wave
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int64_t t = __shfl_up(incl, off, 64);
        if (lane >= off) incl += t;
      }
      if (lane == 63) s_part[wave] = incl;
      __syncthreads();
      int64_t before = carry;
      for (int w = 0; w < wave; ++w) before += s_part[w];
      int64_t chunk = 0;
      for (int w = 0; w < NW; ++w) chunk += s_part[w];
      const int64_t lo_t = before + incl - cnt;
      if (g < p.groups && lid >= lo_t && lid < lo_t + cnt) {
        s_found[0] = g;
        s_found[1] = lo_t;
      }
      carry += chunk;
      __syncthreads();
      if (s_found[0] >= 0) break;
    }
    if (s_found[0] < 0) return;  // beyond the last tile
    const int g = (int)s_found[0];
    const int64_t base = s_found[1];
    m_begin = p.row_off[g];
    m_end = p.row_off[g + 1];
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

  // One stream of K steps: steps 0 .. S-1 are the low path (packed int4,
  // stride ldk), steps S .. S+SO-1 the branch (stride ldo_b).  S and SO are
  // even (rows are padded to 128 bytes), so a pair never mixes the two, and
  // both run through the same two pair buffers: the branch's first pair is
  // already in flight when the low path ends.
  const int S = p.s_low, SO = p.s_out, ST = S + SO;
  // per-lane row offsets of this wave's DMAs for both operand streams
  // (selected per pair with wave-uniform selects, no control flow)
  DmaLoader<BM, BN, NW> ld_lo, ld_br;
  ld_lo.init(wave, lane, m0, m_end, n0, p.n, p.ldk);
  ld_br.init(wave, lane, m0, m_end, n0, p.n, p.ldo_b);
  const uint32_t smem_lds = lds_offset(smem);
  // pair q = steps 2q, 2q+1 -> pair buffer q % 2
  auto issue_from = [&](int q, bool lo) {
    const int t = 2 * q;
    const uint8_t* a = lo ? p.x_low : p.x_out;
    const uint8_t* b = lo ? w_low : w_out;
    const uint32_t so = (uint32_t)(lo ? t : t - S) * 64u;
    const uint32_t buf = smem_lds + (uint32_t)((q & 1) * PAIR);
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const int h = ld_lo.q0 + i;  // wave-uniform
      const uint8_t* base = h < DmaLoader<BM, BN, NW>::AH ? a : b;
      const uint32_t off = lo ? ld_lo.off[i] : ld_br.off[i];
      dma_16B(base, off + so, buf + (uint32_t)(h * 1024));
    }
  };
  auto issue = [&](int q) { issue_from(q, 2 * q < S); };
  // branch pairs only (lets the low path's offsets die after its loop)
  auto issue_br = [&](int q) { issue_from(q, false); };
  // this lane's read offset inside a 2 KiB row block for step parity `sub`:
  // row R = lane % 16, chunk C = lane / 16 + 4 * sub
  uint32_t rd_off[2];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    const int R = lane & 15, C = (lane >> 4) + 4 * sub;
    rd_off[sub] = (uint32_t)((R >> 3) * 1024 + (R & 7) * 128 + 16 * (C ^ pair_swz(R >> 3, R & 7)));
  }
  // the operand fragment of row block rb for step t
  auto frag = [&](int t, int rb) -> v4i {
    return *(const v4i*)(smem + ((t >> 1) & 1) * PAIR + rb * 2048 + rd_off[t & 1]);
  };

  v4i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4i{0, 0, 0, 0};
  // A group's last row tile is mostly empty (its rows end inside it): there
  // each wave runs the MFMAs of its 16-row fragments that hold rows and skips
  // the rest (a wave-uniform branch per fragment; plain tiles never skip).
  int live = TM;
  if constexpr (GROUPED) {
    const int64_t left = m_end - (m0 + wm * WM);
    live = left <= 0 ? 0 : left >= TM * 16 ? TM : (int)((left + 15) >> 4);
    live = __builtin_amdgcn_readfirstlane(live);
  }

  // Pipeline.  A step computes its 64 bytes of K in two halves.  Between
  // them, mid_sync issues the LDS reads of step t+1's B fragments and first A
  // fragment into PB / PA0 (the second half's MFMAs hide their latency); the
  // rest of step t+1's A fragments are read at its start, behind the MFMAs on
  // the prefetched first one.  At the end of a pair (odd t) mid_sync first
  // waits for the next pair to land, crosses the barrier, and refills the
  // buffer of the pair just finished (every wave holds all of it in
  // registers by then) with the pair after next.  The low path widens PB and
  // PA0 completely at the top of a step, so the registers are free again
  // before mid_sync refills them and the loop carries them without a copy.
  v4i PB[TN], PA0;  // prefetched fragments of the next step
  auto prefetch = [&](int t) {
#pragma unroll
    for (int j = 0; j < TN; ++j) PB[j] = frag(t, BM / 16 + wn * TN + j);
    PA0 = frag(t, wm * TM);
  };
  auto mid_sync = [&](int t) {
    if (t & 1) {
      // only the next pair (t+1, t+2) can be in flight here
      wait_vmcnt<0>();
      // every LDS read of this pair has returned (the bf16 branch reads the
      // second half's fragments before this point but uses them after it)
      __builtin_amdgcn_s_waitcnt(0xC07F);
      stage_barrier();
      const int q = (t >> 1) + 2;
      if (2 * q < ST) issue(q);
    }
    prefetch(t + 1);
  };
  // step t's A fragments 1.. from LDS (fragment 0 and B were prefetched)
  auto load_a = [&](int t, v4i (&A)[TM]) {
#pragma unroll
    for (int i = 1; i < TM; ++i) A[i] = frag(t, wm * TM + i);
    // keep the reads at the top of the step: their latency then overlaps
    // the MFMAs on the prefetched fragments instead of stalling each use
    __builtin_amdgcn_sched_barrier(0);
  };
  // int4 pairs (two dwords = 16 codes) -> 16 * int8 (four dwords)
  auto widen = [](uint32_t x, uint32_t y) {
    return v4i{(int)((x << 4) & 0xF0F0F0F0u), (int)(x & 0xF0F0F0F0u),
               (int)((y << 4) & 0xF0F0F0F0u), (int)(y & 0xF0F0F0F0u)};
  };

  // The epilogue's arguments are read with scalar loads.  If one of them were
  // still outstanding during the K loop, the LDS read counter could no longer
  // be waited on in order and every LDS wait there would become a full
  // drain, so they are made to land here.
  {
    const float* y_ = p.y;
    const float* sx_ = p.s_x;
    const float* sxo_ = p.s_xo;
    int32_t* dbg_ = p.acc_dbg;
    const int64_t ldy_ = p.ldy, n_ = p.n;
    asm volatile("" ::"s"(y_), "s"(sx_), "s"(sxo_), "s"(dbg_), "s"(ldy_), "s"(n_), "s"(s_w),
                 "s"(s_wo));
  }

  // prime: both pair buffers, wait for the first
  issue(0);
  if (ST > 2) {
    issue(1);
    wait_vmcnt<PW>();
  } else {
    wait_vmcnt<0>();
  }
  stage_barrier();
  prefetch(0);

  // ---------------- low path: int4 x int4 on int8 MFMA ----------------
  for (int t = 0; t < S; ++t) {
    v4i A[TM], bw[2][TN], a0w[2];
    load_a(t, A);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int j = 0; j < TN; ++j) bw[h][j] = widen((uint32_t)PB[j][2 * h], (uint32_t)PB[j][2 * h + 1]);
      a0w[h] = widen((uint32_t)PA0[2 * h], (uint32_t)PA0[2 * h + 1]);
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      // unconditional, also on the last step (the prefetch then reads a
      // pair buffer whose contents go unused): a conditional refill would
      // keep the old PB / PA0 alive beside the new ones
      if (half == 1) {
        mid_sync(t);
        __builtin_amdgcn_sched_barrier(0);
      }
      // Wave priority: the two waves of a SIMD cross the same barriers and
      // so tend to reach their MFMA runs together.  Each wave raises its
      // priority after its first 16-row fragment and drops it before the
      // last: the raised wave issues its MFMAs back to back while the other
      // one, at the lower level, widens operands and reads LDS (+4-6% on
      // the whole kernel against no priority change, measured).
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        if (GROUPED && i >= live) break;
        if (i == 1) __builtin_amdgcn_s_setprio(1);
        if (i == TM - 1) __builtin_amdgcn_s_setprio(0);
        const v4i aa = i == 0 ? a0w[half]
                              : widen((uint32_t)A[i][2 * half], (uint32_t)A[i][2 * half + 1]);
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aa, bw[half][j], acc[i][j], 0, 0, 0);
      }
      __builtin_amdgcn_s_setprio(0);
    }
  }

  // ---------------- exact int32 -> scaled fp32 ----------------
  // Lane l holds rows 4*(l/16)+r (r < 4) and column l%16 of each 16x16 tile.
  // Row and column indices fit in 32 bits (the host limits operand sizes).
  const int row0 = (int)(m0 - m_begin) + wm * WM + (lane >> 4) * 4;  // tile-local to the group
  const int col0 = (int)n0 + wn * WN + (lane & 15);
  const int mrows = (int)(m_end - m_begin), ncols = (int)p.n;
  const float* s_x = p.s_x + m_begin;
  v4f c[TM][TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int col = col0 + j * 16;
    const float sw = s_w[col < ncols ? col : ncols - 1] * 0.00390625f;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + i * 16 + r;
        if constexpr (DEBUG) {
          if (row < mrows && col < ncols)
            p.acc_dbg[(m_begin + row) * p.n + col] = acc[i][j][r] >> 8;
        }
        c[i][j][r] = (float)acc[i][j][r] * (s_x[row < mrows ? row : mrows - 1] * sw);
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
  // The branch keeps the whole next step in registers: a bf16 step has half
  // the MFMA work of an int4 step, too little to hide the LDS reads of its
  // own A fragments.  CUR holds step t, NXT is read during step t; at the
  // start of an odd step (the second of a pair) the pair sync runs first, so
  // the reads of the following pair's first step come after its barrier.
  auto read_step = [&](int t, v4i (&A)[TM], v4i (&B)[TN]) {
#pragma unroll
    for (int i = 0; i < TM; ++i) A[i] = frag(t, wm * TM + i);
#pragma unroll
    for (int j = 0; j < TN; ++j) B[j] = frag(t, BM / 16 + wn * TN + j);
  };
  auto br_mfma = [&](const v4i (&A)[TM], const v4i (&B)[TN]) {
    if constexpr (BR == kBF16) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        if (GROUPED && i >= live) break;
#pragma unroll
        for (int j = 0; j < TN; ++j)
          c[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(v8bf, A[i]), __builtin_bit_cast(v8bf, B[j]), c[i][j], 0, 0, 0);
      }
    } else {
      // E4M3: two MFMAs (K = 32 each) per 16-byte fragment
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          if (GROUPED && i >= live) break;
          const long a8 = (long)(((uint64_t)(uint32_t)A[i][2 * h + 1] << 32) | (uint32_t)A[i][2 * h]);
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const long b8 = (long)(((uint64_t)(uint32_t)B[j][2 * h + 1] << 32) | (uint32_t)B[j][2 * h]);
            c2[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a8, b8, c2[i][j], 0, 0, 0);
          }
        }
    }
  };
  auto br_sync = [&](int t) {
    wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(0xC07F);
    stage_barrier();
    const int q = (t >> 1) + 2;
    if (2 * q < ST) issue_br(q);
  };
  if (S < ST) {
    // S is even: the branch starts on a pair boundary with step S's B and
    // first A fragment already prefetched
    v4i A0[TM], B0[TN], A1[TM], B1[TN];
    A0[0] = PA0;
#pragma unroll
    for (int j = 0; j < TN; ++j) B0[j] = PB[j];
#pragma unroll
    for (int i = 1; i < TM; ++i) A0[i] = frag(S, wm * TM + i);
    for (int t = S; t < ST; t += 2) {
      // even step t: its successor is in the same pair
      read_step(t + 1, A1, B1);
      br_mfma(A0, B0);
      __builtin_amdgcn_sched_barrier(0);
      // odd step t+1: sync for the next pair, then read its first step
      if (t + 2 < ST) {
        br_sync(t + 1);
        read_step(t + 2, A0, B0);
      }
      br_mfma(A1, B1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---------------- epilogue part 2: fuse and store ----------------
  float* y = p.y + m_begin * p.ldy;
  uint16_t* yb = (uint16_t*)p.y + m_begin * p.ldy;  // (bf16 Y)
  auto fused = [&](int i, int j, int r, int row, int col) {
    float v = c[i][j][r];
    // rows past the end (staged path) read the last row's scale, unused
    if constexpr (BR == kFP8)
      v += (p.s_xo[m_begin + (row < mrows ? row : mrows - 1)] * s_wo[col]) * c2[i][j][r];
    return v;
  };
  const int wrow0 = (int)(m0 - m_begin) + wm * WM, wcol0 = (int)n0 + wn * WN;
  // (grouped: also a tile that ends inside the wave's rows, skipping the
  // rows past the end per 16-row fragment and per row)
  const bool whole = (GROUPED || wrow0 + WM <= mrows) && wcol0 + WN <= ncols &&
                     (p.ldy & 3) == 0 && (((uintptr_t)p.y) & (YB ? 7 : 15)) == 0;
  if (whole) {
    // Y is written once and not read here: non-temporal stores keep it from
    // evicting the operand panels other tiles still stream from L2.
    // Row-contiguous stores: each 16-row slice of the wave tile goes through
    // this wave's part of the pair buffer the K loop no longer uses (the one
    // that held pair NP-2; no DMA targets it any more), padded by 4 floats
    // per row so that both the 4-byte writes and the 16-byte reads are free
    // of bank conflicts, and leaves as 16-byte stores of whole row segments.
    constexpr int LDW = WN + 4;
    static_assert(NW * 16 * LDW * 4 <= PAIR, "staging fits the free pair buffer");
    float* stg = (float*)(smem + ((ST >> 1) & 1) * PAIR) + wave * (16 * LDW);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if (GROUPED && wrow0 + i * 16 >= mrows) break;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          stg[((lane >> 4) * 4 + r) * LDW + j * 16 + (lane & 15)] =
              fused(i, j, r, row0 + i * 16 + r, col0 + j * 16);
#pragma unroll
      for (int k = 0; k < WN / 16; ++k) {
        const int idx = k * 64 + lane, rr = idx / (WN / 4), c4 = idx % (WN / 4);
        const v4f v = *(const v4f*)(stg + rr * LDW + 4 * c4);
        if (!GROUPED || wrow0 + i * 16 + rr < mrows) {
          const int64_t o = (int64_t)(wrow0 + i * 16 + rr) * p.ldy + wcol0 + 4 * c4;
          if constexpr (YB) {
            // v_cvt_pk_bf16_f32: two values per instruction, nearest even
            const v2u h = v2u{__builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{v.x, v.y}, v2bf)),
                              __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{v.z, v.w}, v2bf))};
            __builtin_nontemporal_store(h, (v2u*)(yb + o));
          } else {
            __builtin_nontemporal_store(v, (v4f*)(y + o));
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + i * 16 + r;
        if (row >= mrows) continue;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = col0 + j * 16;
          if (col >= ncols) continue;
          const float v = fused(i, j, r, row, col);
          if constexpr (YB)
            __builtin_nontemporal_store(__builtin_bit_cast(uint16_t, (__bf16)v), yb + (int64_t)row * p.ldy + col);
          else
            __builtin_nontemporal_store(v, y + (int64_t)row * p.ldy + col);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ launch
template <int BM, int BN, int WGM, int WGN, int OCC, int BR, bool GROUPED, bool DEBUG, bool YB>
static hipError_t launch_cfg(const GemmArgs& a, hipStream_t s) {
  int64_t tiles_n = (a.n + BN - 1) / BN;
  int64_t blocks;
  if (GROUPED)  // an upper bound on the tiles, a multiple of the 8 XCDs
    blocks = (((a.m + BM - 1) / BM + a.groups) * tiles_n + 7) & ~(int64_t)7;
  else
    blocks = ((a.m + BM - 1) / BM) * tiles_n;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_dual_gemm<BM, BN, WGM, WGN, OCC, BR, GROUPED, DEBUG, 8, YB>),
                     dim3((unsigned)blocks), dim3(WGM * WGN * 64), 0, s, a);
  return hipGetLastError();
}

template <int BR, bool GROUPED, bool DEBUG, bool YB>
static hipError_t launch_br(const GemmArgs& a, int cfg, hipStream_t s) {
  if constexpr (GROUPED) {
    // expert groups hold a few hundred rows each: 256x256 or 128x128 tiles
    if (BR != kFP8 && cfg == 0) {
      if constexpr (BR != kFP8) return launch_cfg<256, 256, 2, 4, 1, BR, GROUPED, DEBUG, YB>(a, s);
    }
    return launch_cfg<128, 128, 2, 2, 2, BR, GROUPED, DEBUG, YB>(a, s);
  } else {
    // an E4M3 branch keeps a second accumulator set: no 256x256 tile for it
    if (BR == kFP8 && cfg == 0) cfg = 1;
    switch (cfg) {
      case 0:
        if constexpr (BR != kFP8) return launch_cfg<256, 256, 2, 4, 1, BR, GROUPED, DEBUG, YB>(a, s);
        [[fallthrough]];
      case 1:
        return launch_cfg<128, 128, 2, 2, 2, BR, GROUPED, DEBUG, YB>(a, s);
      default:
        return launch_cfg<64, 64, 2, 2, 2, BR, GROUPED, DEBUG, YB>(a, s);
    }
  }
}

// cfg: 0 = 256x256 (8 waves), 1 = 128x128 (4 waves, two blocks per CU),
// 2 = 64x64 (4 waves, two blocks per CU).  ybf16: bf16 Y (not with debug).
template <int BR, bool GROUPED>
static hipError_t launch_mode(const GemmArgs& a, bool debug, bool ybf16, int cfg, hipStream_t s) {
  if (debug) return launch_br<BR, GROUPED, true, false>(a, cfg, s);
  if (ybf16) return launch_br<BR, GROUPED, false, true>(a, cfg, s);
  return launch_br<BR, GROUPED, false, false>(a, cfg, s);
}

hipError_t launch_dual_gemm(const GemmArgs& a, int branch, bool grouped, bool debug, int cfg,
                            hipStream_t s, bool ybf16) {
  if (debug && ybf16) return hipErrorInvalidValue;
  if (branch == kFP8) {
    if (grouped) return launch_mode<kFP8, true>(a, debug, ybf16, cfg, s);
    return launch_mode<kFP8, false>(a, debug, ybf16, cfg, s);
  }
  if (grouped) return launch_mode<kBF16, true>(a, debug, ybf16, cfg, s);
  return launch_mode<kBF16, false>(a, debug, ybf16, cfg, s);
}

}  // namespace sqf
