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
// gfx950 mapping.  The "gather unit" is the decode of each 128-slot K stage of
// a block's W rows into LDS, once per block: a stage of a W row becomes
//   * an int8 low tile: the int4 codes with the marks cleared to 0 (SWAR: a
//     nibble is the mark iff its top bit is set and its low three bits are
//     zero), widened to int8 as 16*code (w << 4 & 0xF0.. and w & 0xF0..) and
//     put back in slot order with two byte permutes per 8 slots;
//   * an int8 tile holding the row's sparse values at their marked slots
//     (zero elsewhere): every 8-slot group is expanded at once from a window
//     of the row's values with byte permutes whose selectors come from a
//     table indexed by the group's mark mask.
// Both tiles and the int8 activations are in natural slot order, so the MFMA
// loop is LDS reads and v_mfma_i32_16x16x64_i8 only: the widening is done
// once per W row per block rather than once per wave that reads it.  The low
// accumulator carries the x16 factor (|acc| <= 16*127*7*k_low < 2^31 for the
// k_low the host accepts); it is removed exactly in the epilogue.
//
// Pipeline.  A block computes 256 x 128 outputs with 8 waves (4 x 2, each
// 64 x 64).  Activations and raw W codes move global -> LDS by DMA
// (global_load_lds_dwordx4) through two-stage rings; the values of a stage
// are fetched the same way, as a 64-byte window per row that starts at the
// row's running value index (known once the previous stage is decoded).
// Iteration s decodes stage s+1 (every wave its own 16 W rows, four lanes per
// row) and runs the MFMAs of stage s in one basic block, so the decode's
// vector ALU work can issue between the MFMAs; one barrier per stage.  The
// DMAs of A stage s+2 and W stage s+3 start right after that barrier, and the
// value window of stage s+2 right after stage s+1 is decoded.
//
// Floating-point form (SQ-format article, section 八: FP8 high-precision
// part, FP4 low part): E4M3 activations, E2M1 weight codes with the same
// 0x8 mark, E4M3 sparse values and branch.  The same pipeline and decode;
// the tiles are laid out for v_mfma_scale_f32_16x16x128_f8f6f4, whose lane
// l of a 16 x 128 operand holds row l%16 and, for FP4, slots 32(l/16) ..
// +31 (16 bytes), for FP8 slots 16(l/16) .. +15 and 64 + 16(l/16) .. +15
// (32 bytes; measured: with one FP8 and one FP4 operand the layouts must
// differ like this, with two FP8 operands any common order works).  The
// clean tile is the raw E2M1 nibbles with the marks cleared (a cleared mark
// is +0); the sparse tile holds the E4M3 values at their slots in the FP8
// order.  The low pass is
// E4M3 x E2M1, the sparse pass and the branch E4M3 x E4M3, all with fp32
// accumulators (not exact).
#include <type_traits>

#include "sqf_device.h"
#include "sqf_launch.h"

namespace sqf {

namespace {

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// eight int4 codes (natural nibble order: slot 2b in the low nibble of byte
// b) -> eight int8 values 16*code in slot order
__device__ __forceinline__ uint2 widen8(uint32_t w) {
  const uint32_t lo = (w << 4) & 0xF0F0F0F0u;  // slots 0, 2, 4, 6
  const uint32_t hi = w & 0xF0F0F0F0u;         // slots 1, 3, 5, 7
  return make_uint2(perm(hi, lo, 0x05010400u), perm(hi, lo, 0x07030602u));
}

// dma_16B for lanes 0..47 only: the exec mask is narrowed and restored inside
// the statement (the wave is converged here), so the caller has no branch
__device__ __forceinline__ void dma_16B_lanes48(const uint8_t* base, uint32_t voff, uint32_t lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds);
  uint64_t saved;
  asm volatile(
      "s_mov_b64 %0, exec\n\t"
      "s_and_b32 exec_hi, exec_hi, 0xffff\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b64 exec, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(base), "{m0}"(m0v)
      : "memory");
}

// LDS barrier that does not wait for outstanding global loads.
__device__ __forceinline__ void sq_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  stage_barrier();
}

// LDS map of one block (bytes).
constexpr int kBM = 256, kBN = 128;
constexpr int kStA = kBM * 128;    // activation stage: 16-row blocks of 16 x 128 B (swizzled)
constexpr int kStW = kBN * 64;     // raw W stage: row-major, 64 B per row
constexpr int kVRow = 48;          // value window per row: three 16-byte blocks
constexpr int kStV = kBN * kVRow;  // value windows: row-major
constexpr int kStS = kBN * 128;    // sparse tile: [row block][K half][entry] x 16 B
template <bool FP>
struct SqLds {
  // clean low tile: E2M1 nibbles [row block][entry] x 16 B (FP), or int8
  // 16*code [row block][K half][entry] x 16 B (integer form)
  static constexpr int kStL = FP ? kBN * 64 : kBN * 128;
  static constexpr int kOffA = 0;
  static constexpr int kOffW = kOffA + 2 * kStA;
  static constexpr int kOffV = kOffW + 2 * kStW;
  static constexpr int kOffL = kOffV + 2 * kStV;
  static constexpr int kOffS = kOffL + 2 * kStL;
  static constexpr int kOffSel = kOffS + 2 * kStS;
  static constexpr int kSmem = kOffSel + 256 * 8;
};
static_assert(SqLds<false>::kSmem <= 160 * 1024 && SqLds<true>::kSmem <= 160 * 1024, "LDS budget");
// A decoded stage image in the workspace: the clean tile, then the sparse
// tile, each exactly as the fused decode leaves it in LDS (24 KiB in the FP
// form, whose clean tile is E2M1 nibbles; 32 KiB in the integer form).
template <bool FP>
constexpr int kImgBytes = SqLds<FP>::kStL + kStS;
// the branch's W tile (128 rows x 128 B, swizzled like A) reuses the raw W
// ring (even branch stages) and the clean-tile ring (odd ones)
static_assert(kBN * 128 <= 2 * kStW && kBN * 128 <= 2 * SqLds<true>::kStL, "branch W tile fits");

// Entry of MFMA lane (16-slot group g, row rr) in a 1 KiB block of a decoded
// integer tile (16 rows x 64 slots of one K half f): 16 g + (rr ^ 4 (g/2 +
// 2 f)).  The 64 lanes of a read cover the 64 entries once; the four lanes of
// a row that write at once (two K halves x two groups) land on four different
// 16-byte bank groups for each of the row's 4 x 4 neighbours.
__device__ __forceinline__ int tile_entry(int g, int rr, int f) {
  return (g << 4) | (rr ^ ((((g >> 1) + 2 * f) << 2) & 15));
}

}  // namespace

typedef int v8i __attribute__((ext_vector_type(8)));

template <bool DEBUG, bool FP, bool PRE>
__global__ __launch_bounds__(512, 1) void k_sq_gemm(SqArgs p) {
  static_assert(!(DEBUG && FP), "the floating-point form has no integer accumulators");
  using AccT = std::conditional_t<FP, v4f, v4i>;
  using L = SqLds<FP>;
  constexpr int kOffA = L::kOffA, kOffW = L::kOffW, kOffV = L::kOffV, kOffL = L::kOffL,
                kOffS = L::kOffS, kOffSel = L::kOffSel, kStL = L::kStL;
  constexpr int TM = 4, TN = 4;
  __shared__ __attribute__((aligned(2048))) uint8_t smem[L::kSmem];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  // rows, columns, stages and byte offsets fit in 32 bits (host limits)
  const int tiles_m = (int)((p.m + kBM - 1) / kBM);
  int lid = blockIdx.x;
  {
    // XCD-aware: hardware block b runs on XCD b % 8; give every XCD a
    // contiguous run of tiles (row tiles fastest: the W tile is shared)
    const int nb = gridDim.x;
    if ((nb & 7) == 0) lid = (lid & 7) * (nb >> 3) + (lid >> 3);
  }
  const int tm = lid % tiles_m, tn = lid / tiles_m;
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int mm = (int)p.m, nn = (int)p.n, nnz = (int)p.nnz;
  const int nst = (int)(p.ldkw / 64);  // 128-slot stages (ldkw is a multiple of 64)
  const uint32_t sbase = lds_offset(smem);

  // ---- DMA lanes ----
  // A: wave w brings the 8-row halves 4w .. 4w+3 of each stage; lane l row
  // 8q + l/8, chunk (l%8) ^ swz(q%2, l/8)
  uint32_t a_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = wave * 4 + i, rl = lane >> 3;
    int row = m0 + q * 8 + rl;
    if (row > mm - 1) row = mm - 1;
    a_off[i] = (uint32_t)row * (uint32_t)p.ldkx + (uint32_t)(((lane & 7) ^ pair_swz(q & 1, rl)) * 16);
  }
  // raw W: wave w brings rows 16w .. 16w+15; lane l row l/4, 16 bytes l%4
  uint32_t w_off;
  {
    int row = n0 + wave * 16 + (lane >> 2);
    if (row > nn - 1) row = nn - 1;
    w_off = (uint32_t)row * (uint32_t)p.ldkw + (uint32_t)((lane & 3) * 16);
  }
  auto issue_a = [&](int s) {
    const uint32_t buf = sbase + kOffA + (uint32_t)((s & 1) * kStA);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dma_16B(p.x_low, a_off[i] + (uint32_t)s * 128u, buf + (uint32_t)((wave * 4 + i) * 1024));
  };
  auto issue_w = [&](int s) {
    dma_16B(p.w_low, w_off + (uint32_t)s * 64u,
            sbase + kOffW + (uint32_t)((s & 1) * kStW) + (uint32_t)(wave * 1024));
  };

  // ---- decode lanes: every wave decodes its own 16 W rows (the rows its
  // raw-W DMA brings), four lanes per row: lane l takes row 16w + l/4 and its
  // 32 slots qq = l % 4 (K half f = qq / 2, 16-slot groups 2(qq%2), +1) ----
  const int r = tid >> 2, qq = tid & 3;
  const int f_own = qq >> 1, g0 = 2 * (qq & 1);
  const int rb = r >> 4, rr = r & 15;
  // floating-point tiles: entry of (row rr, slot group qq) in a 16-row block
  // (clean E2M1 tile); the sparse E4M3 tile takes slots 32qq + 8d .. +7 of
  // this lane to FP8 group g = 2(qq%2) + d/2, bytes 16(qq/2) + 8(d%2) ..
  const int fpos_w = (qq << 4) + (rr ^ (qq << 2));
  auto sp_off = [&](int d) {
    const int g = 2 * (qq & 1) + (d >> 1);
    return ((g << 4) + (rr ^ (g << 2))) * 32 + 16 * (qq >> 1) + 8 * (d & 1);
  };
  const int gn = n0 + r < nn ? n0 + r : nn - 1;
  const int8_t* vrow = p.sq_val + (int64_t)gn * nnz;
  // sq_val is 16-byte aligned (host check); a window starts at the 16-byte
  // boundary at or below the row's next value, and only whole blocks inside
  // the buffer are used.  The buffer has at least one whole block, else every
  // value is read one by one.
  const int64_t vtotal = p.n * p.nnz;
  const bool vdma = vtotal >= 16;
  const uint32_t vlast = (uint32_t)((vtotal & ~(int64_t)15) - 16);  // last whole block
  int vi = 0;  // row r's value index at the next stage to decode (same in its 4 lanes)
  // value window of stage s: lane l < 48 brings 16-byte block l % 3 of row
  // 16w + l / 3 (whose value index it takes from that row's first decode lane)
  const int vr = lane / 3, vb = lane - 3 * vr;
  const int gn_v = n0 + wave * 16 + vr < nn ? n0 + wave * 16 + vr : nn - 1;
  // (lanes 48..63 are switched off inside the DMA statement itself, so the
  // issue adds no branch to the iteration's basic block)
  auto issue_v = [&](int s) {
    const int v_row = __shfl(vi, (4 * vr) & 63, kWave);
    const uint32_t start = (uint32_t)(((int64_t)gn_v * nnz + v_row) & ~(int64_t)15);
    uint32_t off = start + (uint32_t)(vb * 16);
    if (off > vlast) off = vlast;  // past the buffer: any whole block (unused)
    dma_16B_lanes48(vdma ? (const uint8_t*)p.sq_val : p.x_low, vdma ? off : 0u,
                    sbase + kOffV + (uint32_t)((s & 1) * kStV) + (uint32_t)(wave * 16 * kVRow));
  };

  // Expand selectors: for the mark mask m of an 8-slot group, byte p of the
  // group's operand bytes (slot order) takes value number rank(p) (a byte of
  // the pool {hi, lo} of the group's values) if slot p is marked, else zero
  // (selector 0x0C).
  uint2* sSel = (uint2*)(smem + kOffSel);
  if (!PRE && tid < 256) {
    const int m = tid;
    uint32_t sel[2] = {0, 0};
#pragma unroll
    for (int pp = 0; pp < 8; ++pp) {
      const uint32_t b = ((m >> pp) & 1) ? (uint32_t)__builtin_popcount(m & ((1 << pp) - 1)) : 0x0Cu;
      sel[pp >> 2] |= b << (8 * (pp & 3));
    }
    sSel[m] = make_uint2(sel[0], sel[1]);
  }
  // this decode lane's two tile entries (integer form): groups g0, g0 + 1 of
  // K half f_own in row block rb, as LDS pointers into the clean tile of
  // slot 0 (the sparse tile and slot 1 are fixed offsets from them, small
  // enough for the instruction's immediate)
  const int ent0 = (rb * 2 + f_own) * 1024 + 16 * tile_entry(g0, rr, f_own);
  const int ent1 = (rb * 2 + f_own) * 1024 + 16 * tile_entry(g0 + 1, rr, f_own);
  // (LDS-typed, so the stores stay ds_write: a generic pointer would become
  // a flat store, which also makes every LDS wait a full drain)
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  typedef uint32_t lds_v4u_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) lds_v4u_t lds_v4u;
  lds_u8* wb0 = (lds_u8*)(smem + kOffL + ent0);
  lds_u8* wb1 = (lds_u8*)(smem + kOffL + ent1);
  asm volatile("" : "+v"(wb0), "+v"(wb1));

  // decode stage s: raw W and value window from LDS -> clean low tile and
  // sparse tile of buffer s % 2; advances vi
  // (par: the stage's ring slot as a compile-time constant, so that every
  // LDS address is a per-lane base plus an immediate)
  auto decode = [&](auto par) {
    constexpr int b = decltype(par)::value;
    const uint4 rw = *(const uint4*)(smem + kOffW + b * kStW + r * 64 + qq * 16);
    uint32_t wd[4], mk[4];
    int cnt = 0;
    {
      const uint32_t d4[4] = {rw.x, rw.y, rw.z, rw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t x = d4[e];
        const uint32_t nz = ((x & 0x77777777u) + 0x77777777u) & 0x88888888u;
        const uint32_t m8 = x & 0x88888888u & ~nz;  // bit 3 of each marked nibble
        mk[e] = m8;
        wd[e] = x ^ m8;  // a marked nibble is exactly 0x8
        cnt += __builtin_popcount(m8);
      }
    }
    uint8_t* sblk;
    if constexpr (FP) {
      // lane-order entries of the 16-row block rb: (row rr, slot group qq)
      // at fpos (swizzled so the 16 lanes of a row quad hit distinct banks)
      *(uint4*)(smem + kOffL + b * kStL + rb * 1024 + fpos_w * 16) =
          make_uint4(wd[0], wd[1], wd[2], wd[3]);
      sblk = smem + kOffS + b * kStS + rb * 2048;
    } else {
      // int8 16*code, slot order: 16 bytes per entry, one store each
      const uint2 c0 = widen8(wd[0]), c1 = widen8(wd[1]), c2 = widen8(wd[2]), c3 = widen8(wd[3]);
      *(lds_v4u*)(wb0 + b * kStL) = lds_v4u_t{c0.x, c0.y, c1.x, c1.y};
      *(lds_v4u*)(wb1 + b * kStL) = lds_v4u_t{c2.x, c2.y, c3.x, c3.y};
      sblk = smem + kOffS + b * kStS;
    }
    // marks of the row's earlier lanes precede this lane's: an inclusive scan
    // over the row's four lanes with DPP row shifts (no LDS round trip)
    int incl = cnt;
    {
      const int c1 = __builtin_amdgcn_update_dpp(0, incl, 0x111, 0xF, 0xF, true);  // row_shr:1
      if (qq >= 1) incl += c1;
      const int c2 = __builtin_amdgcn_update_dpp(0, incl, 0x112, 0xF, 0xF, true);  // row_shr:2
      if (qq >= 2) incl += c2;
    }
    const int tot = __builtin_amdgcn_update_dpp(0, incl, 0xFF, 0xF, 0xF, true);  // quad_perm [3,3,3,3]
    const int v0 = vi + incl - cnt;  // value index of this lane's first mark
    const int64_t a0 = (int64_t)gn * nnz + vi;
    const int64_t win_lo = a0 & ~(int64_t)15;  // the window the DMA brought
    const int64_t room = vtotal - win_lo;
    const int win_valid = !vdma ? 0 : room >= kVRow ? kVRow : (int)room & ~15;
    const int wo0 = (int)(a0 - win_lo) + (v0 - vi);  // offset of this lane's first value
    {
      const uint8_t* vw = smem + kOffV + b * kStV + r * kVRow;
      auto vdw = [&](int o) { return *(const uint32_t*)(vw + o); };
      int pre = 0;
      uint2 sp[4];  // the four groups' sparse bytes, stored in pairs
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        // byte offset of the group's first value; past the row's window the
        // bytes are not used (those lanes take the path below), so the read
        // only has to stay inside LDS
        const int off = min(wo0 + pre, kVRow);
        const int o4 = off & ~3;
        const uint32_t d0 = vdw(o4), d1 = vdw(o4 + 4), d2 = vdw(o4 + 8);
        const uint32_t lo = __builtin_amdgcn_alignbyte(d1, d0, off & 3);
        const uint32_t hi = __builtin_amdgcn_alignbyte(d2, d1, off & 3);
        // mark bits at 4i + 3 -> bit i: two per byte, then one 4-way
        // weighted byte sum (weights 1, 4, 16, 64)
        const uint32_t t2 = ((mk[d] >> 3) | (mk[d] >> 6)) & 0x03030303u;
        const uint32_t x = __builtin_amdgcn_udot4(t2, 0x40100401u, 0u, false);
        const uint2 sl = sSel[x];
        sp[d] = make_uint2(perm(hi, lo, sl.x), perm(hi, lo, sl.y));
        pre += __builtin_popcount(mk[d]);
      }
      if constexpr (FP) {
        // groups 2e and 2e+1 are the two halves of one 16-byte FP8 slot run
        *(uint4*)(sblk + sp_off(0)) = make_uint4(sp[0].x, sp[0].y, sp[1].x, sp[1].y);
        *(uint4*)(sblk + sp_off(2)) = make_uint4(sp[2].x, sp[2].y, sp[3].x, sp[3].y);
      } else {
        *(lds_v4u*)(wb0 + (kOffS - kOffL) + b * kStS) = lds_v4u_t{sp[0].x, sp[0].y, sp[1].x, sp[1].y};
        *(lds_v4u*)(wb1 + (kOffS - kOffL) + b * kStS) = lds_v4u_t{sp[2].x, sp[2].y, sp[3].x, sp[3].y};
      }
    }
    // rare: values beyond the window (or more marks than values) -> one by one
    if (wo0 + cnt > win_valid || v0 + cnt > nnz) {
      int j = 0;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        uint32_t m8 = mk[d];
        while (m8) {
          const int k = d * 8 + (__builtin_ctz(m8) >> 2);  // slot within the lane's 32
          m8 &= m8 - 1;
          const int8_t v = v0 + j >= nnz ? (int8_t)0 : vrow[v0 + j];
          if constexpr (FP)
            sblk[sp_off(k >> 3) + (k & 7)] = (uint8_t)v;
          else
            sblk[(k < 16 ? ent0 : ent1) + (k & 15)] = (uint8_t)v;
          ++j;
        }
      }
    }
    vi += tot;
  };

  // this lane's read offset inside a 2 KiB block of 16 rows x 128 B for K
  // half f: row R = lane % 16, chunk C = lane / 16 + 4 * f
  uint32_t rd_off[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int R = lane & 15, C = (lane >> 4) + 4 * f;
    rd_off[f] = (uint32_t)((R >> 3) * 1024 + (R & 7) * 128 + 16 * (C ^ pair_swz(R >> 3, R & 7)));
  }

  AccT acc[TM][TN], acs[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = acs[i][j] = AccT{0, 0, 0, 0};

  // floating-point form: this lane's FP8 fragment (row lane%16 of a 16-row
  // block, chunks lane/16 and lane/16 + 4 of the swizzled 128-byte row) and
  // its lane-order tile entry
  uint32_t rdf[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int R = lane & 15, C = (lane >> 4) + 4 * h;
    rdf[h] = (uint32_t)((R >> 3) * 1024 + (R & 7) * 128 + 16 * (C ^ pair_swz(R >> 3, R & 7)));
  }
  const int fpos_r = ((lane >> 4) << 4) + ((lane & 15) ^ ((lane >> 4) << 2));
  // integer form: this lane's entry in the decoded-tile blocks of its wave's
  // columns for K half f (clean tile, slot 0; the sparse tile and slot 1 at
  // immediate offsets), and its A fragment base for K half f
  const uint8_t* rlb[2] = {smem + kOffL + wn * TN * 2048 + 16 * tile_entry(lane >> 4, lane & 15, 0),
                           smem + kOffL + wn * TN * 2048 + 1024 + 16 * tile_entry(lane >> 4, lane & 15, 1)};
  const uint8_t* rab[2] = {smem + kOffA + wm * TM * 2048 + rd_off[0], smem + kOffA + wm * TM * 2048 + rd_off[1]};

  auto ld_a8 = [&](const uint8_t* blk) {
    const v4i lo = *(const v4i*)(blk + rdf[0]), hi = *(const v4i*)(blk + rdf[1]);
    return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  };

  // MFMAs of stage s: low and sparse tiles on the same A
  auto mfma_stage = [&](auto par) {
    constexpr int b = decltype(par)::value;
    if constexpr (FP) {
      const uint8_t* abuf = smem + kOffA + b * kStA;
      const uint8_t* cb = smem + kOffL + b * kStL;
      const uint8_t* sb = smem + kOffS + b * kStS;
      v8i a[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i) a[i] = ld_a8(abuf + (wm * TM + i) * 2048);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int blk = wn * TN + j;
        const v4i l4 = *(const v4i*)(cb + blk * 1024 + fpos_r * 16);
        const v8i bl = v8i{l4.x, l4.y, l4.z, l4.w, 0, 0, 0, 0};
        const v4i s0 = *(const v4i*)(sb + blk * 2048 + fpos_r * 32);
        const v4i s1 = *(const v4i*)(sb + blk * 2048 + fpos_r * 32 + 16);
        const v8i bs = v8i{s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[i], bl, acc[i][j], 0, 4, 0, 0, 0, 0);
          acs[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[i], bs, acs[i][j], 0, 0, 0, 0, 0, 0);
        }
      }
    } else {
      // both decoded tiles and the activations are int8 in slot order: LDS
      // reads (per-lane base + immediate) and MFMAs only.  Eight groups (K
      // half f, column block j) of eight MFMAs; the B fragments of the next
      // group and the A fragments of the next K half are read while the
      // current group multiplies, so no group waits for its own reads.
      v4i a[2][TM], bl[2], bs[2];
      auto ld_b = [&](int g, int slot) {
        const int f = g >> 2, j = g & 3;
        bl[slot] = *(const v4i*)(rlb[f] + b * kStL + j * 2048);
        bs[slot] = *(const v4i*)(rlb[f] + (kOffS - kOffL) + b * kStS + j * 2048);
      };
#pragma unroll
      for (int i = 0; i < TM; ++i) a[0][i] = *(const v4i*)(rab[0] + b * kStA + i * 2048);
      ld_b(0, 0);
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const int f = g >> 2, j = g & 3;
        if (g + 1 < 8) ld_b(g + 1, (g + 1) & 1);
        if (g == 1) {
#pragma unroll
          for (int i = 0; i < TM; ++i) a[1][i] = *(const v4i*)(rab[1] + b * kStA + i * 2048);
        }
        // the reads above stay above this group's MFMAs
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[f][i], bl[g & 1], acc[i][j], 0, 0, 0);
          acs[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[f][i], bs[g & 1], acs[i][j], 0, 0, 0);
        }
      }
    }
  };


  // ---- int8 branch (outlier channels), 128 bytes per row per stage ----
  // Branch stage t takes the A buffer (nst + t) % 2 and, for its W rows (16-row
  // blocks swizzled like A), the raw W ring (t even) or the clean-tile ring
  // (t odd): stages 0 and 1 load while the last low stages compute.  Both
  // operands are in natural slot order.
  auto br_a = [&](int t) { return kOffA + ((nst + t) & 1) * kStA; };
  auto br_w = [&](int t) { return (t & 1) ? kOffL : kOffW; };
  // (lane offsets formed here: they are needed at most a few times)
  auto issue_branch = [&](int t) {
    const int rl = lane >> 3;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = wave * 4 + i;
      int row = m0 + q * 8 + rl;
      if (row > mm - 1) row = mm - 1;
      const uint32_t off = (uint32_t)row * (uint32_t)p.ldo + (uint32_t)(((lane & 7) ^ pair_swz(q & 1, rl)) * 16);
      dma_16B(p.x_out, off + (uint32_t)t * 128u, sbase + (uint32_t)br_a(t) + (uint32_t)(q * 1024));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = wave * 2 + i;
      int row = n0 + q * 8 + rl;
      if (row > nn - 1) row = nn - 1;
      const uint32_t off = (uint32_t)row * (uint32_t)p.ldo + (uint32_t)(((lane & 7) ^ pair_swz(q & 1, rl)) * 16);
      dma_16B(p.w_out, off + (uint32_t)t * 128u, sbase + (uint32_t)br_w(t) + (uint32_t)(q * 1024));
    }
  };

  // ---- PRE: the decoded tiles of each stage come from the call's
  // workspace (k_sq_expand wrote them there), one contiguous image per
  // (column tile, stage): the clean tile, then the sparse tile, each exactly
  // as the decode above would leave it in LDS ----
  constexpr int kImg = kImgBytes<FP>;
  constexpr int kDmaD = kImg / 8192;  // 16-byte DMAs per thread per stage image
  const uint8_t* dec_tile = PRE ? p.dec + (int64_t)tn * nst * kImg : p.x_low;
  auto issue_d = [&](int s) {
    const uint32_t voff = (uint32_t)s * (uint32_t)kImg + (uint32_t)tid * 16u;
#pragma unroll
    for (int i = 0; i < kDmaD; ++i) {
      const uint32_t dst = i * 8192 < kStL
                               ? sbase + kOffL + (uint32_t)((s & 1) * kStL + i * 8192)
                               : sbase + kOffS + (uint32_t)((s & 1) * kStS + i * 8192 - kStL);
      dma_16B(dec_tile, voff + (uint32_t)(i * 8192), dst + (uint32_t)(wave * 1024));
    }
  };

  if constexpr (PRE) {
    // prologue: stages 0 and 1 in flight, wait for stage 0 only
    if (nst > 0) {
      issue_a(0);
      issue_d(0);
      if (nst > 1) {
        issue_a(1);
        issue_d(1);
        wait_vmcnt<4 + kDmaD>();
      } else if (p.s_out > 0) {
        issue_branch(0);
        wait_vmcnt<6>();
      } else {
        wait_vmcnt<0>();
      }
      sq_sync();
    }
    // Iteration s: the MFMAs of stage s; wait for stage s+1; one barrier;
    // then stage s+2 (or the first branch stages) into the slots of stage s.
    auto iteration = [&](int s, auto par) {
      mfma_stage(par);
      wait_vmcnt<0>();
      sq_sync();
      if (s + 2 < nst) {
        issue_a(s + 2);
        issue_d(s + 2);
      } else if (s + 2 - nst < p.s_out) {
        issue_branch(s + 2 - nst);
      }
    };
    for (int s = 0; s < nst; s += 2) {
      iteration(s, std::integral_constant<int, 0>{});
      if (s + 1 < nst) iteration(s + 1, std::integral_constant<int, 1>{});
    }
  } else {
  // ---- prologue: stage 0 decoded, A 1 and W 2 in flight ----
  if (nst > 0) {
    issue_a(0);
    issue_w(0);
    if (nst > 1) issue_w(1);
    issue_v(0);
    wait_vmcnt<0>();
    sq_sync();  // selector table, A 0, W 0 and 1, values 0
    decode(std::integral_constant<int, 0>{});
    if (nst > 1) issue_v(1);
    wait_vmcnt<0>();
    sq_sync();  // decoded stage 0, values 1; W 0 is free
    if (nst > 1) issue_a(1);
    else if (p.s_out > 0) issue_branch(0);
    if (nst > 2) issue_w(2);
  }
  // Iteration s: decode s+1 and the MFMAs of s; one barrier; then the DMAs of
  // A s+2 (into the buffer of A s) and W s+3 (into the buffer of W s+1).
  // Unrolled by two, so that each iteration knows its ring slots.  The values
  // of s+2 are fetched right after the decode of s+1 (for s + 2 == nst: a
  // window nobody reads, into a free slot).  (Measured: having half the
  // waves multiply first, so the two waves of a SIMD alternate decode and
  // matrix work, is slower -- the decode's LDS chains then queue behind the
  // other wave's fragment reads.)
  auto iteration = [&](int s, auto par) {
    constexpr int b = decltype(par)::value;
    if (s + 1 < nst) {
      decode(std::integral_constant<int, 1 - b>{});
      issue_v(s + 2);
    }
    mfma_stage(par);
    // A s+1, W s+2 (issued one iteration ago) and values s+2 have landed
    wait_vmcnt<0>();
    sq_sync();
    if (s + 2 < nst) issue_a(s + 2);
    else if (s + 2 - nst < p.s_out) issue_branch(s + 2 - nst);
    if (s + 3 < nst) issue_w(s + 3);
  };
  for (int s = 0; s < nst; s += 2) {
    iteration(s, std::integral_constant<int, 0>{});
    if (s + 1 < nst) iteration(s + 1, std::integral_constant<int, 1>{});
  }
  }  // !PRE

  // ---- low + masked parts -> fp32 partial (the low accumulator is x16) ----
  // (the fp32 partial reuses the low accumulator's registers)
  const int lr = (lane >> 4) * 4, lc = lane & 15;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = m0 + wm * 64 + i * 16 + lr + q, col = n0 + wn * 64 + j * 16 + lc;
        const int rc = row < mm ? row : mm - 1, cc = col < nn ? col : nn - 1;
        if constexpr (FP) {
          acc[i][j][q] = p.s_x[rc] * (p.s_w4[cc] * acc[i][j][q] + p.s_w8[cc] * acs[i][j][q]);
          acs[i][j][q] = 0.0f;
        } else {
          const int32_t lo = acc[i][j][q] >> 4;
          if (DEBUG && row < mm && col < nn) {
            p.dbg_low[(int64_t)row * nn + col] = lo;
            p.dbg_sp[(int64_t)row * nn + col] = acs[i][j][q];
          }
          acc[i][j][q] = __float_as_int(p.s_x[rc] * (p.s_w4[cc] * (float)lo + p.s_w8[cc] * (float)acs[i][j][q]));
          acs[i][j][q] = 0;
        }
      }

  // ---- int8 branch stages (the first two are already in flight) ----
  {
    int bn = nst >= 1 ? (p.s_out < 2 ? p.s_out : 2) : 0;  // stages issued so far
    for (int t = 0; t < p.s_out; ++t) {
      if (bn == t) {
        issue_branch(t);
        ++bn;
      }
      wait_vmcnt<0>();
      sq_sync();
      if constexpr (FP) {
        // E4M3 x E4M3, one 128-byte K step per instruction
        v8i b[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) b[j] = ld_a8(smem + br_w(t) + (wn * TN + j) * 2048);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const v8i a = ld_a8(smem + br_a(t) + (wm * TM + i) * 2048);
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acs[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b[j], acs[i][j], 0, 0, 0, 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          v4i b[TN];
#pragma unroll
          for (int j = 0; j < TN; ++j) b[j] = *(const v4i*)(smem + br_w(t) + (wn * TN + j) * 2048 + rd_off[f]);
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            const v4i a = *(const v4i*)(smem + br_a(t) + (wm * TM + i) * 2048 + rd_off[f]);
#pragma unroll
            for (int j = 0; j < TN; ++j)
              acs[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b[j], acs[i][j], 0, 0, 0);
          }
        }
      }
      sq_sync();
      // the buffers just read take stage t+2
      if (bn == t + 2 && bn < p.s_out) {
        issue_branch(bn);
        ++bn;
      }
    }
  }

  // ---- fuse and store ----
  // (the fused values replace the float partials in acc)
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int col = n0 + wn * 64 + j * 16 + lc;
    const int cc = col < nn ? col : nn - 1;
    const float swo = p.s_out > 0 ? p.s_wo[cc] : 0.0f;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = m0 + wm * 64 + i * 16 + lr + q;
        const int rc = row < mm ? row : mm - 1;
        if constexpr (FP) {
          if (p.s_out > 0) acc[i][j][q] += (p.s_xo[rc] * swo) * acs[i][j][q];
        } else {
          if (DEBUG && row < mm && col < nn) p.dbg_o[(int64_t)row * nn + col] = acs[i][j][q];
          float v = __int_as_float(acc[i][j][q]);
          if (p.s_out > 0) v += (p.s_xo[rc] * swo) * (float)acs[i][j][q];
          acc[i][j][q] = __float_as_int(v);
        }
      }
  }
  // the fused value of an accumulator element (int form: fp32 bits)
  auto outv = [](auto v) -> float {
    if constexpr (FP) return v;
    else return __int_as_float(v);
  };
  const int wrow0 = m0 + wm * 64, wcol0 = n0 + wn * 64;
  const bool whole = wcol0 + 64 <= nn && (p.ldy & 3) == 0 && (((uintptr_t)p.y) & 15) == 0;
  if (whole) {
    // (non-temporal: Y is written once and not read here)
    // Row-contiguous 16-byte stores: each 16-row slice of the wave tile goes
    // through this wave's rows of the (now free) A ring, padded by 4 floats
    // per row (4-byte writes and 16-byte reads free of bank conflicts).
    constexpr int LDW = 64 + 4;
    float* stg = (float*)(smem + kOffA) + wave * (16 * LDW);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) stg[(lr + q) * LDW + j * 16 + lc] = outv(acc[i][j][q]);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int idx = k * 64 + lane, rr2 = idx >> 4, c4 = idx & 15;
        const v4f v = *(const v4f*)(stg + rr2 * LDW + 4 * c4);
        const int row = wrow0 + i * 16 + rr2;
        if (row < mm) __builtin_nontemporal_store(v, (v4f*)(p.y + (int64_t)row * p.ldy + wcol0 + 4 * c4));
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = wrow0 + i * 16 + lr + q, col = wcol0 + j * 16 + lc;
          if (row < mm && col < nn) __builtin_nontemporal_store(outv(acc[i][j][q]), p.y + (int64_t)row * p.ldy + col);
        }
  }
}

// The gather done once per call (sqf_dual_gemm_sq_ws): every (column tile,
// 128-slot stage) of the weights is decoded into the workspace as the image
// the fused kernel's decode leaves in LDS for that stage -- the clean tile,
// then the sparse tile, same entry order -- so that k_sq_gemm<.., PRE> moves
// it with plain DMAs, and the decode runs once per weight tile instead of
// once per (row tile, weight tile).  A workgroup takes one 16-row block of a
// column tile; its wave w decodes stage 16 t + w of step t for the 16 rows,
// four lanes per row (the fused decode's lane map), so each store
// instruction of a wave writes whole 256-byte runs of the image.  A row's
// value index at a lane comes from a scan over its four lanes, the row's
// counts of the earlier stages of the step (an LDS table) and the steps
// before.  Rows past n are written as zeros.
template <bool FP>
__global__ __launch_bounds__(1024) void k_sq_expand(SqArgs p) {
  constexpr int kStL = SqLds<FP>::kStL, kImg = kImgBytes<FP>;
  __shared__ uint2 sSel[256];
  __shared__ int sCnt[2][16][16];  // [step parity][wave = stage of the step][row]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < 256) {
    // the expand selectors of the fused kernel (one 8-slot group's mark mask)
    const int m = tid;
    uint32_t sel[2] = {0, 0};
#pragma unroll
    for (int pp = 0; pp < 8; ++pp) {
      const uint32_t b = ((m >> pp) & 1) ? (uint32_t)__builtin_popcount(m & ((1 << pp) - 1)) : 0x0Cu;
      sel[pp >> 2] |= b << (8 * (pp & 3));
    }
    sSel[m] = make_uint2(sel[0], sel[1]);
  }
  const int blk16 = blockIdx.x, tn = blk16 >> 3, rb = blk16 & 7;
  const int rr = lane >> 2, qq = lane & 3;
  const int64_t row = (int64_t)blk16 * 16 + rr;
  const bool live = row < p.n;
  const int nst = (int)(p.ldkw / 64), nnz = (int)p.nnz;
  const uint8_t* wrow = p.w_low + (live ? row : 0) * p.ldkw;
  const int64_t vrow = (live ? row : 0) * p.nnz;  // offset of the row's first value
  const int64_t vtotal = p.n * p.nnz;
  uint8_t* img_tile = p.dec + (int64_t)tn * nst * kImg;
  int carry = 0;  // marks of the row in the steps before
  for (int t = 0; t * 16 < nst; ++t) {
    const int s = t * 16 + wave;
    const bool act = s < nst;
    uint4 rw = make_uint4(0u, 0u, 0u, 0u);
    if (act && live) rw = *(const uint4*)(wrow + s * 64 + qq * 16);
    uint32_t wd[4], mk[4];
    int cnt = 0;
    {
      const uint32_t d4[4] = {rw.x, rw.y, rw.z, rw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t x = d4[e];
        const uint32_t nz = ((x & 0x77777777u) + 0x77777777u) & 0x88888888u;
        const uint32_t m8 = x & 0x88888888u & ~nz;  // bit 3 of each marked nibble
        mk[e] = m8;
        wd[e] = x ^ m8;
        cnt += __builtin_popcount(m8);
      }
    }
    // marks of the row's earlier lanes in this stage (DPP scan over the quad)
    int incl = cnt;
    {
      const int c1 = __builtin_amdgcn_update_dpp(0, incl, 0x111, 0xF, 0xF, true);  // row_shr:1
      if (qq >= 1) incl += c1;
      const int c2 = __builtin_amdgcn_update_dpp(0, incl, 0x112, 0xF, 0xF, true);  // row_shr:2
      if (qq >= 2) incl += c2;
    }
    const int tot = __builtin_amdgcn_update_dpp(0, incl, 0xFF, 0xF, 0xF, true);  // quad_perm [3,3,3,3]
    if (qq == 0) sCnt[t & 1][wave][rr] = tot;
    __syncthreads();  // (also orders the selector table before its first use)
    int before = 0, all = 0;
#pragma unroll
    for (int w2 = 0; w2 < 16; ++w2) {
      const int c = sCnt[t & 1][w2][rr];
      before += w2 < wave ? c : 0;
      all += c;
    }
    const int v0 = carry + before + incl - cnt;  // value index of this lane's first mark
    carry += all;
    uint2 sp[4];
    if (v0 + cnt <= nnz && vrow + v0 + cnt + 12 <= vtotal) {
      // three aligned dwords cover a group's (at most 8) values
      int pre = 0;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int64_t off = vrow + v0 + pre;
        const uint32_t* q = (const uint32_t*)(p.sq_val + (off & ~(int64_t)3));
        const uint32_t d0 = q[0], d1 = q[1], d2 = q[2];
        const uint32_t lo = __builtin_amdgcn_alignbyte(d1, d0, (uint32_t)(off & 3));
        const uint32_t hi = __builtin_amdgcn_alignbyte(d2, d1, (uint32_t)(off & 3));
        const uint32_t t2 = ((mk[d] >> 3) | (mk[d] >> 6)) & 0x03030303u;
        const uint32_t x = __builtin_amdgcn_udot4(t2, 0x40100401u, 0u, false);
        const uint2 sl = sSel[x];
        sp[d] = make_uint2(perm(hi, lo, sl.x), perm(hi, lo, sl.y));
        pre += __builtin_popcount(mk[d]);
      }
    } else {
      // near the end of the value buffer, or more marks than values (those
      // take 0): one value at a time
      int j = 0;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        uint32_t w2[2] = {0u, 0u};
#pragma unroll
        for (int pp = 0; pp < 8; ++pp) {
          if ((mk[d] >> (4 * pp + 3)) & 1u) {
            const uint32_t v = v0 + j < nnz ? (uint8_t)p.sq_val[vrow + v0 + j] : 0u;
            w2[pp >> 2] |= v << (8 * (pp & 3));
            ++j;
          }
        }
        sp[d] = make_uint2(w2[0], w2[1]);
      }
    }
    if (act) {
      uint8_t* img = img_tile + (int64_t)s * kImg;
      if constexpr (FP) {
        const int fpos = (qq << 4) + (rr ^ (qq << 2));
        *(uint4*)(img + rb * 1024 + fpos * 16) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
        auto sp_off = [&](int d) {
          const int g = 2 * (qq & 1) + (d >> 1);
          return ((g << 4) + (rr ^ (g << 2))) * 32 + 16 * (qq >> 1) + 8 * (d & 1);
        };
        uint8_t* sblk = img + kStL + rb * 2048;
        *(uint4*)(sblk + sp_off(0)) = make_uint4(sp[0].x, sp[0].y, sp[1].x, sp[1].y);
        *(uint4*)(sblk + sp_off(2)) = make_uint4(sp[2].x, sp[2].y, sp[3].x, sp[3].y);
      } else {
        const int f = qq >> 1, g0 = 2 * (qq & 1);
        const int e0 = (rb * 2 + f) * 1024 + 16 * tile_entry(g0, rr, f);
        const int e1 = (rb * 2 + f) * 1024 + 16 * tile_entry(g0 + 1, rr, f);
        const uint2 c0w = widen8(wd[0]), c1w = widen8(wd[1]), c2w = widen8(wd[2]), c3w = widen8(wd[3]);
        *(uint4*)(img + e0) = make_uint4(c0w.x, c0w.y, c1w.x, c1w.y);
        *(uint4*)(img + e1) = make_uint4(c2w.x, c2w.y, c3w.x, c3w.y);
        *(uint4*)(img + kStL + e0) = make_uint4(sp[0].x, sp[0].y, sp[1].x, sp[1].y);
        *(uint4*)(img + kStL + e1) = make_uint4(sp[2].x, sp[2].y, sp[3].x, sp[3].y);
      }
    }
  }
}

int64_t sq_image_bytes(int64_t n, int64_t ldkw, bool fp) {
  return (n + kBN - 1) / kBN * (ldkw / 64) * (fp ? kImgBytes<true> : kImgBytes<false>);
}

hipError_t launch_sq_gemm(const SqArgs& a, bool debug, bool fp, hipStream_t s) {
  const int64_t blocks = ((a.m + kBM - 1) / kBM) * ((a.n + kBN - 1) / kBN);
  if (blocks <= 0) return hipSuccess;
  if (fp && debug) return hipErrorInvalidValue;
  const dim3 g((unsigned)blocks), b(512);
  if (a.dec) {
    // the gather into the workspace, then the GEMM on the decoded images
    const dim3 ge((unsigned)(((a.n + kBN - 1) / kBN) * (kBN / 16)));
    if (fp) hipLaunchKernelGGL((k_sq_expand<true>), ge, dim3(1024), 0, s, a);
    else hipLaunchKernelGGL((k_sq_expand<false>), ge, dim3(1024), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (fp) hipLaunchKernelGGL((k_sq_gemm<false, true, true>), g, b, 0, s, a);
    else if (debug) hipLaunchKernelGGL((k_sq_gemm<true, false, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((k_sq_gemm<false, false, true>), g, b, 0, s, a);
    return hipGetLastError();
  }
  if (fp) hipLaunchKernelGGL((k_sq_gemm<false, true, false>), g, b, 0, s, a);
  else if (debug) hipLaunchKernelGGL((k_sq_gemm<true, false, false>), g, b, 0, s, a);
  else hipLaunchKernelGGL((k_sq_gemm<false, false, false>), g, b, 0, s, a);
  return hipGetLastError();
}

}  // namespace sqf
