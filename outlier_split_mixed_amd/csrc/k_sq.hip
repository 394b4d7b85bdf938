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
// a block's W rows into LDS: a stage of a W row becomes
//   * an int4 low tile with the marks cleared to 0 (SWAR: a nibble is the
//     mark iff its top bit is set and its low three bits are zero), widened
//     to int8 at MFMA time with the x16 trick (w << 4 & 0xF0.. and
//     w & 0xF0..), which puts a group of 8 slots in the order 0,2,4,6,1,3,5,7;
//   * an int8 tile holding the row's sparse values at their marked slots
//     (zero elsewhere), in that same slot order: every 8-slot group is
//     expanded at once from a window of the row's values with byte permutes
//     whose selectors come from a table indexed by the group's mark mask.
// The int8 activations stay in their natural order in LDS; each A fragment is
// permuted into the widened slot order in registers as it is read, so both
// tiles feed v_mfma_i32_16x16x64_i8 with one A fragment.  The low accumulator
// carries the x16 factor (|acc| <= 16*127*7*k_low < 2^31 for the k_low the
// host accepts); it is removed exactly in the epilogue.
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
#include "sqf_device.h"
#include "sqf_launch.h"

namespace sqf {

namespace {

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// byte position, inside a lane's 16-byte MFMA operand, of slot k (0..15) in
// the widened order 0,2,4,6,1,3,5,7 | 8,10,12,14,9,11,13,15
__device__ __forceinline__ int perm_pos(int k) {
  return (k & 8) + ((k & 1) ? 4 + ((k & 7) >> 1) : ((k & 7) >> 1));
}

// natural slot order -> widened slot order, 16 int8 codes
__device__ __forceinline__ v4i to_widened(v4i u) {
  return v4i{(int)perm((uint32_t)u.y, (uint32_t)u.x, 0x06040200u),
             (int)perm((uint32_t)u.y, (uint32_t)u.x, 0x07050301u),
             (int)perm((uint32_t)u.w, (uint32_t)u.z, 0x06040200u),
             (int)perm((uint32_t)u.w, (uint32_t)u.z, 0x07050301u)};
}

// LDS barrier that does not wait for outstanding global loads.
__device__ __forceinline__ void sq_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  stage_barrier();
}

// LDS map of one block (bytes).
constexpr int kBM = 256, kBN = 128;
constexpr int kStA = kBM * 128;  // activation stage: 16-row blocks of 16 x 128 B (swizzled)
constexpr int kStW = kBN * 64;   // raw W stage: row-major, 64 B per row
constexpr int kStV = kBN * 64;   // value windows: row-major, 64 B per row
constexpr int kStL = kBN * 64;   // clean low tile: [row block][K half][entry] x 8 B
constexpr int kStS = kBN * 128;  // sparse tile: [row block][K half][entry] x 16 B
constexpr int kOffA = 0;
constexpr int kOffW = kOffA + 2 * kStA;
constexpr int kOffV = kOffW + 2 * kStW;
constexpr int kOffL = kOffV + 2 * kStV;
constexpr int kOffS = kOffL + 2 * kStL;
constexpr int kOffSel = kOffS + 2 * kStS;
constexpr int kSmem = kOffSel + 256 * 8;
static_assert(kSmem <= 160 * 1024, "LDS budget");
// the branch's W tile (128 rows x 128 B, swizzled like A) reuses the raw W
// and value rings
static_assert(kBN * 128 <= 2 * kStW + 2 * kStV, "branch W tile fits");

}  // namespace

template <bool DEBUG>
__global__ __launch_bounds__(512, 1) void k_sq_gemm(SqArgs p) {
  constexpr int TM = 4, TN = 4;
  __shared__ __attribute__((aligned(2048))) uint8_t smem[kSmem];

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
  // value window of stage s: lane l brings 16-byte block l % 4 of its own row
  auto issue_v = [&](int s) {
    const uint32_t start = (uint32_t)(((int64_t)gn * nnz + vi) & ~(int64_t)15);
    uint32_t off = start + (uint32_t)(qq * 16);
    if (off > vlast) off = vlast;  // past the buffer: any whole block (unused)
    dma_16B(vdma ? (const uint8_t*)p.sq_val : p.x_low, vdma ? off : 0u,
            sbase + kOffV + (uint32_t)((s & 1) * kStV) + (uint32_t)(wave * 1024));
  };

  // Expand selectors: for the mark mask m of an 8-slot group, byte p of the
  // group's operand bytes (slot order 0,2,4,6,1,3,5,7) takes value number
  // rank(slot) (a byte of the pool {hi, lo} of the group's values) if the
  // slot is marked, else zero (selector 0x0C).
  uint2* sSel = (uint2*)(smem + kOffSel);
  if (tid < 256) {
    const int m = tid;
    uint32_t sel[2] = {0, 0};
#pragma unroll
    for (int pp = 0; pp < 8; ++pp) {
      const int sl = pp < 4 ? 2 * pp : 2 * (pp - 4) + 1;
      const uint32_t b = ((m >> sl) & 1) ? (uint32_t)__builtin_popcount(m & ((1 << sl) - 1)) : 0x0Cu;
      sel[pp >> 2] |= b << (8 * (pp & 3));
    }
    sSel[m] = make_uint2(sel[0], sel[1]);
  }

  // Decoded-tile entry of MFMA lane (16-slot group g, row rr) in a K-half
  // block: g * 16 + (rr ^ 8 (g / 2)), for the clean low tile also with g ^ f
  // (f = K half); the sparse tile's 8-byte halves are swapped for f = 1.  The
  // four lanes of a row write at once: these swizzles spread them over banks.
  auto lpos = [](int g, int rr_, int f) { return ((g ^ f) << 4) + (rr_ ^ ((g >> 1) << 3)); };
  auto spos = [](int g, int rr_) { return (g << 4) + (rr_ ^ ((g >> 1) << 3)); };

  // decode stage s: raw W and value window from LDS -> clean low tile and
  // sparse tile of buffer s % 2; advances vi
  auto decode = [&](int s) {
    const uint4 rw = *(const uint4*)(smem + kOffW + (s & 1) * kStW + r * 64 + qq * 16);
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
    uint2* sL = (uint2*)(smem + kOffL + (s & 1) * kStL) + (rb * 2 + f_own) * 64;
#pragma unroll
    for (int e = 0; e < 2; ++e) sL[lpos(g0 + e, rr, f_own)] = make_uint2(wd[2 * e], wd[2 * e + 1]);
    uint8_t* sblk = smem + kOffS + (s & 1) * kStS + (rb * 2 + f_own) * 1024;
    // marks of the row's earlier lanes precede this lane's
    int incl = cnt;
    {
      const int c1 = __shfl_up(incl, 1, 4);
      if (qq >= 1) incl += c1;
      const int c2 = __shfl_up(incl, 2, 4);
      if (qq >= 2) incl += c2;
    }
    const int tot = __shfl(incl, 3, 4);
    const int v0 = vi + incl - cnt;  // value index of this lane's first mark
    const int64_t a0 = (int64_t)gn * nnz + vi;
    const int64_t win_lo = a0 & ~(int64_t)15;  // the window the DMA brought
    const int64_t room = vtotal - win_lo;
    const int win_valid = !vdma ? 0 : room >= 64 ? 64 : (int)room & ~15;
    const int wo0 = (int)(a0 - win_lo) + (v0 - vi);  // offset of this lane's first value
    {
      const uint8_t* vw = smem + kOffV + (s & 1) * kStV + r * 64;
      auto vdw = [&](int o) { return *(const uint32_t*)(vw + o); };
      int pre = 0;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        // byte offset of the group's first value; past the row's window the
        // bytes are not used (those lanes take the path below), so the read
        // only has to stay inside LDS
        const int off = min(wo0 + pre, 64);
        const int o4 = off & ~3;
        const uint32_t d0 = vdw(o4), d1 = vdw(o4 + 4), d2 = vdw(o4 + 8);
        const uint32_t lo = __builtin_amdgcn_alignbyte(d1, d0, off & 3);
        const uint32_t hi = __builtin_amdgcn_alignbyte(d2, d1, off & 3);
        // mark bits at 4i + 3 -> bit i: two per byte, then one 4-way
        // weighted byte sum (weights 1, 4, 16, 64)
        const uint32_t t2 = ((mk[d] >> 3) | (mk[d] >> 6)) & 0x03030303u;
        const uint32_t x = __builtin_amdgcn_udot4(t2, 0x40100401u, 0u, false);
        const uint2 sl = sSel[x];
        *(uint2*)(sblk + spos(g0 + (d >> 1), rr) * 16 + ((d & 1) ^ f_own) * 8) =
            make_uint2(perm(hi, lo, sl.x), perm(hi, lo, sl.y));
        pre += __builtin_popcount(mk[d]);
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
          sblk[spos(g0 + (k >> 4), rr) * 16 + (perm_pos(k & 15) ^ (f_own * 8))] = (uint8_t)v;
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

  v4i acc[TM][TN], acs[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = acs[i][j] = v4i{0, 0, 0, 0};

  // MFMAs of stage s: both K halves, low and sparse tiles on the same A
  auto mfma_stage = [&](int s) {
    const uint8_t* abuf = smem + kOffA + (s & 1) * kStA;
    const uint2* sL = (const uint2*)(smem + kOffL + (s & 1) * kStL);
    const uint4* sS = (const uint4*)(smem + kOffS + (s & 1) * kStS);
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      v4i a[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i) a[i] = to_widened(*(const v4i*)(abuf + (wm * TM + i) * 2048 + rd_off[f]));
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int blk = ((wn * TN + j) * 2 + f) * 64;
        const uint2 x = sL[blk + lpos(lane >> 4, lane & 15, f)];
        const v4i bl = v4i{(int)((x.x << 4) & 0xF0F0F0F0u), (int)(x.x & 0xF0F0F0F0u),
                           (int)((x.y << 4) & 0xF0F0F0F0u), (int)(x.y & 0xF0F0F0F0u)};
        v4i bs = __builtin_bit_cast(v4i, sS[blk + spos(lane >> 4, lane & 15)]);
        if (f == 1) bs = v4i{bs.z, bs.w, bs.x, bs.y};
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], bl, acc[i][j], 0, 0, 0);
          acs[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], bs, acs[i][j], 0, 0, 0);
        }
      }
    }
  };

  // ---- int8 branch (outlier channels), 128 bytes per row per stage ----
  // Branch stage t takes the A buffer (nst + t) % 2 and, for its W rows (16-row
  // blocks swizzled like A), the raw W ring (t even) or the value ring (t odd):
  // stages 0 and 1 load while the last low stages compute.  Both operands are
  // in natural slot order.
  auto br_a = [&](int t) { return kOffA + ((nst + t) & 1) * kStA; };
  auto br_w = [&](int t) { return (t & 1) ? kOffV : kOffW; };
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

  // ---- prologue: stage 0 decoded, A 1 and W 2 in flight ----
  if (nst > 0) {
    issue_a(0);
    issue_w(0);
    if (nst > 1) issue_w(1);
    issue_v(0);
    wait_vmcnt<0>();
    sq_sync();  // selector table, A 0, W 0 and 1, values 0
    decode(0);
    if (nst > 1) issue_v(1);
    wait_vmcnt<0>();
    sq_sync();  // decoded stage 0, values 1; W 0 is free
    if (nst > 1) issue_a(1);
    else if (p.s_out > 0) issue_branch(0);
    if (nst > 2) issue_w(2);
  }
  // Iteration s: decode s+1 and the MFMAs of s; one barrier; then the DMAs of
  // A s+2 (into the buffer of A s) and W s+3 (into the buffer of W s+1).
  for (int s = 0; s < nst; ++s) {
    if (s + 1 < nst) {
      decode(s + 1);
      if (s + 2 < nst) issue_v(s + 2);
    }
    mfma_stage(s);
    // A s+1, W s+2 (issued one iteration ago) and values s+2 have landed
    wait_vmcnt<0>();
    sq_sync();
    if (s + 2 < nst) issue_a(s + 2);
    else if (s + 2 - nst < p.s_out) issue_branch(s + 2 - nst);
    if (s + 3 < nst) issue_w(s + 3);
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
        const int row = m0 + wm * 64 + i * 16 + lr + q, col = n0 + wn * 64 + j * 16 + lc;
        const int rc = row < mm ? row : mm - 1, cc = col < nn ? col : nn - 1;
        const int32_t lo = acc[i][j][q] >> 4;
        if (DEBUG && row < mm && col < nn) {
          p.dbg_low[(int64_t)row * nn + col] = lo;
          p.dbg_sp[(int64_t)row * nn + col] = acs[i][j][q];
        }
        acc[i][j][q] = __float_as_int(p.s_x[rc] * (p.s_w4[cc] * (float)lo + p.s_w8[cc] * (float)acs[i][j][q]));
        acs[i][j][q] = 0;
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
        if (DEBUG && row < mm && col < nn) p.dbg_o[(int64_t)row * nn + col] = acs[i][j][q];
        float v = __int_as_float(acc[i][j][q]);
        if (p.s_out > 0) v += (p.s_xo[rc] * swo) * (float)acs[i][j][q];
        acc[i][j][q] = __float_as_int(v);
      }
  }
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
        for (int q = 0; q < 4; ++q) stg[(lr + q) * LDW + j * 16 + lc] = __int_as_float(acc[i][j][q]);
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
          if (row < mm && col < nn) __builtin_nontemporal_store(__int_as_float(acc[i][j][q]), p.y + (int64_t)row * p.ldy + col);
        }
  }
}

hipError_t launch_sq_gemm(const SqArgs& a, bool debug, hipStream_t s) {
  const int64_t blocks = ((a.m + kBM - 1) / kBM) * ((a.n + kBN - 1) / kBN);
  if (blocks <= 0) return hipSuccess;
  if (debug) hipLaunchKernelGGL(k_sq_gemm<true>, dim3((unsigned)blocks), dim3(512), 0, s, a);
  else hipLaunchKernelGGL(k_sq_gemm<false>, dim3((unsigned)blocks), dim3(512), 0, s, a);
  return hipGetLastError();
}

}  // namespace sqf
