// sqf_api.hip -- the C ABI of libsqf (declared in include/sqf.h).
//
// Every entry point validates its arguments on the host before launching
// anything; a failure returns a status and sets a thread-local message.  No
// entry point allocates device memory or keeps a pointer after it returns.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/sqf.h"
#include "sqf_device.h"
#include "sqf_launch.h"

// The allocation-free channel choice (sqf_select_channels_noalloc) keeps its
// scores in this array: one copy per GPU, held from the library's first use
// on that GPU until the process ends.  Host code never uses the array's name
// as an address (on the host it is only a stand-in): the device address comes
// from hipGetSymbolAddress, looked up once per device (scratch_scores below).
constexpr int64_t kScratchScores = 65536;  // channels (512 KiB of fp64 scores)
static __device__ __align__(256) double scratch[kScratchScores];

namespace {

thread_local std::string g_err;

sqf_status fail(sqf_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

sqf_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return SQF_OK;
  return fail(SQF_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// The low path sums int4 products scaled by 256 in int32: 49 * 256 * k_low
// must stay below 2^31.
constexpr int64_t kMaxKLow = 171000;
// weight-side format: |acc| <= 16 * 127 * 7 * k_low < 2^31
constexpr int64_t kMaxKLowSq = 150000;
// Banked weight-side format: each slot ranks itself within its bank (bank^2
// work per bank in the packer).
constexpr int64_t kMaxSqBank = 1024;
// Kernels address operands with 32-bit byte offsets.
constexpr int64_t kMaxOperandBytes = ((int64_t)1 << 31) - 1;

int branch_esz(int32_t b) { return b == SQF_BF16 ? 2 : 1; }
bool branch_ok(int32_t b) { return b == SQF_BF16 || b == SQF_FP8_E4M3 || b == SQF_I8; }

bool tile_ok(int32_t t) { return t >= SQF_TILE_AUTO && t <= SQF_TILE_64; }

// Bytes per row of a low operand: packed nibbles (and E2M1 pairs) pad/2, int8
// pad, 6-bit E2M3 fields pad*3/4 (E2M3 and E2M1 stored K-blocked, see sqf.h).
int64_t low_ldk(int64_t k_low, int32_t low) {
  const int64_t pad = sqf_pad_k_low(k_low);
  return (low == SQF_I8 || low == SQF_FP8_E4M3) ? pad : low == SQF_I4_E2M3 ? pad / 4 * 3 : pad / 2;
}
// Rows of a low operand's storage (the K-blocked layout pads them).
bool low_kblocked(int32_t low) { return low == SQF_I4_E2M3 || low == SQF_MXFP4; }
int64_t low_rows(int64_t rows, int32_t low) { return low_kblocked(low) ? sqf_pad_rows(rows) : rows; }
// Bytes of an MXFP4 operand's E8M0 scale array: one per 32 slots of every
// stored row.
int64_t mx_scale_bytes(int64_t k_low, int64_t rows) { return sqf_pad_k_low(k_low) / 32 * sqf_pad_rows(rows); }

// Tile configuration for the channel-split GEMM: the caller's sqf_tile, or
// (SQF_TILE_AUTO) the largest tile that still gives the 256 CUs enough tiles.
// The E4M3 branch runs on 128x128 tiles: it needs a second accumulator set.
int pick_cfg(int64_t m, int64_t n, int32_t branch, int32_t tile) {
  int cfg;
  if (tile != SQF_TILE_AUTO)
    cfg = tile;
  else if (((m + 255) / 256) * ((n + 255) / 256) >= 448)
    cfg = 0;
  else if (((m + 127) / 128) * ((n + 127) / 128) >= 256)
    cfg = 1;
  else
    cfg = 2;
  if (branch == SQF_FP8_E4M3 && cfg == 0) cfg = 1;  // only when chosen automatically
  return cfg;
}

sqf_status check_weights(const sqf_weights* wt, const char* who) {
  if (!wt) return fail(SQF_ERR_INVALID_ARG, "%s: weights descriptor is NULL", who);
  if (wt->k < 1 || wt->n < 1 || wt->k_low < 0 || wt->k_out < 0 || wt->k_low + wt->k_out != wt->k)
    return fail(SQF_ERR_SHAPE, "%s: inconsistent weight shape k=%lld n=%lld k_low=%lld k_out=%lld",
                who, (long long)wt->k, (long long)wt->n, (long long)wt->k_low,
                (long long)wt->k_out);
  if (!branch_ok(wt->branch))
    return fail(SQF_ERR_INVALID_ARG, "%s: bad branch dtype %d", who, wt->branch);
  if (wt->groups < 1) return fail(SQF_ERR_SHAPE, "%s: groups must be >= 1", who);
  if (wt->low != SQF_I4X2 && wt->low != SQF_I4_E2M3 && wt->low != SQF_MXFP4 &&
      wt->low != SQF_FP4_E2M1)
    return fail(SQF_ERR_INVALID_ARG, "%s: bad low dtype %d for weights", who, wt->low);
  if (wt->low == SQF_FP4_E2M1 && (wt->sq_nnz == 0 || wt->branch != SQF_FP8_E4M3 || wt->groups != 1))
    return fail(SQF_ERR_UNSUPPORTED, "%s: SQF_FP4_E2M1 weights are the floating-point weight-side "
                "format (sq_nnz > 0, SQF_FP8_E4M3 branch, one weight set)", who);
  if (low_kblocked(wt->low) && (wt->groups != 1 || wt->branch != SQF_BF16 || wt->sq_nnz != 0))
    return fail(SQF_ERR_UNSUPPORTED, "%s: the K-blocked low layouts (E2M3, MXFP4) are built for "
                "one weight set, a bf16 branch and the channel-split format", who);
  if (wt->k_low > kMaxKLow)
    return fail(SQF_ERR_SHAPE, "%s: k_low=%lld exceeds %lld", who, (long long)wt->k_low,
                (long long)kMaxKLow);
  const int64_t want_wldk = low_ldk(wt->k_low, wt->low);
  if (wt->ldk != want_wldk)
    return fail(SQF_ERR_SHAPE, "%s: ldk=%lld, expected %lld", who, (long long)wt->ldk,
                (long long)want_wldk);
  if (wt->ldo != sqf_pad_k_out(wt->k_out, wt->branch))
    return fail(SQF_ERR_SHAPE, "%s: ldo=%lld, expected %lld", who, (long long)wt->ldo,
                (long long)sqf_pad_k_out(wt->k_out, wt->branch));
  if (wt->k_low > 0 && !wt->w_low) return fail(SQF_ERR_INVALID_ARG, "%s: w_low is NULL", who);
  if (wt->k_low > 0 && !aligned16(wt->w_low))
    return fail(SQF_ERR_ALIGN, "%s: w_low must be 16-byte aligned", who);
  if (wt->low == SQF_MXFP4) {
    if (wt->k_low > 0 && !wt->s_wb) return fail(SQF_ERR_INVALID_ARG, "%s: s_wb is NULL", who);
    if (wt->k_low > 0 && !aligned16(wt->s_wb))
      return fail(SQF_ERR_ALIGN, "%s: s_wb must be 16-byte aligned", who);
    if (mx_scale_bytes(wt->k_low, wt->n) > kMaxOperandBytes)
      return fail(SQF_ERR_SHAPE, "%s: the weight scales exceed 2 GiB", who);
  } else if (!wt->s_w) {
    return fail(SQF_ERR_INVALID_ARG, "%s: s_w is NULL", who);
  }
  if (wt->k_out > 0 && !wt->w_out) return fail(SQF_ERR_INVALID_ARG, "%s: w_out is NULL", who);
  if (wt->k_out > 0 && !aligned16(wt->w_out))
    return fail(SQF_ERR_ALIGN, "%s: w_out must be 16-byte aligned", who);
  if (wt->k_out > 0 && wt->branch != SQF_BF16 && !wt->s_wo)
    return fail(SQF_ERR_INVALID_ARG, "%s: s_wo is required for a scaled branch", who);
  if (low_rows(wt->n, wt->low) * wt->ldk * wt->groups > kMaxOperandBytes ||
      wt->n * wt->ldo * branch_esz(wt->branch) * wt->groups > kMaxOperandBytes)
    return fail(SQF_ERR_SHAPE, "%s: a weight operand exceeds 2 GiB", who);
  if (wt->sq_nnz < 0 || wt->sq_nnz > wt->k_low)
    return fail(SQF_ERR_SHAPE, "%s: sq_nnz=%lld outside [0, k_low]", who, (long long)wt->sq_nnz);
  if (wt->sq_nnz > 0) {
    if (wt->groups != 1)
      return fail(SQF_ERR_UNSUPPORTED, "%s: the weight-side format needs groups == 1", who);
    if (!((wt->low == SQF_I4X2 && wt->branch == SQF_I8) ||
          (wt->low == SQF_FP4_E2M1 && wt->branch == SQF_FP8_E4M3)))
      return fail(SQF_ERR_UNSUPPORTED, "%s: the weight-side format is int4 codes with an SQF_I8 "
                  "branch, or SQF_FP4_E2M1 codes with an SQF_FP8_E4M3 branch", who);
    if (!wt->sq_val || !wt->s_w8)
      return fail(SQF_ERR_INVALID_ARG, "%s: sq_val and s_w8 are required", who);
    if (wt->sq_bank != 0 && wt->sq_bank != wt->k_low) {
      if (wt->sq_bank < 64 || wt->sq_bank % 64 != 0 || wt->k_low % wt->sq_bank != 0 ||
          wt->sq_nnz % (wt->k_low / wt->sq_bank) != 0)
        return fail(SQF_ERR_SHAPE, "%s: sq_bank=%lld must be a multiple of 64 dividing k_low=%lld, "
                    "and sq_nnz=%lld a multiple of the %lld banks", who, (long long)wt->sq_bank,
                    (long long)wt->k_low, (long long)wt->sq_nnz,
                    (long long)(wt->sq_bank > 0 ? wt->k_low / wt->sq_bank : 0));
      if (wt->sq_bank > kMaxSqBank)
        return fail(SQF_ERR_UNSUPPORTED, "%s: sq_bank=%lld: banks of up to %lld slots (or the "
                    "whole row) are built", who, (long long)wt->sq_bank, (long long)kMaxSqBank);
    }
    if (!aligned16(wt->sq_val))
      return fail(SQF_ERR_ALIGN, "%s: sq_val must be 16-byte aligned", who);
  } else if (wt->branch == SQF_I8) {
    return fail(SQF_ERR_UNSUPPORTED,
                "%s: an int8 branch is only built for the weight-side format", who);
  }
  return SQF_OK;
}

sqf_status check_acts(const sqf_acts* a, const char* who) {
  if (!a) return fail(SQF_ERR_INVALID_ARG, "%s: activation descriptor is NULL", who);
  if (a->m < 0 || a->k_low < 0 || a->k_out < 0 || a->k_low + a->k_out < 1)
    return fail(SQF_ERR_SHAPE, "%s: bad activation shape m=%lld k_low=%lld k_out=%lld", who,
                (long long)a->m, (long long)a->k_low, (long long)a->k_out);
  if (a->low != SQF_I4X2 && a->low != SQF_I8 && a->low != SQF_I4_E2M3 && a->low != SQF_MXFP4 &&
      a->low != SQF_FP8_E4M3)
    return fail(SQF_ERR_INVALID_ARG, "%s: bad low dtype %d", who, a->low);
  if (a->low == SQF_FP8_E4M3 && a->branch != SQF_FP8_E4M3)
    return fail(SQF_ERR_UNSUPPORTED, "%s: E4M3 low codes (the floating-point weight-side format) "
                "come with an SQF_FP8_E4M3 branch", who);
  if (low_kblocked(a->low) && a->branch != SQF_BF16)
    return fail(SQF_ERR_UNSUPPORTED, "%s: the K-blocked low layouts (E2M3, MXFP4) come with a "
                "bf16 branch", who);
  if (!branch_ok(a->branch))
    return fail(SQF_ERR_INVALID_ARG, "%s: bad branch dtype %d", who, a->branch);
  if (a->k_low > kMaxKLow)
    return fail(SQF_ERR_SHAPE, "%s: k_low exceeds %lld", who, (long long)kMaxKLow);
  const int64_t want_ldk = low_ldk(a->k_low, a->low);
  if (a->ldk != want_ldk)
    return fail(SQF_ERR_SHAPE, "%s: ldk=%lld, expected %lld", who, (long long)a->ldk,
                (long long)want_ldk);
  if (a->ldo != sqf_pad_k_out(a->k_out, a->branch))
    return fail(SQF_ERR_SHAPE, "%s: ldo=%lld, expected %lld", who, (long long)a->ldo,
                (long long)sqf_pad_k_out(a->k_out, a->branch));
  if (a->m > 0) {
    if (a->k_low > 0 && !a->x_low) return fail(SQF_ERR_INVALID_ARG, "%s: x_low is NULL", who);
    if (a->k_low > 0 && !aligned16(a->x_low))
      return fail(SQF_ERR_ALIGN, "%s: x_low must be 16-byte aligned", who);
    if (a->low == SQF_MXFP4) {
      if (a->k_low > 0 && !a->s_xb) return fail(SQF_ERR_INVALID_ARG, "%s: s_xb is NULL", who);
      if (a->k_low > 0 && !aligned16(a->s_xb))
        return fail(SQF_ERR_ALIGN, "%s: s_xb must be 16-byte aligned", who);
    } else if (!a->s_x) {
      return fail(SQF_ERR_INVALID_ARG, "%s: s_x is NULL", who);
    }
    if (a->k_out > 0 && !a->x_out) return fail(SQF_ERR_INVALID_ARG, "%s: x_out is NULL", who);
    if (a->k_out > 0 && !aligned16(a->x_out))
      return fail(SQF_ERR_ALIGN, "%s: x_out must be 16-byte aligned", who);
    if (a->k_out > 0 && a->branch != SQF_BF16 && !a->s_xo)
      return fail(SQF_ERR_INVALID_ARG, "%s: s_xo is required for a scaled branch", who);
  }
  if (low_rows(a->m, a->low) * a->ldk > kMaxOperandBytes ||
      a->m * a->ldo * branch_esz(a->branch) > kMaxOperandBytes ||
      (a->low == SQF_MXFP4 && mx_scale_bytes(a->k_low, a->m) > kMaxOperandBytes))
    return fail(SQF_ERR_SHAPE, "%s: an activation operand exceeds 2 GiB", who);
  return SQF_OK;
}

sqf_status quantize_common(const void* x, int32_t x_dtype, int64_t ldx, int64_t groups,
                           const int64_t* row_off, const int32_t* map, sqf_acts* a, bool grouped,
                           void* stream, const char* who, const float* gamma = nullptr,
                           float eps = 0.0f) {
  g_err.clear();
  sqf_status st = check_acts(a, who);
  if (st != SQF_OK) return st;
  if (a->m == 0) return SQF_OK;
  if (!x || !map) return fail(SQF_ERR_INVALID_ARG, "%s: x and map are required", who);
  if (x_dtype != SQF_F32 && x_dtype != SQF_BF16)
    return fail(SQF_ERR_INVALID_ARG, "%s: x_dtype must be SQF_F32 or SQF_BF16", who);
  const int64_t k = a->k_low + a->k_out;
  if (k > 65536) return fail(SQF_ERR_SHAPE, "%s: k=%lld exceeds 65536", who, (long long)k);
  const bool norm = gamma != nullptr;
  if (norm) {
    if (a->branch != SQF_BF16 || (a->low != SQF_I4X2 && a->low != SQF_I4_E2M3))
      return fail(SQF_ERR_UNSUPPORTED, "%s: the fused norm comes with a bf16 branch and int4 codes "
                  "(SQF_I4X2 or SQF_I4_E2M3)", who);
    if (!(eps >= 0.0f) || eps > 1.0f)
      return fail(SQF_ERR_INVALID_ARG, "%s: eps must be in [0, 1]", who);
    if ((uintptr_t)gamma & 3u) return fail(SQF_ERR_ALIGN, "%s: gamma must be 4-byte aligned", who);
  }
  if (sqf::act_split_lds_bytes(a->ldk, a->k_out, a->low, norm ? k : 0) > 160 * 1024)
    return fail(SQF_ERR_SHAPE, "%s: k_low=%lld, k_out=%lld exceed the kernel's LDS staging%s", who,
                (long long)a->k_low, (long long)a->k_out, norm ? " (with gamma)" : "");
  if (ldx < k) return fail(SQF_ERR_SHAPE, "%s: ldx=%lld < k=%lld", who, (long long)ldx, (long long)k);
  if (((uintptr_t)x & (x_dtype == SQF_BF16 ? 1u : 3u)) || ((uintptr_t)map & 3u))
    return fail(SQF_ERR_ALIGN, "%s: x and map must be aligned to their element size", who);
  // 8-channel chunks with 16-byte loads need k, ldx and x aligned to them;
  // anything else takes the element-wise load path
  const bool ragged = k % 8 != 0 || ldx % 8 != 0 || !aligned16(x) || !aligned16(map);
  if (ragged && grouped)
    return fail(SQF_ERR_UNSUPPORTED, "%s: grouped rows need k and ldx multiples of 8 and "
                "16-byte aligned x and maps", who);
  if (grouped && (groups < 1 || !row_off))
    return fail(SQF_ERR_INVALID_ARG, "%s: groups >= 1 and row_off are required", who);
  if (grouped && a->low != SQF_I4X2)
    return fail(SQF_ERR_UNSUPPORTED, "%s: grouped activations are packed int4 only", who);
  sqf::ActArgs args{x, ldx, map, row_off, a->m, k, a->k_low, a->k_out, sqf_pad_k_low(a->k_low),
                    a->ldk, a->ldo, low_kblocked(a->low) ? sqf_pad_rows(a->m) : 0,
                    (int32_t)(grouped ? groups : 1), a->x_low, a->s_x, (uint8_t*)a->x_out, a->s_xo,
                    a->s_xb, gamma, eps};
  return hip_status(sqf::launch_act_split(args, x_dtype, a->low, a->branch, grouped, ragged, norm,
                                          (hipStream_t)stream),
                    who);
}

sqf_status check_pair(const sqf_acts* a, const sqf_weights* w, const void* y, int64_t ldy,
                      const char* who) {
  sqf_status st = check_acts(a, who);
  if (st != SQF_OK) return st;
  st = check_weights(w, who);
  if (st != SQF_OK) return st;
  if (a->k_low != w->k_low || a->k_out != w->k_out || a->branch != w->branch)
    return fail(SQF_ERR_INVALID_ARG, "%s: activations and weights disagree on k_low/k_out/branch",
                who);
  if (w->sq_nnz > 0 && !((w->low == SQF_I4X2 && a->low == SQF_I8) ||
                         (w->low == SQF_FP4_E2M1 && a->low == SQF_FP8_E4M3)))
    return fail(SQF_ERR_INVALID_ARG, "%s: the weight-side format needs int8 activations (int4 "
                "weights) or E4M3 activations (E2M1 weights)", who);
  if (w->sq_nnz == 0 && (a->low == SQF_I8 || a->low == SQF_FP8_E4M3))
    return fail(SQF_ERR_INVALID_ARG, "%s: 8-bit low activations belong to the weight-side format",
                who);
  if (w->sq_nnz == 0 && a->low != w->low)
    return fail(SQF_ERR_INVALID_ARG, "%s: activations (low %d) and weights (low %d) disagree on "
                "the low storage", who, a->low, w->low);
  if (a->m > 0 && !y) return fail(SQF_ERR_INVALID_ARG, "%s: y is NULL", who);
  if (ldy < w->n) return fail(SQF_ERR_SHAPE, "%s: ldy=%lld < n=%lld", who, (long long)ldy,
                              (long long)w->n);
  return SQF_OK;
}

// Y is fp32 (float*) or, with ybf16, bf16 (uint16_t* bit patterns); ldy in
// elements of Y's type.
sqf_status dual_gemm_impl(const sqf_acts* a, const sqf_weights* w, void* y, bool ybf16,
                          int64_t ldy, int32_t tile, int32_t* acc_low_dbg, int32_t* acc_sp_dbg,
                          int32_t* acc_out_dbg, void* stream, const char* who,
                          void* ws = nullptr, int64_t ws_bytes = 0, bool ws_call = false) {
  sqf_status st = check_pair(a, w, y, ldy, who);
  if (st != SQF_OK) return st;
  if (ws_call) {
    if (w->sq_nnz <= 0)
      return fail(SQF_ERR_INVALID_ARG, "%s: the workspace call is for the weight-side format", who);
    const int64_t need = sqf::sq_image_bytes(w->n, w->ldk, w->low == SQF_FP4_E2M1);
    if (!ws) return fail(SQF_ERR_INVALID_ARG, "%s: workspace is NULL", who);
    if ((((uintptr_t)ws) & 255) != 0)
      return fail(SQF_ERR_ALIGN, "%s: workspace must be 256-byte aligned", who);
    if (ws_bytes < need)
      return fail(SQF_ERR_SHAPE, "%s: workspace of %lld bytes, %lld needed", who, (long long)ws_bytes,
                  (long long)need);
  }
  if (!tile_ok(tile)) return fail(SQF_ERR_INVALID_ARG, "%s: bad tile %d", who, tile);
  if (ybf16 && (acc_low_dbg || acc_sp_dbg || acc_out_dbg))
    return fail(SQF_ERR_INVALID_ARG, "%s: debug outputs need fp32 Y", who);
  if (w->branch == SQF_FP8_E4M3 && tile == SQF_TILE_256)
    return fail(SQF_ERR_UNSUPPORTED, "%s: the E4M3 branch has no 256x256 tile", who);
  if (w->groups != 1) return fail(SQF_ERR_INVALID_ARG, "%s: use sqf_dual_gemm_grouped", who);
  if (a->m == 0) return SQF_OK;
  const bool debug = acc_low_dbg || acc_sp_dbg || acc_out_dbg;
  if (w->sq_nnz > 0) {
    if (ybf16) return fail(SQF_ERR_UNSUPPORTED, "%s: the weight-side format writes fp32 Y", who);
    const bool fp = w->low == SQF_FP4_E2M1;
    if (fp && debug)
      return fail(SQF_ERR_UNSUPPORTED, "%s: the floating-point weight-side format has no integer "
                  "accumulators", who);
    // int8 activations x (16 x int4 weights) in an int32 accumulator
    if (w->k_low > kMaxKLowSq)
      return fail(SQF_ERR_UNSUPPORTED, "%s: k_low=%lld exceeds %lld for the weight-side format", who,
                  (long long)w->k_low, (long long)kMaxKLowSq);
    if (debug && !(acc_low_dbg && acc_sp_dbg && acc_out_dbg))
      return fail(SQF_ERR_INVALID_ARG, "%s: the weight-side debug path writes all three accumulators", who);
    if (tile != SQF_TILE_AUTO)
      return fail(SQF_ERR_UNSUPPORTED, "%s: the weight-side GEMM has one tile shape", who);
    sqf::SqArgs sa{a->x_low, a->s_x, (const uint8_t*)a->x_out, a->s_xo, w->w_low, w->s_w,
                   w->sq_val, w->s_w8, (const uint8_t*)w->w_out, w->s_wo, (float*)y,
                   acc_low_dbg, acc_sp_dbg, acc_out_dbg, a->m, w->n, a->ldk, w->ldk, w->ldo, ldy,
                   w->sq_nnz, (int32_t)(w->ldk / 128), (int32_t)(w->ldo / 128),
                   ws_call ? (uint8_t*)ws : nullptr};
    return hip_status(sqf::launch_sq_gemm(sa, debug, fp, (hipStream_t)stream), who);
  }
  if (acc_sp_dbg || acc_out_dbg)
    return fail(SQF_ERR_INVALID_ARG, "%s: acc_sp/acc_out debug outputs need the weight-side format", who);
  if (low_kblocked(w->low)) {
    if (tile != SQF_TILE_AUTO && tile != SQF_TILE_256)
      return fail(SQF_ERR_UNSUPPORTED, "%s: the K-blocked low paths have 256x256 tiles only", who);
    if (w->low == SQF_MXFP4 && acc_low_dbg)
      return fail(SQF_ERR_UNSUPPORTED, "%s: the MXFP4 low path has no integer accumulators", who);
    sqf::Gemm6Args ga{a->x_low, a->s_x, a->s_xb, (const uint8_t*)a->x_out, w->w_low, w->s_w,
                      w->s_wb, (const uint8_t*)w->w_out, (float*)y, acc_low_dbg, a->m, w->n,
                      sqf_pad_rows(a->m), sqf_pad_rows(w->n), w->ldo * 2, ldy,
                      (int32_t)(sqf_pad_k_low(w->k_low) / 128), (int32_t)(w->ldo / 32)};
    return hip_status(sqf::launch_gemm6(ga, w->low == SQF_MXFP4 ? sqf::kMXFP4 : sqf::kI4E2M3, debug,
                                        ybf16, (hipStream_t)stream),
                      who);
  }
  const int64_t ldo_b = w->ldo * branch_esz(w->branch);
  sqf::GemmArgs ga{a->x_low, a->s_x, (const uint8_t*)a->x_out, a->s_xo, w->w_low, w->s_w,
                   (const uint8_t*)w->w_out, w->s_wo, (float*)y, acc_low_dbg, nullptr, a->m, w->n, w->ldk,
                   ldo_b, ldy, 0, 0, 0, (int32_t)(w->ldk / 64), (int32_t)(ldo_b / 64), 1};
  return hip_status(sqf::launch_dual_gemm(ga, w->branch, false, debug,
                                          pick_cfg(a->m, w->n, w->branch, tile), (hipStream_t)stream,
                                          ybf16),
                    who);
}

sqf_status grouped_impl(const sqf_acts* a, const sqf_weights* w, int64_t groups,
                        const int64_t* row_off, void* y, bool ybf16, int64_t ldy, int32_t tile,
                        int32_t* acc_low_dbg, void* stream, const char* who) {
  sqf_status st = check_pair(a, w, y, ldy, who);
  if (st != SQF_OK) return st;
  if (!tile_ok(tile)) return fail(SQF_ERR_INVALID_ARG, "%s: bad tile %d", who, tile);
  if (tile == SQF_TILE_64)
    return fail(SQF_ERR_UNSUPPORTED, "%s: grouped tiles are 256x256 or 128x128", who);
  if (ybf16 && acc_low_dbg) return fail(SQF_ERR_INVALID_ARG, "%s: debug outputs need fp32 Y", who);
  if (w->branch == SQF_FP8_E4M3 && tile == SQF_TILE_256)
    return fail(SQF_ERR_UNSUPPORTED, "%s: the E4M3 branch has no 256x256 tile", who);
  if (groups < 1 || w->groups != groups || !row_off)
    return fail(SQF_ERR_INVALID_ARG, "%s: need groups >= 1 == w->groups and row_off", who);
  if (w->sq_nnz > 0) return fail(SQF_ERR_UNSUPPORTED, "%s: channel-split format only", who);
  if (w->low != SQF_I4X2)
    return fail(SQF_ERR_UNSUPPORTED, "%s: grouped weights are packed int4 only", who);
  if (a->m == 0) return SQF_OK;
  const int64_t ldo_b = w->ldo * branch_esz(w->branch);
  // 256x256 tiles when the groups average 384 rows or more (bf16 branch),
  // else 128x128, unless the caller forces one
  sqf::GemmArgs ga{a->x_low, a->s_x, (const uint8_t*)a->x_out, a->s_xo, w->w_low, w->s_w,
                   (const uint8_t*)w->w_out, w->s_wo, (float*)y, acc_low_dbg, row_off, a->m, w->n,
                   w->ldk, ldo_b, ldy, w->n * w->ldk, w->n * ldo_b, w->n,
                   (int32_t)(w->ldk / 64), (int32_t)(ldo_b / 64), (int32_t)groups};
  int cfg = tile != SQF_TILE_AUTO ? tile : (a->m / groups >= 384) ? 0 : 1;
  if (w->branch == SQF_FP8_E4M3) cfg = 1;
  return hip_status(sqf::launch_dual_gemm(ga, w->branch, true, acc_low_dbg != nullptr, cfg,
                                          (hipStream_t)stream, ybf16),
                    who);
}

sqf_status check_select(const float* x_cal, int64_t m_cal, int64_t k, const float* w, int64_t n,
                        int64_t k_out, const int32_t* idx_out, const int32_t* map_out,
                        const char* who) {
  if (!x_cal || !w || !map_out)
    return fail(SQF_ERR_INVALID_ARG, "%s: x_cal, w and map_out are required", who);
  if (m_cal < 1 || n < 1 || k < 1 || k > 1048576)
    return fail(SQF_ERR_SHAPE, "%s: need m_cal>=1, n>=1, 1<=k<=1048576 (got %lld, %lld, %lld)",
                who, (long long)m_cal, (long long)n, (long long)k);
  if (k_out < 0 || k_out > k)
    return fail(SQF_ERR_SHAPE, "%s: k_out=%lld outside [0, k=%lld]", who, (long long)k_out,
                (long long)k);
  if (k_out > 0 && !idx_out) return fail(SQF_ERR_INVALID_ARG, "%s: idx_out is NULL", who);
  return SQF_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
double* g_scratch_ptr[kMaxDevices] = {};

// The device address of the current device's `scratch`, looked up on the
// first call on that device (with that device current).
sqf_status scratch_scores(double** out, const char* who) {
  int dev = -1;
  sqf_status st = hip_status(hipGetDevice(&dev), who);
  if (st != SQF_OK) return st;
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SQF_ERR_UNSUPPORTED, "%s: device %d beyond the %d this library tracks", who, dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    st = hip_status(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), who);
    if (st != SQF_OK) return st;
    if (!ptr) return fail(SQF_ERR_HIP, "%s: no device address for the score array", who);
    g_scratch_ptr[dev] = (double*)ptr;
  }
  *out = g_scratch_ptr[dev];
  return SQF_OK;
}

}  // namespace

extern "C" {

int sqf_abi_version(void) { return SQF_ABI_VERSION; }

const char* sqf_last_error(void) { return g_err.c_str(); }

int64_t sqf_pad_k_low(int64_t k_low) {
  if (k_low < 0) return -1;
  return (k_low + 255) / 256 * 256;
}

int64_t sqf_pad_rows(int64_t rows) {
  if (rows < 0) return -1;
  return (rows + 255) / 256 * 256;
}

int64_t sqf_pad_k_out(int64_t k_out, int32_t branch) {
  if (k_out < 0 || !branch_ok(branch)) return -1;
  const int64_t step = 128 / branch_esz(branch);
  return (k_out + step - 1) / step * step;
}

sqf_status sqf_select_channels(const float* x_cal, int64_t m_cal, int64_t k, const float* w,
                               int64_t n, int64_t k_out, int32_t* idx_out, int32_t* map_out,
                               double* score_out, float* hdiag_out, void* stream) {
  g_err.clear();
  const char* who = "sqf_select_channels";
  sqf_status vst = check_select(x_cal, m_cal, k, w, n, k_out, idx_out, map_out, who);
  if (vst != SQF_OK) return vst;
  hipStream_t s = (hipStream_t)stream;
  double* score = score_out;
  if (!score) {
    // the scores are the kernels' workspace: borrow them from the
    // stream-ordered pool for the duration of the call
    sqf_status st = hip_status(hipMallocAsync((void**)&score, (size_t)k * sizeof(double), s), who);
    if (st != SQF_OK) return st;
  }
  sqf_status st = hip_status(sqf::launch_select(x_cal, m_cal, k, w, n, k_out, idx_out, map_out,
                                                score, hdiag_out, s),
                             who);
  if (!score_out) {
    const sqf_status fst = hip_status(hipFreeAsync(score, s), who);
    if (st == SQF_OK) st = fst;
  }
  return st;
}

sqf_status sqf_select_channels_noalloc(const float* x_cal, int64_t m_cal, int64_t k,
                                       const float* w, int64_t n, int64_t k_out, int32_t* idx_out,
                                       int32_t* map_out, float* hdiag_out, void* stream) {
  g_err.clear();
  const char* who = "sqf_select_channels_noalloc";
  sqf_status vst = check_select(x_cal, m_cal, k, w, n, k_out, idx_out, map_out, who);
  if (vst != SQF_OK) return vst;
  if (k > kScratchScores)
    return fail(SQF_ERR_SHAPE, "%s: k=%lld exceeds the %lld channels of the library's static "
                "score array (use sqf_select_channels)", who, (long long)k,
                (long long)kScratchScores);
  double* score = nullptr;
  sqf_status st = scratch_scores(&score, who);
  if (st != SQF_OK) return st;
  // every score[c], c < k, is written by the first kernel before it is read:
  // nothing left by an earlier call needs clearing
  return hip_status(sqf::launch_select(x_cal, m_cal, k, w, n, k_out, idx_out, map_out, score,
                                       hdiag_out, (hipStream_t)stream),
                    who);
}

sqf_status sqf_pack_weights(const float* w, const int32_t* map, const float* hdiag,
                            sqf_weights* wt, void* stream) {
  g_err.clear();
  const char* who = "sqf_pack_weights";
  if (!w || !map) return fail(SQF_ERR_INVALID_ARG, "%s: w and map are required", who);
  sqf_status st = check_weights(wt, who);
  if (st != SQF_OK) return st;
  if (wt->sq_nnz > 0) {
    if (!hdiag) return fail(SQF_ERR_INVALID_ARG, "%s: hdiag is required", who);
    if (wt->k_low * 9 + wt->k_out * 4 + 16 > 150 * 1024)
      return fail(SQF_ERR_SHAPE, "%s: a weight-side row (k_low=%lld) does not fit in LDS", who,
                  (long long)wt->k_low);
  }
  sqf::PackArgs a{w, map, hdiag, wt->k, wt->n, wt->k_low, wt->k_out, wt->ldk, wt->ldo,
                  wt->sq_nnz, wt->sq_bank == wt->k_low ? 0 : wt->sq_bank, low_kblocked(wt->low) ? sqf_pad_rows(wt->n) : 0, wt->w_low, wt->s_w,
                  wt->s_wb, (uint8_t*)wt->w_out, wt->s_wo, wt->sq_val, wt->s_w8};
  return hip_status(sqf::launch_pack(a, wt->branch, wt->low, wt->groups, (hipStream_t)stream), who);
}

sqf_status sqf_quantize_split_act(const void* x, int32_t x_dtype, int64_t ldx, const int32_t* map,
                                  sqf_acts* a, void* stream) {
  return quantize_common(x, x_dtype, ldx, 1, nullptr, map, a, false, stream,
                         "sqf_quantize_split_act");
}

sqf_status sqf_slot_order(const int32_t* map, int64_t k, int32_t* perm_out,
                          int32_t* slice_map_out, void* stream) {
  g_err.clear();
  const char* who = "sqf_slot_order";
  if (!map || !perm_out || !slice_map_out)
    return fail(SQF_ERR_INVALID_ARG, "%s: map, perm_out and slice_map_out are required", who);
  if (k < 1 || k > 1048576)
    return fail(SQF_ERR_SHAPE, "%s: need 1 <= k <= 1048576 (got %lld)", who, (long long)k);
  return hip_status(sqf::launch_slot_order(map, k, perm_out, slice_map_out, (hipStream_t)stream),
                    who);
}

sqf_status sqf_permute_channels(const float* src, int64_t rows, int64_t cols, int64_t ld_src,
                                const int32_t* perm, int32_t axis, float* dst, int64_t ld_dst,
                                void* stream) {
  g_err.clear();
  const char* who = "sqf_permute_channels";
  if (!src || !perm || !dst) return fail(SQF_ERR_INVALID_ARG, "%s: src, perm and dst are required", who);
  if (axis != 0 && axis != 1) return fail(SQF_ERR_INVALID_ARG, "%s: axis must be 0 or 1", who);
  if (rows < 0 || cols < 0 || ld_src < cols || ld_dst < cols)
    return fail(SQF_ERR_SHAPE, "%s: bad shape rows=%lld cols=%lld ld_src=%lld ld_dst=%lld", who,
                (long long)rows, (long long)cols, (long long)ld_src, (long long)ld_dst);
  if ((const void*)src == (const void*)dst)
    return fail(SQF_ERR_INVALID_ARG, "%s: src and dst must not be the same buffer", who);
  return hip_status(sqf::launch_permute(src, rows, cols, ld_src, perm, axis, dst, ld_dst,
                                        (hipStream_t)stream),
                    who);
}

sqf_status sqf_rmsnorm_quantize_split_act(const void* x, int32_t x_dtype, int64_t ldx,
                                          const float* gamma, float eps, const int32_t* map,
                                          sqf_acts* a, void* stream) {
  if (!gamma) {
    g_err.clear();
    return fail(SQF_ERR_INVALID_ARG, "sqf_rmsnorm_quantize_split_act: gamma is required");
  }
  return quantize_common(x, x_dtype, ldx, 1, nullptr, map, a, false, stream,
                         "sqf_rmsnorm_quantize_split_act", gamma, eps);
}

sqf_status sqf_quantize_split_act_grouped(const void* x, int32_t x_dtype, int64_t ldx,
                                          int64_t groups, const int64_t* row_off,
                                          const int32_t* maps, sqf_acts* a, void* stream) {
  return quantize_common(x, x_dtype, ldx, groups, row_off, maps, a, true, stream,
                         "sqf_quantize_split_act_grouped");
}

sqf_status sqf_dual_gemm(const sqf_acts* a, const sqf_weights* w, float* y, int64_t ldy,
                         int32_t* acc_low_dbg, int32_t* acc_sp_dbg, int32_t* acc_out_dbg,
                         void* stream) {
  g_err.clear();
  return dual_gemm_impl(a, w, y, false, ldy, SQF_TILE_AUTO, acc_low_dbg, acc_sp_dbg, acc_out_dbg,
                        stream, "sqf_dual_gemm");
}

int64_t sqf_sq_workspace_bytes(const sqf_weights* w) {
  if (!w || w->sq_nnz <= 0 || w->n < 1 || w->ldk < 0 || w->ldk % 64 != 0) return -1;
  return sqf::sq_image_bytes(w->n, w->ldk, w->low == SQF_FP4_E2M1);
}

sqf_status sqf_dual_gemm_sq_ws(const sqf_acts* a, const sqf_weights* w, float* y, int64_t ldy,
                               void* workspace, int64_t workspace_bytes, int32_t* acc_low_dbg,
                               int32_t* acc_sp_dbg, int32_t* acc_out_dbg, void* stream) {
  return dual_gemm_impl(a, w, y, false, ldy, SQF_TILE_AUTO, acc_low_dbg, acc_sp_dbg, acc_out_dbg,
                        stream, "sqf_dual_gemm_sq_ws", workspace, workspace_bytes, true);
}

sqf_status sqf_dual_gemm_y(const sqf_acts* a, const sqf_weights* w, void* y, int32_t y_dtype,
                           int64_t ldy, void* stream) {
  g_err.clear();
  const char* who = "sqf_dual_gemm_y";
  if (y_dtype != SQF_F32 && y_dtype != SQF_BF16)
    return fail(SQF_ERR_INVALID_ARG, "%s: y_dtype %d is neither SQF_F32 nor SQF_BF16", who, y_dtype);
  return dual_gemm_impl(a, w, y, y_dtype == SQF_BF16, ldy, SQF_TILE_AUTO, nullptr, nullptr,
                        nullptr, stream, who);
}

sqf_status sqf_dual_gemm_grouped(const sqf_acts* a, const sqf_weights* w, int64_t groups,
                                 const int64_t* row_off, float* y, int64_t ldy,
                                 int32_t* acc_low_dbg, void* stream) {
  g_err.clear();
  return grouped_impl(a, w, groups, row_off, y, false, ldy, SQF_TILE_AUTO, acc_low_dbg, stream,
                      "sqf_dual_gemm_grouped");
}

sqf_status sqf_dual_gemm_grouped_y(const sqf_acts* a, const sqf_weights* w, int64_t groups,
                                   const int64_t* row_off, void* y, int32_t y_dtype, int64_t ldy,
                                   void* stream) {
  g_err.clear();
  const char* who = "sqf_dual_gemm_grouped_y";
  if (y_dtype != SQF_F32 && y_dtype != SQF_BF16)
    return fail(SQF_ERR_INVALID_ARG, "%s: y_dtype %d is neither SQF_F32 nor SQF_BF16", who, y_dtype);
  return grouped_impl(a, w, groups, row_off, y, y_dtype == SQF_BF16, ldy, SQF_TILE_AUTO, nullptr,
                      stream, who);
}

sqf_status sqf_dual_gemm_ex(const sqf_acts* a, const sqf_weights* w, void* y, int32_t y_dtype,
                            int64_t ldy, int32_t tile, int32_t* acc_low_dbg, int32_t* acc_sp_dbg,
                            int32_t* acc_out_dbg, void* stream) {
  g_err.clear();
  const char* who = "sqf_dual_gemm_ex";
  if (y_dtype != SQF_F32 && y_dtype != SQF_BF16)
    return fail(SQF_ERR_INVALID_ARG, "%s: y_dtype %d is neither SQF_F32 nor SQF_BF16", who, y_dtype);
  return dual_gemm_impl(a, w, y, y_dtype == SQF_BF16, ldy, tile, acc_low_dbg, acc_sp_dbg,
                        acc_out_dbg, stream, who);
}

sqf_status sqf_dual_gemm_grouped_ex(const sqf_acts* a, const sqf_weights* w, int64_t groups,
                                    const int64_t* row_off, void* y, int32_t y_dtype, int64_t ldy,
                                    int32_t tile, int32_t* acc_low_dbg, void* stream) {
  g_err.clear();
  const char* who = "sqf_dual_gemm_grouped_ex";
  if (y_dtype != SQF_F32 && y_dtype != SQF_BF16)
    return fail(SQF_ERR_INVALID_ARG, "%s: y_dtype %d is neither SQF_F32 nor SQF_BF16", who, y_dtype);
  return grouped_impl(a, w, groups, row_off, y, y_dtype == SQF_BF16, ldy, tile, acc_low_dbg,
                      stream, who);
}

}  // extern "C"
