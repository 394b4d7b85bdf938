// sqf_api.hip -- the C ABI of libsqf (declared in include/sqf.h).
//
// Every entry point validates its arguments on the host before launching
// anything; a failure returns a status and sets a thread-local message.  No
// entry point allocates device memory or keeps a pointer after it returns.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <string>

#include "../../include/sqf.h"
#include "sqf_device.h"
#include "sqf_launch.h"

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
// Kernels address operands with 32-bit byte offsets.
constexpr int64_t kMaxOperandBytes = ((int64_t)1 << 31) - 1;

int branch_esz(int32_t b) { return b == SQF_BF16 ? 2 : 1; }
bool branch_ok(int32_t b) { return b == SQF_BF16 || b == SQF_FP8_E4M3 || b == SQF_I8; }

// Tile configuration for the channel-split GEMM.  SQF_GEMM_TILE=0/1/2 forces
// 256x256 / 128x128 / 64x64 (a tuning and test aid, read on every call);
// otherwise the largest tile that still gives the 256 CUs enough tiles.
int pick_cfg(int64_t m, int64_t n, int32_t branch) {
  const char* env = getenv("SQF_GEMM_TILE");
  const int forced = env ? atoi(env) : -1;
  int cfg;
  if (forced >= 0 && forced <= 2)
    cfg = forced;
  else if (((m + 255) / 256) * ((n + 255) / 256) >= 448)
    cfg = 0;
  else if (((m + 127) / 128) * ((n + 127) / 128) >= 256)
    cfg = 1;
  else
    cfg = 2;
  if (branch == SQF_FP8_E4M3 && cfg == 0) cfg = 1;  // it needs a second accumulator set
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
  if (wt->k_low > kMaxKLow)
    return fail(SQF_ERR_SHAPE, "%s: k_low=%lld exceeds %lld", who, (long long)wt->k_low,
                (long long)kMaxKLow);
  if (wt->ldk != sqf_pad_k_low(wt->k_low) / 2)
    return fail(SQF_ERR_SHAPE, "%s: ldk=%lld, expected %lld", who, (long long)wt->ldk,
                (long long)(sqf_pad_k_low(wt->k_low) / 2));
  if (wt->ldo != sqf_pad_k_out(wt->k_out, wt->branch))
    return fail(SQF_ERR_SHAPE, "%s: ldo=%lld, expected %lld", who, (long long)wt->ldo,
                (long long)sqf_pad_k_out(wt->k_out, wt->branch));
  if (wt->k_low > 0 && !wt->w_low) return fail(SQF_ERR_INVALID_ARG, "%s: w_low is NULL", who);
  if (wt->k_low > 0 && !aligned16(wt->w_low))
    return fail(SQF_ERR_ALIGN, "%s: w_low must be 16-byte aligned", who);
  if (!wt->s_w) return fail(SQF_ERR_INVALID_ARG, "%s: s_w is NULL", who);
  if (wt->k_out > 0 && !wt->w_out) return fail(SQF_ERR_INVALID_ARG, "%s: w_out is NULL", who);
  if (wt->k_out > 0 && !aligned16(wt->w_out))
    return fail(SQF_ERR_ALIGN, "%s: w_out must be 16-byte aligned", who);
  if (wt->k_out > 0 && wt->branch != SQF_BF16 && !wt->s_wo)
    return fail(SQF_ERR_INVALID_ARG, "%s: s_wo is required for a scaled branch", who);
  if (wt->n * wt->ldk * wt->groups > kMaxOperandBytes ||
      wt->n * wt->ldo * branch_esz(wt->branch) * wt->groups > kMaxOperandBytes)
    return fail(SQF_ERR_SHAPE, "%s: a weight operand exceeds 2 GiB", who);
  if (wt->sq_nnz < 0 || wt->sq_nnz > wt->k_low)
    return fail(SQF_ERR_SHAPE, "%s: sq_nnz=%lld outside [0, k_low]", who, (long long)wt->sq_nnz);
  if (wt->sq_nnz > 0) {
    if (wt->groups != 1)
      return fail(SQF_ERR_UNSUPPORTED, "%s: the weight-side format needs groups == 1", who);
    if (wt->branch != SQF_I8)
      return fail(SQF_ERR_UNSUPPORTED, "%s: the weight-side format needs an SQF_I8 branch", who);
    if (!wt->sq_val || !wt->s_w8 || !wt->sq_tile_off)
      return fail(SQF_ERR_INVALID_ARG, "%s: sq_val, s_w8 and sq_tile_off are required", who);
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
  if (a->low != SQF_I4X2 && a->low != SQF_I8)
    return fail(SQF_ERR_INVALID_ARG, "%s: bad low dtype %d", who, a->low);
  if (!branch_ok(a->branch))
    return fail(SQF_ERR_INVALID_ARG, "%s: bad branch dtype %d", who, a->branch);
  if (a->k_low > kMaxKLow)
    return fail(SQF_ERR_SHAPE, "%s: k_low exceeds %lld", who, (long long)kMaxKLow);
  const int64_t pad = sqf_pad_k_low(a->k_low);
  const int64_t want_ldk = a->low == SQF_I4X2 ? pad / 2 : pad;
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
    if (!a->s_x) return fail(SQF_ERR_INVALID_ARG, "%s: s_x is NULL", who);
    if (a->k_out > 0 && !a->x_out) return fail(SQF_ERR_INVALID_ARG, "%s: x_out is NULL", who);
    if (a->k_out > 0 && !aligned16(a->x_out))
      return fail(SQF_ERR_ALIGN, "%s: x_out must be 16-byte aligned", who);
    if (a->k_out > 0 && a->branch != SQF_BF16 && !a->s_xo)
      return fail(SQF_ERR_INVALID_ARG, "%s: s_xo is required for a scaled branch", who);
  }
  if (a->m * a->ldk > kMaxOperandBytes ||
      a->m * a->ldo * branch_esz(a->branch) > kMaxOperandBytes)
    return fail(SQF_ERR_SHAPE, "%s: an activation operand exceeds 2 GiB", who);
  return SQF_OK;
}

sqf_status quantize_common(const void* x, int32_t x_dtype, int64_t ldx, int64_t groups,
                           const int64_t* row_off, const int32_t* map, sqf_acts* a, bool grouped,
                           void* stream, const char* who) {
  g_err.clear();
  sqf_status st = check_acts(a, who);
  if (st != SQF_OK) return st;
  if (a->m == 0) return SQF_OK;
  if (!x || !map) return fail(SQF_ERR_INVALID_ARG, "%s: x and map are required", who);
  if (x_dtype != SQF_F32 && x_dtype != SQF_BF16)
    return fail(SQF_ERR_INVALID_ARG, "%s: x_dtype must be SQF_F32 or SQF_BF16", who);
  const int64_t k = a->k_low + a->k_out;
  if (k % 8 != 0 || k > 65536)
    return fail(SQF_ERR_SHAPE, "%s: k=%lld must be a multiple of 8 and <= 65536", who,
                (long long)k);
  if (sqf::act_split_lds_bytes(a->ldk, a->k_out) > 160 * 1024)
    return fail(SQF_ERR_SHAPE, "%s: k_low=%lld, k_out=%lld exceed the kernel's LDS staging", who,
                (long long)a->k_low, (long long)a->k_out);
  if (ldx < k || ldx % 8 != 0)
    return fail(SQF_ERR_SHAPE, "%s: ldx=%lld must be >= k and a multiple of 8", who,
                (long long)ldx);
  if (!aligned16(x) || !aligned16(map))
    return fail(SQF_ERR_ALIGN, "%s: x and map must be 16-byte aligned", who);
  if (grouped && (groups < 1 || !row_off))
    return fail(SQF_ERR_INVALID_ARG, "%s: groups >= 1 and row_off are required", who);
  if (grouped && a->low != SQF_I4X2)
    return fail(SQF_ERR_UNSUPPORTED, "%s: grouped activations are int4 only", who);
  sqf::ActArgs args{x, ldx, map, row_off, a->m, k, a->k_low, a->k_out, sqf_pad_k_low(a->k_low),
                    a->ldk, a->ldo, (int32_t)(grouped ? groups : 1), a->x_low, a->s_x,
                    (uint8_t*)a->x_out, a->s_xo};
  return hip_status(
      sqf::launch_act_split(args, x_dtype, a->low, a->branch, grouped, (hipStream_t)stream), who);
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
  if ((w->sq_nnz > 0) != (a->low == SQF_I8))
    return fail(SQF_ERR_INVALID_ARG,
                "%s: weight-side format needs int8 activations and the channel split int4", who);
  if (a->m > 0 && !y) return fail(SQF_ERR_INVALID_ARG, "%s: y is NULL", who);
  if (ldy < w->n) return fail(SQF_ERR_SHAPE, "%s: ldy=%lld < n=%lld", who, (long long)ldy,
                              (long long)w->n);
  return SQF_OK;
}

// Y is fp32 (float*) or, with ybf16, bf16 (uint16_t* bit patterns); ldy in
// elements of Y's type.
sqf_status dual_gemm_impl(const sqf_acts* a, const sqf_weights* w, void* y, bool ybf16,
                          int64_t ldy, int32_t* acc_low_dbg, int32_t* acc_sp_dbg,
                          int32_t* acc_out_dbg, void* stream, const char* who) {
  sqf_status st = check_pair(a, w, y, ldy, who);
  if (st != SQF_OK) return st;
  if (w->groups != 1) return fail(SQF_ERR_INVALID_ARG, "%s: use sqf_dual_gemm_grouped", who);
  if (a->m == 0) return SQF_OK;
  const bool debug = acc_low_dbg || acc_sp_dbg || acc_out_dbg;
  if (w->sq_nnz > 0) {
    if (ybf16) return fail(SQF_ERR_UNSUPPORTED, "%s: the weight-side format writes fp32 Y", who);
    // int8 activations x (16 x int4 weights) in an int32 accumulator
    if (w->k_low > kMaxKLowSq)
      return fail(SQF_ERR_UNSUPPORTED, "%s: k_low=%lld exceeds %lld for the weight-side format", who,
                  (long long)w->k_low, (long long)kMaxKLowSq);
    if (debug && !(acc_low_dbg && acc_sp_dbg && acc_out_dbg))
      return fail(SQF_ERR_INVALID_ARG, "%s: the weight-side debug path writes all three accumulators", who);
    sqf::SqArgs sa{a->x_low, a->s_x, (const uint8_t*)a->x_out, a->s_xo, w->w_low, w->s_w,
                   w->sq_val, w->s_w8, w->sq_tile_off, (const uint8_t*)w->w_out, w->s_wo, (float*)y,
                   acc_low_dbg, acc_sp_dbg, acc_out_dbg, a->m, w->n, a->ldk, w->ldk, w->ldo, ldy,
                   w->sq_nnz, (int32_t)(w->ldk / 128), (int32_t)(w->ldo / 128)};
    return hip_status(sqf::launch_sq_gemm(sa, debug, (hipStream_t)stream), who);
  }
  if (acc_sp_dbg || acc_out_dbg)
    return fail(SQF_ERR_INVALID_ARG, "%s: acc_sp/acc_out debug outputs need the weight-side format", who);
  const int64_t ldo_b = w->ldo * branch_esz(w->branch);
  sqf::GemmArgs ga{a->x_low, a->s_x, (const uint8_t*)a->x_out, a->s_xo, w->w_low, w->s_w,
                   (const uint8_t*)w->w_out, w->s_wo, (float*)y, acc_low_dbg, nullptr, a->m, w->n, w->ldk,
                   ldo_b, ldy, 0, 0, 0, (int32_t)(w->ldk / 64), (int32_t)(ldo_b / 64), 1};
  return hip_status(sqf::launch_dual_gemm(ga, w->branch, false, debug,
                                          pick_cfg(a->m, w->n, w->branch), (hipStream_t)stream, ybf16),
                    who);
}

sqf_status grouped_impl(const sqf_acts* a, const sqf_weights* w, int64_t groups,
                        const int64_t* row_off, void* y, bool ybf16, int64_t ldy,
                        int32_t* acc_low_dbg, void* stream, const char* who) {
  sqf_status st = check_pair(a, w, y, ldy, who);
  if (st != SQF_OK) return st;
  if (groups < 1 || w->groups != groups || !row_off)
    return fail(SQF_ERR_INVALID_ARG, "%s: need groups >= 1 == w->groups and row_off", who);
  if (w->sq_nnz > 0) return fail(SQF_ERR_UNSUPPORTED, "%s: channel-split format only", who);
  if (a->m == 0) return SQF_OK;
  const int64_t ldo_b = w->ldo * branch_esz(w->branch);
  // 256x256 tiles when the groups average 384 rows or more (bf16 branch),
  // else 128x128; SQF_GEMM_TILE=0/1 forces one
  sqf::GemmArgs ga{a->x_low, a->s_x, (const uint8_t*)a->x_out, a->s_xo, w->w_low, w->s_w,
                   (const uint8_t*)w->w_out, w->s_wo, (float*)y, acc_low_dbg, row_off, a->m, w->n,
                   w->ldk, ldo_b, ldy, w->n * w->ldk, w->n * ldo_b, w->n,
                   (int32_t)(w->ldk / 64), (int32_t)(ldo_b / 64), (int32_t)groups};
  const char* env = getenv("SQF_GEMM_TILE");
  int cfg = (a->m / groups >= 384) ? 0 : 1;
  if (env && (atoi(env) == 0 || atoi(env) == 1)) cfg = atoi(env);
  if (w->branch == SQF_FP8_E4M3) cfg = 1;
  return hip_status(sqf::launch_dual_gemm(ga, w->branch, true, acc_low_dbg != nullptr, cfg,
                                          (hipStream_t)stream, ybf16),
                    who);
}

}  // namespace

extern "C" {

int sqf_abi_version(void) { return SQF_ABI_VERSION; }

const char* sqf_last_error(void) { return g_err.c_str(); }

int64_t sqf_pad_k_low(int64_t k_low) {
  if (k_low < 0) return -1;
  return (k_low + 255) / 256 * 256;
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
  if (!x_cal || !w || !map_out || !score_out)
    return fail(SQF_ERR_INVALID_ARG, "%s: x_cal, w, map_out and score_out are required", who);
  if (m_cal < 1 || n < 1 || k < 1 || k > 1048576)
    return fail(SQF_ERR_SHAPE, "%s: need m_cal>=1, n>=1, 1<=k<=1048576 (got %lld, %lld, %lld)",
                who, (long long)m_cal, (long long)n, (long long)k);
  if (k_out < 0 || k_out > k)
    return fail(SQF_ERR_SHAPE, "%s: k_out=%lld outside [0, k=%lld]", who, (long long)k_out,
                (long long)k);
  if (k_out > 0 && !idx_out) return fail(SQF_ERR_INVALID_ARG, "%s: idx_out is NULL", who);
  return hip_status(sqf::launch_select(x_cal, m_cal, k, w, n, k_out, idx_out, map_out, score_out,
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
                  wt->sq_nnz, wt->w_low, wt->s_w, (uint8_t*)wt->w_out, wt->s_wo, wt->sq_val,
                  wt->s_w8, wt->sq_tile_off};
  return hip_status(sqf::launch_pack(a, wt->branch, wt->groups, (hipStream_t)stream), who);
}

sqf_status sqf_quantize_split_act(const void* x, int32_t x_dtype, int64_t ldx, const int32_t* map,
                                  sqf_acts* a, void* stream) {
  return quantize_common(x, x_dtype, ldx, 1, nullptr, map, a, false, stream,
                         "sqf_quantize_split_act");
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
  return dual_gemm_impl(a, w, y, false, ldy, acc_low_dbg, acc_sp_dbg, acc_out_dbg, stream,
                        "sqf_dual_gemm");
}

sqf_status sqf_dual_gemm_y(const sqf_acts* a, const sqf_weights* w, void* y, int32_t y_dtype,
                           int64_t ldy, void* stream) {
  g_err.clear();
  const char* who = "sqf_dual_gemm_y";
  if (y_dtype != SQF_F32 && y_dtype != SQF_BF16)
    return fail(SQF_ERR_INVALID_ARG, "%s: y_dtype %d is neither SQF_F32 nor SQF_BF16", who, y_dtype);
  return dual_gemm_impl(a, w, y, y_dtype == SQF_BF16, ldy, nullptr, nullptr, nullptr, stream, who);
}

sqf_status sqf_dual_gemm_grouped(const sqf_acts* a, const sqf_weights* w, int64_t groups,
                                 const int64_t* row_off, float* y, int64_t ldy,
                                 int32_t* acc_low_dbg, void* stream) {
  g_err.clear();
  return grouped_impl(a, w, groups, row_off, y, false, ldy, acc_low_dbg, stream,
                      "sqf_dual_gemm_grouped");
}

sqf_status sqf_dual_gemm_grouped_y(const sqf_acts* a, const sqf_weights* w, int64_t groups,
                                   const int64_t* row_off, void* y, int32_t y_dtype, int64_t ldy,
                                   void* stream) {
  g_err.clear();
  const char* who = "sqf_dual_gemm_grouped_y";
  if (y_dtype != SQF_F32 && y_dtype != SQF_BF16)
    return fail(SQF_ERR_INVALID_ARG, "%s: y_dtype %d is neither SQF_F32 nor SQF_BF16", who, y_dtype);
  return grouped_impl(a, w, groups, row_off, y, y_dtype == SQF_BF16, ldy, nullptr, stream, who);
}

}  // extern "C"
