// sqf_launch.h -- internal launch interface between the C ABI (sqf_api.hip)
// and the kernel translation units.  Not installed, not part of the ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sqf {

struct PackArgs {
  const float* w;      // [groups][k][n]
  const int32_t* map;  // [groups][k]
  const float* hdiag;  // [k] (weight-side format)
  int64_t k, n, k_low, k_out, ldk, ldo, nnz;
  uint8_t* w_low;
  float* s_w;
  uint8_t* w_out;
  float* s_wo;
  int8_t* sq_val;
  float* s_w8;
  int32_t* tile_off;
};

struct ActArgs {
  const void* x;
  int64_t ldx;
  const int32_t* map;  // [groups][k]
  const int64_t* row_off;
  int64_t m, k, k_low, k_out, pad_lo, ldk, ldo;
  int32_t groups;
  uint8_t* x_low;
  float* s_x;
  uint8_t* x_out;
  float* s_xo;
};

struct GemmArgs {
  const uint8_t* x_low;
  const float* s_x;
  const uint8_t* x_out;
  const float* s_xo;
  const uint8_t* w_low;
  const float* s_w;
  const uint8_t* w_out;
  const float* s_wo;
  float* y;
  int32_t* acc_dbg;
  const int64_t* row_off;  // grouped: [groups+1]
  int64_t m, n, ldk, ldo_b, ldy;
  int64_t w_stride_low, w_stride_out, w_stride_s;  // per-group strides (bytes, bytes, elems)
  int32_t s_low, s_out, groups;  // 64-byte K stages of the low / branch operands
};

struct SqArgs {
  const uint8_t* x_low;  // int8 [m][ldkx]
  const float* s_x;
  const uint8_t* x_out;  // int8 [m][ldo]
  const float* s_xo;
  const uint8_t* w_low;  // int4 [n][ldkw]
  const float* s_w4;
  const int8_t* sq_val;  // [n][nnz]
  const float* s_w8;
  const int32_t* tile_off;  // [n][tiles+1]
  const uint8_t* w_out;     // int8 [n][ldo]
  const float* s_wo;
  float* y;
  int32_t* dbg_low;
  int32_t* dbg_sp;
  int32_t* dbg_o;
  int64_t m, n, ldkx, ldkw, ldo, ldy, nnz;
  int32_t s_low, s_out;
};

hipError_t launch_select(const float* x_cal, int64_t m_cal, int64_t k, const float* w, int64_t n,
                         int64_t k_out, int32_t* idx, int32_t* map, double* score, float* hdiag,
                         hipStream_t s);
hipError_t launch_pack(const PackArgs& a, int branch, int groups, hipStream_t s);
hipError_t launch_act_split(const ActArgs& a, int x_dtype, int low, int branch, bool grouped,
                            hipStream_t s);
// dynamic LDS bytes the activation kernel needs for one block
size_t act_split_lds_bytes(int64_t ldk, int64_t k_out);
// cfg: 0 = 256x256 tiles (8 waves), 1 = 128x128 (4 waves), 2 = 64x64 (4 waves)
// ybf16: Y written as bf16 (not together with debug)
hipError_t launch_dual_gemm(const GemmArgs& a, int branch, bool grouped, bool debug, int cfg,
                            hipStream_t s, bool ybf16);
hipError_t launch_sq_gemm(const SqArgs& a, bool debug, hipStream_t s);

}  // namespace sqf
