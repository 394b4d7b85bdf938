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
  int64_t bank;      // weight-side format: slots per bank (0 = the whole row)
  int64_t rows_pad;  // K-blocked layouts: rows of each K block (0 otherwise)
  uint8_t* w_low;
  float* s_w;
  uint8_t* s_wb;  // MXFP4: E8M0 block scales, K-blocked [pad/128][rows_pad/64][4][16][4]
  uint8_t* w_out;
  float* s_wo;
  int8_t* sq_val;
  float* s_w8;
};

struct ActArgs {
  const void* x;
  int64_t ldx;
  const int32_t* map;  // [groups][k]
  const int64_t* row_off;
  int64_t m, k, k_low, k_out, pad_lo, ldk, ldo;
  int64_t rows_pad;  // K-blocked 6-bit layout: rows of each K block (0 otherwise)
  int32_t groups;
  uint8_t* x_low;
  float* s_x;
  uint8_t* x_out;
  float* s_xo;
  uint8_t* s_xb;  // MXFP4: E8M0 block scales, K-blocked [pad/128][rows_pad/64][4][16][4]
  const float* gamma;  // fused RMS norm: [k] weights (NULL: no norm)
  float eps;
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
  const uint8_t* w_out;  // int8 [n][ldo]
  const float* s_wo;
  float* y;
  int32_t* dbg_low;
  int32_t* dbg_sp;
  int32_t* dbg_o;
  int64_t m, n, ldkx, ldkw, ldo, ldy, nnz;
  int32_t s_low, s_out;
  // NULL: the GEMM decodes each stage itself; else the call's workspace of
  // sq_image_bytes(n, ldkw, fp) bytes, which the decode fills first (once
  // per call) and the GEMM then reads
  uint8_t* dec;
};

// The dual GEMM with int4 codes in 6-bit E2M3 fields (K-blocked) and a bf16
// branch, on the FP6 matrix unit; one 256 x 256 tile shape.
struct Gemm6Args {
  const uint8_t* x6;     // K-blocked low codes: E2M3 [s_low][x_rows][96] or E2M1 [s_low][x_rows][64]
  const float* s_x;      // E2M3: per-token scale
  const uint8_t* x_sc;   // E2M1: E8M0 block scales [s_low][x_rows/64][4][16][4]
  const uint8_t* x_out;  // bf16 [m][ldo]
  const uint8_t* w6;
  const float* s_w;
  const uint8_t* w_sc;
  const uint8_t* w_out;  // bf16 [n][ldo]
  float* y;
  int32_t* acc_dbg;
  int64_t m, n, x_rows, w_rows, ldo_b, ldy;
  int32_t s_low, s_br;  // 128-slot low stages, 32-channel branch stages
};

hipError_t launch_select(const float* x_cal, int64_t m_cal, int64_t k, const float* w, int64_t n,
                         int64_t k_out, int32_t* idx, int32_t* map, double* score, float* hdiag,
                         hipStream_t s);
hipError_t launch_pack(const PackArgs& a, int branch, int low, int groups, hipStream_t s);
// ragged: k, ldx or x not aligned to 8-channel chunks; element-wise loads
// norm: RMS-normalise each row with a.gamma / a.eps first (fused)
hipError_t launch_act_split(const ActArgs& a, int x_dtype, int low, int branch, bool grouped,
                            bool ragged, bool norm, hipStream_t s);
// dynamic LDS bytes the activation kernel needs for one block
size_t act_split_lds_bytes(int64_t ldk, int64_t k_out, int low, int64_t norm_k);
// cfg: 0 = 256x256 tiles (8 waves), 1 = 128x128 (4 waves), 2 = 64x64 (4 waves)
// ybf16: Y written as bf16 (not together with debug)
hipError_t launch_dual_gemm(const GemmArgs& a, int branch, bool grouped, bool debug, int cfg,
                            hipStream_t s, bool ybf16);
hipError_t launch_sq_gemm(const SqArgs& a, bool debug, bool fp, hipStream_t s);
// Workspace bytes of the decoded stage images of an n-row weight-side operand
// with ldkw bytes per row.
int64_t sq_image_bytes(int64_t n, int64_t ldkw, bool fp);
// low: kI4E2M3 (int4 codes as E2M3 subnormals, exact sums; debug dumps them)
// or kMXFP4 (E2M1 with E8M0 block scales; no debug output)
hipError_t launch_gemm6(const Gemm6Args& a, int low, bool debug, bool ybf16, hipStream_t s);

// slot order of a channel map (perm[p] = channel at position p) and the
// slice map of the reordered axis
hipError_t launch_slot_order(const int32_t* map, int64_t k, int32_t* perm, int32_t* slice_map,
                             hipStream_t s);
// gather along one axis of a row-major fp32 matrix by perm (axis 1: columns,
// axis 0: rows)
hipError_t launch_permute(const float* src, int64_t rows, int64_t cols, int64_t ld_src,
                          const int32_t* perm, int axis, float* dst, int64_t ld_dst, hipStream_t s);

}  // namespace sqf
