/*
 * sqf.h -- C ABI of libsqf, the MI355X (gfx950) outlier-separated dual-path
 * GEMM:   Y = Xlow(int4) . Wlow(int4)  +  Xout(high precision) . Wout(high precision)
 *
 * The method (cited by page title and section):
 *   [SQF-art] SQ-format press article (91haoming.cn): section 二 (weight and
 *             activation selection strategies), 三 (two parallel paths; the
 *             low part keeps its dense layout and a reserved mask value marks
 *             high-precision positions), 五 (static activation strategy,
 *             calibration, no online top-k), 九 (format definition, reserved
 *             code, banked top-(1-s) selection, column reordering).
 *   [SQF-abs] "SQ-format: A Unified Sparse-Quantized Hardware-friendly Data
 *             Format for LLMs", abstract.
 *   [OSC]     "OSC: Hardware Efficient W4A4 Quantization via Outlier
 *             Separation in Channel Dimension", abstract and method framework
 *             (offline channel identification, online structured sub-tensor
 *             extraction, 4-bit GEMM + 16-bit branch GEMM, result fusion,
 *             FP8 fallback for the down-projection input).
 *
 * Layout conventions (all row-major):
 *   X      [m][ldx]  activations, fp32 or bf16, token rows.
 *   W      [k][n]    fp32 weights, input-channel rows (Y = X . W).
 *   map    [k] int32 channel map: map[c] = j >= 0 -> low slot j (low channels
 *          keep ascending channel order); map[c] = -(t+1) -> outlier slot t
 *          (outliers ascending).  Produced by sqf_select_channels.
 *   x_low  [m][ldk] bytes: int4 codes in [-7,7], two's complement, slot 2i in
 *          the low nibble of byte i, slot 2i+1 in the high nibble (SQF_I4X2);
 *          or one int8 code per byte (SQF_I8).  Padding slots are 0.
 *   w_low  [n][ldk] bytes: int4 codes, same packing; nibble 0x8 is the
 *          reserved "high precision here" mark (weight-side format only).
 *   x_out  [m][ldo], w_out [n][ldo]: branch operands (bf16, E4M3 or int8).
 *   Y      [m][ldy] fp32.
 *   Low slots are padded to sqf_pad_k_low(k_low) (a multiple of 256); branch
 *   rows to sqf_pad_k_out(k_out, dtype) elements (128 bytes per stage).
 *
 * Quantisation: symmetric, per token (activations) and per output channel
 * (weights): a = max|v| over the vector, inv = Q/a in fp32, code =
 * clamp(rint(v*inv), -Q, Q), scale = a/Q; a = 0 gives codes 0, scale 0.
 * Q = 7 (int4), 127 (int8); E4M3 codes are the nearest-even E4M3 value of
 * v*448/a, saturated.  The low absmax excludes the outlier channels (and the
 * marked weight positions).  The bf16 branch is unscaled (round to nearest
 * even); E4M3 / int8 branches carry per-token and per-output-channel scales.
 * Output:  y = s_x[m]*s_w[n]*acc_low (+ s_x[m]*s_w8[n]*acc_sp)
 *              + (s_xo[m]*s_wo[n]) * acc_out           (bf16: s = 1)
 *
 * Ownership: every buffer is caller-allocated device memory unless stated;
 * the library keeps no pointer after a call returns and allocates nothing.
 * Streams: `stream` is a hipStream_t (NULL = default stream); every call is
 * asynchronous on it.  Errors: arguments are validated on the host before
 * any launch; a failing call returns a non-zero sqf_status, launches nothing
 * and sets a thread-local message (sqf_last_error).  A HIP launch failure is
 * SQF_ERR_HIP.  Inputs must be finite; NaN / Inf give unspecified output.
 * Calls on different streams may run concurrently; calls that share output
 * buffers must be ordered by the caller.
 */
#ifndef SQF_H_
#define SQF_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SQF_ABI_VERSION 1

typedef enum {
  SQF_OK = 0,
  SQF_ERR_INVALID_ARG = 1, /* null pointer, bad enum, inconsistent descriptor */
  SQF_ERR_SHAPE = 2,       /* size out of range or leading dimension too small */
  SQF_ERR_UNSUPPORTED = 3, /* valid request this build does not implement */
  SQF_ERR_HIP = 4,         /* HIP runtime error (text in sqf_last_error) */
  SQF_ERR_ALIGN = 5        /* pointer or leading dimension misaligned */
} sqf_status;

typedef enum {
  SQF_F32 = 0,
  SQF_BF16 = 1,
  SQF_FP8_E4M3 = 2, /* OCP E4M3 (max 448, no infinities) */
  SQF_I8 = 3,
  SQF_I4X2 = 4 /* two int4 codes per byte */
} sqf_dtype;

/* Quantised weights, caller-allocated.  `groups` weight sets of identical
 * shape may be stacked back to back (grouped GEMM); every array then gains a
 * leading [groups] dimension. */
typedef struct sqf_weights {
  int64_t k;      /* input channels */
  int64_t n;      /* output channels */
  int64_t k_low;  /* low channels, k - k_out */
  int64_t k_out;  /* outlier channels */
  int64_t ldk;    /* bytes per w_low row = sqf_pad_k_low(k_low) / 2 */
  int64_t ldo;    /* elements per w_out row = sqf_pad_k_out(k_out, branch) */
  int32_t branch; /* SQF_BF16 | SQF_FP8_E4M3 | SQF_I8 */
  int32_t groups; /* >= 1 */
  uint8_t* w_low; /* [groups][n][ldk] int4 codes */
  float* s_w;     /* [groups][n] low scale (s_w4 of the weight-side format) */
  void* w_out;    /* [groups][n][ldo] branch codes; NULL when k_out == 0 */
  float* s_wo;    /* [groups][n] branch scale; NULL for SQF_BF16 */
  /* weight-side SQ-format ([SQF-art] 九): sq_nnz > 0 marks, per output row,
   * the sq_nnz most important low slots with nibble 0x8 and stores their
   * int8 values in ascending slot order.  groups must be 1. */
  int64_t sq_nnz;       /* 0 = channel-split (OSC) format */
  int8_t* sq_val;       /* [n][sq_nnz], 16-byte aligned */
  float* s_w8;          /* [n] scale of sq_val */
  int32_t* sq_tile_off; /* [n][ldk/128 + 1]: count of marked slots before
                           each 256-slot tile (derived, written by pack) */
} sqf_weights;

/* Quantised activations, caller-allocated. */
typedef struct sqf_acts {
  int64_t m;      /* token rows */
  int64_t k_low;  /* low channels */
  int64_t k_out;  /* outlier channels */
  int64_t ldk;    /* bytes per x_low row: pad/2 (SQF_I4X2) or pad (SQF_I8) */
  int64_t ldo;    /* elements per x_out row */
  int32_t low;    /* SQF_I4X2 | SQF_I8 (SQF_I8 only with weight-side format) */
  int32_t branch; /* SQF_BF16 | SQF_FP8_E4M3 | SQF_I8 */
  uint8_t* x_low; /* [m][ldk] */
  float* s_x;     /* [m] */
  void* x_out;    /* [m][ldo]; NULL when k_out == 0 */
  float* s_xo;    /* [m]; NULL for SQF_BF16 */
} sqf_acts;

/* Version of this header's layouts; a library built from another header
 * returns a different number. */
int sqf_abi_version(void);

/* Text of the last non-OK status returned on the calling thread ("" if none). */
const char* sqf_last_error(void);

/* Padded low-slot count: round_up(k_low, 256); 0 stays 0; -1 if k_low < 0. */
int64_t sqf_pad_k_low(int64_t k_low);

/* Padded branch row length in elements: round_up(k_out, 64) for SQF_BF16,
 * round_up(k_out, 128) for SQF_FP8_E4M3 / SQF_I8 (128 bytes per stage);
 * 0 stays 0; -1 for a bad argument. */
int64_t sqf_pad_k_out(int64_t k_out, int32_t branch);

/* a0 -- offline outlier-channel choice ([SQF-art] 二, 五; [OSC] offline
 * channel identification).  From calibration tokens x_cal [m_cal][k] (fp32)
 * and weights w [k][n] (fp32):
 *   score[c] = (sum_m |x_cal[m,c]| / m_cal) * sqrt(sum_j w[c,j]^2)   (fp64,
 *              both sums taken sequentially in index order)
 *   hdiag[c] = (float) sum_m x_cal[m,c]^2                            (fp64 sum)
 * The k_out channels of highest score (ties: lower index) become outliers.
 * Outputs: idx_out [k_out] ascending (may be NULL if k_out == 0), map_out
 * [k] (required: holds the rank counts until the map is written),
 * score_out [k] (required: also used as workspace), hdiag_out [k] or
 * NULL.  Asynchronous; k <= 1048576, m_cal >= 1, 0 <= k_out <= k. */
sqf_status sqf_select_channels(const float* x_cal, int64_t m_cal, int64_t k, const float* w,
                               int64_t n, int64_t k_out, int32_t* idx_out, int32_t* map_out,
                               double* score_out, float* hdiag_out, void* stream);

/* a1 -- offline weight conversion.  w: [groups][k][n] fp32, map: [groups][k]
 * (one map per group).  Fills every array of `wt` (shape fields must be set
 * and consistent with map).  Channel-split format ([OSC]): per output row,
 * the low channels' values in slot order are quantised to int4, the outlier
 * channels' values stored in the branch type.  Weight-side format
 * (wt->sq_nnz > 0, [SQF-art] 九): hdiag [k] required, branch must be SQF_I8;
 * per output row the sq_nnz low slots with the largest w^2 * hdiag (ties:
 * lower slot) are marked 0x8 and kept as int8 (own scale s_w8), the others
 * quantised to int4 with an absmax over the unmarked slots. */
sqf_status sqf_pack_weights(const float* w, const int32_t* map, const float* hdiag,
                            sqf_weights* wt, void* stream);

/* a2 -- online per-token quantisation + outlier extraction ([OSC]
 * structured sub-tensor extraction).  x: [a->m][ldx] of x_dtype (SQF_F32 |
 * SQF_BF16), k = a->k_low + a->k_out must be a multiple of 8 and at most
 * 65536.  One pass over x writes x_low, s_x, x_out (and s_xo). */
sqf_status sqf_quantize_split_act(const void* x, int32_t x_dtype, int64_t ldx, const int32_t* map,
                                  sqf_acts* a, void* stream);

/* a3-a5 (and the weight-side masked path) -- the fused dual GEMM.
 * y: [a->m][ldy] fp32, ldy >= n.  The low path runs on int8 MFMA with exact
 * int32 accumulation (int4 codes unpacked in registers); the branch on
 * bf16 / FP8 / int8 MFMA; the epilogue applies the scales and sums the paths
 * ([SQF-art] 三 two paths and fusion; [OSC] result fusion).
 * Debug outputs (NULL in normal use) receive the exact int32 accumulators
 * [m][n] (row stride n): acc_low_dbg (low path), acc_sp_dbg (weight-side
 * masked path), acc_out_dbg (int8 branch only). */
sqf_status sqf_dual_gemm(const sqf_acts* a, const sqf_weights* w, float* y, int64_t ldy,
                         int32_t* acc_low_dbg, int32_t* acc_sp_dbg, int32_t* acc_out_dbg,
                         void* stream);

/* Grouped (mixture-of-experts) variants: rows of group g are
 * [row_off[g], row_off[g+1]) of the concatenated activations (row_off: device
 * int64 [groups+1], non-decreasing, row_off[0] = 0, row_off[groups] = a->m).
 * Each group has its own map (maps: [groups][k]) and its own stacked weight
 * set (w->groups == groups).  Channel-split format only. */
sqf_status sqf_quantize_split_act_grouped(const void* x, int32_t x_dtype, int64_t ldx,
                                          int64_t groups, const int64_t* row_off,
                                          const int32_t* maps, sqf_acts* a, void* stream);
sqf_status sqf_dual_gemm_grouped(const sqf_acts* a, const sqf_weights* w, int64_t groups,
                                 const int64_t* row_off, float* y, int64_t ldy,
                                 int32_t* acc_low_dbg, void* stream);

/* The same fused epilogue ([OSC] result fusion) with a choice of output
 * type: y_dtype SQF_F32 (y is float*, as above) or SQF_BF16 (y holds bf16
 * bit patterns, each the round-to-nearest-even of the fp32 value the fp32
 * call writes: half the output bytes, for a consumer that reads bf16).
 * ldy counts elements of y's type.  No debug outputs.  Channel-split format
 * only for SQF_BF16 (the weight-side format returns SQF_ERR_UNSUPPORTED);
 * any other y_dtype returns SQF_ERR_INVALID_ARG. */
sqf_status sqf_dual_gemm_y(const sqf_acts* a, const sqf_weights* w, void* y, int32_t y_dtype,
                           int64_t ldy, void* stream);
sqf_status sqf_dual_gemm_grouped_y(const sqf_acts* a, const sqf_weights* w, int64_t groups,
                                   const int64_t* row_off, void* y, int32_t y_dtype, int64_t ldy,
                                   void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SQF_H_ */
