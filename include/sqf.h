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
 *          SQF_I4_E2M3 holds the same int4 codes, each in a 6-bit OCP E2M3
 *          field read as a subnormal (value code/8: field = sign << 5 | |code|),
 *          32 slots per 24 bytes (slot i of a 32-group at bits 6i..6i+5,
 *          little-endian), K-blocked with P = sqf_pad_rows(m): for K block
 *          kb (slots 128kb..128kb+127) and rows 32p..32p+31 the 3072 bytes at
 *          (kb*P/32 + p)*3072 hold, for row r of them (h = (r/16)%2, lane =
 *          16g + r%16, g the 32-slot group), bytes 0..15 of its 24 at
 *          h*1024 + 16*lane and bytes 16..23 at 2048 + 16*lane + 8h (the
 *          6-bit matrix unit's lane order).  Rows beyond m are never written
 *          and never reach an output.
          SQF_MXFP4 holds OCP MXFP4 ([OSC] abstract: the low path on 4-bit
 *          micro-scaling hardware): every 32 slots 32b..32b+31 of a row are
 *          one block of E2M1 codes (sign bit 3, exponent bits 2..1 with bias
 *          1, mantissa bit 0) sharing one E8M0 scale byte (value 2^(s-127)).
 *          Codes two per byte (slot 2i in the low nibble), K-blocked
 *          [ldk/64][P/16][4][16][16]: the 16 bytes of slot group g (slots
 *          32g..32g+31) of K block kb of row r at
 *          (((kb*P/16 + r/16)*4 + g)*16 + r%16)*16.  Scales K-blocked
 *          [ldk/64][P/64][4][16][4]: the scale of that block of row r at
 *          (((kb*P/64 + r/64)*4 + g)*16 + r%16)*4 + (r/16)%4 (s_xb / s_wb).
 *   w_low  [n][ldk] bytes: int4 codes, same packings (SQF_I4_E2M3 and
 *          SQF_MXFP4: K-blocked with P = sqf_pad_rows(n));
 *          nibble 0x8 is the reserved "high precision here" mark
 *          (weight-side format only; in the floating-point form, SQF_FP4_E2M1,
 *          the mark is 0x8 = E2M1 -0, which the encoder never produces).
 *   x_out  [m][ldo], w_out [n][ldo]: branch operands (bf16, E4M3 or int8).
 *   Y      [m][ldy] fp32.
 *   Low slots are padded to sqf_pad_k_low(k_low) (a multiple of 256); branch
 *   rows to sqf_pad_k_out(k_out, dtype) elements (128 bytes per stage).
 *
 * Quantisation: symmetric, per token (activations) and per output channel
 * (weights): a = max|v| over the vector, inv = Q/a in fp32, code =
 * clamp(rint(v*inv), -Q, Q), scale = a/Q; a = 0 gives codes 0, scale 0.
 * MXFP4 instead quantises each 32-slot block of a row: X = floor(log2
 * max|v|) - 2 clamped to >= -127 (an all-zero block: -127), scale byte X+127,
 * code = the E2M1 value nearest v / 2^X (ties to the even code, saturating
 * at 6).
 * Q = 7 (int4), 127 (int8); E4M3 codes are the nearest-even E4M3 value of
 * v*448/a, saturated.  The low absmax excludes the outlier channels (and the
 * marked weight positions).  The bf16 branch is unscaled (round to nearest
 * even); E4M3 / int8 branches carry per-token and per-output-channel scales.
 * Output:  y = s_x[m]*s_w[n]*acc_low (+ s_x[m]*s_w8[n]*acc_sp)
 *              + (s_xo[m]*s_wo[n]) * acc_out           (bf16: s = 1)
 *          MXFP4: y = sum_j 2^Xx(j/32) e2m1(cx_j) * 2^Xw(j/32) e2m1(cw_j)
 *              + acc_out  (fp32 sums, not exact)
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

#define SQF_ABI_VERSION 6

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
  SQF_I4X2 = 4,    /* two int4 codes per byte */
  SQF_I4_E2M3 = 5, /* int4 codes, one per 6-bit E2M3 field, K-blocked (see above) */
  SQF_MXFP4 = 6,   /* OCP MXFP4: E2M1 codes + one E8M0 scale per 32 slots */
  SQF_FP4_E2M1 = 7 /* OCP E2M1 codes packed like SQF_I4X2, one scale per row
                      (the floating-point weight-side format) */
} sqf_dtype;

/* GEMM tile choice of the *_ex calls.  SQF_TILE_AUTO picks by problem size;
 * the others force 256x256, 128x128 or 64x64 output tiles (the E4M3 branch
 * and the SQF_I4_E2M3 / SQF_MXFP4 low paths have one tile shape each: a
 * forced tile they do not have returns SQF_ERR_UNSUPPORTED). */
typedef enum {
  SQF_TILE_AUTO = -1,
  SQF_TILE_256 = 0,
  SQF_TILE_128 = 1,
  SQF_TILE_64 = 2
} sqf_tile;

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
  int32_t low;    /* SQF_I4X2 | SQF_I4_E2M3 | SQF_MXFP4 | SQF_FP4_E2M1 (the
                     floating-point weight-side format) */
  int32_t reserved0;
  uint8_t* w_low; /* [groups][n][ldk] int4 codes (see the layouts above) */
  float* s_w;     /* [groups][n] low scale (s_w4 of the weight-side format);
                     unused (may be NULL) for SQF_MXFP4 */
  uint8_t* s_wb;  /* SQF_MXFP4 only: E8M0 block scales, K-blocked (see above),
                     16-byte aligned */
  void* w_out;    /* [groups][n][ldo] branch codes; NULL when k_out == 0 */
  float* s_wo;    /* [groups][n] branch scale; NULL for SQF_BF16 */
  /* weight-side SQ-format ([SQF-art] 六, 七, 九): sq_nnz > 0 marks, per
   * output row, the most important low slots of every bank with nibble 0x8
   * and stores their int8 values in ascending slot order.  groups must be 1,
   * low SQF_I4X2. */
  int64_t sq_nnz;  /* 0 = channel-split (OSC) format; else marked slots per
                      row, an equal share in every bank */
  int64_t sq_bank; /* slots per bank: 0 (or k_low) = the whole row is one
                      bank; else a multiple of 64, at most 1024, that
                      divides k_low, with sq_nnz a multiple of the bank count
                      k_low / sq_bank: sq_nnz * sq_bank / k_low marks in
                      every bank (SQF_ERR_SHAPE otherwise; larger banks
                      SQF_ERR_UNSUPPORTED) */
  int8_t* sq_val;  /* [n][sq_nnz], 16-byte aligned, in ascending slot order
                      (so bank by bank) */
  float* s_w8;     /* [n] scale of sq_val */
} sqf_weights;

/* Quantised activations, caller-allocated. */
typedef struct sqf_acts {
  int64_t m;      /* token rows */
  int64_t k_low;  /* low channels */
  int64_t k_out;  /* outlier channels */
  int64_t ldk;    /* bytes per x_low row: pad/2 (SQF_I4X2) or pad (SQF_I8) */
  int64_t ldo;    /* elements per x_out row */
  int32_t low;    /* SQF_I4X2 | SQF_I8 (weight-side format only) |
                     SQF_I4_E2M3 | SQF_MXFP4 | SQF_FP8_E4M3 (E4M3 codes, one
                     per byte, ldk = pad: the floating-point weight-side
                     format, with an SQF_FP8_E4M3 branch) */
  int32_t branch; /* SQF_BF16 | SQF_FP8_E4M3 | SQF_I8 */
  uint8_t* x_low; /* [m][ldk], or K-blocked for SQF_I4_E2M3 (see above) */
  float* s_x;     /* [m]; unused (may be NULL) for SQF_MXFP4 */
  uint8_t* s_xb;  /* SQF_MXFP4 only: E8M0 block scales, K-blocked (see above),
                     16-byte aligned */
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

/* Row count of the K-blocked SQF_I4_E2M3 arrays: round_up(rows, 256); 0
 * stays 0; -1 if rows < 0. */
int64_t sqf_pad_rows(int64_t rows);

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
 * score_out [k] or NULL, hdiag_out [k] or NULL.  The scores double as the
 * call's workspace; with score_out == NULL the call takes k doubles from
 * the stream-ordered allocator (hipMallocAsync on `stream`) and returns
 * them (hipFreeAsync) before it returns.  Asynchronous on `stream` either
 * way; k <= 1048576, m_cal >= 1, 0 <= k_out <= k. */
sqf_status sqf_select_channels(const float* x_cal, int64_t m_cal, int64_t k, const float* w,
                               int64_t n, int64_t k_out, int32_t* idx_out, int32_t* map_out,
                               double* score_out, float* hdiag_out, void* stream);

/* a0 without allocation, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same channel choice and outputs as sqf_select_channels
 * (bit for bit), with the scores kept in a static array of the library
 * (65536 fp64 values per GPU, held until the process ends) instead of
 * score_out or a stream-ordered workspace.  No call allocates or frees
 * memory.  k <= 65536, else SQF_ERR_SHAPE; other checks and the asynchrony
 * as sqf_select_channels; `stream` must belong to the current device.  Every
 * call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (other streams, other threads) race and must be ordered by the caller. */
sqf_status sqf_select_channels_noalloc(const float* x_cal, int64_t m_cal, int64_t k,
                                       const float* w, int64_t n, int64_t k_out, int32_t* idx_out,
                                       int32_t* map_out, float* hdiag_out, void* stream);

/* a1 -- offline weight conversion.  w: [groups][k][n] fp32, map: [groups][k]
 * (one map per group).  Fills every array of `wt` (shape fields must be set
 * and consistent with map).  Channel-split format ([OSC]): per output row,
 * the low channels' values in slot order are quantised to int4, the outlier
 * channels' values stored in the branch type.  Weight-side format
 * (wt->sq_nnz > 0, [SQF-art] 六, 七, 九: banks of sq_bank slots, the same
 * count of high-precision values in each): hdiag [k] required, branch must
 * be SQF_I8, low SQF_I4X2; in every bank of every output row the
 * sq_nnz / banks slots with the largest w^2 * hdiag (ties: lower slot) are
 * marked 0x8 and kept as int8 (one scale s_w8 per row over all its marked
 * values), the others quantised to int4 with an absmax over the unmarked
 * slots.  Floating-point weight-side format ([SQF-art] 八: FP8 high, FP4
 * low): low SQF_FP4_E2M1 and an SQF_FP8_E4M3 branch; the same marks, the
 * kept values as E4M3 codes of v*448/a8 (s_w8 = a8/448, sq_val holds the
 * E4M3 bytes), the others as E2M1 codes of v*6/a4 (s_w = a4/6), the branch
 * E4M3 per row; it pairs with E4M3 activations (low SQF_FP8_E4M3, per-token
 * scale a/448) and its GEMM has fp32 sums (no debug outputs).  SQF_I4_E2M3 weights hold the channel-split int4 codes in the
 * K-blocked 6-bit layout; SQF_MXFP4 weights quantise each 32-slot block of
 * a row's low values to E2M1 with a shared E8M0 scale (OCP MX), K-blocked.
 * Both need groups == 1 and a bf16 branch. */
sqf_status sqf_pack_weights(const float* w, const int32_t* map, const float* hdiag,
                            sqf_weights* wt, void* stream);

/* a2 -- online per-token quantisation + outlier extraction ([OSC]
 * structured sub-tensor extraction).  x: [a->m][ldx] of x_dtype (SQF_F32 |
 * SQF_BF16), 1 <= k = a->k_low + a->k_out <= 65536, ldx >= k.  One pass over
 * x writes x_low, s_x (or s_xb for SQF_MXFP4), x_out (and s_xo).  A k or
 * ldx that is not a multiple of 8, or an x that is not 16-byte aligned,
 * takes a slower element-wise load path with the same results. */
sqf_status sqf_quantize_split_act(const void* x, int32_t x_dtype, int64_t ldx, const int32_t* map,
                                  sqf_acts* a, void* stream);

/* Producer-side reordering ([SQF-art] 九: weight columns reordered by the
 * importance mask).  sqf_slot_order: from a channel map [k] (device),
 * perm_out[p] = the channel at position p of the slot order (the low
 * channels in slot order, then the outlier channels in branch order) and
 * slice_map_out [k] = the map of the reordered axis (p for p < k_low,
 * -(p - k_low + 1) after), with which the split is a slice.  Reordering the
 * producer's output channels (its weight columns and its norm's gamma) and
 * the consumer's input channels (the rows of W) by perm leaves every product
 * unchanged: the packed weights, the quantised activations and Y are the
 * same bit for bit.  1 <= k <= 1048576; the map must be a valid channel map.
 * sqf_permute_channels: dst = src gathered along one axis of a row-major
 * fp32 matrix [rows][cols]: axis 1, dst[r][p] = src[r][perm[p]]; axis 0,
 * dst[p][j] = src[perm[p]][j] (perm has cols resp. rows entries); src and
 * dst distinct, ld >= cols.  Both asynchronous on `stream`. */
sqf_status sqf_slot_order(const int32_t* map, int64_t k, int32_t* perm_out, int32_t* slice_map_out,
                          void* stream);
sqf_status sqf_permute_channels(const float* src, int64_t rows, int64_t cols, int64_t ld_src,
                                const int32_t* perm, int32_t axis, float* dst, int64_t ld_dst,
                                void* stream);

/* a2 fused with the norm in front of it (producer-side fusion): each row is
 * RMS-normalised, xn[c] = (x[c] * r) * gamma[c] in fp32 with r = 1 /
 * sqrt(mean_c x[c]^2 + eps) (the mean of squares in fp64, r rounded once to
 * fp32), and xn is split and quantised exactly as sqf_quantize_split_act
 * would quantise it (the norm that precedes the linear layers of the
 * Llama / Qwen models is RMSNorm; [OSC] structured sub-tensor extraction).
 * gamma: [k] fp32 device array, 4-byte aligned; 0 <= eps <= 1.  Bf16 branch
 * and SQF_I4X2 / SQF_I4_E2M3 low codes only (SQF_ERR_UNSUPPORTED otherwise);
 * gamma is staged in LDS, so k is bounded by the kernel's LDS budget
 * (SQF_ERR_SHAPE beyond it; about 30000 channels).  Other arguments and
 * errors as sqf_quantize_split_act. */
sqf_status sqf_rmsnorm_quantize_split_act(const void* x, int32_t x_dtype, int64_t ldx,
                                          const float* gamma, float eps, const int32_t* map,
                                          sqf_acts* a, void* stream);

/* a3-a5 (and the weight-side masked path) -- the fused dual GEMM.
 * y: [a->m][ldy] fp32, ldy >= n.  The low path runs on int8 MFMA with exact
 * int32 accumulation (SQF_I4X2: int4 codes unpacked in registers), on the
 * FP6 matrix unit with exact sums (SQF_I4_E2M3) or on the FP4 matrix unit
 * with the block scales applied per product (SQF_MXFP4, no debug output:
 * SQF_ERR_UNSUPPORTED); the branch on bf16 / FP8 / int8 MFMA; the epilogue
 * applies the scales and sums the paths ([SQF-art] 三 two paths and fusion;
 * [OSC] result fusion).
 * Debug outputs (NULL in normal use) receive the exact int32 accumulators
 * [m][n] (row stride n): acc_low_dbg (low path), acc_sp_dbg (weight-side
 * masked path), acc_out_dbg (int8 branch only). */
sqf_status sqf_dual_gemm(const sqf_acts* a, const sqf_weights* w, float* y, int64_t ldy,
                         int32_t* acc_low_dbg, int32_t* acc_sp_dbg, int32_t* acc_out_dbg,
                         void* stream);

/* a7 with the gather done once per call ([SQF-art] 三 and 七: the gather
 * unit feeds the sparse high-precision values to the matrix units; 九: the
 * format).  The same product, accumulators and Y as sqf_dual_gemm on
 * weight-side (sq_nnz > 0) weights, bit for bit in the integer form (the FP8 /
 * FP4 form sums in fp32 the same way).  The decode of every 128-slot K stage
 * of every 128-row weight tile -- the clean low tile and the sparse tile --
 * is written once into `workspace` by a first kernel, and the GEMM then
 * reads the decoded tiles instead of decoding each stage in every
 * 256-row activation tile; for m above a few hundred rows this is the faster
 * call.  workspace: device memory of at least sqf_sq_workspace_bytes(w)
 * bytes, 256-byte aligned, owned by the caller, overwritten by the call and
 * free again once the call's work on `stream` is done (calls that share a
 * workspace must be ordered).  Errors: SQF_ERR_INVALID_ARG for weights
 * without the weight-side format or a NULL workspace, SQF_ERR_ALIGN,
 * SQF_ERR_SHAPE for a workspace that is too small; the rest as
 * sqf_dual_gemm.  Asynchronous on `stream`. */
int64_t sqf_sq_workspace_bytes(const sqf_weights* w); /* -1: not weight-side weights */
sqf_status sqf_dual_gemm_sq_ws(const sqf_acts* a, const sqf_weights* w, float* y, int64_t ldy,
                               void* workspace, int64_t workspace_bytes, int32_t* acc_low_dbg,
                               int32_t* acc_sp_dbg, int32_t* acc_out_dbg, void* stream);

/* Grouped (mixture-of-experts) variants ([OSC] abstract: evaluation on the
 * Qwen3 mixture-of-experts model, whose experts each see their own tokens;
 * the FP8 fallback is for the input of the experts' down projection W2):
 * rows of group g are
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

/* The dual GEMM with every option explicit: the output type (as
 * sqf_dual_gemm_y), the tile (sqf_tile) and the debug accumulators (as
 * sqf_dual_gemm; SQF_F32 output only).  sqf_dual_gemm, sqf_dual_gemm_y and
 * their grouped forms are this call with SQF_TILE_AUTO.  No call reads the
 * environment or any other process-wide setting. */
sqf_status sqf_dual_gemm_ex(const sqf_acts* a, const sqf_weights* w, void* y, int32_t y_dtype,
                            int64_t ldy, int32_t tile, int32_t* acc_low_dbg, int32_t* acc_sp_dbg,
                            int32_t* acc_out_dbg, void* stream);
sqf_status sqf_dual_gemm_grouped_ex(const sqf_acts* a, const sqf_weights* w, int64_t groups,
                                    const int64_t* row_off, void* y, int32_t y_dtype, int64_t ldy,
                                    int32_t tile, int32_t* acc_low_dbg, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SQF_H_ */
