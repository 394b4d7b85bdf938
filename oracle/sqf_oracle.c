/*
 * sqf_oracle.c -- plain, slow, scalar CPU oracle for the outlier-separated
 * dual-path GEMM (SQ-format / OSC).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the parity reference.  Only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg may load
 * it.  It shares no code, header, table or constant with the GPU library.
 *
 * Sources (cited by page title and section):
 *   [SQF-art]  SQ-format press article (91haoming.cn), sections numbered
 *              二 (two selection strategies), 三 (hardware: two paths, mask
 *              code), 五 (static strategy), 九 (technical details).
 *   [SQF-abs]  "SQ-format: A Unified Sparse-Quantized Hardware-friendly Data
 *              Format for LLMs", abstract.
 *   [OSC-abs]  "OSC: Hardware Efficient W4A4 Quantization via Outlier
 *              Separation in Channel Dimension", abstract and the section
 *              on the method framework.
 *
 * Everything is written as scalar loops, in the order the method states it.
 * Floating point: quantisation decisions are taken in fp32 (the precision
 * the kernels use, so both sides decide integer codes identically); sums
 * and the final output are formed in fp64.  Build flags:
 *   -O2 -fno-fast-math -ffp-contract=off -fopenmp
 *
 * Conventions where the pages are silent (each is a stated reading):
 *   - symmetric quantisation to [-Q, Q] with Q = 7 (int4) or 127 (int8);
 *     the int4 code 0x8 (-8) is never produced by quantisation and is the
 *     reserved "high precision here" mark of the weight-side format;
 *   - inv = Q / absmax as one fp32 division, code = clamp(rint(v*inv)),
 *     scale = absmax / Q as one fp32 division; absmax 0 gives codes 0 and
 *     scale 0;
 *   - ties in any ranking go to the lower index;
 *   - packed int4: slot 2i in the low nibble of byte i, slot 2i+1 in the
 *     high nibble; rows zero-padded to their leading dimension.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_FP8 2
#define ORC_I8 3
#define ORC_I4 4

/* ------------------------------------------------------------------ */
/* Number formats                                                      */
/* ------------------------------------------------------------------ */

static float f32_from_bits(uint32_t b) {
  float f;
  memcpy(&f, &b, 4);
  return f;
}
static uint32_t bits_from_f32(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  return b;
}

/* memset(p, 0, n) that is also defined for n == 0 with p == NULL (an empty
 * array passed from the caller) */
static void zero_bytes(void* p, int64_t n) {
  if (n > 0) memset(p, 0, (size_t)n);
}

/* bf16 -> fp32 is exact: the bf16 pattern is the top half of the fp32 one. */
double orc_bf16_to_double(uint16_t h) { return (double)f32_from_bits((uint32_t)h << 16); }

/* fp32 -> bf16, round to nearest, ties to even mantissa.  Finite inputs. */
uint16_t orc_bf16_from_float(float v) {
  uint32_t b = bits_from_f32(v);
  uint32_t upper = b >> 16, lower = b & 0xFFFFu;
  if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
  return (uint16_t)upper;
}

/* OCP FP8 E4M3 ("fn" variant): 1 sign, 4 exponent bits (bias 7), 3 mantissa
 * bits, no infinities, 0x7F / 0xFF are NaN, largest finite 448 (0x7E).  The
 * value of a non-negative code is computed from that definition. */
double orc_e4m3_to_double(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 0xF, m = c & 7;
  double v;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6); /* subnormal: 0.m * 2^(1-7) */
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

/* fp32 -> E4M3, round to nearest with ties to the even code, saturating to
 * +-448.  Written as a search over every finite non-negative code, which is
 * the definition of round-to-nearest rather than a bit trick. */
uint8_t orc_e4m3_from_float(float v) {
  double a = fabs((double)v);
  int best = 0;
  double best_err = a; /* code 0 has value 0 */
  for (int c = 1; c <= 0x7E; ++c) {
    double err = fabs(orc_e4m3_to_double((uint8_t)c) - a);
    if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
      best = c;
      best_err = err;
    }
  }
  if (a > 448.0) best = 0x7E; /* saturate */
  return (uint8_t)(best | ((v < 0.0f && best != 0) ? 0x80 : 0));
}

/* OCP E2M1 (FP4) conversions, defined with the MXFP4 steps below. */
double orc_e2m1_to_double(uint8_t c);
uint8_t orc_e2m1_from_double(double t);

/* Signed int4 nibble -> code.  0x8 is the reserved mark; it contributes 0 to
 * the dense low-precision product [SQF-art section 三: the low part is
 * consumed by ordinary matrix units, the marked positions by a separate
 * gather of high-precision values]. */
static int nib_code(uint8_t nib) {
  nib &= 0xF;
  if (nib == 0x8) return 0;
  return (nib & 0x8) ? (int)nib - 16 : (int)nib;
}

/* ------------------------------------------------------------------ */
/* Step: symmetric quantisation of one vector                          */
/* ------------------------------------------------------------------ */

/* Quantise v[0..len) symmetrically to [-q, q].  Per-token for activations,
 * per-output-channel for weights.  fmt selects the code type: ORC_I4 / ORC_I8
 * give integer codes clamp(rint(v*inv)); ORC_FP8 gives E4M3 codes of v*inv
 * (q = 448).  Returns the scale; codes[i] receives the signed integer code
 * (int formats) or the raw E4M3 byte (fp8). */
float orc_quantize_vec(const float* v, int64_t len, int fmt, int32_t* codes) {
  int q = fmt == ORC_I4 ? 7 : (fmt == ORC_I8 ? 127 : 448);
  float a = 0.0f;
  for (int64_t i = 0; i < len; ++i) {
    float t = fabsf(v[i]);
    if (t > a) a = t;
  }
  if (a == 0.0f) {
    for (int64_t i = 0; i < len; ++i) codes[i] = 0;
    return 0.0f;
  }
  float inv = (float)q / a;
  for (int64_t i = 0; i < len; ++i) {
    float p = v[i] * inv;
    if (fmt == ORC_FP8) {
      codes[i] = orc_e4m3_from_float(p);
    } else {
      float r = rintf(p);
      if (r > (float)q) r = (float)q;
      if (r < (float)-q) r = (float)-q;
      codes[i] = (int32_t)r;
    }
  }
  return a / (float)q;
}

/* ------------------------------------------------------------------ */
/* Step a0: static outlier-channel selection                           */
/* ------------------------------------------------------------------ */

static const double* g_sort_score;
static int cmp_rank(const void* pa, const void* pb) {
  int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
  double sa = g_sort_score[a], sb = g_sort_score[b];
  if (sa > sb) return -1;
  if (sa < sb) return 1;
  return a < b ? -1 : (a > b ? 1 : 0);
}
static int cmp_i32(const void* pa, const void* pb) {
  int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
  return a < b ? -1 : (a > b ? 1 : 0);
}

/* Channel importance from calibration data [SQF-art sections 二 and 五: mean
 * activation per channel weighted by the channel's contribution through the
 * weights; chosen offline so no online top-k is needed] and [OSC-abs: outlier
 * channels identified offline, token-persistent].
 *   score_c = (sum_m |x[m,c]| / m_cal) * sqrt(sum_n W[c,n]^2)
 * sums in fp64 in index order.  hdiag_c = (float) sum_m x[m,c]^2 (the
 * diagonal of X^T X, used by the weight-side score).  The k_out best channels
 * (score descending, lower index first on ties) are the outliers; idx lists
 * them ascending; map[c] = low slot j >= 0, or -(t+1) for outlier slot t.
 * score / hdiag may be NULL. */
void orc_select_channels(const float* x_cal, int64_t m_cal, int64_t k, const float* w, int64_t n,
                         int64_t k_out, int32_t* idx, int32_t* map, double* score_out,
                         float* hdiag_out) {
  double* score = (double*)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
  for (int64_t c = 0; c < k; ++c) {
    double sa = 0.0, s2 = 0.0, sw = 0.0;
    for (int64_t m = 0; m < m_cal; ++m) {
      double x = (double)x_cal[m * k + c];
      sa += fabs(x);
      s2 += x * x;
    }
    for (int64_t j = 0; j < n; ++j) {
      double t = (double)w[c * n + j];
      sw += t * t;
    }
    double mean_abs = sa / (double)m_cal;
    score[c] = mean_abs * sqrt(sw);
    if (score_out) score_out[c] = score[c];
    if (hdiag_out) hdiag_out[c] = (float)s2;
  }
  int32_t* order = (int32_t*)malloc(sizeof(int32_t) * (size_t)(k > 0 ? k : 1));
  for (int64_t c = 0; c < k; ++c) order[c] = (int32_t)c;
  g_sort_score = score;
  qsort(order, (size_t)k, sizeof(int32_t), cmp_rank);
  for (int64_t t = 0; t < k_out; ++t) idx[t] = order[t];
  qsort(idx, (size_t)k_out, sizeof(int32_t), cmp_i32);
  for (int64_t c = 0; c < k; ++c) map[c] = 0;
  for (int64_t t = 0; t < k_out; ++t) map[idx[t]] = (int32_t)(-(t + 1));
  int32_t j = 0;
  for (int64_t c = 0; c < k; ++c)
    if (map[c] >= 0) map[c] = j++;
  free(order);
  free(score);
}

/* ------------------------------------------------------------------ */
/* Packing helpers                                                     */
/* ------------------------------------------------------------------ */

static void pack_i4_row(const int32_t* codes, int64_t len, uint8_t* row, int64_t ldk) {
  zero_bytes(row, ldk);
  for (int64_t j = 0; j < len; ++j) {
    uint8_t nib = (uint8_t)(codes[j] & 0xF);
    if (j & 1)
      row[j >> 1] |= (uint8_t)(nib << 4);
    else
      row[j >> 1] |= nib;
  }
}

/* Store one branch vector (the outlier slots of a row) in the branch format. */
static float store_branch_row(const float* vals, int64_t k_out, int fmt, void* dst_row,
                              int64_t ldo, int32_t* tmp) {
  float scale = 1.0f;
  if (fmt == ORC_BF16) {
    uint16_t* d = (uint16_t*)dst_row;
    for (int64_t t = 0; t < ldo; ++t) d[t] = t < k_out ? orc_bf16_from_float(vals[t]) : 0;
    return scale;
  }
  scale = orc_quantize_vec(vals, k_out, fmt, tmp);
  uint8_t* d = (uint8_t*)dst_row;
  for (int64_t t = 0; t < ldo; ++t) d[t] = t < k_out ? (uint8_t)(tmp[t] & 0xFF) : 0;
  return scale;
}

/* ------------------------------------------------------------------ */
/* Step a1: weight format (outlier-channel split, OSC-style)          */
/* ------------------------------------------------------------------ */

/* For every output channel nn: the values W[c, nn] of the low channels, in
 * slot order, are quantised per output channel to int4 and packed
 * (w_low[nn][ldk]); the outlier-channel values form the branch row
 * w_out[nn][ldo] in bf16 (no scale), FP8 or int8 (scale s_wo[nn]).
 * [OSC-abs: low-precision 4-bit path plus a high-precision branch over the
 * outlier channels.] */
void orc_pack_weights(const float* w, int64_t k, int64_t n, const int32_t* map, int64_t k_low,
                      int64_t k_out, int64_t ldk, int64_t ldo, int branch_fmt, uint8_t* w_low,
                      float* s_w, void* w_out, float* s_wo) {
  float* lo = (float*)malloc(sizeof(float) * (size_t)(k_low + 1));
  float* hi = (float*)malloc(sizeof(float) * (size_t)(k_out + 1));
  int32_t* codes = (int32_t*)malloc(sizeof(int32_t) * (size_t)(k + 1));
  size_t esz = branch_fmt == ORC_BF16 ? 2 : 1;
  for (int64_t nn = 0; nn < n; ++nn) {
    for (int64_t c = 0; c < k; ++c) {
      int32_t s = map[c];
      float v = w[c * n + nn];
      if (s >= 0)
        lo[s] = v;
      else
        hi[-s - 1] = v;
    }
    s_w[nn] = orc_quantize_vec(lo, k_low, ORC_I4, codes);
    pack_i4_row(codes, k_low, w_low + nn * ldk, ldk);
    if (ldo > 0) {
      float sc = store_branch_row(hi, k_out, branch_fmt, (uint8_t*)w_out + (size_t)nn * ldo * esz,
                                  ldo, codes);
      if (s_wo) s_wo[nn] = sc;
    } else if (s_wo) {
      s_wo[nn] = 0.0f;
    }
  }
  free(codes);
  free(hi);
  free(lo);
}

/* ------------------------------------------------------------------ */
/* Step a1 (weight-side SQ-format): int4 with a reserved mask code     */
/* ------------------------------------------------------------------ */

/* Weight-side SQ-format for one output channel, generic in the low bit
 * width (bits = 2 or 4).  [SQF-art section 九: the format is a quantised
 * dense matrix, a sparse high-precision matrix and a mask; symmetric
 * quantisation leaves the largest unsigned code unused and that code marks
 * the high-precision positions; the positions are the top fraction of each
 * bank by an importance score built from the weight and the Hessian
 * diagonal; section 七: banks keep the work of every bank equal.]
 *   key_j = w_j^2 * hdiag_j in fp64 (orders exactly like |w_j| * sqrt(hdiag_j))
 * The row is split into banks of `bank` consecutive slots (bank <= 0 or
 * bank == k_low: one bank, the whole row; otherwise bank divides k_low and
 * nnz is a multiple of the bank count); in every bank the nnz / banks
 * largest keys (lower slot first on ties) are kept at high precision: int8
 * per-row quantisation of all kept values in ascending slot order ->
 * v8[0..nnz), scale *s8.  The remaining slots are quantised to
 * [-(2^(bits-1)-1), 2^(bits-1)-1] with their own scale *s_low; the kept
 * slots receive the reserved code 2^(bits-1) (as an unsigned field).
 * codes_out[j] holds the unsigned field value of slot j. */
void orc_sq_row(const float* wrow, const float* hdiag, int64_t k_low, int64_t nnz, int64_t bank,
                int bits, uint8_t* codes_out, int8_t* v8, float* s8, float* s_low) {
  double* key = (double*)malloc(sizeof(double) * (size_t)(k_low + 1));
  int32_t* order = (int32_t*)malloc(sizeof(int32_t) * (size_t)(k_low + 1));
  uint8_t* keep = (uint8_t*)calloc((size_t)(k_low + 1), 1);
  float* tmp = (float*)malloc(sizeof(float) * (size_t)(k_low + 1));
  int32_t* codes = (int32_t*)malloc(sizeof(int32_t) * (size_t)(k_low + 1));
  for (int64_t j = 0; j < k_low; ++j) {
    double wj = (double)wrow[j];
    key[j] = wj * wj * (double)hdiag[j];
    order[j] = (int32_t)j;
  }
  if (bank <= 0 || bank > k_low) bank = k_low;
  const int64_t banks = k_low > 0 ? k_low / bank : 0;
  const int64_t per_bank = banks > 0 ? nnz / banks : 0;
  g_sort_score = key;
  for (int64_t b = 0; b < banks; ++b) {
    /* rank the bank's slots on their own and keep its per_bank largest */
    qsort(order + b * bank, (size_t)bank, sizeof(int32_t), cmp_rank);
    for (int64_t i = 0; i < per_bank; ++i) keep[order[b * bank + i]] = 1;
  }
  /* high-precision values, ascending slot order */
  int64_t c = 0;
  for (int64_t j = 0; j < k_low; ++j)
    if (keep[j]) tmp[c++] = wrow[j];
  *s8 = orc_quantize_vec(tmp, nnz, ORC_I8, codes);
  for (int64_t i = 0; i < nnz; ++i) v8[i] = (int8_t)codes[i];
  /* low-precision part over the remaining slots */
  int q = (1 << (bits - 1)) - 1;
  float a = 0.0f;
  for (int64_t j = 0; j < k_low; ++j)
    if (!keep[j] && fabsf(wrow[j]) > a) a = fabsf(wrow[j]);
  float inv = a == 0.0f ? 0.0f : (float)q / a;
  *s_low = a == 0.0f ? 0.0f : a / (float)q;
  uint32_t field_mask = (1u << bits) - 1u;
  for (int64_t j = 0; j < k_low; ++j) {
    if (keep[j]) {
      codes_out[j] = (uint8_t)(1u << (bits - 1)); /* reserved mark */
    } else {
      int32_t cq = 0;
      if (a != 0.0f) {
        float r = rintf(wrow[j] * inv);
        if (r > (float)q) r = (float)q;
        if (r < (float)-q) r = (float)-q;
        cq = (int32_t)r;
      }
      codes_out[j] = (uint8_t)((uint32_t)cq & field_mask);
    }
  }
  free(codes);
  free(tmp);
  free(keep);
  free(order);
  free(key);
}

/* Weight-side SQ-format for a whole weight matrix with a static outlier
 * channel split on the activation side: low slots -> int4 codes with the
 * reserved mark + int8 sparse values (sq_val[nn][nnz], scale s_w8); outlier
 * channels -> int8 branch rows w_out[nn][ldo] with scale s_wo. */
void orc_pack_weights_sq(const float* w, int64_t k, int64_t n, const int32_t* map,
                         const float* hdiag_k, int64_t k_low, int64_t k_out, int64_t ldk,
                         int64_t ldo, int64_t nnz, int64_t bank, uint8_t* w_low, float* s_w4, int8_t* sq_val,
                         float* s_w8, int8_t* w_out, float* s_wo) {
  float* lo = (float*)malloc(sizeof(float) * (size_t)(k_low + 1));
  float* hlo = (float*)malloc(sizeof(float) * (size_t)(k_low + 1));
  float* hi = (float*)malloc(sizeof(float) * (size_t)(k_out + 1));
  uint8_t* fields = (uint8_t*)malloc((size_t)(k_low + 1));
  int32_t* codes = (int32_t*)malloc(sizeof(int32_t) * (size_t)(k + 1));
  for (int64_t c = 0; c < k; ++c)
    if (map[c] >= 0) hlo[map[c]] = hdiag_k[c];
  for (int64_t nn = 0; nn < n; ++nn) {
    for (int64_t c = 0; c < k; ++c) {
      int32_t s = map[c];
      float v = w[c * n + nn];
      if (s >= 0)
        lo[s] = v;
      else
        hi[-s - 1] = v;
    }
    orc_sq_row(lo, hlo, k_low, nnz, bank, 4, fields, sq_val + nn * nnz, &s_w8[nn], &s_w4[nn]);
    uint8_t* row = w_low + nn * ldk;
    zero_bytes(row, ldk);
    for (int64_t j = 0; j < k_low; ++j)
      row[j >> 1] |= (uint8_t)((j & 1) ? (fields[j] << 4) : fields[j]);
    if (ldo > 0) {
      s_wo[nn] = store_branch_row(hi, k_out, ORC_I8, (uint8_t*)w_out + nn * ldo, ldo, codes);
    } else {
      s_wo[nn] = 0.0f;
    }
  }
  free(codes);
  free(fields);
  free(hi);
  free(hlo);
  free(lo);
}

/* ------------------------------------------------------------------ */
/* Floating-point weight-side SQ-format: FP4 low part, FP8 sparse part */
/* ------------------------------------------------------------------ */

/* [SQF-art section 八: the format with floating-point types, FP8 for the
 * high-precision part and FP4 for the low part at 87.5% sparsity, about 5
 * bits per weight.]  Readings: FP4 = OCP E2M1, FP8 = OCP E4M3; the reserved
 * mark of the dense FP4 codes is 0x8 (E2M1 negative zero, which the encoder
 * never produces: a value that rounds to zero is +0); one scale per output
 * row for each part, as in the integer form: the kept values are E4M3 codes
 * of v * 448/a8 (s_w8 = a8/448), the others E2M1 codes of v * inv4 with
 * inv4 = 6/a4 as one fp32 division (s_w4 = a4/6), a4 the absmax over the
 * unmarked slots.  The marks are chosen exactly as in the integer form
 * (orc_sq_row: key w^2 * hdiag, banks, ties to the lower slot).  fields[j]
 * receives the 4-bit field of slot j, v8[0..nnz) the E4M3 bytes in slot
 * order. */
void orc_sqf_row(const float* wrow, const float* hdiag, int64_t k_low, int64_t nnz, int64_t bank,
                 uint8_t* fields, uint8_t* v8, float* s8, float* s4) {
  int8_t* dummy8 = (int8_t*)malloc((size_t)(nnz + 1));
  float* tmp = (float*)malloc(sizeof(float) * (size_t)(k_low + 1));
  int32_t* codes = (int32_t*)malloc(sizeof(int32_t) * (size_t)(k_low + 1));
  float s_int8, s_int4;
  /* the marks: the integer form's choice (its codes are not used) */
  orc_sq_row(wrow, hdiag, k_low, nnz, bank, 4, fields, dummy8, &s_int8, &s_int4);
  int64_t c = 0;
  for (int64_t j = 0; j < k_low; ++j)
    if (fields[j] == 0x8) tmp[c++] = wrow[j];
  *s8 = orc_quantize_vec(tmp, c, ORC_FP8, codes);
  for (int64_t i = 0; i < c; ++i) v8[i] = (uint8_t)(codes[i] & 0xFF);
  float a = 0.0f;
  for (int64_t j = 0; j < k_low; ++j)
    if (fields[j] != 0x8 && fabsf(wrow[j]) > a) a = fabsf(wrow[j]);
  float inv = a == 0.0f ? 0.0f : 6.0f / a;
  *s4 = a == 0.0f ? 0.0f : a / 6.0f;
  for (int64_t j = 0; j < k_low; ++j)
    if (fields[j] != 0x8) fields[j] = orc_e2m1_from_double((double)(wrow[j] * inv));
  free(codes);
  free(tmp);
  free(dummy8);
}

/* Whole weight matrix in the floating-point SQ-format with an E4M3 branch
 * over the outlier channels (scale s_wo per output row). */
void orc_pack_weights_sqf(const float* w, int64_t k, int64_t n, const int32_t* map,
                          const float* hdiag_k, int64_t k_low, int64_t k_out, int64_t ldk,
                          int64_t ldo, int64_t nnz, int64_t bank, uint8_t* w_low, float* s_w4,
                          uint8_t* sq_val, float* s_w8, uint8_t* w_out, float* s_wo) {
  float* lo = (float*)malloc(sizeof(float) * (size_t)(k_low + 1));
  float* hlo = (float*)malloc(sizeof(float) * (size_t)(k_low + 1));
  float* hi = (float*)malloc(sizeof(float) * (size_t)(k_out + 1));
  uint8_t* fields = (uint8_t*)malloc((size_t)(k_low + 1));
  int32_t* codes = (int32_t*)malloc(sizeof(int32_t) * (size_t)(k + 1));
  for (int64_t c = 0; c < k; ++c)
    if (map[c] >= 0) hlo[map[c]] = hdiag_k[c];
  for (int64_t nn = 0; nn < n; ++nn) {
    for (int64_t c = 0; c < k; ++c) {
      if (map[c] >= 0)
        lo[map[c]] = w[c * n + nn];
      else
        hi[-map[c] - 1] = w[c * n + nn];
    }
    orc_sqf_row(lo, hlo, k_low, nnz, bank, fields, sq_val + nn * nnz, &s_w8[nn], &s_w4[nn]);
    uint8_t* row = w_low + nn * ldk;
    zero_bytes(row, ldk);
    for (int64_t j = 0; j < k_low; ++j)
      row[j >> 1] |= (uint8_t)((j & 1) ? (fields[j] << 4) : fields[j]);
    if (ldo > 0)
      s_wo[nn] = store_branch_row(hi, k_out, ORC_FP8, w_out + nn * ldo, ldo, codes);
    else
      s_wo[nn] = 0.0f;
  }
  free(codes);
  free(fields);
  free(hi);
  free(hlo);
  free(lo);
}

/* y of the floating-point SQ-format for the token rows rows[0..nr): E4M3
 * activations (per-token scale s_x over the low channels), E2M1 weights with
 * the 0x8 mark, E4M3 sparse values, E4M3 branch:
 *   acc_low = sum_j e4m3(cx_j) * e2m1(cw_j)        (unmarked slots)
 *   acc_sp  = sum_i e4m3(cx_pos_i) * e4m3(v8_i)     (i-th marked slot)
 *   acc_o   = sum_t e4m3(xo_t) * e4m3(wo_t)
 *   y = s_x * (s_w4 * acc_low + s_w8 * acc_sp) + (s_xo * s_wo) * acc_o
 * in fp64 (every product and these sums are exact there), rounded once to
 * fp32.  [SQF-art section 三: two paths summed; 八: the FP8/FP4 form.] */
void orc_dual_gemm_sqf(int64_t n, int64_t k_low, int64_t k_out, const int64_t* rows, int64_t nr,
                       const uint8_t* x_low, int64_t ldk_x, const float* s_x, const uint8_t* x_out,
                       int64_t ldo, const float* s_xo, const uint8_t* w_low, int64_t ldk_w,
                       const float* s_w4, int64_t nnz, const uint8_t* sq_val, const float* s_w8,
                       const uint8_t* w_out, const float* s_wo, float* y, int64_t ldy) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t r = 0; r < nr; ++r) {
    for (int64_t nn = 0; nn < n; ++nn) {
      int64_t mm = rows[r];
      double acc = 0.0, acc_sp = 0.0, acc_o = 0.0;
      int64_t i_sp = 0;
      for (int64_t j = 0; j < k_low; ++j) {
        double vx = orc_e4m3_to_double(x_low[mm * ldk_x + j]);
        uint8_t b = w_low[nn * ldk_w + (j >> 1)];
        uint8_t f = (uint8_t)(((j & 1) ? (b >> 4) : b) & 0xF);
        if (f == 0x8) {
          acc_sp += vx * orc_e4m3_to_double(sq_val[nn * nnz + i_sp]);
          ++i_sp;
        } else {
          acc += vx * orc_e2m1_to_double(f);
        }
      }
      for (int64_t t = 0; t < k_out; ++t)
        acc_o += orc_e4m3_to_double(x_out[mm * ldo + t]) * orc_e4m3_to_double(w_out[nn * ldo + t]);
      double out = (double)s_x[mm] * ((double)s_w4[nn] * acc + (double)s_w8[nn] * acc_sp);
      if (k_out > 0) out += ((double)s_xo[mm] * (double)s_wo[nn]) * acc_o;
      y[r * ldy + nn] = (float)out;
    }
  }
}

/* ------------------------------------------------------------------ */
/* Step a2: per-token quantisation and outlier extraction             */
/* ------------------------------------------------------------------ */

/* For every token m: the low channels (slot order) are quantised per token to
 * int4 (low_fmt ORC_I4, packed, ldk bytes per row) or int8 (ORC_I8, one byte
 * per slot); the outlier channels are gathered into the compact dense
 * branch row x_out[m][ldo] (bf16, or FP8 / int8 with a per-token scale).
 * [OSC-abs: structured sub-tensor extraction gathers the scattered outlier
 * channels online into a compact dense tensor.]  x is fp32 (x_fmt ORC_F32)
 * or bf16 bit patterns (ORC_BF16), row stride ldx elements. */
void orc_quantize_split_act(const void* x, int x_fmt, int64_t m, int64_t k, int64_t ldx,
                            const int32_t* map, int64_t k_low, int64_t k_out, int64_t ldk,
                            int64_t ldo, int low_fmt, int branch_fmt, uint8_t* x_low, float* s_x,
                            void* x_out, float* s_xo) {
  float* row = (float*)malloc(sizeof(float) * (size_t)(k + 1));
  float* lo = (float*)malloc(sizeof(float) * (size_t)(k_low + 1));
  float* hi = (float*)malloc(sizeof(float) * (size_t)(k_out + 1));
  int32_t* codes = (int32_t*)malloc(sizeof(int32_t) * (size_t)(k + 1));
  size_t esz = branch_fmt == ORC_BF16 ? 2 : 1;
  for (int64_t mm = 0; mm < m; ++mm) {
    for (int64_t c = 0; c < k; ++c) {
      if (x_fmt == ORC_BF16)
        row[c] = (float)orc_bf16_to_double(((const uint16_t*)x)[mm * ldx + c]);
      else
        row[c] = ((const float*)x)[mm * ldx + c];
    }
    for (int64_t c = 0; c < k; ++c) {
      if (map[c] >= 0)
        lo[map[c]] = row[c];
      else
        hi[-map[c] - 1] = row[c];
    }
    s_x[mm] = orc_quantize_vec(lo, k_low, low_fmt, codes);
    uint8_t* dst = x_low + mm * ldk;
    if (low_fmt == ORC_I4) {
      pack_i4_row(codes, k_low, dst, ldk);
    } else {
      zero_bytes(dst, ldk);
      for (int64_t j = 0; j < k_low; ++j) dst[j] = (uint8_t)(codes[j] & 0xFF);
    }
    if (ldo > 0) {
      float sc = store_branch_row(hi, k_out, branch_fmt, (uint8_t*)x_out + (size_t)mm * ldo * esz,
                                  ldo, codes);
      if (s_xo) s_xo[mm] = sc;
    } else if (s_xo) {
      s_xo[mm] = 0.0f;
    }
  }
  free(codes);
  free(hi);
  free(lo);
  free(row);
}

/* ------------------------------------------------------------------ */
/* Producer side: the norm that feeds the split, and the channel order */
/* ------------------------------------------------------------------ */

/* RMS normalisation of each row (the norm in front of the linear layers of
 * the Llama / Qwen models the workloads are shaped after; the pages name no
 * norm, so this is a reading): out[m][c] = (x[m][c] * r_m) * gamma[c] in
 * fp32, r_m = 1 / sqrt(mean_c x[m][c]^2 + eps) formed in fp64 (the squares of
 * fp32 values are exact there) and rounded once to fp32.  x is fp32 (x_fmt
 * ORC_F32) or bf16 patterns (ORC_BF16), row stride ldx; out is [m][k]. */
void orc_rmsnorm(const void* x, int x_fmt, int64_t m, int64_t k, int64_t ldx, const float* gamma,
                 float eps, float* out) {
  for (int64_t mm = 0; mm < m; ++mm) {
    double ss = 0.0;
    for (int64_t c = 0; c < k; ++c) {
      double v = x_fmt == ORC_BF16 ? orc_bf16_to_double(((const uint16_t*)x)[mm * ldx + c])
                                   : (double)((const float*)x)[mm * ldx + c];
      ss += v * v;
    }
    float r = (float)(1.0 / sqrt(ss / (double)k + (double)eps));
    for (int64_t c = 0; c < k; ++c) {
      float v = x_fmt == ORC_BF16 ? (float)orc_bf16_to_double(((const uint16_t*)x)[mm * ldx + c])
                                  : ((const float*)x)[mm * ldx + c];
      float t = v * r;
      out[mm * k + c] = t * gamma[c];
    }
  }
}

/* The channel order that makes the split a slice [SQ-format article,
 * section 九: weight columns reordered by the importance mask]: position p
 * of the reordered axis holds channel perm[p]; the low channels first in slot
 * order (p = map[c]), then the outlier channels in branch order (p = k_low +
 * t for map[c] = -(t+1)).  Reordering the producer's output channels and the
 * consumer's input channels this way leaves every product of the layer
 * unchanged, and the consumer's map becomes the slice map: p -> p for
 * p < k_low, p -> -(p - k_low + 1) after. */
void orc_slot_order(const int32_t* map, int64_t k, int32_t* perm, int32_t* slice_map) {
  int64_t k_low = 0;
  for (int64_t c = 0; c < k; ++c)
    if (map[c] >= 0) ++k_low;
  for (int64_t c = 0; c < k; ++c) {
    int64_t p = map[c] >= 0 ? map[c] : k_low + (-map[c] - 1);
    perm[p] = (int32_t)c;
  }
  for (int64_t p = 0; p < k; ++p) slice_map[p] = p < k_low ? (int32_t)p : (int32_t)(-(p - k_low + 1));
}

/* ------------------------------------------------------------------ */
/* Storage of int4 codes in 6-bit OCP E2M3 fields (K-blocked layout)   */
/* ------------------------------------------------------------------ */

/* OCP MX E2M3: 1 sign bit (bit 5), 2 exponent bits (bits 4..3, bias 1), 3
 * mantissa bits (bits 2..0); exponent 0 is subnormal with value
 * (-1)^s * 2^(1-1) * m/8.  An int4 code c in [-7, 7] is held as the
 * subnormal of magnitude |c|/8: field = (c < 0) << 5 | |c|.  The arithmetic
 * on the codes is unchanged: this is how the same integers are stored for
 * a 6-bit matrix unit (the product of two fields is c_x * c_w / 64). */
uint8_t orc_e2m3_field_of_code(int code) {
  int a = code < 0 ? -code : code;
  return (uint8_t)(((code < 0) ? 0x20 : 0) | (a & 7));
}

/* Re-encode packed int4 rows (the layout of orc_quantize_split_act /
 * orc_pack_weights: [rows][ldk], slot 2i in the low nibble of byte i) into
 * the K-blocked E2M3 storage.  The 32 slots 32g .. 32g+31 of K block kb
 * (slots 128kb .. 128kb+127) of row r form a 24-byte group, field j%32 at
 * bits 6*(j%32), little-endian.  Rows are taken in pairs of 16-row groups:
 * for K block kb and rows 32p .. 32p+31 (p = r/32, h = (r/16)%2, lane =
 * 16g + r%16) the 3072 bytes at (kb * rows_pad/32 + p) * 3072 hold
 *   bytes 0..15 of the group at h*1024 + lane*16   (the two "head" KiB),
 *   bytes 16..23 of the group at 2048 + lane*16 + 8h   (the "tail" KiB).
 * (A storage convention of this implementation, not of the method: it lets
 * each lane read its 24 bytes with 16-byte loads.)  pad = 2*ldk slots per
 * row; rows_pad >= rows, a multiple of 32; the rows past `rows` are left
 * zero. */
void orc_i4x2_to_e2m3(const uint8_t* packed, int64_t rows, int64_t ldk, int64_t rows_pad,
                      uint8_t* out) {
  const int64_t pad = 2 * ldk, nblk = pad / 128, npair = rows_pad / 32;
  zero_bytes(out, nblk * rows_pad * 96);
  uint8_t grp[24];
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t kb = 0; kb < nblk; ++kb) {
      for (int64_t g = 0; g < 4; ++g) {
        memset(grp, 0, sizeof grp);
        for (int64_t i = 0; i < 32; ++i) {
          int64_t j = kb * 128 + g * 32 + i;
          uint8_t b = packed[r * ldk + (j >> 1)];
          uint8_t nib = (uint8_t)(((j & 1) ? (b >> 4) : b) & 0xF);
          int code = (nib & 0x8) ? (int)nib - 16 : (int)nib;
          uint32_t f = orc_e2m3_field_of_code(code);
          int64_t bit = 6 * i;
          for (int t = 0; t < 6; ++t)
            if ((f >> t) & 1u) grp[(bit + t) >> 3] |= (uint8_t)(1u << ((bit + t) & 7));
        }
        const int64_t lane = g * 16 + r % 16, h = (r / 16) % 2;
        uint8_t* base = out + (kb * npair + r / 32) * 3072;
        memcpy(base + h * 1024 + lane * 16, grp, 16);
        memcpy(base + 2048 + lane * 16 + 8 * h, grp + 16, 8);
      }
    }
  }
}

/* ------------------------------------------------------------------ */
/* MXFP4 low path (OCP Microscaling: E2M1 elements, E8M0 block scales) */
/* ------------------------------------------------------------------ */

/* [OSC-abs: the low path fits 4-bit micro-scaling hardware.]  The pages do
 * not define the format; the plain reading is the OCP Microscaling (MX)
 * specification's MXFP4: blocks of 32 consecutive values share one E8M0
 * scale 2^X, and each value is stored as an FP4 E2M1 element.
 *
 * E2M1: 1 sign bit (bit 3), 2 exponent bits (bits 2..1, bias 1), 1 mantissa
 * bit (bit 0), no infinities or NaN; exponent 0 is subnormal with value
 * (-1)^s * m/2, otherwise (-1)^s * 2^(e-1) * (1 + m/2).  The value of a code
 * is computed from that definition. */
double orc_e2m1_to_double(uint8_t c) {
  int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
  double v = e == 0 ? (double)m / 2.0 : ldexp(1.0 + (double)m / 2.0, e - 1);
  return s ? -v : v;
}

/* Nearest E2M1 value to t, ties to the code with mantissa bit 0, saturating
 * to +-6 (the largest finite element); written as a search over the eight
 * non-negative codes.  A value that rounds to zero gives +0 (0x0). */
uint8_t orc_e2m1_from_double(double t) {
  double a = fabs(t);
  int best = 0;
  double best_err = a;
  for (int c = 1; c <= 7; ++c) {
    double err = fabs(orc_e2m1_to_double((uint8_t)c) - a);
    if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
      best = c;
      best_err = err;
    }
  }
  if (a > 6.0) best = 7; /* saturate */
  return (uint8_t)(best | ((t < 0.0 && best != 0) ? 0x8 : 0));
}

/* One MX block v[0..len) (len <= 32; absent positions count as 0): the
 * shared exponent is X = floor(log2(max|v|)) - 2, 2 being the exponent of
 * the largest E2M1 normal (6 = 1.5 * 2^2), clamped to the E8M0 range
 * [-127, 127]; an all-zero block takes X = -127.  Element i is the E2M1
 * code of v_i / 2^X (so the block's absmax lands in [4, 8) and saturates
 * to 6 above 6).  codes[i] receives the 4-bit code; the return value is the
 * E8M0 byte X + 127. */
uint8_t orc_mx_block(const float* v, int64_t len, uint8_t* codes) {
  double amax = 0.0;
  for (int64_t i = 0; i < len; ++i)
    if (fabs((double)v[i]) > amax) amax = fabs((double)v[i]);
  int x = -127;
  if (amax > 0.0) {
    int e;
    frexp(amax, &e); /* amax = f * 2^e, f in [0.5, 1): floor(log2 amax) = e - 1 */
    x = (e - 1) - 2;
    if (x < -127) x = -127;
    if (x > 127) x = 127;
  }
  for (int64_t i = 0; i < len; ++i) codes[i] = orc_e2m1_from_double(ldexp((double)v[i], -x));
  return (uint8_t)(x + 127);
}

/* Quantise a row of `len` values in slot order into MXFP4 over `pad` slots
 * (pad a multiple of 32; slots >= len are 0): codes packed two per byte
 * (slot 2i in the low nibble of byte i) into row[pad/2], scales[pad/32]. */
static void mx_row(const float* vals, int64_t len, int64_t pad, uint8_t* row, uint8_t* scales) {
  float blk[32];
  uint8_t c[32];
  zero_bytes(row, pad / 2);
  for (int64_t b = 0; b < pad / 32; ++b) {
    for (int i = 0; i < 32; ++i) {
      int64_t j = b * 32 + i;
      blk[i] = j < len ? vals[j] : 0.0f;
    }
    scales[b] = orc_mx_block(blk, 32, c);
    for (int i = 0; i < 32; ++i) {
      int64_t j = b * 32 + i;
      row[j >> 1] |= (uint8_t)((j & 1) ? (c[i] << 4) : c[i]);
    }
  }
}

/* Weights for the MXFP4 low path: per output channel nn, the low channels'
 * values in slot order -> MXFP4 (codes w_low[nn][pad/2], scales
 * s_wb[nn][pad/32]); the outlier channels -> bf16 branch row w_out[nn][ldo]. */
void orc_pack_weights_mx(const float* w, int64_t k, int64_t n, const int32_t* map, int64_t k_low,
                         int64_t k_out, int64_t pad, int64_t ldo, uint8_t* w_low, uint8_t* s_wb,
                         uint16_t* w_out) {
  float* lo = (float*)malloc(sizeof(float) * (size_t)(k_low + 1));
  float* hi = (float*)malloc(sizeof(float) * (size_t)(k_out + 1));
  int32_t* tmp = (int32_t*)malloc(sizeof(int32_t) * (size_t)(k_out + 1));
  for (int64_t nn = 0; nn < n; ++nn) {
    for (int64_t c = 0; c < k; ++c) {
      int32_t s = map[c];
      float v = w[c * n + nn];
      if (s >= 0)
        lo[s] = v;
      else
        hi[-s - 1] = v;
    }
    if (pad > 0) mx_row(lo, k_low, pad, w_low + nn * (pad / 2), s_wb + nn * (pad / 32));
    if (ldo > 0) store_branch_row(hi, k_out, ORC_BF16, w_out + nn * ldo, ldo, tmp);
  }
  free(tmp);
  free(hi);
  free(lo);
}

/* Activations for the MXFP4 low path: per token, the low channels' values in
 * slot order -> MXFP4 (x_low[m][pad/2], s_xb[m][pad/32]); the outlier
 * channels -> bf16 branch row x_out[m][ldo] (no scale).  x as in
 * orc_quantize_split_act. */
void orc_quantize_split_act_mx(const void* x, int x_fmt, int64_t m, int64_t k, int64_t ldx,
                               const int32_t* map, int64_t k_low, int64_t k_out, int64_t pad,
                               int64_t ldo, uint8_t* x_low, uint8_t* s_xb, uint16_t* x_out) {
  float* lo = (float*)malloc(sizeof(float) * (size_t)(k_low + 1));
  float* hi = (float*)malloc(sizeof(float) * (size_t)(k_out + 1));
  int32_t* tmp = (int32_t*)malloc(sizeof(int32_t) * (size_t)(k_out + 1));
  for (int64_t mm = 0; mm < m; ++mm) {
    for (int64_t c = 0; c < k; ++c) {
      float v = x_fmt == ORC_BF16 ? (float)orc_bf16_to_double(((const uint16_t*)x)[mm * ldx + c])
                                  : ((const float*)x)[mm * ldx + c];
      if (map[c] >= 0)
        lo[map[c]] = v;
      else
        hi[-map[c] - 1] = v;
    }
    if (pad > 0) mx_row(lo, k_low, pad, x_low + mm * (pad / 2), s_xb + mm * (pad / 32));
    if (ldo > 0) store_branch_row(hi, k_out, ORC_BF16, x_out + mm * ldo, ldo, tmp);
  }
  free(tmp);
  free(hi);
  free(lo);
}

/* The MXFP4 rows in the K-blocked storage the 4-bit matrix unit reads:
 *   codes  [pad/128][rows_pad/16][4][16][16]: the 16 bytes of slots
 *          32g .. 32g+31 of K block kb of row r (bytes 64kb+16g .. +15 of
 *          the packed row) at (((kb * rows_pad/16 + r/16) * 4 + g) * 16 +
 *          r%16) * 16;
 *   scales [pad/128][rows_pad/64][4][16][4]: the scale of that block of
 *          row r at (((kb * rows_pad/64 + r/64) * 4 + g) * 16 + r%16) * 4 +
 *          (r/16)%4.
 * rows_pad >= rows, a multiple of 64; rows past `rows` are left zero. */
void orc_mx_storage(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t pad,
                    int64_t rows_pad, uint8_t* codes_out, uint8_t* scales_out) {
  const int64_t nblk = pad / 128;
  zero_bytes(codes_out, nblk * rows_pad * 64);
  zero_bytes(scales_out, nblk * rows_pad * 4);
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t kb = 0; kb < nblk; ++kb)
      for (int64_t g = 0; g < 4; ++g) {
        memcpy(codes_out + (((kb * (rows_pad / 16) + r / 16) * 4 + g) * 16 + r % 16) * 16,
               codes + r * (pad / 2) + kb * 64 + g * 16, 16);
        scales_out[(((kb * (rows_pad / 64) + r / 64) * 4 + g) * 16 + r % 16) * 4 + (r / 16) % 4] =
            scales[r * (pad / 32) + kb * 4 + g];
      }
}

/* y[r][nn] of the MXFP4 dual GEMM for the token rows rows[0..nr):
 *   y = sum_j (2^(X_x(b)) * e2m1(cx_j)) * (2^(X_w(b)) * e2m1(cw_j))
 *       + sum_t xo[t] * wo[t]                   (b = block of slot j = j/32)
 * in fp64, rounded once to fp32.  [OSC-abs: 4-bit path plus 16-bit branch,
 * results summed; the micro-scaling block scales multiply each block's
 * products.]  Codes packed [rows][pad/2], scales [rows][pad/32] (the
 * logical layout of orc_quantize_split_act_mx / orc_pack_weights_mx). */
void orc_dual_gemm_mx(int64_t n, int64_t k_low, int64_t k_out, int64_t pad, const int64_t* rows,
                      int64_t nr, const uint8_t* x_low, const uint8_t* s_xb,
                      const uint16_t* x_out, int64_t ldo, const uint8_t* w_low,
                      const uint8_t* s_wb, const uint16_t* w_out, float* y, int64_t ldy) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t r = 0; r < nr; ++r) {
    for (int64_t nn = 0; nn < n; ++nn) {
      int64_t mm = rows[r];
      double acc = 0.0;
      for (int64_t j = 0; j < k_low; ++j) {
        uint8_t bx = x_low[mm * (pad / 2) + (j >> 1)], bw = w_low[nn * (pad / 2) + (j >> 1)];
        uint8_t cx = (uint8_t)(((j & 1) ? bx >> 4 : bx) & 0xF);
        uint8_t cw = (uint8_t)(((j & 1) ? bw >> 4 : bw) & 0xF);
        double vx = ldexp(orc_e2m1_to_double(cx), (int)s_xb[mm * (pad / 32) + j / 32] - 127);
        double vw = ldexp(orc_e2m1_to_double(cw), (int)s_wb[nn * (pad / 32) + j / 32] - 127);
        acc += vx * vw;
      }
      for (int64_t t = 0; t < k_out; ++t)
        acc += orc_bf16_to_double(x_out[mm * ldo + t]) * orc_bf16_to_double(w_out[nn * ldo + t]);
      y[r * ldy + nn] = (float)acc;
    }
  }
}

/* ------------------------------------------------------------------ */
/* Steps a3-a5 (and the weight-side masked path): the dual GEMM        */
/* ------------------------------------------------------------------ */

static double branch_val(const void* base, int64_t ld, int64_t r, int64_t t, int fmt) {
  if (fmt == ORC_BF16) return orc_bf16_to_double(((const uint16_t*)base)[r * ld + t]);
  uint8_t b = ((const uint8_t*)base)[r * ld + t];
  if (fmt == ORC_FP8) return orc_e4m3_to_double(b);
  return (double)(int8_t)b;
}

/* Decoded low code of slot j of a packed (int4) or byte (int8) row. */
static int low_code(const uint8_t* row, int64_t j, int fmt) {
  if (fmt == ORC_I8) return (int)(int8_t)row[j];
  uint8_t b = row[j >> 1];
  return nib_code((j & 1) ? (uint8_t)(b >> 4) : b);
}

/* y[r][nn] for the token rows listed in rows[0..nr) (row r of the outputs is
 * token rows[r]) and every output channel nn < n:
 *   acc_low = sum_j qx[j] * qw[j]            (exact integer, mark -> 0)
 *   acc_sp  = sum_i qx[pos_i] * v8[i]         (weight-side format only; pos_i
 *                                              = i-th marked slot of the row)
 *   acc_o   = sum_t xo[t] * wo[t]             (branch; integer for int8,
 *                                              fp64 for bf16 / FP8)
 *   y = s_x*s_w*acc_low [+ s_x*s_w8*acc_sp] + (s_xo*s_wo)*acc_o
 * formed in fp64 and rounded once to fp32.  [SQF-art section 三: two parallel
 * paths whose results are summed; OSC method framework: result fusion.]
 * x_low_fmt: ORC_I4 (packed) or ORC_I8.  branch_fmt: ORC_BF16 / ORC_FP8 /
 * ORC_I8 (the bf16 branch has no scales).  sq_nnz > 0 selects the
 * weight-side format (w_low holds marks, sq_val/s_w8 the sparse values).
 * Debug accumulators (NULL to skip) are int64 [nr][n]; acc_o is only filled
 * for an int8 branch. */
void orc_dual_gemm(int64_t n, int64_t k_low, int64_t k_out, const int64_t* rows, int64_t nr,
                   const uint8_t* x_low, int64_t ldk_x, int x_low_fmt, const float* s_x,
                   const void* x_out, int64_t ldo, int branch_fmt, const float* s_xo,
                   const uint8_t* w_low, int64_t ldk_w, const float* s_w, const void* w_out,
                   const float* s_wo, int64_t sq_nnz, const int8_t* sq_val, const float* s_w8,
                   float* y, int64_t ldy, int64_t* acc_low_dbg, int64_t* acc_sp_dbg,
                   int64_t* acc_o_dbg) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t r = 0; r < nr; ++r) {
    for (int64_t nn = 0; nn < n; ++nn) {
      int64_t mm = rows[r];
      const uint8_t* xr = x_low + mm * ldk_x;
      const uint8_t* wr = w_low + nn * ldk_w;
      int64_t acc = 0, acc_sp = 0, acc_o_i = 0;
      double acc_o = 0.0;
      int64_t i_sp = 0;
      for (int64_t j = 0; j < k_low; ++j) {
        int qx = low_code(xr, j, x_low_fmt);
        if (sq_nnz > 0) {
          uint8_t b = wr[j >> 1];
          uint8_t nib = (uint8_t)(((j & 1) ? (b >> 4) : b) & 0xF);
          if (nib == 0x8) {
            acc_sp += (int64_t)qx * (int64_t)sq_val[nn * sq_nnz + i_sp];
            ++i_sp;
            continue;
          }
        }
        acc += (int64_t)qx * (int64_t)low_code(wr, j, ORC_I4);
      }
      for (int64_t t = 0; t < k_out; ++t) {
        if (branch_fmt == ORC_I8) {
          acc_o_i += (int64_t)(int8_t)((const uint8_t*)x_out)[mm * ldo + t] *
                     (int64_t)(int8_t)((const uint8_t*)w_out)[nn * ldo + t];
        } else {
          acc_o += branch_val(x_out, ldo, mm, t, branch_fmt) *
                   branch_val(w_out, ldo, nn, t, branch_fmt);
        }
      }
      double br;
      if (branch_fmt == ORC_BF16)
        br = acc_o;
      else if (branch_fmt == ORC_FP8)
        br = ((double)s_xo[mm] * (double)s_wo[nn]) * acc_o;
      else
        br = ((double)s_xo[mm] * (double)s_wo[nn]) * (double)acc_o_i;
      if (k_out == 0) br = 0.0;
      double low = (double)s_x[mm] * (double)s_w[nn] * (double)acc;
      if (sq_nnz > 0) low += (double)s_x[mm] * (double)s_w8[nn] * (double)acc_sp;
      y[r * ldy + nn] = (float)(low + br);
      if (acc_low_dbg) acc_low_dbg[r * n + nn] = acc;
      if (acc_sp_dbg) acc_sp_dbg[r * n + nn] = acc_sp;
      if (acc_o_dbg) acc_o_dbg[r * n + nn] = acc_o_i;
    }
  }
}

/* Threads the OpenMP loops above use (reported with CPU timings). */
int orc_num_threads(void) { return omp_get_max_threads(); }
