/*
 * nvfp4_oracle.c -- plain CPU reference for the NVFP4 quantizer and the
 * block-scaled FP4 GEMM.  TEST INFRASTRUCTURE ONLY (see nvfp4_oracle.h for
 * the sources cited as [NVFP4], [RHT], [2D], [SR], [ACC], [E2M1], [E4M3],
 * [PHILOX]).
 *
 * Written to be checked by eye, not to be fast:
 *   - every fp32 step is one IEEE-754 binary32 operation rounded to nearest
 *     even (build with -ffp-contract=off, no fast-math; x86-64 SSE keeps
 *     float temporaries in float);
 *   - rounding to a format is an argmin over that format's value table, with
 *     the tie rule applied to adjacent table entries; no bit tricks;
 *   - the GEMM is the definition: a double-precision sum of products of the
 *     dequantized operands.
 * The only parallelism is independent rows split over OpenMP threads.
 *
 * Readings taken where the pages are silent (each one is listed in the
 * design notes with its reason):
 *   R1  S_enc = fl(2688 / amax): 2688 = 6 * 448 puts the tensor's amax at the
 *       top of the range one block can express (E2M1 max times E4M3 max).
 *       amax == 0 gives S_enc = 1; an overflowing quotient gives FLT_MAX.
 *   R2  block scale s = fl(fl(amax_b * S_enc) / 6), stored as E4M3 with
 *       round-to-nearest-even and saturation to 448.
 *   R3  per-block multiplier inv = fl(S_enc / decode(byte)), 0 when the byte
 *       decodes to 0, clamped to FLT_MAX; element y = fl(x * inv).
 *   R4  E2M1 round-to-nearest-even: ties go to the code with mantissa bit 0,
 *       |y| >= 6 saturates to 6, the sign of y (also of zero) is kept.
 *   R5  stochastic rounding: with lo <= |y| < hi adjacent grid values and
 *       f = (|y| - lo) / (hi - lo), round up iff u < f * 2^16 for a 16-bit
 *       random u.
 *   R6  random bits: Philox4x32-10 keyed by the seed; counter
 *       (g lo, g hi, stream, 0) with g = index >> 3; element index i takes
 *       16-bit half (i & 1) of output word (i & 7) >> 1.  Streams: 0 rowwise
 *       (and 2D), 1 columnwise copy, 2 Hadamard signs.
 *   R7  RHT: per contiguous 16-chunk v <- 1/4 * H16 * diag(sigma) * v,
 *       H16 Sylvester-ordered, evaluated by the in-place butterfly with
 *       h = 1, 2, 4, 8 in fp32; one sign vector per seed shared by all chunks.
 *   R8  layouts: two codes per byte, the even element in the low nibble;
 *       codes [rows][cols/2], scales [rows][cols/16]; a 2D tile's byte is
 *       stored on each of its 16 rows.
 */
#include "nvfp4_oracle.h"

#include <float.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* [E2M1] magnitudes, indexed by the low three bits of a code */
static const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* format codecs                                                       */
/* ------------------------------------------------------------------ */

double orc_e2m1_value(int code) {
  double v = kE2M1[code & 7];
  return (code & 8) ? -v : v;
}

/* [E4M3] sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0
 * holds the subnormals m * 2^-9; 0x7F and 0xFF are NaN. */
double orc_e4m3_value(int byte) {
  int s = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/* Nearest non-negative finite E4M3 value to s >= 0, ties to the even byte
 * (the even byte is the one whose mantissa LSB is 0).  Values above 448 go to
 * 448 (0x7E): the argmin over finite values saturates by itself; +inf is
 * handled explicitly.  Distances are taken in double: near a tie both are
 * exact (a half-spacing is a power of two), elsewhere rounding is monotone
 * and cannot reorder two distances that differ by at least one fp32 ulp. */
int orc_e4m3_encode(float s) {
  if (!(s >= 0.0f)) return -1; /* negative or NaN: not a scale */
  if (s >= 448.0f) return 0x7E;
  int best = 0;
  double best_d = fabs((double)s - orc_e4m3_value(0));
  for (int b = 1; b <= 0x7E; ++b) {
    double d = fabs((double)s - orc_e4m3_value(b));
    if (d < best_d || (d == best_d && (b % 2) == 0)) {
      best = b;
      best_d = d;
    }
  }
  return best;
}

/* R4: nearest grid magnitude, ties to the even index, saturate at 6, keep the
 * sign bit (so -0 and small negatives that round to 0 give code 0x8). */
int orc_e2m1_encode_rne(float y) {
  double m = fabs((double)y);
  int idx;
  if (m >= 6.0) {
    idx = 7;
  } else {
    idx = 0;
    double best_d = m;
    for (int i = 1; i < 8; ++i) {
      double d = fabs(m - kE2M1[i]);
      if (d < best_d || (d == best_d && (i % 2) == 0)) {
        idx = i;
        best_d = d;
      }
    }
  }
  return (signbit(y) ? 8 : 0) | idx;
}

/* R5: [SR] round |y| up to the next grid value with probability equal to the
 * fractional distance.  m - lo is exact (Sterbenz, or lo = 0) and hi - lo is
 * 0.5, 1 or 2, so f and f * 65536 are exact. */
int orc_e2m1_encode_sr(float y, uint32_t u16) {
  double m = fabs((double)y);
  int idx;
  if (m >= 6.0) {
    idx = 7;
  } else {
    int lo = 0;
    for (int i = 1; i < 8; ++i)
      if (kE2M1[i] <= m) lo = i;
    double f = (m - kE2M1[lo]) / (kE2M1[lo + 1] - kE2M1[lo]);
    idx = ((double)u16 < f * 65536.0) ? lo + 1 : lo;
  }
  return (signbit(y) ? 8 : 0) | idx;
}

/* array forms of the three encoders, for exhaustive checks */
int orc_e4m3_encode_n(const float* s, int64_t n, uint8_t* out) {
  if (!s || !out) return ORC_E_ARG;
  int bad = 0;
#pragma omp parallel for reduction(| : bad)
  for (int64_t i = 0; i < n; ++i) {
    const int b = orc_e4m3_encode(s[i]);
    if (b < 0) bad = 1;
    out[i] = (uint8_t)b;
  }
  return bad ? ORC_E_ARG : ORC_OK;
}

int orc_e2m1_encode_rne_n(const float* y, int64_t n, uint8_t* out) {
  if (!y || !out) return ORC_E_ARG;
#pragma omp parallel for
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)orc_e2m1_encode_rne(y[i]);
  return ORC_OK;
}

int orc_e2m1_encode_sr_n(const float* y, const uint16_t* u, int64_t n, uint8_t* out) {
  if (!y || !u || !out) return ORC_E_ARG;
#pragma omp parallel for
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)orc_e2m1_encode_sr(y[i], u[i]);
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* [PHILOX] Philox4x32-10                                               */
/* ------------------------------------------------------------------ */

/* One round: the two 32x32->64 products of counter words 0 and 2 with the
 * round multipliers; the high halves are xored with the other two counter
 * words and the key words, and the words are permuted. */
static void philox_round(uint32_t c[4], const uint32_t k[2]) {
  const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
  const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
  const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
  const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
  uint32_t n0 = hi1 ^ c[1] ^ k[0];
  uint32_t n1 = lo1;
  uint32_t n2 = hi0 ^ c[3] ^ k[1];
  uint32_t n3 = lo0;
  c[0] = n0;
  c[1] = n1;
  c[2] = n2;
  c[3] = n3;
}

/* Ten rounds; the key is bumped by the Weyl constants between rounds. */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
  uint32_t k[2] = {key[0], key[1]};
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k[0] += 0x9E3779B9u;
      k[1] += 0xBB67AE85u;
    }
    philox_round(c, k);
  }
  memcpy(out, c, sizeof c);
}

/* R6 */
uint32_t orc_sr_bits(uint64_t seed, uint32_t stream, uint64_t index) {
  const uint64_t g = index >> 3;
  const uint32_t ctr[4] = {(uint32_t)g, (uint32_t)(g >> 32), stream, 0u};
  const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  orc_philox4x32_10(ctr, key, out);
  const uint32_t word = out[(index & 7) >> 1];
  return (index & 1) ? (word >> 16) : (word & 0xFFFFu);
}

/* R6/R7: sign j of the Hadamard diagonal is -1 iff bit j of word 0 of
 * Philox(counter (0,0,2,0), key(rht_seed)) is set. */
int orc_sr_bits_n(uint64_t seed, uint32_t stream, uint64_t first, int64_t n, uint16_t* out) {
  if (!out) return ORC_E_ARG;
#pragma omp parallel for
  for (int64_t i = 0; i < n; ++i) out[i] = (uint16_t)orc_sr_bits(seed, stream, first + (uint64_t)i);
  return ORC_OK;
}

uint32_t orc_rht_sign_mask(uint64_t rht_seed) {
  const uint32_t ctr[4] = {0u, 0u, 2u, 0u};
  const uint32_t key[2] = {(uint32_t)rht_seed, (uint32_t)(rht_seed >> 32)};
  uint32_t out[4];
  orc_philox4x32_10(ctr, key, out);
  return out[0] & 0xFFFFu;
}

/* ------------------------------------------------------------------ */
/* inputs, transform, scales                                           */
/* ------------------------------------------------------------------ */

static float load_elem(const void* x, int dtype, int64_t i) {
  if (dtype == ORC_F32) return ((const float*)x)[i];
  /* bf16 is the top half of an fp32: widening is exact */
  uint32_t bits = (uint32_t)((const uint16_t*)x)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return f;
}

static int check_input(const void* x, int dtype, int64_t n) {
  int bad = 0;
#pragma omp parallel for reduction(| : bad)
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(load_elem(x, dtype, i))) bad = 1;
  return bad ? ORC_E_NONFINITE : ORC_OK;
}

/* R7: [RHT] one 16-chunk, in place. */
static void rht16(float v[16], uint32_t sign_mask) {
  for (int j = 0; j < 16; ++j)
    if ((sign_mask >> j) & 1u) v[j] = -v[j];
  for (int h = 1; h < 16; h <<= 1) {
    for (int i = 0; i < 16; ++i) {
      if (i & h) continue;
      const float a = v[i], b = v[i + h];
      v[i] = a + b;
      v[i + h] = a - b;
    }
  }
  for (int j = 0; j < 16; ++j) v[j] = 0.25f * v[j];
}

int orc_rht(const void* x, int dtype, int64_t rows, int64_t cols, uint64_t rht_seed, float* y) {
  if (!x || !y || (dtype != ORC_F32 && dtype != ORC_BF16)) return ORC_E_ARG;
  if (rows <= 0 || cols <= 0 || cols % 16) return ORC_E_SHAPE;
  int st = check_input(x, dtype, rows * cols);
  if (st) return st;
  const uint32_t mask = orc_rht_sign_mask(rht_seed);
#pragma omp parallel for
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t c0 = 0; c0 < cols; c0 += 16) {
      float v[16];
      for (int j = 0; j < 16; ++j) v[j] = load_elem(x, dtype, r * cols + c0 + j);
      rht16(v, mask);
      for (int j = 0; j < 16; ++j) y[r * cols + c0 + j] = v[j];
    }
  }
  return ORC_OK;
}

/* R1: [NVFP4] the FP32 per-tensor scale */
float orc_tensor_scale(float amax) {
  if (amax == 0.0f) return 1.0f;
  float s = 2688.0f / amax;
  if (isinf(s)) s = FLT_MAX;
  return s;
}

/* R2 and R3 for one block: returns the scale byte, writes the multiplier. */
static int block_scale(float amax_b, float s_enc, float* inv) {
  const float t = amax_b * s_enc;
  const float s = t / 6.0f;
  const int byte = orc_e4m3_encode(s);
  const float sb = (float)orc_e4m3_value(byte);
  if (sb == 0.0f) {
    *inv = 0.0f;
  } else {
    float q = s_enc / sb;
    *inv = isinf(q) ? FLT_MAX : q;
  }
  return byte;
}

static int encode(float x, float inv, int rounding, uint64_t seed, uint32_t stream, uint64_t index) {
  const float y = x * inv;
  if (rounding == ORC_RNE) return orc_e2m1_encode_rne(y);
  return orc_e2m1_encode_sr(y, orc_sr_bits(seed, stream, index));
}

static void put_code(uint8_t* row, int64_t k, int code) {
  if (k & 1)
    row[k >> 1] = (uint8_t)((row[k >> 1] & 0x0F) | (code << 4));
  else
    row[k >> 1] = (uint8_t)((row[k >> 1] & 0xF0) | code);
}

static float tensor_amax(const float* v, int64_t n) {
  float amax = 0.0f;
#pragma omp parallel for reduction(max : amax)
  for (int64_t i = 0; i < n; ++i) {
    const float a = fabsf(v[i]);
    if (a > amax) amax = a;
  }
  return amax;
}

/* widen (and optionally transform) the input into a float array */
static float* to_float(const void* x, int dtype, int64_t rows, int64_t cols, int rht, uint64_t rht_seed) {
  float* v = (float*)malloc((size_t)(rows * cols) * sizeof(float));
  if (!v) return NULL;
  if (rht) {
    orc_rht(x, dtype, rows, cols, rht_seed, v);
  } else {
#pragma omp parallel for
    for (int64_t i = 0; i < rows * cols; ++i) v[i] = load_elem(x, dtype, i);
  }
  return v;
}

/* ------------------------------------------------------------------ */
/* quantizers                                                          */
/* ------------------------------------------------------------------ */

int orc_quantize_1d(const void* x, int dtype, int64_t rows, int64_t cols,
                    int rounding, uint64_t seed, int rht, uint64_t rht_seed,
                    uint8_t* codes, uint8_t* scales, float* tensor_scale,
                    uint8_t* codes_t, uint8_t* scales_t) {
  if (!x || !codes || !scales || !tensor_scale) return ORC_E_ARG;
  if (dtype != ORC_F32 && dtype != ORC_BF16) return ORC_E_ARG;
  if (rounding != ORC_RNE && rounding != ORC_SR) return ORC_E_ARG;
  if (rht != 0 && rht != 1) return ORC_E_ARG;
  if ((codes_t == NULL) != (scales_t == NULL)) return ORC_E_ARG;
  if (rows <= 0 || cols <= 0 || cols % 16) return ORC_E_SHAPE;
  if (codes_t && rht) return ORC_E_ARG;
  if (codes_t && rows % 16) return ORC_E_SHAPE;
  int st = check_input(x, dtype, rows * cols);
  if (st) return st;

  float* v = to_float(x, dtype, rows, cols, rht, rht_seed);
  if (!v) return ORC_E_ARG;
  const float amax = tensor_amax(v, rows * cols);
  const float s_enc = orc_tensor_scale(amax);
  tensor_scale[0] = s_enc;
  tensor_scale[1] = amax;

  /* rowwise: blocks of 16 consecutive elements of a row; SR stream 0,
   * element index r * cols + c */
#pragma omp parallel for
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < cols / 16; ++b) {
      const float* blk = v + r * cols + b * 16;
      float amax_b = 0.0f;
      for (int j = 0; j < 16; ++j)
        if (fabsf(blk[j]) > amax_b) amax_b = fabsf(blk[j]);
      float inv;
      scales[r * (cols / 16) + b] = (uint8_t)block_scale(amax_b, s_enc, &inv);
      for (int j = 0; j < 16; ++j) {
        const int64_t c = b * 16 + j;
        put_code(codes + r * (cols / 2), c,
                 encode(blk[j], inv, rounding, seed, 0u, (uint64_t)(r * cols + c)));
      }
    }
  }

  /* columnwise copy: blocks of 16 consecutive rows of a column, written as
   * rows of the transposed tensor; SR stream 1, index c * rows + r */
  if (codes_t) {
#pragma omp parallel for
    for (int64_t c = 0; c < cols; ++c) {
      for (int64_t b = 0; b < rows / 16; ++b) {
        float amax_b = 0.0f;
        for (int j = 0; j < 16; ++j) {
          const float a = fabsf(v[(b * 16 + j) * cols + c]);
          if (a > amax_b) amax_b = a;
        }
        float inv;
        scales_t[c * (rows / 16) + b] = (uint8_t)block_scale(amax_b, s_enc, &inv);
        for (int j = 0; j < 16; ++j) {
          const int64_t r = b * 16 + j;
          put_code(codes_t + c * (rows / 2), r,
                   encode(v[r * cols + c], inv, rounding, seed, 1u, (uint64_t)(c * rows + r)));
        }
      }
    }
  }
  free(v);
  return ORC_OK;
}

int orc_quantize_2d(const void* w, int dtype, int64_t rows, int64_t cols,
                    int rounding, uint64_t seed,
                    uint8_t* codes, uint8_t* scales, float* tensor_scale,
                    uint8_t* codes_t, uint8_t* scales_t) {
  if (!w || !codes || !scales || !tensor_scale) return ORC_E_ARG;
  if (dtype != ORC_F32 && dtype != ORC_BF16) return ORC_E_ARG;
  if (rounding != ORC_RNE && rounding != ORC_SR) return ORC_E_ARG;
  if ((codes_t == NULL) != (scales_t == NULL)) return ORC_E_ARG;
  if (rows <= 0 || cols <= 0 || rows % 16 || cols % 16) return ORC_E_SHAPE;
  int st = check_input(w, dtype, rows * cols);
  if (st) return st;

  float* v = to_float(w, dtype, rows, cols, 0, 0);
  if (!v) return ORC_E_ARG;
  const float amax = tensor_amax(v, rows * cols);
  const float s_enc = orc_tensor_scale(amax);
  tensor_scale[0] = s_enc;
  tensor_scale[1] = amax;

  /* [2D] one scale per aligned 16x16 tile; each element is encoded once (SR
   * index r * cols + c of W, stream 0) and the same code goes to both
   * copies, so the transposed copy is W^T's quantization exactly. */
#pragma omp parallel for
  for (int64_t tr = 0; tr < rows / 16; ++tr) {
    for (int64_t tc = 0; tc < cols / 16; ++tc) {
      float amax_t = 0.0f;
      for (int i = 0; i < 16; ++i)
        for (int j = 0; j < 16; ++j) {
          const float a = fabsf(v[(tr * 16 + i) * cols + tc * 16 + j]);
          if (a > amax_t) amax_t = a;
        }
      float inv;
      const uint8_t byte = (uint8_t)block_scale(amax_t, s_enc, &inv);
      for (int i = 0; i < 16; ++i) {
        const int64_t r = tr * 16 + i;
        scales[r * (cols / 16) + tc] = byte;
        for (int j = 0; j < 16; ++j) {
          const int64_t c = tc * 16 + j;
          const int code = encode(v[r * cols + c], inv, rounding, seed, 0u, (uint64_t)(r * cols + c));
          put_code(codes + r * (cols / 2), c, code);
          if (codes_t) put_code(codes_t + c * (rows / 2), r, code);
        }
      }
      if (scales_t)
        for (int j = 0; j < 16; ++j) scales_t[(tc * 16 + j) * (rows / 16) + tr] = byte;
    }
  }
  free(v);
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* dequantize and GEMM                                                 */
/* ------------------------------------------------------------------ */

static double deq(const uint8_t* codes, const uint8_t* scales, double s_enc, int64_t K,
                  int64_t i, int64_t k) {
  const uint8_t byte = codes[i * (K / 2) + k / 2];
  const int code = (k & 1) ? (byte >> 4) : (byte & 0x0F);
  return orc_e2m1_value(code) * orc_e4m3_value(scales[i * (K / 16) + k / 16]) / s_enc;
}

int orc_dequantize(const uint8_t* codes, const uint8_t* scales, float s_enc,
                   int64_t rows, int64_t cols, double* out) {
  if (!codes || !scales || !out) return ORC_E_ARG;
  if (rows <= 0 || cols <= 0 || cols % 16) return ORC_E_SHAPE;
#pragma omp parallel for
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) out[r * cols + c] = deq(codes, scales, s_enc, cols, r, c);
  return ORC_OK;
}

/* [ACC] C_ij = sum_k deq(A)_ik * deq(B)_jk, accumulated in double */
static void dot(const uint8_t* a_codes, const uint8_t* a_scales, double sa,
                const uint8_t* b_codes, const uint8_t* b_scales, double sb,
                int64_t K, int64_t i, int64_t j, double* c, double* abs_sum) {
  double acc = 0.0, acc_abs = 0.0;
  for (int64_t k = 0; k < K; ++k) {
    const double p = deq(a_codes, a_scales, sa, K, i, k) * deq(b_codes, b_scales, sb, K, j, k);
    acc += p;
    acc_abs += fabs(p);
  }
  *c = acc;
  *abs_sum = acc_abs;
}

int orc_gemm(const uint8_t* a_codes, const uint8_t* a_scales, float a_s_enc,
             const uint8_t* b_codes, const uint8_t* b_scales, float b_s_enc,
             int64_t M, int64_t N, int64_t K, double* c, double* abs_sum) {
  if (!a_codes || !a_scales || !b_codes || !b_scales || !c || !abs_sum) return ORC_E_ARG;
  if (M <= 0 || N <= 0 || K <= 0 || K % 16) return ORC_E_SHAPE;
#pragma omp parallel for
  for (int64_t i = 0; i < M; ++i)
    for (int64_t j = 0; j < N; ++j)
      dot(a_codes, a_scales, a_s_enc, b_codes, b_scales, b_s_enc, K, i, j, &c[i * N + j],
          &abs_sum[i * N + j]);
  return ORC_OK;
}

int orc_gemm_sample(const uint8_t* a_codes, const uint8_t* a_scales, float a_s_enc,
                    const uint8_t* b_codes, const uint8_t* b_scales, float b_s_enc,
                    int64_t M, int64_t N, int64_t K,
                    const int64_t* ii, const int64_t* jj, int64_t count,
                    double* c, double* abs_sum) {
  if (!a_codes || !a_scales || !b_codes || !b_scales || !ii || !jj || !c || !abs_sum)
    return ORC_E_ARG;
  if (M <= 0 || N <= 0 || K <= 0 || K % 16) return ORC_E_SHAPE;
  for (int64_t t = 0; t < count; ++t)
    if (ii[t] < 0 || ii[t] >= M || jj[t] < 0 || jj[t] >= N) return ORC_E_ARG;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < count; ++t)
    dot(a_codes, a_scales, a_s_enc, b_codes, b_scales, b_s_enc, K, ii[t], jj[t], &c[t], &abs_sum[t]);
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* MXFP4 (the format the pages compare NVFP4 against)                  */
/* ------------------------------------------------------------------ */

/* [MX] E8M0 scale exponent of a 32-element block: floor(log2(amax)) - 2,
 * where 2 is the exponent of E2M1's largest normal (6 = 1.5 * 2^2), clamped
 * to the E8M0 range [-127, 127]; an all-zero block takes -127 (byte 0). */
static int mx_scale_exponent(float amax) {
  if (amax == 0.0f) return -127;
  int e;
  frexp((double)amax, &e); /* amax = f * 2^e with f in [0.5, 1): floor(log2) = e - 1 */
  int s = (e - 1) - 2;
  if (s < -127) s = -127;
  if (s > 127) s = 127;
  return s;
}

/* [MX] 1D MXFP4 along cols: each block of 32 consecutive elements of a row
 * gets the E8M0 byte s + 127 and each element the E2M1 code of V / 2^s by R4
 * (nearest, ties to the even code, saturating at 6, sign kept).  V / 2^s is
 * formed exactly in double; narrowing it to float changes only values below
 * 2^-126, which encode to a signed zero either way. */
int orc_mx_quantize(const void* x, int dtype, int64_t rows, int64_t cols, uint8_t* codes,
                    uint8_t* scales) {
  if (!x || !codes || !scales) return ORC_E_ARG;
  if (dtype != ORC_F32 && dtype != ORC_BF16) return ORC_E_ARG;
  if (rows <= 0 || cols <= 0 || cols % 32) return ORC_E_SHAPE;
  int st = check_input(x, dtype, rows * cols);
  if (st) return st;
#pragma omp parallel for
  for (int64_t r = 0; r < rows; ++r) {
    uint8_t* crow = codes + r * (cols / 2);
    for (int64_t b = 0; b < cols / 32; ++b) {
      float amax = 0.0f;
      for (int k = 0; k < 32; ++k) {
        const float a = fabsf(load_elem(x, dtype, r * cols + 32 * b + k));
        if (a > amax) amax = a;
      }
      const int s = mx_scale_exponent(amax);
      scales[r * (cols / 32) + b] = (uint8_t)(s + 127);
      for (int k = 0; k < 32; ++k) {
        const double y = ldexp((double)load_elem(x, dtype, r * cols + 32 * b + k), -s);
        put_code(crow, 32 * b + k, orc_e2m1_encode_rne((float)y));
      }
    }
  }
  return ORC_OK;
}

/* [MX] value of an E8M0 byte: 2^(byte - 127); 0xFF is NaN */
double orc_e8m0_value(int byte) {
  if ((byte & 0xFF) == 0xFF) return NAN;
  return ldexp(1.0, (byte & 0xFF) - 127);
}

static double mx_deq(const uint8_t* codes, const uint8_t* scales, int64_t K, int64_t i, int64_t k) {
  const uint8_t byte = codes[i * (K / 2) + k / 2];
  const int code = (k & 1) ? (byte >> 4) : (byte & 0x0F);
  return orc_e2m1_value(code) * orc_e8m0_value(scales[i * (K / 32) + k / 32]);
}

/* out[r][c] = e2m1(code) * 2^(scale - 127), in double */
int orc_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                      double* out) {
  if (!codes || !scales || !out) return ORC_E_ARG;
  if (rows <= 0 || cols <= 0 || cols % 32) return ORC_E_SHAPE;
#pragma omp parallel for
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) out[r * cols + c] = mx_deq(codes, scales, cols, r, c);
  return ORC_OK;
}

/* [ACC] C_ij = sum_k deq(A)_ik * deq(B)_jk in double, for the (ii, jj) pairs
 * given (or every pair when ii == NULL: count must be M * N, row-major). */
int orc_mx_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, const int64_t* ii,
                const int64_t* jj, int64_t count, double* c, double* abs_sum) {
  if (!a_codes || !a_scales || !b_codes || !b_scales || !c || !abs_sum) return ORC_E_ARG;
  if (M <= 0 || N <= 0 || K <= 0 || K % 32) return ORC_E_SHAPE;
  if (!ii != !jj) return ORC_E_ARG;
  if (!ii && count != M * N) return ORC_E_ARG;
  for (int64_t t = 0; ii && t < count; ++t)
    if (ii[t] < 0 || ii[t] >= M || jj[t] < 0 || jj[t] >= N) return ORC_E_ARG;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < count; ++t) {
    const int64_t i = ii ? ii[t] : t / N, j = jj ? jj[t] : t % N;
    double acc = 0.0, acc_abs = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      const double p = mx_deq(a_codes, a_scales, K, i, k) * mx_deq(b_codes, b_scales, K, j, k);
      acc += p;
      acc_abs += fabs(p);
    }
    c[t] = acc;
    abs_sum[t] = acc_abs;
  }
  return ORC_OK;
}
