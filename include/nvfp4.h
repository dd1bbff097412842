/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 quantizer and block-scaled
 * FP4 GEMM library (libnvfp4.so).
 *
 * What the calls compute (sources cited by page title and section):
 *   "Pretraining Large Language Models with NVFP4" (gist.science summary),
 *   Technische samenvatting:
 *     2A   NVFP4: E2M1 (4-bit) elements in blocks of 16, one E4M3 scale per
 *          block, one FP32 scale per tensor that brings the whole tensor into
 *          the range one block can express;
 *     2B.2 a 16x16 random Hadamard transform on the inputs of the Wgrad GEMM;
 *     2B.3 16x16 blocks for weights, so W and W^T quantize identically; 1x16
 *          blocks for activations and gradients;
 *     2B.4 stochastic rounding for gradients, round-to-nearest-even otherwise.
 *   "NVIDIA acelera el preentrenamiento de LLM: NVFP4 en Blackwell junto con
 *   JAX y MaxText", "Como Funciona Mixed-Precision con NVFP4": NVFP4 GEMMs
 *   on weights and activations with FP32 (or BF16) accumulation.
 *
 * Quantized tensor of R x C elements, quantized along C (rows of 16):
 *   codes   uint8 [R][C/2]   two E2M1 codes per byte, element 2k in the low
 *                            nibble; code = sign << 3 | index into
 *                            {0, .5, 1, 1.5, 2, 3, 4, 6}
 *   scales  uint8 [R][C/16]  OCP E4M3 (bias 7, max 448) block scales
 *   tensor_scale float[2]    [0] = S_enc = 2688 / amax (1 if amax == 0,
 *                            FLT_MAX if the quotient overflows),
 *                            [1] = amax (the kernel's reduction target)
 *   value(r, c) = e2m1(code) * e4m3(scale) / S_enc
 * The block scale is E4M3_RNE_sat(amax_b * S_enc / 6); each element is
 * encoded from y = x * (S_enc / block_scale) (0 for a zero scale, at most
 * FLT_MAX).  Random bits for stochastic rounding: Philox4x32-10 keyed by the
 * seed; element i draws 16 bits (half i & 1 of word (i & 7) >> 1 of counter
 * (i >> 3, stream, 0)) and rounds |y| up iff they are below 2^16 times its
 * fractional position between the two neighbouring E2M1 values.
 *
 * Conventions for every call:
 *   - All buffers are DEVICE pointers owned by the caller; the library never
 *     allocates, frees or synchronizes.  Outputs must not overlap inputs or
 *     each other.  Work is enqueued on `stream` (a hipStream_t, NULL for the
 *     default stream) and is asynchronous.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     negative status means nothing was enqueued.  NVFP4_ERR_HIP means a
 *     launch failed (text in nvfp4_last_error()).  Faults during execution
 *     surface at the caller's next synchronization.
 *   - Inputs must be finite: NaN or Inf inputs are outside the contract and
 *     are not detected.
 *   - Sizes: a tensor holds at most 2^40 elements (rows * cols); a GEMM's
 *     M * K, N * K and M * N are each at most 2^40, with M at most
 *     65535 * 128 (NVFP4) or 65535 * 64 (MXFP4).  Larger sizes give
 *     NVFP4_ERR_SHAPE.
 *   - Thread-safe: no state besides a per-device cache of the CU count and
 *     each thread's last error text.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum nvfp4_status {
  NVFP4_OK = 0,
  NVFP4_ERR_ARG = -1,   /* null pointer, bad enum, or an invalid combination */
  NVFP4_ERR_SHAPE = -2, /* size <= 0, not a multiple of 16 where required, or too large */
  NVFP4_ERR_ALIGN = -3, /* pointer alignment below what the call states */
  NVFP4_ERR_HIP = -4    /* a HIP call failed; see nvfp4_last_error() */
};

enum nvfp4_dtype { NVFP4_F32 = 0, NVFP4_BF16 = 1 };
enum nvfp4_rounding { NVFP4_RNE = 0, NVFP4_SR = 1 };

/*
 * 1D NVFP4 quantization of x [rows][cols] (row-major, dtype f32 or bf16)
 * along cols: blocks of 16 consecutive elements of a row (2A, 2B.3 1x16).
 *   rounding  NVFP4_RNE or NVFP4_SR (2B.4); SR draws Philox stream 0 with
 *             element index r * cols + c.
 *   rht       1: every contiguous 16-chunk of every row is first replaced by
 *             1/4 * H16 * diag(sigma) * chunk (2B.2), H16 the Sylvester
 *             Hadamard matrix, evaluated in fp32 by the butterfly with
 *             h = 1, 2, 4, 8; sigma_j = -1 iff bit j of the low 16 bits of
 *             word 0 of Philox(key = rht_seed, counter (0, 0, 2, 0)).  The
 *             amax is taken after the transform.
 *   codes [rows][cols/2], scales [rows][cols/16], tensor_scale[2]: outputs.
 *   codes_t [cols][rows/2], scales_t [cols][rows/16]: optional columnwise
 *             copy (both NULL or both set): blocks of 16 consecutive rows of
 *             each column, stored as rows of the transpose, same S_enc; SR
 *             uses stream 1 with element index c * rows + r.  Requires
 *             rows % 16 == 0 and rht == 0.
 * Shapes: rows >= 1, cols >= 16, cols % 16 == 0.
 * Alignment: x 16 bytes; codes, codes_t 8 bytes; tensor_scale 4 bytes.
 */
int nvfp4_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int rounding,
                   uint64_t seed, int rht, uint64_t rht_seed, uint8_t* codes, uint8_t* scales,
                   float* tensor_scale, uint8_t* codes_t, uint8_t* scales_t, void* stream);

/*
 * 2D NVFP4 quantization of a weight w [rows][cols] with one E4M3 scale per
 * aligned 16x16 tile (2B.3).  Each element is encoded once (SR: stream 0,
 * index r * cols + c) and written to both copies, so the transposed copy is
 * the transpose of w's codes and scales under either rounding.  With RNE it
 * is also exactly nvfp4_quantize_2d(w^T); with SR it is not, since that
 * call would draw element (r, c) of w at index c * rows + r.
 *   codes [rows][cols/2], scales [rows][cols/16] (a tile's byte is stored on
 *   each of its 16 rows, so GEMM operands have one layout), tensor_scale[2].
 *   codes_t [cols][rows/2], scales_t [cols][rows/16]: transposed copy, both
 *   NULL or both set.
 * Shapes: rows, cols >= 16 and multiples of 16.  Alignment as nvfp4_quantize.
 */
int nvfp4_quantize_2d(const void* w, int dtype, int64_t rows, int64_t cols, int rounding,
                      uint64_t seed, uint8_t* codes, uint8_t* scales, float* tensor_scale,
                      uint8_t* codes_t, uint8_t* scales_t, void* stream);

/*
 * Cast-transpose: the two NVFP4 copies of x [rows][cols] that a training
 * step uses, made from x in its own layout (x^T is never formed; x is read
 * once per pass instead of once per copy and pass).  2B.2 puts the Hadamard
 * transform on the Wgrad inputs only, and Wgrad contracts over the rows of
 * x, so the columnwise copy is the one that may take it:
 *   codes [rows][cols/2], scales [rows][cols/16], tensor_scale[2]: exactly
 *     nvfp4_quantize(x, dtype, rows, cols, rounding, seed, rht = 0);
 *   codes_t [cols][rows/2], scales_t [cols][rows/16], tensor_scale_t[2]:
 *     exactly nvfp4_quantize(x^T, dtype, cols, rows, rounding, seed_t,
 *     rht_t, rht_seed), i.e. blocks of 16 consecutive rows of a column, with
 *     their own amax (after the transform when rht_t = 1) and S_enc; SR draws
 *     stream 0 of seed_t with element index c * rows + r.
 * Pass a seed_t different from seed for draws independent of the rowwise
 * copy's.  All six outputs are required.
 * Shapes: rows >= 16, rows % 16 == 0, cols >= 16, cols % 16 == 0.
 * Alignment: x 16 bytes; codes, codes_t 8 bytes; tensor scales 4 bytes.
 */
int nvfp4_quantize_cast_transpose(const void* x, int dtype, int64_t rows, int64_t cols, int rounding,
                                  uint64_t seed, uint64_t seed_t, int rht_t, uint64_t rht_seed,
                                  uint8_t* codes, uint8_t* scales, float* tensor_scale,
                                  uint8_t* codes_t, uint8_t* scales_t, float* tensor_scale_t,
                                  void* stream);

/*
 * The random Hadamard transform of nvfp4_quantize (rht = 1) alone: y [rows]
 * [cols] fp32 = transform of every contiguous 16-chunk of every row of x.
 * nvfp4_quantize(x, rht = 1) equals nvfp4_quantize(y as f32, rht = 0) bit
 * for bit.  Shapes: rows >= 1, cols % 16 == 0.  Alignment: x, y 16 bytes.
 */
int nvfp4_rht(const void* x, int dtype, int64_t rows, int64_t cols, uint64_t rht_seed, float* y,
              void* stream);

/*
 * Dequantization of an NVFP4 tensor of rows x cols (codes [rows][cols/2],
 * scales [rows][cols/16], tensor_scale[0] = S_enc, read on the device):
 * out[r][c] = e2m1(code) * e4m3(scale) / S_enc (2A: the block scale and the
 * tensor scale undo the encoding's scaling).  The product is exact in fp32,
 * so an fp32 output is the correctly rounded quotient; out_dtype NVFP4_BF16
 * writes that fp32 value rounded to nearest-even bf16.  Scale bytes are those
 * the quantizers produce (0x00 .. 0x7E).  Works for any copy, rowwise or
 * transposed (a transposed copy dequantizes to x^T).
 * Shapes: rows >= 1, cols >= 16, cols % 16 == 0.
 * Alignment: codes 8 bytes, tensor_scale 4 bytes, out 16 bytes.
 */
int nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                     int64_t rows, int64_t cols, int out_dtype, void* out, void* stream);

/*
 * C [M][N] fp32 = deq(A) . deq(B)^T with FP32 accumulation, where A is an
 * NVFP4 tensor of M x K (codes [M][K/2], scales [M][K/16], tensor scale
 * a_tensor_scale[0]) and B one of N x K, both quantized along K.  Tensor
 * scales are read on the device (the outputs of the quantizers), so no host
 * synchronization is needed.  Any result within
 * 1e-5 * sum_k |deq(A)_ik deq(B)_jk| of the exact sum is correct.
 * Error model: each operand value code * scale is exact in fp16 and every
 * product exact in fp32; each 16-element block's products are added to an
 * fp32 accumulator by one matrix instruction, and the two tensor scales are
 * then applied as (acc * (1 / S_A)) * (1 / S_B).  The accumulation rounds
 * about once per block, so the error is at most about
 * (K / 16 + 2) * 2^-24 * sum_k |a_ik b_jk| (while the sum, acc / S_A and
 * the result stay within fp32's normal range).  That worst case, in which
 * every rounding has the same sign, guarantees the 1e-5 tolerance for K up
 * to about 2,600.  Beyond it the tolerance is met by data whose roundings
 * do not all align, and has been measured over every output: 1e-8 .. 7e-8
 * of the sum for the layer's fprop, dgrad and wgrad GEMMs (K = 5120,
 * 20480, 8192), and 2.7e-6 when every product is non-negative at K = 20480
 * (no cancellation at all).  Scale
 * bytes are those the quantizers produce (0x00 .. 0x7E); the kernels read
 * the low seven bits of a byte.
 * Shapes: M, N >= 1, K >= 16, K % 16 == 0.  Alignment: codes 8 bytes, C 4
 * bytes (16-byte aligned codes and scales, M and N multiples of 256 and
 * K % 512 == 0 take the fast path).
 */
int nvfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_tensor_scale,
               const uint8_t* b_codes, const uint8_t* b_scales, const float* b_tensor_scale,
               int64_t M, int64_t N, int64_t K, float* c, void* stream);

/*
 * MXFP4, the format the NVFP4 recipe is measured against (2A: blocks of 32
 * elements with a UE8M0 scale instead of 16 with E4M3, and no per-tensor
 * scale).  Conversion as OCP Microscaling Formats (MX) v1.0, section 6.3:
 * a block of 32 consecutive elements of a row with absolute maximum amax
 * shares X = 2^(floor(log2 amax) - 2), stored as the E8M0 byte
 * log2(X) + 127 clamped to >= 0 (0 for an all-zero block); each element is
 * x / X rounded to E2M1, nearest-even, saturating at 6, sign kept.
 *   codes [rows][cols/2] (element 2k in the low nibble), scales [rows][cols/32].
 * Shapes: rows >= 1, cols >= 32, cols % 32 == 0.  Alignment: x 16, codes 8.
 */
int mxfp4_quantize(const void* x, int dtype, int64_t rows, int64_t cols, uint8_t* codes,
                   uint8_t* scales, void* stream);

/*
 * out [rows][cols] = e2m1(code) * 2^(scale - 127), exact in fp32; bf16 output
 * (out_dtype NVFP4_BF16) is that value rounded to nearest-even.  Shapes as
 * mxfp4_quantize.  Alignment: codes 8 bytes, out 16 bytes.
 */
int mxfp4_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                     int out_dtype, void* out, void* stream);

/*
 * C [M][N] fp32 = deq(A) . deq(B)^T for MXFP4 A [M x K] and B [N x K], both
 * quantized along K, with FP32 accumulation on gfx950's scaled FP4 matrix
 * instruction (products of E2M1 values and power-of-two scales are exact).
 * Any result within 1e-5 * sum_k |deq(A)_ik deq(B)_jk| of the exact sum is
 * correct.  Shapes: M, N >= 1, K >= 32, K % 32 == 0 (M, N and K multiples
 * of 256 with 8-byte aligned scales take the fast path).
 * Alignment: codes 16 bytes, C 4 bytes.
 */
int mxfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
               const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, float* c, void* stream);

/*
 * nvfp4_gemm with epilogue options (for a training step: gradient
 * accumulation, a 16-bit output, and the amax the next quantization needs):
 *   C [M][N] = deq(A) . deq(B)^T + beta * C_old, where the product term is
 *   computed as nvfp4_gemm does (fp32, then times 1/S_a and 1/S_b), C_old is
 *   read only when beta != 0, and the sum is one fp32 add of the rounded
 *   beta * C_old;
 *   c_dtype NVFP4_F32 stores fp32, NVFP4_BF16 the fp32 result rounded to
 *   nearest-even bf16 (C_old is then read as bf16);
 *   c_amax (NULL or a device float): set to max |stored C| over the call,
 *   so a following nvfp4_quantize_with_amax of C can skip its amax pass.
 * Shapes as nvfp4_gemm.  beta must be finite.  Alignment: codes 8 bytes, C 4
 * (fp32) or 2 (bf16) bytes, c_amax 4 bytes.
 */
int nvfp4_gemm_ex(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_tensor_scale,
                  const uint8_t* b_codes, const uint8_t* b_scales, const float* b_tensor_scale,
                  int64_t M, int64_t N, int64_t K, void* c, int c_dtype, float beta, float* c_amax,
                  void* stream);

/*
 * nvfp4_quantize without its first pass: tensor_scale[1] must already hold
 * the amax that nvfp4_quantize would compute (of x, or of its transform
 * when rht = 1), e.g. the c_amax of the nvfp4_gemm_ex that produced x.
 * With that amax the outputs are bit-identical to nvfp4_quantize's, from a
 * single read of x.  No transposed copy.  Arguments otherwise as
 * nvfp4_quantize.
 */
int nvfp4_quantize_with_amax(const void* x, int dtype, int64_t rows, int64_t cols, int rounding,
                             uint64_t seed, int rht, uint64_t rht_seed, uint8_t* codes,
                             uint8_t* scales, float* tensor_scale, void* stream);

/* Static text for a status code. */
const char* nvfp4_status_string(int status);
/* Text of the last NVFP4_ERR_HIP on the calling thread ("" if none). */
const char* nvfp4_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4_H */
