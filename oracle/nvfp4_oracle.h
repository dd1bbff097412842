/*
 * nvfp4_oracle.h -- plain CPU reference ("the oracle") for the NVFP4 quantizer
 * and the block-scaled FP4 GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  The product (the HIP
 * library under bit_block_scaled_quant_amd/) shares no code, header, table or
 * constant with it and never calls it.
 *
 * Sources (the pages cite no equations; every step below is either the
 * format's published definition or the plainest reading of a page passage):
 *   [NVFP4]  "Pretraining Large Language Models with NVFP4" (gist.science
 *            summary), Technische samenvatting, section 2A "Het NVFP4 Formaat":
 *            16-element blocks, E4M3 block scale, FP32 per-tensor scale,
 *            two-level scaling.
 *   [RHT]    same page, section 2B.2 "Random Hadamard Transforms": 16x16
 *            transform on the inputs of the Wgrad GEMM.
 *   [2D]     same page, section 2B.3 "Twee-dimensionale (2D) Blokschaling":
 *            16x16 weight blocks so W and W^T quantize identically.
 *   [SR]     same page, section 2B.4 "Stochastisch Afronden" and the lay part
 *            "De Vier Slimme Trucs" (the 3.4 -> 3 or 4 example): stochastic
 *            rounding of gradients, probability of rounding up equals the
 *            fractional distance.
 *   [ACC]    "NVIDIA acelera el preentrenamiento de LLM: NVFP4 en Blackwell
 *            junto con JAX y MaxText", section "Como Funciona Mixed-Precision
 *            con NVFP4": NVFP4 on weights and activations in the GEMMs, BF16
 *            or FP32 accumulators.
 *   [E2M1], [E4M3]  OCP Microscaling Formats (MX) v1.0 and OCP 8-bit Floating
 *            Point (OFP8) specifications: FP4 E2M1 magnitudes
 *            {0,0.5,1,1.5,2,3,4,6}; E4M3 bias 7, max 448, subnormals m*2^-9,
 *            0x7F/0xFF NaN.
 *   [PHILOX] Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
 *            1, 2, 3", SC'11: Philox4x32 with 10 rounds.
 *   [MX]     OCP Microscaling Formats (MX) v1.0, section 6.3 (conversion of a
 *            vector to an MX block): MXFP4 = 32-element blocks of E2M1 with an
 *            E8M0 (power-of-two) scale 2^(floor(log2(amax)) - emax_elem), the
 *            format "Pretraining Large Language Models with NVFP4",
 *            Technische samenvatting 2A, compares NVFP4 against (32 vs 16
 *            elements, UE8M0 vs E4M3 scales).
 *
 * Parity status: every function here is pinned by tests/test_oracle_*.py
 * (closed forms, exhaustive codec checks, invariants, library routines,
 * brute force).  None is "parity unpinned" except where a test file says so.
 *
 * All functions return 0 on success or a negative ORC_E_* code.
 */
#ifndef NVFP4_ORACLE_H
#define NVFP4_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  ORC_OK = 0,
  ORC_E_ARG = -1,      /* null pointer or bad enum */
  ORC_E_SHAPE = -2,    /* size not a positive multiple of 16 where required */
  ORC_E_NONFINITE = -3 /* NaN or Inf in the input: outside the contract */
};

/* dtype of a quantizer input */
enum { ORC_F32 = 0, ORC_BF16 = 1 };
/* rounding mode of the element encode */
enum { ORC_RNE = 0, ORC_SR = 1 };

/* --- format codecs --------------------------------------------------- */
double orc_e2m1_value(int code);          /* 4-bit code -> value      */
double orc_e4m3_value(int byte);          /* 8-bit code -> value (NaN for 0x7F/0xFF) */
int orc_e4m3_encode(float s);             /* s >= 0 -> byte, RNE, saturating */
int orc_e2m1_encode_rne(float y);         /* -> 4-bit code            */
int orc_e2m1_encode_sr(float y, uint32_t u16); /* u16 in [0, 65535]  */
/* the same over arrays (exhaustive checks) */
int orc_e4m3_encode_n(const float* s, int64_t n, uint8_t* out);
int orc_e2m1_encode_rne_n(const float* y, int64_t n, uint8_t* out);
int orc_e2m1_encode_sr_n(const float* y, const uint16_t* u, int64_t n, uint8_t* out);

/* --- random bits ----------------------------------------------------- */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
uint32_t orc_sr_bits(uint64_t seed, uint32_t stream, uint64_t index);
/* out[t] = orc_sr_bits(seed, stream, first + t) */
int orc_sr_bits_n(uint64_t seed, uint32_t stream, uint64_t first, int64_t n, uint16_t* out);
uint32_t orc_rht_sign_mask(uint64_t rht_seed); /* bit j set => sign j is -1 */

/* --- transform and scales -------------------------------------------- */
/* y[r][c] = RHT of every contiguous 16-chunk of every row, fp32 */
int orc_rht(const void* x, int dtype, int64_t rows, int64_t cols, uint64_t rht_seed, float* y);
float orc_tensor_scale(float amax);

/* --- quantizers ------------------------------------------------------ */
/* 1D blocks of 16 along cols.  codes [rows][cols/2], scales [rows][cols/16],
 * tensor_scale[0] = S_enc, [1] = amax.  If codes_t is non-NULL, also the
 * columnwise copy (blocks of 16 rows per column): codes_t [cols][rows/2],
 * scales_t [cols][rows/16]; requires rows % 16 == 0 and rht == 0. */
int orc_quantize_1d(const void* x, int dtype, int64_t rows, int64_t cols,
                    int rounding, uint64_t seed, int rht, uint64_t rht_seed,
                    uint8_t* codes, uint8_t* scales, float* tensor_scale,
                    uint8_t* codes_t, uint8_t* scales_t);
/* 2D 16x16 tiles.  scales [rows][cols/16] carry each tile's byte on all 16 of
 * its rows; codes_t/scales_t (may be NULL) are the exact transposes. */
int orc_quantize_2d(const void* w, int dtype, int64_t rows, int64_t cols,
                    int rounding, uint64_t seed,
                    uint8_t* codes, uint8_t* scales, float* tensor_scale,
                    uint8_t* codes_t, uint8_t* scales_t);
/* out[r][c] = e2m1(code) * e4m3(scale) / S_enc, in double */
int orc_dequantize(const uint8_t* codes, const uint8_t* scales, float s_enc,
                   int64_t rows, int64_t cols, double* out);

/* --- GEMM ------------------------------------------------------------ */
/* C = deq(A) . deq(B)^T in double; abs_sum[i][j] = sum_k |deq(A)_ik deq(B)_jk|.
 * A: codes [M][K/2], scales [M][K/16]; B: codes [N][K/2], scales [N][K/16]. */
int orc_gemm(const uint8_t* a_codes, const uint8_t* a_scales, float a_s_enc,
             const uint8_t* b_codes, const uint8_t* b_scales, float b_s_enc,
             int64_t M, int64_t N, int64_t K, double* c, double* abs_sum);
/* the same for a list of (i, j) output positions */
int orc_gemm_sample(const uint8_t* a_codes, const uint8_t* a_scales, float a_s_enc,
                    const uint8_t* b_codes, const uint8_t* b_scales, float b_s_enc,
                    int64_t M, int64_t N, int64_t K,
                    const int64_t* ii, const int64_t* jj, int64_t count,
                    double* c, double* abs_sum);

int orc_num_threads(void);

/* --- MXFP4 ([MX]) ---------------------------------------------------- */
/* 1D along cols (cols % 32 == 0): codes [rows][cols/2] (two per byte, even
 * element low), scales [rows][cols/32] E8M0 bytes; round-to-nearest-even. */
int orc_mx_quantize(const void* x, int dtype, int64_t rows, int64_t cols, uint8_t* codes,
                    uint8_t* scales);
double orc_e8m0_value(int byte);
int orc_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                      double* out);
/* C_ij in double for the given (ii[t], jj[t]) pairs, or all M*N (ii = jj = NULL) */
int orc_mx_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, const int64_t* ii,
                const int64_t* jj, int64_t count, double* c, double* abs_sum);

#ifdef __cplusplus
}
#endif
#endif
