// Launchers shared by the C-ABI entry points (host side of the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace nvfp4 {

struct QuantArgs {
  const void* x;
  bool bf16;
  int64_t rows, cols;
  int rounding;  // 0 RNE, 1 SR
  uint64_t seed;
  bool rht;
  uint32_t rht_mask;
  bool two_d;
  uint8_t* codes;
  uint8_t* scales;
  float* tensor_scale;
  uint8_t* codes_t;  // may be null
  uint8_t* scales_t;
  bool amax_given;   // tensor_scale[1] already holds the amax: skip pass 1
};

void launch_quantize(const QuantArgs& a, int cus, hipStream_t st);

// x [rows][cols] quantized rowwise (no transform) and columnwise (the rows
// of x^T, with the transform when rht_t) in one pair of passes
struct CastTransposeArgs {
  const void* x;
  bool bf16;
  int64_t rows, cols;
  int rounding;  // 0 RNE, 1 SR (both copies)
  uint64_t seed, seed_t;
  bool rht_t;
  uint32_t rht_mask;
  uint8_t* codes;
  uint8_t* scales;
  float* tensor_scale;
  uint8_t* codes_t;
  uint8_t* scales_t;
  float* tensor_scale_t;  // may equal tensor_scale when rht_t is off
  uint32_t stream_t;      // SR stream of the columnwise copy: 0, or 1 for nvfp4_quantize's copy
};

void launch_cast_transpose(const CastTransposeArgs& a, int cus, hipStream_t st);
void launch_rht(const void* x, bool bf16, int64_t rows, int64_t cols, uint32_t mask, float* y, int cus,
                hipStream_t st);
void launch_dequantize(const uint8_t* codes, const uint8_t* scales, const float* ts, int64_t rows, int64_t cols,
                       bool bf16_out, void* out, int cus, hipStream_t st);

struct GemmArgs {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const float* a_ts;
  const uint8_t* b_codes;
  const uint8_t* b_scales;
  const float* b_ts;
  int64_t M, N, K;
  float* c;            // fp32 output, or
  uint16_t* c16;       // bf16 output (exactly one of c, c16 is set)
  float beta;          // C = A.B^T + beta * C_old (C_old not read when beta == 0)
  unsigned* amax;      // optional: max |stored C| as float bits (cleared by launch_gemm)
};

void launch_gemm(const GemmArgs& g, int cus, hipStream_t st);

// MXFP4: 32-element blocks of E2M1 codes with E8M0 (power-of-two) scales
struct MxGemmArgs {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const uint8_t* b_codes;
  const uint8_t* b_scales;
  int64_t M, N, K;
  float* c;
};

void launch_mx_quantize(const void* x, bool bf16, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                        int cus, hipStream_t st);
void launch_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols, bool bf16_out,
                          void* out, int cus, hipStream_t st);
void launch_mx_gemm(const MxGemmArgs& g, hipStream_t st);

}  // namespace nvfp4
