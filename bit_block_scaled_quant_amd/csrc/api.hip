// C-ABI entry points of libnvfp4.so (declared in include/nvfp4.h): host-side
// argument validation, then the kernel launches of quantize.hip and gemm.hip
// on the caller's stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <cmath>

#include "../../include/nvfp4.h"
#include "internal.hpp"
#include "nvfp4_device.hpp"

namespace {

thread_local char g_last_error[256] = "";

int set_hip_error(hipError_t e, const char* where) {
  std::snprintf(g_last_error, sizeof g_last_error, "%s: %s", where, hipGetErrorString(e));
  return NVFP4_ERR_HIP;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

// compute-unit count of the current device, cached per device
int device_cus(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_hip_error(e, "hipGetDevice");
  if (dev >= 0 && dev < kMaxDevices) {
    int v = g_cus[dev].load(std::memory_order_relaxed);
    if (v > 0) {
      *cus = v;
      return NVFP4_OK;
    }
  }
  int v = 0;
  e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return set_hip_error(e, "hipDeviceGetAttribute");
  if (v <= 0) v = 1;
  if (dev >= 0 && dev < kMaxDevices) g_cus[dev].store(v, std::memory_order_relaxed);
  *cus = v;
  return NVFP4_OK;
}

int check_launch(const char* where) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_hip_error(e, where);
  return NVFP4_OK;
}

// rows * cols must fit comfortably in int64 arithmetic
bool size_ok(int64_t rows, int64_t cols) { return rows <= (INT64_C(1) << 40) / cols; }

int validate_quant(const void* x, int dtype, int64_t rows, int64_t cols, int rounding, uint8_t* codes,
                   uint8_t* scales, float* tensor_scale, uint8_t* codes_t, uint8_t* scales_t) {
  if (!x || !codes || !scales || !tensor_scale) return NVFP4_ERR_ARG;
  if (dtype != NVFP4_F32 && dtype != NVFP4_BF16) return NVFP4_ERR_ARG;
  if (rounding != NVFP4_RNE && rounding != NVFP4_SR) return NVFP4_ERR_ARG;
  if ((codes_t == nullptr) != (scales_t == nullptr)) return NVFP4_ERR_ARG;
  if (rows <= 0 || cols <= 0 || cols % 16 != 0 || !size_ok(rows, cols)) return NVFP4_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(codes, 8) || !aligned(tensor_scale, 4)) return NVFP4_ERR_ALIGN;
  if (codes_t && !aligned(codes_t, 8)) return NVFP4_ERR_ALIGN;
  return NVFP4_OK;
}

}  // namespace

extern "C" {

const char* nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_ARG: return "invalid argument";
    case NVFP4_ERR_SHAPE: return "invalid shape";
    case NVFP4_ERR_ALIGN: return "misaligned pointer";
    case NVFP4_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* nvfp4_last_error(void) { return g_last_error; }

int nvfp4_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int rounding, uint64_t seed,
                   int rht, uint64_t rht_seed, uint8_t* codes, uint8_t* scales, float* tensor_scale,
                   uint8_t* codes_t, uint8_t* scales_t, void* stream) {
  int st = validate_quant(x, dtype, rows, cols, rounding, codes, scales, tensor_scale, codes_t, scales_t);
  if (st) return st;
  if (rht != 0 && rht != 1) return NVFP4_ERR_ARG;
  if (codes_t && rht) return NVFP4_ERR_ARG;
  if (codes_t && rows % 16 != 0) return NVFP4_ERR_SHAPE;
  int cus = 0;
  if ((st = device_cus(&cus))) return st;
  nvfp4::QuantArgs a{x,      dtype == NVFP4_BF16, rows,   cols,   rounding,     seed,    rht == 1,
                     rht ? nvfp4::rht_sign_mask(rht_seed) : 0u,  false, codes, scales, tensor_scale,
                     codes_t, scales_t, false};
  nvfp4::launch_quantize(a, cus, (hipStream_t)stream);
  return check_launch("nvfp4_quantize");
}

int nvfp4_quantize_with_amax(const void* x, int dtype, int64_t rows, int64_t cols, int rounding, uint64_t seed,
                             int rht, uint64_t rht_seed, uint8_t* codes, uint8_t* scales, float* tensor_scale,
                             void* stream) {
  int st = validate_quant(x, dtype, rows, cols, rounding, codes, scales, tensor_scale, nullptr, nullptr);
  if (st) return st;
  if (rht != 0 && rht != 1) return NVFP4_ERR_ARG;
  int cus = 0;
  if ((st = device_cus(&cus))) return st;
  nvfp4::QuantArgs a{x,       dtype == NVFP4_BF16, rows,    cols,   rounding,     seed,    rht == 1,
                     rht ? nvfp4::rht_sign_mask(rht_seed) : 0u,   false, codes, scales, tensor_scale,
                     nullptr, nullptr,             true};
  nvfp4::launch_quantize(a, cus, (hipStream_t)stream);
  return check_launch("nvfp4_quantize_with_amax");
}

int nvfp4_quantize_2d(const void* w, int dtype, int64_t rows, int64_t cols, int rounding, uint64_t seed,
                      uint8_t* codes, uint8_t* scales, float* tensor_scale, uint8_t* codes_t,
                      uint8_t* scales_t, void* stream) {
  int st = validate_quant(w, dtype, rows, cols, rounding, codes, scales, tensor_scale, codes_t, scales_t);
  if (st) return st;
  if (rows % 16 != 0) return NVFP4_ERR_SHAPE;
  int cus = 0;
  if ((st = device_cus(&cus))) return st;
  nvfp4::QuantArgs a{w,      dtype == NVFP4_BF16, rows, cols,   rounding,     seed,    false,
                     0u,     true,                codes, scales, tensor_scale, codes_t, scales_t, false};
  nvfp4::launch_quantize(a, cus, (hipStream_t)stream);
  return check_launch("nvfp4_quantize_2d");
}

int nvfp4_quantize_cast_transpose(const void* x, int dtype, int64_t rows, int64_t cols, int rounding,
                                  uint64_t seed, uint64_t seed_t, int rht_t, uint64_t rht_seed, uint8_t* codes,
                                  uint8_t* scales, float* tensor_scale, uint8_t* codes_t, uint8_t* scales_t,
                                  float* tensor_scale_t, void* stream) {
  if (!codes_t || !tensor_scale_t) return NVFP4_ERR_ARG;
  int st = validate_quant(x, dtype, rows, cols, rounding, codes, scales, tensor_scale, codes_t, scales_t);
  if (st) return st;
  if (rht_t != 0 && rht_t != 1) return NVFP4_ERR_ARG;
  if (rows % 16 != 0) return NVFP4_ERR_SHAPE;
  if (!aligned(tensor_scale_t, 4)) return NVFP4_ERR_ALIGN;
  int cus = 0;
  if ((st = device_cus(&cus))) return st;
  nvfp4::CastTransposeArgs a{x,      dtype == NVFP4_BF16, rows,   cols,         rounding, seed,     seed_t,
                             rht_t == 1, rht_t ? nvfp4::rht_sign_mask(rht_seed) : 0u, codes, scales,
                             tensor_scale, codes_t, scales_t, tensor_scale_t, 0u};
  nvfp4::launch_cast_transpose(a, cus, (hipStream_t)stream);
  return check_launch("nvfp4_quantize_cast_transpose");
}

int nvfp4_rht(const void* x, int dtype, int64_t rows, int64_t cols, uint64_t rht_seed, float* y,
              void* stream) {
  if (!x || !y) return NVFP4_ERR_ARG;
  if (dtype != NVFP4_F32 && dtype != NVFP4_BF16) return NVFP4_ERR_ARG;
  if (rows <= 0 || cols <= 0 || cols % 16 != 0 || !size_ok(rows, cols)) return NVFP4_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(y, 16)) return NVFP4_ERR_ALIGN;
  int cus = 0;
  int st = device_cus(&cus);
  if (st) return st;
  nvfp4::launch_rht(x, dtype == NVFP4_BF16, rows, cols, nvfp4::rht_sign_mask(rht_seed), y, cus,
                    (hipStream_t)stream);
  return check_launch("nvfp4_rht");
}

int nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale, int64_t rows,
                     int64_t cols, int out_dtype, void* out, void* stream) {
  if (!codes || !scales || !tensor_scale || !out) return NVFP4_ERR_ARG;
  if (out_dtype != NVFP4_F32 && out_dtype != NVFP4_BF16) return NVFP4_ERR_ARG;
  if (rows <= 0 || cols <= 0 || cols % 16 != 0 || !size_ok(rows, cols)) return NVFP4_ERR_SHAPE;
  if (!aligned(codes, 8) || !aligned(tensor_scale, 4) || !aligned(out, 16)) return NVFP4_ERR_ALIGN;
  int cus = 0;
  int st = device_cus(&cus);
  if (st) return st;
  nvfp4::launch_dequantize(codes, scales, tensor_scale, rows, cols, out_dtype == NVFP4_BF16, out, cus,
                           (hipStream_t)stream);
  return check_launch("nvfp4_dequantize");
}

int nvfp4_gemm_ex(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_tensor_scale,
                  const uint8_t* b_codes, const uint8_t* b_scales, const float* b_tensor_scale, int64_t M,
                  int64_t N, int64_t K, void* c, int c_dtype, float beta, float* c_amax, void* stream) {
  if (!a_codes || !a_scales || !a_tensor_scale || !b_codes || !b_scales || !b_tensor_scale || !c)
    return NVFP4_ERR_ARG;
  if (c_dtype != NVFP4_F32 && c_dtype != NVFP4_BF16) return NVFP4_ERR_ARG;
  if (!(beta == beta) || beta == INFINITY || beta == -INFINITY) return NVFP4_ERR_ARG;
  if (M <= 0 || N <= 0 || K <= 0 || K % 16 != 0) return NVFP4_ERR_SHAPE;
  if (!size_ok(M, K) || !size_ok(N, K) || !size_ok(M, N)) return NVFP4_ERR_SHAPE;
  if (M > INT64_C(65535) * 128) return NVFP4_ERR_SHAPE;  // grid.y limit
  if (!aligned(a_codes, 8) || !aligned(b_codes, 8) || !aligned(c, c_dtype == NVFP4_F32 ? 4 : 2) ||
      !aligned(a_tensor_scale, 4) || !aligned(b_tensor_scale, 4) || (c_amax && !aligned(c_amax, 4)))
    return NVFP4_ERR_ALIGN;
  int cus = 0;
  int st = device_cus(&cus);
  if (st) return st;
  const bool f32 = c_dtype == NVFP4_F32;
  nvfp4::GemmArgs g{a_codes, a_scales, a_tensor_scale, b_codes, b_scales, b_tensor_scale, M, N, K,
                    f32 ? static_cast<float*>(c) : nullptr, f32 ? nullptr : static_cast<uint16_t*>(c), beta,
                    reinterpret_cast<unsigned*>(c_amax)};
  nvfp4::launch_gemm(g, cus, (hipStream_t)stream);
  return check_launch("nvfp4_gemm_ex");
}

int mxfp4_quantize(const void* x, int dtype, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                   void* stream) {
  if (!x || !codes || !scales) return NVFP4_ERR_ARG;
  if (dtype != NVFP4_F32 && dtype != NVFP4_BF16) return NVFP4_ERR_ARG;
  if (rows <= 0 || cols <= 0 || cols % 32 != 0 || !size_ok(rows, cols)) return NVFP4_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(codes, 8)) return NVFP4_ERR_ALIGN;
  int cus = 0;
  int st = device_cus(&cus);
  if (st) return st;
  nvfp4::launch_mx_quantize(x, dtype == NVFP4_BF16, rows, cols, codes, scales, cus, (hipStream_t)stream);
  return check_launch("mxfp4_quantize");
}

int mxfp4_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols, int out_dtype,
                     void* out, void* stream) {
  if (!codes || !scales || !out) return NVFP4_ERR_ARG;
  if (out_dtype != NVFP4_F32 && out_dtype != NVFP4_BF16) return NVFP4_ERR_ARG;
  if (rows <= 0 || cols <= 0 || cols % 32 != 0 || !size_ok(rows, cols)) return NVFP4_ERR_SHAPE;
  if (!aligned(codes, 8) || !aligned(out, 16)) return NVFP4_ERR_ALIGN;
  int cus = 0;
  int st = device_cus(&cus);
  if (st) return st;
  nvfp4::launch_mx_dequantize(codes, scales, rows, cols, out_dtype == NVFP4_BF16, out, cus, (hipStream_t)stream);
  return check_launch("mxfp4_dequantize");
}

int mxfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes, const uint8_t* b_scales,
               int64_t M, int64_t N, int64_t K, float* c, void* stream) {
  if (!a_codes || !a_scales || !b_codes || !b_scales || !c) return NVFP4_ERR_ARG;
  if (M <= 0 || N <= 0 || K <= 0 || K % 32 != 0) return NVFP4_ERR_SHAPE;
  if (!size_ok(M, K) || !size_ok(N, K) || !size_ok(M, N)) return NVFP4_ERR_SHAPE;
  if (M > INT64_C(65535) * 64) return NVFP4_ERR_SHAPE;  // grid.y of the general path
  if (!aligned(a_codes, 16) || !aligned(b_codes, 16) || !aligned(c, 4)) return NVFP4_ERR_ALIGN;
  nvfp4::MxGemmArgs g{a_codes, a_scales, b_codes, b_scales, M, N, K, c};
  nvfp4::launch_mx_gemm(g, (hipStream_t)stream);
  return check_launch("mxfp4_gemm");
}

int nvfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_tensor_scale,
               const uint8_t* b_codes, const uint8_t* b_scales, const float* b_tensor_scale, int64_t M,
               int64_t N, int64_t K, float* c, void* stream) {
  if (!a_codes || !a_scales || !a_tensor_scale || !b_codes || !b_scales || !b_tensor_scale || !c)
    return NVFP4_ERR_ARG;
  if (M <= 0 || N <= 0 || K <= 0 || K % 16 != 0) return NVFP4_ERR_SHAPE;
  if (!size_ok(M, K) || !size_ok(N, K) || !size_ok(M, N)) return NVFP4_ERR_SHAPE;
  if (M > INT64_C(65535) * 128) return NVFP4_ERR_SHAPE;  // grid.y limit
  if (!aligned(a_codes, 8) || !aligned(b_codes, 8) || !aligned(c, 4) || !aligned(a_tensor_scale, 4) ||
      !aligned(b_tensor_scale, 4))
    return NVFP4_ERR_ALIGN;
  int cus = 0;
  int st = device_cus(&cus);
  if (st) return st;
  nvfp4::GemmArgs g{a_codes, a_scales, a_tensor_scale, b_codes, b_scales, b_tensor_scale, M, N, K, c, nullptr,
                    0.0f,    nullptr};
  nvfp4::launch_gemm(g, cus, (hipStream_t)stream);
  return check_launch("nvfp4_gemm");
}

}  // extern "C"
