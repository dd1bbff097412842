// NVFP4 dequantization for CDNA4 (gfx950): out[r][c] = e2m1(code) *
// e4m3(scale) / S_enc ("Pretraining Large Language Models with NVFP4",
// Technische samenvatting, 2A: the per-block E4M3 scale and the per-tensor
// FP32 scale together bring a block back to its original range).
//
// The product e2m1 * e4m3 has at most 6 significant bits and is exact in
// fp32, so the value is one correctly rounded division.  A tensor has one
// S_enc and a value depends only on the scale byte and the code magnitude:
// every workgroup divides the 128 x 8 possible products once into an LDS
// table, and each element is then a table read and a sign flip.  bf16 output
// is that fp32 value rounded to nearest-even.
//
// Layout: a thread takes four consecutive elements (two code bytes, one
// scale byte shared by four neighbouring threads), so a wave's store
// instruction writes 1 KB (fp32) or 512 B (bf16) of contiguous output, with
// the nontemporal hint (measured 3.9 -> 6.0 TB/s for bf16, 4.4 -> 6.3 for fp32
// on an 8192 x 20480 tensor).
#include "internal.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

constexpr int kDqThreads = 256;
constexpr int kDqTable = 128 * 8;  // [scale byte & 0x7F][code magnitude]

template <bool BF16OUT>
__global__ __launch_bounds__(kDqThreads) void k_dequantize(const uint8_t* __restrict__ codes,
                                                           const uint8_t* __restrict__ scales,
                                                           const float* __restrict__ ts, int64_t nquad,
                                                           void* __restrict__ out) {
  __shared__ float tab[kDqTable];
  const float s_enc = ts[0];
  for (int i = threadIdx.x; i < kDqTable; i += kDqThreads) {
    const float p = e2m1_magnitude(i & 7) * e4m3_decode((uint32_t)(i >> 3));  // exact
    tab[i] = __fdiv_rn(p, s_enc);
  }
  __syncthreads();
  const int64_t stride = (int64_t)gridDim.x * kDqThreads;
  for (int64_t q = (int64_t)blockIdx.x * kDqThreads + threadIdx.x; q < nquad; q += stride) {
    // elements 4q .. 4q + 3: code bytes 2q, 2q + 1; block (4q) / 16
    const uint32_t cw = *reinterpret_cast<const uint16_t*>(codes + 2 * q);
    const uint32_t base = (uint32_t)(scales[q >> 2] & 0x7Fu) << 3;
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t c = (cw >> (4 * j)) & 15u;
      v[j] = __uint_as_float(__float_as_uint(tab[base + (c & 7u)]) | ((c & 8u) << 28));
    }
    // streaming stores: the output is written once and not read here
    if (BF16OUT) {
      const u32x2_t w = {bf16_rne(v[0]) | bf16_rne(v[1]) << 16, bf16_rne(v[2]) | bf16_rne(v[3]) << 16};
      __builtin_nontemporal_store(w, reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(out) + 4 * q));
    } else {
      typedef float f32x4_t __attribute__((ext_vector_type(4)));
      const f32x4_t w = {v[0], v[1], v[2], v[3]};
      __builtin_nontemporal_store(w, reinterpret_cast<f32x4_t*>(static_cast<float*>(out) + 4 * q));
    }
  }
}

void launch_dequantize(const uint8_t* codes, const uint8_t* scales, const float* ts, int64_t rows, int64_t cols,
                       bool bf16_out, void* out, int cus, hipStream_t st) {
  const int64_t nquad = rows * cols / 4;
  const int blocks = (int)std::max<int64_t>(
      1, std::min<int64_t>((nquad + kDqThreads - 1) / kDqThreads, (int64_t)cus * 8));
  if (bf16_out)
    hipLaunchKernelGGL(k_dequantize<true>, dim3(blocks), dim3(kDqThreads), 0, st, codes, scales, ts, nquad, out);
  else
    hipLaunchKernelGGL(k_dequantize<false>, dim3(blocks), dim3(kDqThreads), 0, st, codes, scales, ts, nquad, out);
}

}  // namespace nvfp4
