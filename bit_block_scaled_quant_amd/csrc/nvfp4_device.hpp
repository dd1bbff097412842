// Device-side building blocks of the NVFP4 quantizer for CDNA4 (gfx950).
//
// Format and method (cited by page title and section):
//   "Pretraining Large Language Models with NVFP4" (gist.science summary),
//   Technische samenvatting:
//     2A   16-element blocks, an E4M3 scale per block, an FP32 scale per
//          tensor (two-level scaling);
//     2B.2 16-point random Hadamard transform on the Wgrad inputs;
//     2B.3 16x16 blocks for weights, 1x16 for activations and gradients;
//     2B.4 stochastic rounding of gradients, round-to-nearest-even otherwise.
//   E2M1 and E4M3 bit layouts: OCP Microscaling Formats v1.0 and OCP 8-bit
//   Floating Point.  Random bits: Philox4x32-10 (Salmon et al., SC'11).
//
// Conventions fixed here (the pages do not give them):
//   S_enc = 2688 / amax (2688 = 6 * 448), 1 for an all-zero tensor, FLT_MAX
//   on overflow; block scale s = (amax_b * S_enc) / 6 rounded to E4M3 (RNE,
//   saturating); inv = S_enc / decode(s) (0 for a zero scale, at most
//   FLT_MAX); y = x * inv; E2M1 RNE with ties to the even code, saturating at
//   6 and keeping the sign; SR rounds |y| up iff u16 < f * 2^16 where f is
//   the fractional position of |y| between its grid neighbours; the random
//   u16 of element i is half (i & 1) of word (i & 7) >> 1 of
//   Philox(key = seed, counter = (i >> 3, stream, 0)).
//
// Every fp32 step is a single correctly rounded operation: the library is
// compiled with -ffp-contract=off and divisions use __fdiv_rn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

constexpr float kFltMax = 3.40282346638528859812e+38f;

// ---------------------------------------------------------------- E4M3 ---
// s >= 0, finite or +inf.  Round to nearest even, saturate to 448 (0x7E).
__device__ __forceinline__ uint32_t e4m3_encode(float s) {
  if (!(s < 448.0f)) return 0x7Eu;
  const uint32_t b = __float_as_uint(s);
  if (b < 0x3C800000u) {  // s < 2^-6: subnormal range, multiples of 2^-9
    // s * 512 is exact; rintf rounds half to even; 8 is the smallest normal
    return (uint32_t)__builtin_rintf(s * 512.0f);
  }
  // keep 3 mantissa bits, round to nearest even on the discarded 20 bits
  const uint32_t r = b + 0x7FFFFu + ((b >> 20) & 1u);
  const uint32_t e = (r >> 23) - 120u;  // E4M3 exponent field (bias 7)
  return (e << 3) | ((r >> 20) & 7u);
}

__device__ __forceinline__ float e4m3_decode(uint32_t byte) {
  const uint32_t e = (byte >> 3) & 15u, m = byte & 7u;
  if (e == 0) return (float)m * 0.001953125f;  // m * 2^-9, exact
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// ---------------------------------------------------------- scales -------
__device__ __forceinline__ float tensor_scale_from_amax(float amax) {
  if (amax == 0.0f) return 1.0f;
  const float s = __fdiv_rn(2688.0f, amax);
  return fminf(s, kFltMax);
}

// block scale byte and element multiplier for a block with amax amax_b
__device__ __forceinline__ uint32_t block_scale(float amax_b, float s_enc, float* inv) {
  const float t = amax_b * s_enc;
  const float s = __fdiv_rn(t, 6.0f);
  const uint32_t byte = e4m3_encode(s);
  const float sb = e4m3_decode(byte);
  *inv = (sb == 0.0f) ? 0.0f : fminf(__fdiv_rn(s_enc, sb), kFltMax);
  return byte;
}

// ---------------------------------------------------------------- E2M1 ---
// Round-to-nearest-even of |y| onto {0,.5,1,1.5,2,3,4,6}: adding 2^22, 2^23
// or 2^24 (for |y| < 2, < 4, <= 6) rounds |y| to a multiple of 0.5, 1 or 2
// with the hardware's ties-to-even, and the low bits of the sum count those
// multiples; ties to even multiples are ties to even codes.
__device__ __forceinline__ uint32_t e2m1_rne(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 28) & 8u;
  const float m = fminf(fabsf(y), 6.0f);
  const uint32_t mb = __float_as_uint(m);
  const uint32_t magic = max(0x4A800000u, (mb & 0x7F800000u) + (22u << 23));
  const uint32_t t = __float_as_uint(m + __uint_as_float(magic));
  const uint32_t idx = (t - magic) + 2u * ((magic >> 23) - 149u);
  return sign | idx;
}

// Stochastic rounding with a 16-bit random u: the grid step is 0.5, 1 or 2
// below 2, 4 and 6; t = |y| / step is exact, its integer part picks lo and
// its fraction f decides: up iff u < f * 65536 (exact comparison).
__device__ __forceinline__ uint32_t e2m1_sr(float y, uint32_t u) {
  const uint32_t sign = (__float_as_uint(y) >> 28) & 8u;
  const float m = fminf(fabsf(y), 6.0f);
  const uint32_t ef = min(max(__float_as_uint(m) >> 23, 127u), 129u);
  const float inv_step = __uint_as_float((255u - ef) << 23);  // 2, 1, 0.5
  const float t = m * inv_step;
  const uint32_t n = (uint32_t)t;  // truncation of t >= 0
  const float f = t - (float)n;
  const uint32_t up = ((float)u < f * 65536.0f) ? 1u : 0u;
  return sign | (n + 2u * (ef - 127u) + up);
}

// ---------------------------------------------------------- Philox -------
struct Philox4 {
  uint32_t x, y, z, w;
};

__host__ __device__ __forceinline__ uint32_t mulhi32(uint32_t a, uint32_t b) {
  return (uint32_t)(((uint64_t)a * b) >> 32);
}

// Ten rounds; in each, words 0 and 2 are multiplied by the round constants,
// the high halves are xored with words 1 and 3 and the key, and the key is
// advanced by the Weyl increments.
__host__ __device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                          uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t lo0 = 0xD2511F53u * c0, hi0 = mulhi32(0xD2511F53u, c0);
    const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = mulhi32(0xCD9E8D57u, c2);
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return {c0, c1, c2, c3};
}

// Hadamard sign mask of a seed: the low 16 bits of word 0 of stream 2,
// counter 0 (bit j set => sign j is -1)
__host__ __device__ __forceinline__ uint32_t rht_sign_mask(uint64_t rht_seed) {
  return philox4x32_10(0u, 0u, 2u, 0u, (uint32_t)rht_seed, (uint32_t)(rht_seed >> 32)).x & 0xFFFFu;
}

// the eight 16-bit draws of elements 8g .. 8g+7 of a stream
__device__ __forceinline__ Philox4 sr_draws(uint64_t seed, uint32_t stream, uint64_t g) {
  return philox4x32_10((uint32_t)g, (uint32_t)(g >> 32), stream, 0u, (uint32_t)seed,
                       (uint32_t)(seed >> 32));
}

__device__ __forceinline__ uint32_t draw16(const Philox4& p, int j) {  // j in 0..7
  const uint32_t w = (j >> 1) == 0 ? p.x : (j >> 1) == 1 ? p.y : (j >> 1) == 2 ? p.z : p.w;
  return (j & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// ------------------------------------------------------------- RHT -------
// v <- 1/4 * H16 * diag(sigma) * v, in-place butterfly h = 1, 2, 4, 8, in
// fp32; sign j flips when bit j of mask is set.
__device__ __forceinline__ void rht16(float v[16], uint32_t mask) {
#pragma unroll
  for (int j = 0; j < 16; ++j)
    v[j] = __uint_as_float(__float_as_uint(v[j]) ^ (((mask >> j) & 1u) << 31));
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i & h) continue;
      const float a = v[i], b = v[i + h];
      v[i] = a + b;
      v[i + h] = a - b;
    }
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = 0.25f * v[j];
}

// ----------------------------------------------------------- loads -------
// Streaming 16-byte load with the nontemporal hint: the quantizer reads
// every input byte once per pass, and on MI355X such loads sustain about
// twice the bandwidth of cached ones.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 16 consecutive elements starting at element e (e % 16 == 0) as fp32
template <bool BF16>
__device__ __forceinline__ void load16(const void* __restrict__ x, int64_t e, float v[16]) {
  if (BF16) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + e);
    const uint4 a = ld_stream(p), b = ld_stream(p + 1);
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(x) + e);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 q = ld_stream(p + i);
      v[4 * i] = __uint_as_float(q.x);
      v[4 * i + 1] = __uint_as_float(q.y);
      v[4 * i + 2] = __uint_as_float(q.z);
      v[4 * i + 3] = __uint_as_float(q.w);
    }
  }
}

__device__ __forceinline__ float amax16(const float v[16]) {
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) m = fmaxf(m, fabsf(v[j]));
  return m;
}

// Round-to-nearest-even of eight values with the gfx950 conversion
// v_cvt_scalef32_pk_fp4_f32 (scale 1.0: no scaling), two values per
// instruction, even element in the low nibble of each byte.  Its rounding
// equals e2m1_rne above for every fp32 input (ties to even, saturation at 6,
// sign kept); the exhaustive device test checks that against the oracle.
__device__ __forceinline__ uint32_t e2m1_rne8(const float* y) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], 1.0f, 3);
  return w;
}

// encode 16 elements of one block; codes packed two per byte, even element
// in the low nibble, into two 32-bit words
template <bool SR>
__device__ __forceinline__ uint2 encode16(const float v[16], float inv, uint64_t seed,
                                          uint32_t stream, uint64_t index0) {
  uint32_t lo = 0, hi = 0;
  if (SR) {
    const Philox4 p0 = sr_draws(seed, stream, index0 >> 3);
    const Philox4 p1 = sr_draws(seed, stream, (index0 >> 3) + 1);
#pragma unroll
    for (int j = 0; j < 8; ++j) lo |= e2m1_sr(v[j] * inv, draw16(p0, j)) << (4 * j);
#pragma unroll
    for (int j = 0; j < 8; ++j) hi |= e2m1_sr(v[8 + j] * inv, draw16(p1, j)) << (4 * j);
  } else {
    float y[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) y[j] = v[j] * inv;
    lo = e2m1_rne8(y);
    hi = e2m1_rne8(y + 8);
  }
  return make_uint2(lo, hi);
}

}  // namespace nvfp4
