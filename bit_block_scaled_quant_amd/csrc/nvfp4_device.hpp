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
// compiled with -ffp-contract=off, divisions use __fdiv_rn, and the one
// division by a constant (by 6, in the block scale) uses a correction step
// that is exact where it matters (div6).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

constexpr float kFltMax = 3.40282346638528859812e+38f;

// ---------------------------------------------------------------- E4M3 ---
// s >= 0, finite or +inf.  Round to nearest even, saturate to 448 (0x7E):
// gfx950's fp8 conversion (OCP E4M3, round to nearest even, subnormals kept)
// of min(s, 448).  A device probe found it equal to a bit-level
// round-to-nearest-even encoder for every non-negative fp32 pattern up to
// +inf; the tests check the scale bytes of the quantizers against the
// oracle's argmin encoder, around every E4M3 rounding boundary and over
// whole tensors.
__device__ __forceinline__ uint32_t e4m3_encode(float s) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(s, 448.0f), 0.0f, 0, false) & 0xFFu;
}

__device__ __forceinline__ float e4m3_decode(uint32_t byte) {
  const uint32_t e = (byte >> 3) & 15u, m = byte & 7u;
  const float sub = (float)m * 0.001953125f;  // m * 2^-9, exact
  const float nrm = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return e == 0 ? sub : nrm;
}

// ---------------------------------------------------------- scales -------
__device__ __forceinline__ float tensor_scale_from_amax(float amax) {
  if (amax == 0.0f) return 1.0f;
  const float s = __fdiv_rn(2688.0f, amax);
  return fminf(s, kFltMax);
}

// t / 6 for t >= 0 in three operations: the product with fl(1/6), corrected
// once by its exact fma residual (Markstein's correction step).  The result
// is the correctly rounded quotient for every t in [2^-125, FLT_MAX] (checked
// exhaustively on the host over all those bit patterns).  Below 2^-125 it may
// miss by an ulp of a subnormal, and +inf gives NaN: in both cases the E4M3
// byte of the quotient is unchanged (0x00 below 2^-10; 0x7E, since
// min(NaN, 448) is 448).
__device__ __forceinline__ float div6(float t) {
  const float c = 0.16666667163372039795f;  // fl(1/6)
  const float q0 = t * c;
  return __builtin_fmaf(__builtin_fmaf(-q0, 6.0f, t), c, q0);
}

// Table of the element multiplier for each scale byte: inv = S_enc / sb
// rounded once, at most FLT_MAX, and 0 for the zero scale.  Every encode
// workgroup builds it in LDS before its first block (the first 128 threads,
// then a barrier), so a block's multiplier is one LDS read instead of a
// decode and a division.
constexpr int kInvTable = 128;

__device__ __forceinline__ float inv_table_entry(uint32_t byte, float s_enc) {
  return byte == 0 ? 0.0f : fminf(__fdiv_rn(s_enc, e4m3_decode(byte)), kFltMax);
}

__device__ __forceinline__ void build_inv_table(float* tab, float s_enc) {
  if (threadIdx.x < kInvTable) tab[threadIdx.x] = inv_table_entry(threadIdx.x, s_enc);
  __syncthreads();
}

// block scale byte and element multiplier for a block with amax amax_b
__device__ __forceinline__ uint32_t block_scale(float amax_b, float s_enc, const float* inv_tab,
                                                float* inv) {
  const uint32_t byte = e4m3_encode(div6(amax_b * s_enc));
  *inv = inv_tab[byte];
  return byte;
}

// ---------------------------------------------------------- Philox -------
struct Philox4 {
  uint32_t x, y, z, w;
};

// a ^ b ^ c; one v_bitop3_b32 on the device
__host__ __device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
#else
  return a ^ b ^ c;
#endif
}

// Ten rounds; in each, words 0 and 2 are multiplied by the round constants,
// the high halves are xored with words 1 and 3 and the key, and the key is
// advanced by the Weyl increments.  Each product is one 32 x 32 -> 64-bit
// multiply (a single v_mad_u64_u32 on the device, which measures about 25%
// faster than the separate low and high multiplies).
__host__ __device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                          uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = xor3((uint32_t)(p1 >> 32), c1, k0), n2 = xor3((uint32_t)(p0 >> 32), c3, k1);
    c0 = n0;
    c1 = (uint32_t)p1;
    c2 = n2;
    c3 = (uint32_t)p0;
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
// hadamard16: v <- 1/4 * H16 * v: the in-place butterfly h = 1, 2, 4, 8 in
// fp32, then the factor 1/4 (H16 / 4 is orthonormal).
__device__ __forceinline__ void hadamard16(float v[16]) {
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

// max_j |(H16 v)_j| for the amax pass.  The last stage (h = 8) turns the pair
// a = v[j], b = v[j + 8] into a + b and a - b, and max(|fl(a + b)|,
// |fl(a - b)|) = fl(|a| + |b|) exactly: one of the two is a sum of the
// magnitudes, the other a difference no larger, and rounding is symmetric
// and monotone.  So that stage and the maxima over its 16 outputs become
// eight additions of magnitudes and a maximum over eight, with the same
// result bits.
__device__ __forceinline__ float hadamard16_absmax(float v[16]) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i & h) continue;
      const float a = v[i], b = v[i + h];
      v[i] = a + b;
      v[i + h] = a - b;
    }
  }
  uint32_t s[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) s[j] = __float_as_uint(__builtin_fabsf(v[j]) + __builtin_fabsf(v[j + 8]));
  // non-negative floats order like their bit patterns
  const uint32_t a = max(max(s[0], s[1]), s[2]), b = max(max(s[3], s[4]), s[5]);
  return __uint_as_float(max(max(a, b), max(s[6], s[7])));
}

// rht16: v <- 1/4 * H16 * diag(sigma) * v; sign j flips when bit j of mask
// is set.
__device__ __forceinline__ void rht16(float v[16], uint32_t mask) {
#pragma unroll
  for (int j = 0; j < 16; ++j)
    v[j] = __uint_as_float(__float_as_uint(v[j]) ^ (((mask >> j) & 1u) << 31));
  hadamard16(v);
}

// The same transform on a block held by a lane pair: the even lane holds
// elements 0..7, the odd lane 8..15.  Stages h = 1, 2, 4 stay inside the
// lane; stage h = 8 pairs element j of the two lanes through a DPP swap of
// lanes 2k and 2k + 1 (all lanes of the wave must be active).  Every value
// takes the same operations in the same order as rht16.
__device__ __forceinline__ float lane_pair_swap(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}

__device__ __forceinline__ void rht16_pair(float v[8], uint32_t mask, bool odd) {
  const uint32_t m8 = odd ? (mask >> 8) : mask;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = __uint_as_float(__float_as_uint(v[j]) ^ (((m8 >> j) & 1u) << 31));
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i & h) continue;
      const float a = v[i], b = v[i + h];
      v[i] = a + b;
      v[i + h] = a - b;
    }
  }
  // h = 8: even lane a + b (a its own), odd lane a - b (b its own)
  const uint32_t neg = odd ? 0x80000000u : 0u;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float p = lane_pair_swap(v[j]);
    v[j] = p + __uint_as_float(__float_as_uint(v[j]) ^ neg);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = 0.25f * v[j];
}

// max_j |(H16 sigma v)_j| over a block held by a lane pair (the transform of
// rht16_pair without the final 1/4), with the last stage and the maximum
// merged as in hadamard16_absmax; both lanes of the pair return the block's
// maximum.
__device__ __forceinline__ float rht16_pair_absmax(float v[8], uint32_t mask, bool odd) {
  const uint32_t m8 = odd ? (mask >> 8) : mask;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = __uint_as_float(__float_as_uint(v[j]) ^ (((m8 >> j) & 1u) << 31));
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i & h) continue;
      const float a = v[i], b = v[i + h];
      v[i] = a + b;
      v[i + h] = a - b;
    }
  }
  uint32_t s[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    s[j] = __float_as_uint(__builtin_fabsf(lane_pair_swap(v[j])) + __builtin_fabsf(v[j]));
  const uint32_t a = max(max(s[0], s[1]), s[2]), b = max(max(s[3], s[4]), s[5]);
  return __uint_as_float(max(max(a, b), max(s[6], s[7])));
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

// the same for 8 bytes
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 ld_stream8(const void* p) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v.x, v.y);
}

// 16 / 8 bytes, streaming or as ordinary cached loads.  A first pass over a
// tensor that fits in the 256 MB MALL reads it with cached loads (a few
// percent slower) so that the second pass finds it there.
template <bool CACHED>
__device__ __forceinline__ uint4 ld16(const void* p) {
  if (CACHED) return *reinterpret_cast<const uint4*>(p);
  return ld_stream(p);
}
template <bool CACHED>
__device__ __forceinline__ uint2 ld8(const void* p) {
  if (CACHED) return *reinterpret_cast<const uint2*>(p);
  return ld_stream8(p);
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

// raw storage of eight consecutive input elements (e % 8 == 0)
template <bool BF16>
struct Raw8 {
  uint4 a, b;  // b unused for bf16
};

template <bool BF16, bool CACHED = false>
__device__ __forceinline__ Raw8<BF16> load8_raw(const void* __restrict__ x, int64_t e) {
  Raw8<BF16> r;
  if (BF16) {
    r.a = ld16<CACHED>(static_cast<const uint16_t*>(x) + e);
    r.b = make_uint4(0u, 0u, 0u, 0u);
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(x) + e);
    r.a = ld16<CACHED>(p);
    r.b = ld16<CACHED>(p + 1);
  }
  return r;
}

template <bool BF16>
__device__ __forceinline__ void unpack8(const Raw8<BF16>& r, float v[8]) {
  if (BF16) {
    const uint32_t w[4] = {r.a.x, r.a.y, r.a.z, r.a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    v[0] = __uint_as_float(r.a.x); v[1] = __uint_as_float(r.a.y); v[2] = __uint_as_float(r.a.z);
    v[3] = __uint_as_float(r.a.w); v[4] = __uint_as_float(r.b.x); v[5] = __uint_as_float(r.b.y);
    v[6] = __uint_as_float(r.b.z); v[7] = __uint_as_float(r.b.w);
  }
}

// max(|a|, |b|, |c|) in one v_max3_f32 with absolute-value modifiers.
// Inputs are finite (the calls' contract), so the NaN-quieting moves the
// compiler puts before fmaxf of values it cannot prove canonical are not
// needed.
__device__ __forceinline__ float max3_abs(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, |%1|, |%2|, |%3|" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// max of two non-negative floats as an integer max of their bit patterns
__device__ __forceinline__ float max_nonneg(float a, float b) {
  return __uint_as_float(max(__float_as_uint(a), __float_as_uint(b)));
}

// max |v| as a tree (independent max3 chains rather than one serial chain)
__device__ __forceinline__ float max_abs8(const float v[8]) {
  const float a = max3_abs(v[0], v[1], v[2]);
  const float b = max3_abs(v[3], v[4], v[5]);
  return max_nonneg(b, max3_abs(v[6], v[7], a));
}

__device__ __forceinline__ float max_abs16(const float v[16]) {
  const float a = max3_abs(v[0], v[1], v[2]), b = max3_abs(v[3], v[4], v[5]), c = max3_abs(v[6], v[7], v[8]);
  const float d = max3_abs(v[9], v[10], v[11]), e = max3_abs(v[12], v[13], v[14]);
  return max_nonneg(max3_abs(a, b, v[15]), max3_abs(c, d, e));
}

// the maximum of a non-negative value and its neighbour's in the lane pair
// (2k, 2k + 1): one integer max with a DPP quad swap
__device__ __forceinline__ float pair_max(float m) {
  const uint32_t b = __float_as_uint(m);
  const uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)b, 0xB1, 0xF, 0xF, true);
  return __uint_as_float(max(b, o));
}

// E2M1 magnitude of index m (0..7): 0, 0.5, 1, 1.5, 2, 3, 4, 6
__device__ __forceinline__ float e2m1_magnitude(uint32_t m) {
  const float sub = 0.5f * (float)m;                                          // m < 4
  const float nrm = __uint_as_float(((m >> 1) + 126u) << 23 | (m & 1u) << 22);  // 2^(m/2 - 1) * (1 + (m & 1) / 2)
  return m < 4 ? sub : nrm;
}

__device__ __forceinline__ uint32_t bf16_rne(float v) {  // finite or inf
  const uint32_t b = __float_as_uint(v);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
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
// is round-to-nearest-even onto the E2M1 grid for every fp32 input (ties to the even code, saturation at 6,
// sign kept); the exhaustive device test checks that against the oracle.
__device__ __forceinline__ uint32_t e2m1_rne8(const float* y) {
  // the four conversions write all four bytes: the word starts as whatever
  // its register holds (an empty asm defines it without an instruction)
  uint32_t w;
  asm("" : "=v"(w));
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], 1.0f, 3);
  return w;
}

// Stochastic rounding of eight values (the eight draws of one Philox call)
// with the gfx950 conversion v_cvt_scalef32_sr_pk_fp4_f32, one value per
// instruction (the second input is 0.0, whose code is 0).  Measured on the
// device: the instruction divides its input by the scale operand and rounds
// |v| up iff its discarded bits, read as a fraction of the E2M1 step, plus
// rand[31:10] / 2^22 reach 1.  With rand = ~(u << 16) that is exactly
// "u < f * 2^16" whenever the step leaves 22 discarded bits (|v| >= 1);
// below that the hardware ignores the discarded bits past the 22nd, so |v|
// is first rounded up to a multiple of 2^-23 (exact, sign kept), which moves
// every fraction f*2^16 in (u, u+2^-6) to a value the 22-bit comparison
// orders the same way.  The rounded value is passed as the integer
// ceil(|v| 2^23) (with v's sign) and scale 2^23.  An exhaustive device test
// checks the result against the oracle's rule for every fp32 value in
// [2^-9, 6] and a sample of smaller ones.
typedef float float2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float sr_prepare(float v) {
  return __builtin_copysignf(__builtin_ceilf(__builtin_fabsf(v) * 8388608.0f), v);
}

// One conversion into byte K of w; the other bytes of w are kept.  Written
// as inline assembly with w tied to the destination: the compiler's builtin
// for this instruction does not place the old value in the destination
// register, so the kept bytes would be stale register contents.  op_sel
// [.., .., b0, b1] selects the byte, as the compiler encodes it.
template <int K>
__device__ __forceinline__ void sr_cvt(uint32_t& w, float v, uint32_t rand) {
  const float2v src = {sr_prepare(v), 0.0f};
  const float sc = 8388608.0f;  // 2^23
  if (K == 0)
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3" : "+v"(w) : "v"(src), "v"(rand), "s"(sc));
  if (K == 1)
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,1,0]" : "+v"(w) : "v"(src), "v"(rand), "s"(sc));
  if (K == 2)
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,0,1]" : "+v"(w) : "v"(src), "v"(rand), "s"(sc));
  if (K == 3)
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,1,1]" : "+v"(w) : "v"(src), "v"(rand), "s"(sc));
}

// ~(w << 16), i.e. the complemented low half of w in the high half and ones
// below, in one instruction: v_mad_i32_i24 forms sext24(w) * -2^16 - 1, whose
// low 32 bits depend on the low 16 bits of w only.  (Written out, the
// compiler emits a shift and a complement.)
__device__ __forceinline__ uint32_t not_low_half_up(uint32_t w) {
  uint32_t r;
  asm("v_mad_i32_i24 %0, %1, %2, -1" : "=v"(r) : "v"(w), "s"(-65536));
  return r;
}

// elements 2K (draw: low half of word w) and 2K + 1 (high half) into byte K
// of the even / odd code words; rand = ~(u << 16) for draw u
template <int K>
__device__ __forceinline__ void sr_pair(const float* y, uint32_t w, uint32_t& we, uint32_t& wo) {
  sr_cvt<K>(we, y[2 * K], not_low_half_up(w));
  sr_cvt<K>(wo, y[2 * K + 1], ~w | 0xFFFFu);
}

__device__ __forceinline__ uint32_t e2m1_sr8(const float* y, const Philox4& p) {
  uint32_t we = 0, wo = 0;  // codes of even / odd elements, one per byte
  sr_pair<0>(y, p.x, we, wo);
  sr_pair<1>(y, p.y, we, wo);
  sr_pair<2>(y, p.z, we, wo);
  sr_pair<3>(y, p.w, we, wo);
  return we | (wo << 4);
}

// encode 16 elements of one block; codes packed two per byte, even element
// in the low nibble, into two 32-bit words
template <bool SR>
__device__ __forceinline__ uint2 encode16(const float v[16], float inv, uint64_t seed,
                                          uint32_t stream, uint64_t index0) {
  float y[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) y[j] = v[j] * inv;
  if (SR) {
    const Philox4 p0 = sr_draws(seed, stream, index0 >> 3);
    const Philox4 p1 = sr_draws(seed, stream, (index0 >> 3) + 1);
    return make_uint2(e2m1_sr8(y, p0), e2m1_sr8(y + 8, p1));
  }
  return make_uint2(e2m1_rne8(y), e2m1_rne8(y + 8));
}

}  // namespace nvfp4
