// Block-scaled NVFP4 GEMM for CDNA4 (gfx950): C[M][N] = deq(A) . deq(B)^T,
// A = codes [M][K/2] + E4M3 scales [M][K/16] + FP32 tensor scale, B likewise
// with N rows; FP32 accumulation, FP32 output.
//
// "NVIDIA acelera el preentrenamiento de LLM: NVFP4 en Blackwell junto con JAX
// y MaxText", section "Como Funciona Mixed-Precision con NVFP4": NVFP4 feeds
// the GEMMs on weights and activations, accumulators stay in BF16 or FP32.
// "Pretraining Large Language Models with NVFP4", section 2A: a value is its
// E2M1 code times its block's E4M3 scale, divided by the tensor's FP32 scale.
//
// Exactness: an E2M1 magnitude has 2 significant bits and an E4M3 scale 4,
// so code * scale has at most 6 significant bits and lies in [2^-10, 2688]:
// it is an exact, normal fp16 number.  Each operand element is rebuilt
// exactly in fp16 in registers and multiplied on the fp16 MFMA
// (v_mfma_f32_16x16x32_f16) with fp32 accumulation; the two tensor scales are
// applied once in the epilogue.  (gfx950's scaled FP4 MFMA takes power-of-two
// scales per 32 elements, which cannot represent E4M3 scales per 16.)
//
// Tiling: a 256-thread workgroup owns a 256x256 tile of C and walks K in
// steps of 128.  Packed codes and scale bytes are staged through LDS (double
// buffered, 16-byte chunks XOR-swizzled against bank conflicts); each wave
// owns a 128x128 sub-tile (accumulators in AGPRs), reads its packed
// fragments from LDS and expands them in registers: per 128x128x32 of MFMA
// work a lane converts 64 elements, which hides under the matrix cores.  Lane group g = lane / 16 of a fragment covers the 32
// K-elements [32g, 32g+32) of a step; its word s feeds MFMA slice s.  A and B
// use the same lane-to-K map, so the products pair up correctly.
#include "internal.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kGemmThreads = 256;  // 4 waves in a 2 x 2 grid
constexpr int kBK = 128;           // K-elements per step
constexpr int kRowBytes = kBK / 2;  // 64 bytes of codes per row per step
constexpr int kRowScales = kBK / 16;

template <int BM, int BN>
struct __align__(16) GemmStage {
  uint8_t a[BM * kRowBytes];
  uint8_t b[BN * kRowBytes];
  uint8_t as[BM * kRowScales];
  uint8_t bs[BN * kRowScales];
};

// 16-byte chunk c of row r lives at chunk c ^ ((r >> 1) & 3): eight
// consecutive rows reading the same chunk hit eight distinct bank groups
__device__ __forceinline__ int swz(int r, int c) { return r * kRowBytes + ((c ^ ((r >> 1) & 3)) << 4); }

// Eight E2M1 codes (element 2k in the low nibble of byte k) -> eight exact
// fp16 values times the block scale, in element order.  The gfx950
// conversion v_cvt_scalef32_pk_f16_fp4 turns one byte into two fp16 values
// times a power-of-two scale exactly (checked for all 256 bytes); here the
// scale is 2^8.  The E4M3 scale byte b enters as the fp16 whose bits are
// (b & 0x7F) << 7, which is its value times 2^-8 (subnormal E4M3 bytes become
// fp16 subnormals), so one packed multiply yields code * scale exactly: the
// product has at most 6 significant bits and lies in [2^-10, 2688].
__device__ __forceinline__ half8 unpack8(uint32_t w, half2v sc) {
  const half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 0) * sc;
  const half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 1) * sc;
  const half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 2) * sc;
  const half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 3) * sc;
  return half8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// E4M3 byte -> (scale * 2^-8, scale * 2^-8) as packed fp16 bits
__device__ __forceinline__ half2v scale_h2(uint32_t byte) {
  return __builtin_bit_cast(half2v, (byte & 0x7Fu) * 0x00800080u);
}

// ---- global -> registers -> LDS -----------------------------------------
template <bool ALIGNED>
__device__ __forceinline__ uint4 load_chunk(const uint8_t* __restrict__ codes, int64_t row, int64_t K,
                                            int64_t kk) {
  const uint8_t* p = codes + row * (K / 2) + kk / 2;
  if (ALIGNED) return *reinterpret_cast<const uint4*>(p);
  uint4 v = make_uint4(0, 0, 0, 0);
  if (kk + 32 <= K) {
    const uint2 x0 = reinterpret_cast<const uint2*>(p)[0], x1 = reinterpret_cast<const uint2*>(p)[1];
    v = make_uint4(x0.x, x0.y, x1.x, x1.y);
  } else if (kk + 16 <= K) {
    const uint2 x0 = reinterpret_cast<const uint2*>(p)[0];
    v = make_uint4(x0.x, x0.y, 0, 0);
  }
  return v;
}

// the 8 scale bytes of one row for K-elements [k0, k0 + 128)
template <bool ALIGNED>
__device__ __forceinline__ uint2 load_scales(const uint8_t* __restrict__ scales, int64_t row, int64_t K,
                                             int64_t k0) {
  const uint8_t* p = scales + row * (K / 16) + k0 / 16;
  if (ALIGNED) return *reinterpret_cast<const uint2*>(p);
  uint32_t w[2] = {0, 0};
  for (int j = 0; j < 8; ++j)
    if (k0 / 16 + j < K / 16) w[j >> 2] |= (uint32_t)p[j] << (8 * (j & 3));
  return make_uint2(w[0], w[1]);
}

template <int BM, int BN>
struct Staged {
  static constexpr int kA = BM * 4 / kGemmThreads, kB = BN * 4 / kGemmThreads;
  static constexpr int kS = (BM + BN) / kGemmThreads;  // scale rows per thread
  uint4 a[kA], b[kB];
  uint2 s[kS];
};

template <int BM, int BN, bool ALIGNED>
__device__ __forceinline__ void stage_load(const GemmArgs& g, int64_t m0, int64_t n0, int64_t k0,
                                           Staged<BM, BN>& st) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < Staged<BM, BN>::kA; ++i) {
    const int idx = t + i * kGemmThreads;
    const int row = idx >> 2, chunk = idx & 3;
    const int64_t kk = k0 + chunk * 32;
    st.a[i] = (ALIGNED || kk < g.K) ? load_chunk<ALIGNED>(g.a_codes, min(m0 + row, g.M - 1), g.K, kk)
                                    : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < Staged<BM, BN>::kB; ++i) {
    const int idx = t + i * kGemmThreads;
    const int row = idx >> 2, chunk = idx & 3;
    const int64_t kk = k0 + chunk * 32;
    st.b[i] = (ALIGNED || kk < g.K) ? load_chunk<ALIGNED>(g.b_codes, min(n0 + row, g.N - 1), g.K, kk)
                                    : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < Staged<BM, BN>::kS; ++i) {
    const int r = t + i * kGemmThreads;  // rows 0..BM-1 of A, then BN rows of B
    if (r < BM)
      st.s[i] = load_scales<ALIGNED>(g.a_scales, min(m0 + r, g.M - 1), g.K, k0);
    else
      st.s[i] = load_scales<ALIGNED>(g.b_scales, min(n0 + r - BM, g.N - 1), g.K, k0);
  }
}

// LDS position of scale byte (row r, block column c) of a BM-row operand:
// column-major over the 8 block columns, and inside a column the rows of
// each wave half ordered (lane row li, tile i), so that a lane reads the
// scales of all its tiles for one column with a single 8-byte load.
template <int BM>
__device__ __forceinline__ int scale_pos(int r, int c) {
  constexpr int TI = BM / 32;
  return c * BM + (r / (BM / 2)) * (BM / 2) + (r & 15) * TI + ((r % (BM / 2)) >> 4);
}

template <int BM, int BN>
__device__ __forceinline__ void stage_store(GemmStage<BM, BN>& sm, const Staged<BM, BN>& st) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < Staged<BM, BN>::kA; ++i) {
    const int idx = t + i * kGemmThreads;
    *reinterpret_cast<uint4*>(sm.a + swz(idx >> 2, idx & 3)) = st.a[i];
  }
#pragma unroll
  for (int i = 0; i < Staged<BM, BN>::kB; ++i) {
    const int idx = t + i * kGemmThreads;
    *reinterpret_cast<uint4*>(sm.b + swz(idx >> 2, idx & 3)) = st.b[i];
  }
#pragma unroll
  for (int i = 0; i < Staged<BM, BN>::kS; ++i) {
    const int r = t + i * kGemmThreads;
    const uint32_t w[2] = {st.s[i].x, st.s[i].y};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint8_t v = (uint8_t)(w[c >> 2] >> (8 * (c & 3)));
      if (r < BM)
        sm.as[scale_pos<BM>(r, c)] = v;
      else
        sm.bs[scale_pos<BN>(r - BM, c)] = v;
    }
  }
}

// ---- the kernel ---------------------------------------------------------
// BM x BN tile per workgroup, (BM/2) x (BN/2) per wave.
template <int BM, int BN, bool ALIGNED>
__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm(GemmArgs g) {
  constexpr int TI = BM / 32, TJ = BN / 32;  // 16x16 MFMA tiles per wave
  __shared__ GemmStage<BM, BN> smem[2];
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 15, lg = lane >> 4;

  floatx4 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int64_t nk = (g.K + kBK - 1) / kBK;
  Staged<BM, BN> st;
  stage_load<BM, BN, ALIGNED>(g, m0, n0, 0, st);
  stage_store<BM, BN>(smem[0], st);
  __syncthreads();

  for (int64_t kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) stage_load<BM, BN, ALIGNED>(g, m0, n0, (kt + 1) * kBK, st);
    const GemmStage<BM, BN>& sm = smem[kt & 1];

    // two halves of the step: words 2h, 2h+1 of each fragment share the
    // scale byte h (K-elements 32g + 16h .. 32g + 16h + 15)
#pragma unroll 1
    for (int h = 0; h < 2; ++h) {
      uint2 qa[TI], qb[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i)
        qa[i] = *reinterpret_cast<const uint2*>(sm.a + swz(wm * (BM / 2) + i * 16 + li, lg) + 8 * h);
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        qb[j] = *reinterpret_cast<const uint2*>(sm.b + swz(wn * (BN / 2) + j * 16 + li, lg) + 8 * h);
      // scale bytes of block column 2g + h for all tiles of this lane
      const uint8_t* pa = sm.as + (2 * lg + h) * BM + wm * (BM / 2) + li * TI;
      const uint8_t* pb = sm.bs + (2 * lg + h) * BN + wn * (BN / 2) + li * TJ;
      uint8_t ba[TI], bb[TJ];
      *reinterpret_cast<uint2*>(ba) = *reinterpret_cast<const uint2*>(pa);
      *reinterpret_cast<uint2*>(bb) = *reinterpret_cast<const uint2*>(pb);
      half2v sa[TI], sb[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i) sa[i] = scale_h2(ba[i]);
#pragma unroll
      for (int j = 0; j < TJ; ++j) sb[j] = scale_h2(bb[j]);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        half8 fa[TI], fb[TJ];
#pragma unroll
        for (int i = 0; i < TI; ++i) fa[i] = unpack8(s ? qa[i].y : qa[i].x, sa[i]);
#pragma unroll
        for (int j = 0; j < TJ; ++j) fb[j] = unpack8(s ? qb[j].y : qb[j].x, sb[j]);
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      }
    }
    if (more) stage_store<BM, BN>(smem[(kt + 1) & 1], st);
    __syncthreads();
  }

  // epilogue: C = acc / (S_a * S_b), lane holds rows 4*lg .. 4*lg+3 of column li
  const float inv_a = __fdiv_rn(1.0f, g.a_ts[0]), inv_b = __fdiv_rn(1.0f, g.b_ts[0]);
#pragma unroll
  for (int i = 0; i < TI; ++i) {
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int64_t n = n0 + wn * (BN / 2) + j * 16 + li;
      if (n >= g.N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm * (BM / 2) + i * 16 + lg * 4 + r;
        if (m < g.M) g.c[m * g.N + n] = (acc[i][j][r] * inv_a) * inv_b;
      }
    }
  }
}

void launch_gemm(const GemmArgs& g, int cus, hipStream_t st) {
  (void)cus;
  constexpr int BM = 256, BN = 256;
  const dim3 grid((unsigned)((g.N + BN - 1) / BN), (unsigned)((g.M + BM - 1) / BM));
  const bool aligned = g.K % kBK == 0 && ((uintptr_t)g.a_codes % 16 == 0) &&
                       ((uintptr_t)g.b_codes % 16 == 0) && ((uintptr_t)g.a_scales % 8 == 0) &&
                       ((uintptr_t)g.b_scales % 8 == 0);
  if (aligned)
    hipLaunchKernelGGL((k_gemm<BM, BN, true>), grid, dim3(kGemmThreads), 0, st, g);
  else
    hipLaunchKernelGGL((k_gemm<BM, BN, false>), grid, dim3(kGemmThreads), 0, st, g);
}

}  // namespace nvfp4
