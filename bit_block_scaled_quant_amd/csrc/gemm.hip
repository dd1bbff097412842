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
// Tiling: a 256-thread workgroup owns a 128x128 tile of C and walks K in
// steps of 128.  Packed codes and scale bytes are staged through LDS (double
// buffered, 16-byte chunks XOR-swizzled against bank conflicts); each wave
// owns a 64x64 sub-tile, reads its packed fragments from LDS and expands
// them in registers.  Lane group g = lane / 16 of a fragment covers the 32
// K-elements [32g, 32g+32) of a step; its word s feeds MFMA slice s.  A and B
// use the same lane-to-K map, so the products pair up correctly.
#include "internal.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kGemmThreads = 256;
constexpr int kBM = 128, kBN = 128;
constexpr int kBK = 128;           // K-elements per step
constexpr int kRowBytes = kBK / 2;  // 64 bytes of codes per row per step
constexpr int kRowScales = kBK / 16;

struct __align__(16) GemmStage {
  uint8_t a[kBM * kRowBytes];
  uint8_t b[kBN * kRowBytes];
  uint8_t as[kBM * kRowScales];
  uint8_t bs[kBN * kRowScales];
};

// 16-byte chunk c of row r lives at chunk c ^ ((r >> 1) & 3): eight
// consecutive rows reading the same chunk hit eight distinct bank groups
__device__ __forceinline__ int swz(int r, int c) { return r * kRowBytes + ((c ^ ((r >> 1) & 3)) << 4); }

// Eight E2M1 codes (element 2k in the low nibble of byte k) -> eight exact
// fp16 values times the block scale, in the lane order
// [n0, n4, n1, n5, n2, n6, n3, n7].  Magnitudes come from a byte table via
// v_perm (fp16 high bytes of 0, .5, 1, 1.5, 2, 3, 4, 6; low bytes are 0),
// the sign bit is moved into place, and one packed multiply applies the
// scale (exact: at most 6 significant bits).
__device__ __forceinline__ half8 unpack8(uint32_t w, half2v sc) {
  const uint32_t lo = w & 0x07070707u;         // n0 n2 n4 n6
  const uint32_t hi = (w >> 4) & 0x07070707u;  // n1 n3 n5 n7
  const uint32_t z = 0x0C0C0C0Cu;              // selector 0x0C yields 0x00
  const uint32_t tlo = 0x3E3C3800u, thi = 0x46444240u;
  const uint32_t s0 = __builtin_amdgcn_perm(z, lo, 0x02040004u);  // [0C n0 0C n4]
  const uint32_t s1 = __builtin_amdgcn_perm(z, hi, 0x02040004u);  // [0C n1 0C n5]
  const uint32_t s2 = __builtin_amdgcn_perm(z, lo, 0x03040104u);  // [0C n2 0C n6]
  const uint32_t s3 = __builtin_amdgcn_perm(z, hi, 0x03040104u);  // [0C n3 0C n7]
  uint32_t d[4];
  d[0] = __builtin_amdgcn_perm(thi, tlo, s0) | ((w << 12) & 0x80008000u);
  d[1] = __builtin_amdgcn_perm(thi, tlo, s1) | ((w << 8) & 0x80008000u);
  d[2] = __builtin_amdgcn_perm(thi, tlo, s2) | ((w << 4) & 0x80008000u);
  d[3] = __builtin_amdgcn_perm(thi, tlo, s3) | (w & 0x80008000u);
  half8 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    half2v p = __builtin_bit_cast(half2v, d[i]) * sc;
    out[2 * i] = p[0];
    out[2 * i + 1] = p[1];
  }
  return out;
}

__device__ __forceinline__ half2v scale_h2(uint32_t byte) {
  const _Float16 h = (_Float16)e4m3_decode(byte);  // exact: 2^-9 .. 448
  return half2v{h, h};
}

// ---- global -> registers -> LDS -----------------------------------------
struct Staged {
  uint4 a[2], b[2];
  uint2 s;  // threads 0..127: 8 A scale bytes of a row; 128..255: B
};

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

template <bool ALIGNED>
__device__ __forceinline__ void stage_load(const GemmArgs& g, int64_t m0, int64_t n0, int64_t k0,
                                           Staged& st) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = t + i * kGemmThreads;
    const int row = idx >> 2, chunk = idx & 3;
    const int64_t kk = k0 + chunk * 32;
    const int64_t ra = min(m0 + row, g.M - 1), rb = min(n0 + row, g.N - 1);
    st.a[i] = (ALIGNED || kk < g.K) ? load_chunk<ALIGNED>(g.a_codes, ra, g.K, kk) : make_uint4(0, 0, 0, 0);
    st.b[i] = (ALIGNED || kk < g.K) ? load_chunk<ALIGNED>(g.b_codes, rb, g.K, kk) : make_uint4(0, 0, 0, 0);
  }
  if (t < kBM)
    st.s = load_scales<ALIGNED>(g.a_scales, min(m0 + t, g.M - 1), g.K, k0);
  else
    st.s = load_scales<ALIGNED>(g.b_scales, min(n0 + t - kBM, g.N - 1), g.K, k0);
}

__device__ __forceinline__ void stage_store(GemmStage& sm, const Staged& st) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = t + i * kGemmThreads;
    const int row = idx >> 2, chunk = idx & 3;
    *reinterpret_cast<uint4*>(sm.a + swz(row, chunk)) = st.a[i];
    *reinterpret_cast<uint4*>(sm.b + swz(row, chunk)) = st.b[i];
  }
  if (t < kBM)
    *reinterpret_cast<uint2*>(sm.as + t * kRowScales) = st.s;
  else
    *reinterpret_cast<uint2*>(sm.bs + (t - kBM) * kRowScales) = st.s;
}

// ---- the kernel ---------------------------------------------------------
template <bool ALIGNED>
__global__ __launch_bounds__(kGemmThreads) void k_gemm(GemmArgs g) {
  __shared__ GemmStage smem[2];
  const int64_t m0 = (int64_t)blockIdx.y * kBM, n0 = (int64_t)blockIdx.x * kBN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 15, lg = lane >> 4;

  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int64_t nk = (g.K + kBK - 1) / kBK;
  Staged st;
  stage_load<ALIGNED>(g, m0, n0, 0, st);
  stage_store(smem[0], st);
  __syncthreads();

  for (int64_t kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) stage_load<ALIGNED>(g, m0, n0, (kt + 1) * kBK, st);
    const GemmStage& sm = smem[kt & 1];

    uint4 qa[4], qb[4];
    uint32_t sa[4], sb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ra = wm * 64 + i * 16 + li, rb = wn * 64 + i * 16 + li;
      qa[i] = *reinterpret_cast<const uint4*>(sm.a + swz(ra, lg));
      qb[i] = *reinterpret_cast<const uint4*>(sm.b + swz(rb, lg));
      sa[i] = *reinterpret_cast<const uint16_t*>(sm.as + ra * kRowScales + 2 * lg);
      sb[i] = *reinterpret_cast<const uint16_t*>(sm.bs + rb * kRowScales + 2 * lg);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      half8 fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t wa = s == 0 ? qa[i].x : s == 1 ? qa[i].y : s == 2 ? qa[i].z : qa[i].w;
        const uint32_t wb = s == 0 ? qb[i].x : s == 1 ? qb[i].y : s == 2 ? qb[i].z : qb[i].w;
        fa[i] = unpack8(wa, scale_h2((sa[i] >> (8 * (s >> 1))) & 0xFFu));
        fb[i] = unpack8(wb, scale_h2((sb[i] >> (8 * (s >> 1))) & 0xFFu));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (more) stage_store(smem[(kt + 1) & 1], st);
    __syncthreads();
  }

  // epilogue: C = acc / (S_a * S_b), lane holds rows 4*lg .. 4*lg+3 of column li
  const float inv_a = __fdiv_rn(1.0f, g.a_ts[0]), inv_b = __fdiv_rn(1.0f, g.b_ts[0]);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + wn * 64 + j * 16 + li;
      if (n >= g.N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm * 64 + i * 16 + lg * 4 + r;
        if (m < g.M) g.c[m * g.N + n] = (acc[i][j][r] * inv_a) * inv_b;
      }
    }
  }
}

void launch_gemm(const GemmArgs& g, int cus, hipStream_t st) {
  (void)cus;
  const dim3 grid((unsigned)((g.N + kBN - 1) / kBN), (unsigned)((g.M + kBM - 1) / kBM));
  const bool aligned = g.K % kBK == 0 && ((uintptr_t)g.a_codes % 16 == 0) &&
                       ((uintptr_t)g.b_codes % 16 == 0) && ((uintptr_t)g.a_scales % 8 == 0) &&
                       ((uintptr_t)g.b_scales % 8 == 0);
  if (aligned)
    hipLaunchKernelGGL(k_gemm<true>, grid, dim3(kGemmThreads), 0, st, g);
  else
    hipLaunchKernelGGL(k_gemm<false>, grid, dim3(kGemmThreads), 0, st, g);
}

}  // namespace nvfp4
