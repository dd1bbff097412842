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
// with fp32 accumulation; the two tensor scales are
// applied once in the epilogue.  (gfx950's scaled FP4 MFMA takes power-of-two
// scales per 32 elements, which cannot represent E4M3 scales per 16.)
//
// Two kernels.  k_gemm (any shape): a 256-thread workgroup owns a 256x256
// tile of C (128x128 when 256x256 tiles would not fill the CUs) and walks K
// in steps of 128; packed codes and scale bytes are staged through
// registers into LDS (double buffered, 16-byte chunks XOR-swizzled against
// bank conflicts); each wave owns a quarter of the tile,
// reads its packed fragments from LDS and expands them in registers for
// v_mfma_f32_16x16x32_f16.  Lane group g = lane / 16 of a fragment covers the
// 32 K-elements [32g, 32g+32) of a step; its word s feeds MFMA slice s.
// k_gemm_m32 (256-multiples, below) is the fast path.
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
//
// The four conversions go to four registers before any multiply: written as
// one conversion-multiply pair per byte, the compiler reused one temporary
// register, so every multiply waited on the conversion just before it and
// the next conversion on that multiply.
__device__ __forceinline__ half8 unpack8(uint32_t w, half2v sc) {
  half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 0);
  half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 1);
  half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 2);
  half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 3);
  asm volatile("" : "+v"(p0), "+v"(p1), "+v"(p2), "+v"(p3));  // all four are live at once
  p0 = p0 * sc;
  p1 = p1 * sc;
  p2 = p2 * sc;
  p3 = p3 * sc;
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

// ---- epilogue -------------------------------------------------------------
// One output element: v = (acc / S_a) / S_b as two multiplies by the
// reciprocals; with beta != 0, v + beta * C_old (C_old as stored, fp32 or
// bf16); stored as fp32, or rounded to nearest-even bf16.  m collects
// |stored value| for the optional output amax.
__device__ __forceinline__ void store_c(const GemmArgs& g, int64_t idx, float v, float& m, bool streaming) {
  if (g.c16) {
    if (g.beta != 0.0f) v = v + g.beta * __uint_as_float((uint32_t)g.c16[idx] << 16);
    const uint32_t h = bf16_rne(v);
    g.c16[idx] = (uint16_t)h;
    m = fmaxf(m, fabsf(__uint_as_float(h << 16)));
  } else {
    if (g.beta != 0.0f) v = v + g.beta * g.c[idx];
    if (streaming)
      __builtin_nontemporal_store(v, &g.c[idx]);  // written once, not read here (+2.5% measured)
    else
      g.c[idx] = v;
    m = fmaxf(m, fabsf(v));
  }
}

// the wave's maximum into *g.amax (float bits; non-negative floats order
// like their bit patterns); the atomic only when it can raise the value
__device__ __forceinline__ void amax_to(const GemmArgs& g, float m) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) {
    const unsigned bits = __float_as_uint(m);
    if (bits > __hip_atomic_load(g.amax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(g.amax, bits);
  }
}

__global__ void k_zero_amax(unsigned* p) { *p = 0u; }

// the T scale bytes (T = 4 or 8) a lane reads for its tiles of one block
// column, as one 4- or 8-byte LDS read
template <int T>
__device__ __forceinline__ void read_scale_bytes(const uint8_t* p, uint32_t w[2]) {
  static_assert(T == 4 || T == 8, "tiles per wave half");
  if (T == 8) {
    const uint2 x = *reinterpret_cast<const uint2*>(p);
    w[0] = x.x;
    w[1] = x.y;
  } else {
    w[0] = *reinterpret_cast<const uint32_t*>(p);
    w[1] = 0u;
  }
}

// ---- the kernel ---------------------------------------------------------
// BM x BN tile per workgroup (256 x 256, or 128 x 128 for problems whose
// 256 x 256 tiles would not fill the CUs), (BM/2) x (BN/2) per wave.
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
      uint32_t wa[2], wb[2];
      read_scale_bytes<TI>(pa, wa);
      read_scale_bytes<TJ>(pb, wb);
      half2v sa[TI], sb[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i) sa[i] = scale_h2((uint8_t)(wa[i >> 2] >> (8 * (i & 3))));
#pragma unroll
      for (int j = 0; j < TJ; ++j) sb[j] = scale_h2((uint8_t)(wb[j >> 2] >> (8 * (j & 3))));
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

  // epilogue: C = acc / (S_a * S_b), lane holds rows 4*lg .. 4*lg+3 of column li.
  // The loops are fully unrolled, so every accumulator index is a constant:
  // a row's offset is formed once per (i, r) and a column's once per j.  With
  // the 64-bit index of each value formed inside one loop around store_c,
  // the unrolled body exceeded the compiler's limit, the loop stayed, the
  // accumulators were indexed at run time and moved to scratch memory (1 KB
  // per lane), and a 256 x 256 x 256 product took 83 us.
  const float inv_a = __fdiv_rn(1.0f, g.a_ts[0]), inv_b = __fdiv_rn(1.0f, g.b_ts[0]);
  float cmax = 0.0f;
  const int64_t mrow = m0 + wm * (BM / 2) + lg * 4, ncol = n0 + wn * (BN / 2) + li;
  auto each = [&](auto&& put) {
#pragma unroll
    for (int i = 0; i < TI; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = mrow + i * 16 + r;
        const int64_t row = m * g.N + ncol;
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          if (m < g.M && ncol + j * 16 < g.N) put(row + j * 16, (acc[i][j][r] * inv_a) * inv_b);
      }
    }
  };
  if (!g.c16 && g.beta == 0.0f) {
    each([&](int64_t idx, float v) {
      g.c[idx] = v;
      cmax = fmaxf(cmax, fabsf(v));
    });
  } else {
    each([&](int64_t idx, float v) { store_c(g, idx, v, cmax, false); });
  }
  if (g.amax) amax_to(g, cmax);
}

// ---- fast path: direct-to-LDS stages, 32 x 32 x 16 MFMA, pipelined unpack --
// For M, N multiples of 256, K a multiple of 512 and aligned operands.
//  - A stage holds 256 K-elements of both operands (128 code bytes and 16
//    scale bytes per row, 72 KB); two stages are double buffered in LDS.
//  - Operand bytes go from global memory straight into LDS
//    (global_load_lds_dwordx4, 16 bytes per lane): no staging registers and
//    no LDS store instructions.  Code rows are 8 XOR-swizzled 16-byte
//    chunks, so the 8 rows a wave reads at once hit distinct banks.
//  - Four waves, one per SIMD, each own 128 x 128 of the 256 x 256 tile as
//    4 x 4 tiles of v_mfma_f32_32x32x16_f16 (accumulators in AGPRs).
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

constexpr int kDirBK = 256;                     // K-elements per stage
constexpr int kDirRow = kDirBK / 2;             // 128 code bytes per row

// physical 16-byte chunk of logical chunk c in row r (8 chunks per row)
__device__ __forceinline__ int dswz(int r, int c) { return r * kDirRow + ((c ^ ((r ^ (r >> 3)) & 7)) << 4); }

// Lane l feeds row l % 32 of a fragment; its lane group g = l / 32 covers the
// NVFP4 blocks 8g .. 8g + 7 of a stage, so MFMA step t = 2p + s takes half s
// of block 8g + p from each group (A and B use the same map, so the products
// pair up).  A step's fragments take 32 VGPRs, which leaves room to unpack
// step t + 1 while step t multiplies: the unpack and the LDS reads of the
// next block are interleaved instruction by instruction with the 16 MFMAs of
// a step (sched_group_barrier), so the vector ALU works under the matrix
// core.  The barrier that publishes the next stage sits before a stage's
// last step, whose MFMAs then cover the next stage's first reads and unpack.
typedef float floatx16 __attribute__((ext_vector_type(16)));

// NT = 32-column MFMA tiles per wave along N: 4 for a 256 x 256 workgroup
// tile; 2 (256 x 128) or 1 (256 x 64) for the last, partial wave of tiles.
template <int NT>
struct M32 {
  static constexpr int kBN = 64 * NT;                 // tile width
  static constexpr int kOffB = 256 * kDirRow;         // B codes after 32 KB of A codes
  static constexpr int kOffAS = kOffB + kBN * kDirRow;  // A scales, 4 KB
  static constexpr int kOffBS = kOffAS + 4096;          // B scales, NT KB
  static constexpr int kStage = kOffBS + 1024 * NT;
};

template <int NT>
struct M32Frag { half8 a[4], b[NT]; };
template <int NT>
struct M32Raw { uint4 a[4], b[NT]; };  // blocks 8g + 2Q (.x, .y) and 8g + 2Q + 1 (.z, .w)
template <int NT>
struct M32Scales { uint4 a[2], b[(NT + 1) / 2]; };  // dword 2i + q: blocks 8g + 4q .. + 3 of tile-row i

// A stage's scale bytes sit in LDS in their global order: row r's 16 bytes
// (blocks 0 .. 15 of the stage) at 16 r.  A wave loads 64 rows with one
// 16-byte-per-lane load (with 4-byte loads into a lane-shuffled layout a
// stage took 4 + NT load instructions per wave instead of 1 + 1, and every
// load instruction costs issue cycles beside the MFMAs).
template <int ROWS>
__device__ __forceinline__ void m32_issue_scales(const uint8_t* s0, int64_t ks, uint8_t* dst) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (64 * wave >= ROWS) return;  // wave-uniform: a 128-row operand takes two waves
  const uint32_t off = (uint32_t)((64 * wave + lane) * ks);
  __builtin_amdgcn_global_load_lds((glb_void_t*)(s0 + off), (lds_void_t*)(dst + 1024 * wave), 16, 0, 0);
}

// Part U (0..7) of a stage's loads: A block 8 * wave + U, B block
// 2 NT * wave + U (U < 2 NT), and with U = 0 / 1 the wave's rows of A / B
// scales.  A stage is issued as eight such parts spread over the
// first four step pairs: issued all at once, the 24 loads of every wave
// backed up in the texture unit and stalled the waves' MFMA issue (about 57
// cycles per load instruction, by counters).
template <int NT, int U>
__device__ __forceinline__ void m32_issue_part(const GemmArgs& g, int64_t m0, int64_t n0, int64_t k0,
                                               uint8_t* buf) {
  using L = M32<NT>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t kb = g.K / 2, ks = g.K / 16;
  {
    const uint8_t* a0 = g.a_codes + m0 * kb + k0 / 2;
    const int blk = 8 * wave + U;
    const int row = 8 * blk + (lane >> 3);
    const int chunk = (lane & 7) ^ ((row ^ (row >> 3)) & 7);
    const uint32_t off = (uint32_t)(row * kb + 16 * chunk);
    __builtin_amdgcn_global_load_lds((glb_void_t*)(a0 + off), (lds_void_t*)(buf + 1024 * blk), 16, 0, 0);
  }
  if (U < 2 * NT) {
    const uint8_t* b0 = g.b_codes + n0 * kb + k0 / 2;
    const int bb = 2 * NT * wave + U, brow = 8 * bb + (lane >> 3);
    const int bchunk = (lane & 7) ^ ((brow ^ (brow >> 3)) & 7);
    const uint32_t boff = (uint32_t)(brow * kb + 16 * bchunk);
    __builtin_amdgcn_global_load_lds((glb_void_t*)(b0 + boff), (lds_void_t*)(buf + L::kOffB + 1024 * bb), 16,
                                     0, 0);
  }
  if (U == 0) m32_issue_scales<256>(g.a_scales + m0 * ks + k0 / 16, ks, buf + L::kOffAS);
  if (U == 1) m32_issue_scales<64 * NT>(g.b_scales + n0 * ks + k0 / 16, ks, buf + L::kOffBS);
}

template <int NT>
__device__ __forceinline__ void m32_issue(const GemmArgs& g, int64_t m0, int64_t n0, int64_t k0,
                                          uint8_t* buf) {
  m32_issue_part<NT, 0>(g, m0, n0, k0, buf);
  m32_issue_part<NT, 1>(g, m0, n0, k0, buf);
  m32_issue_part<NT, 2>(g, m0, n0, k0, buf);
  m32_issue_part<NT, 3>(g, m0, n0, k0, buf);
  m32_issue_part<NT, 4>(g, m0, n0, k0, buf);
  m32_issue_part<NT, 5>(g, m0, n0, k0, buf);
  m32_issue_part<NT, 6>(g, m0, n0, k0, buf);
  m32_issue_part<NT, 7>(g, m0, n0, k0, buf);
}

template <int NT>
__device__ __forceinline__ void m32_read_scales(const uint8_t* buf, int wm, int wn, int r, int gq,
                                                M32Scales<NT>& d) {
  using L = M32<NT>;
  // tile-row i of A is row wm * 128 + 32 i + r; lane group gq takes blocks
  // 8 gq .. 8 gq + 7, i.e. bytes 8 gq .. 8 gq + 7 of the row (a read
  // instruction covers 512 contiguous bytes: no bank conflicts)
  const uint8_t* pa = buf + L::kOffAS + 16 * (wm * 128 + r) + 8 * gq;
  const uint8_t* pb = buf + L::kOffBS + 16 * (wn * 32 * NT + r) + 8 * gq;
  uint2 ra[4], rb[NT];
#pragma unroll
  for (int i = 0; i < 4; ++i) ra[i] = *reinterpret_cast<const uint2*>(pa + 16 * 32 * i);
#pragma unroll
  for (int j = 0; j < NT; ++j) rb[j] = *reinterpret_cast<const uint2*>(pb + 16 * 32 * j);
  d.a[0] = make_uint4(ra[0].x, ra[0].y, ra[1].x, ra[1].y);
  d.a[1] = make_uint4(ra[2].x, ra[2].y, ra[3].x, ra[3].y);
#pragma unroll
  for (int k = 0; k < (NT + 1) / 2; ++k) {
    const uint2 hi = 2 * k + 1 < NT ? rb[2 * k + 1 < NT ? 2 * k + 1 : 0] : make_uint2(0u, 0u);
    d.b[k] = make_uint4(rb[2 * k].x, rb[2 * k].y, hi.x, hi.y);
  }
}

// raw codes of blocks 8g + 2Q and 8g + 2Q + 1 (one 16-byte chunk) for the
// lane's four A and NT B rows; the eight rows of a swizzle group hit eight
// distinct chunk positions, so a 16-byte read is free of bank conflicts
template <int Q, int NT>
__device__ __forceinline__ void m32_read_raw(const uint8_t* buf, int wm, int wn, int r, int gq,
                                             M32Raw<NT>& q) {
  const int c = 4 * gq + Q;
#pragma unroll
  for (int i = 0; i < 4; ++i) q.a[i] = *reinterpret_cast<const uint4*>(buf + dswz(wm * 128 + i * 32 + r, c));
#pragma unroll
  for (int j = 0; j < NT; ++j)
    q.b[j] = *reinterpret_cast<const uint4*>(buf + M32<NT>::kOffB + dswz(wn * 32 * NT + j * 32 + r, c));
}

__device__ __forceinline__ uint32_t raw_word(const uint4& v, int k) {
  return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}

__device__ __forceinline__ uint32_t m32_dword(const uint4& v0, const uint4& v1, int k) {
  return k == 0 ? v0.x : k == 1 ? v0.y : k == 2 ? v0.z : k == 3 ? v0.w : k == 4 ? v1.x : k == 5 ? v1.y
       : k == 6 ? v1.z : v1.w;
}

// step (P, S): half S of block 8g + P
template <int P, int S, int NT>
__device__ __forceinline__ void m32_unpack(const M32Raw<NT>& q, const M32Scales<NT>& d, M32Frag<NT>& f) {
  constexpr int kw = 2 * (P & 1) + S;  // word of the 16-byte chunk
#pragma unroll
  for (int i = 0; i < 4; ++i)
    f.a[i] = unpack8(raw_word(q.a[i], kw),
                     scale_h2(m32_dword(d.a[0], d.a[1], 2 * i + (P >> 2)) >> (8 * (P & 3))));
#pragma unroll
  for (int j = 0; j < NT; ++j)
    f.b[j] = unpack8(raw_word(q.b[j], kw),
                     scale_h2(m32_dword(d.b[0], d.b[(NT + 1) / 2 - 1], 2 * j + (P >> 2)) >> (8 * (P & 3))));
}

template <int NT>
__device__ __forceinline__ void m32_mfma(const M32Frag<NT>& f, floatx16 (&acc)[4][NT]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

// Instruction order of one step of 4 NT MFMAs; READS groups of LDS reads ride
// on the first MFMAs; with DEP the unpack waits on them behind a few MFMAs.
// A step's unpack is about 10 VALU per fragment (4 + NT fragments).
template <int READS, bool DEP, int NT>
__device__ __forceinline__ void m32_order() {
  constexpr int kMfma = 4 * NT;
#pragma unroll
  for (int k = 0; k < READS; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, DEP ? 2 : 1, 0);
    if (!DEP) __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
  }
  constexpr int kCover = DEP ? (NT == 4 ? 3 : 2) : 0;
#pragma unroll
  for (int k = 0; k < kCover; ++k) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  constexpr int kRest = kMfma - READS - kCover;
  constexpr int kValu = NT == 4 ? (DEP ? 8 : 5) : (DEP ? 14 : 7);  // group sizes tuned by measurement
#pragma unroll
  for (int k = 0; k < kRest; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);
  }
}

// pair P of a stage: steps 2P and 2P + 1.  In: f = step (P, 0), q = raw of
// quad P / 2 (pairs P & ~1 and P | 1).  An even pair also reads the next
// quad into qn; an odd pair hands it over.
template <int P, int NT>
__device__ __forceinline__ void m32_pair(const uint8_t* cur, M32Frag<NT>& f, M32Raw<NT>& q, M32Raw<NT>& qn,
                                         const M32Scales<NT>& d, floatx16 (&acc)[4][NT], int wm, int wn,
                                         int r, int gq) {
  constexpr bool kRead = (P & 1) == 0 && P < 6;
  M32Frag<NT> f1;
  m32_mfma<NT>(f, acc);
  if (kRead) m32_read_raw<P / 2 + 1, NT>(cur, wm, wn, r, gq, qn);
  m32_unpack<P, 1, NT>(q, d, f1);
  m32_order<kRead ? 4 + NT : 0, false, NT>();
  __builtin_amdgcn_sched_barrier(0);
  m32_mfma<NT>(f1, acc);
  if (P & 1) {
    m32_unpack<P + 1, 0, NT>(qn, d, f);
    q = qn;
  } else {
    m32_unpack<P + 1, 0, NT>(q, d, f);
  }
  m32_order<0, false, NT>();
  __builtin_amdgcn_sched_barrier(0);
}

// One stage from cur.  In: f = step (0, 0), q = raw 0, d = scales.  Out: the
// same for the stage in nxt.  When issue is set, the stage at (m0, n0,
// k_issue) streams into nxt after the first pair of steps: every wave passed
// the barrier that ended the previous stage, the last reader of nxt.  The
// barrier before the last step waits for those loads.  No load is then in
// flight at a loop back edge, where the compiler's wait insertion would
// otherwise make the first LDS reads of cur wait for the loads into nxt.
template <int NT>
__device__ __forceinline__ void m32_stage(const GemmArgs& g, int64_t m0, int64_t n0, bool issue,
                                          int64_t k_issue, const uint8_t* cur, uint8_t* nxt, M32Frag<NT>& f,
                                          M32Raw<NT>& q, M32Scales<NT>& d, floatx16 (&acc)[4][NT], int wm,
                                          int wn, int r, int gq) {
  M32Raw<NT> qn;
  m32_pair<0, NT>(cur, f, q, qn, d, acc, wm, wn, r, gq);
  if (issue) {
    m32_issue_part<NT, 0>(g, m0, n0, k_issue, nxt);
    m32_issue_part<NT, 1>(g, m0, n0, k_issue, nxt);
  }
  __builtin_amdgcn_sched_barrier(0);
  m32_pair<1, NT>(cur, f, q, qn, d, acc, wm, wn, r, gq);
  if (issue) {
    m32_issue_part<NT, 2>(g, m0, n0, k_issue, nxt);
    m32_issue_part<NT, 3>(g, m0, n0, k_issue, nxt);
  }
  __builtin_amdgcn_sched_barrier(0);
  m32_pair<2, NT>(cur, f, q, qn, d, acc, wm, wn, r, gq);
  if (issue) {
    m32_issue_part<NT, 4>(g, m0, n0, k_issue, nxt);
    m32_issue_part<NT, 5>(g, m0, n0, k_issue, nxt);
  }
  __builtin_amdgcn_sched_barrier(0);
  m32_pair<3, NT>(cur, f, q, qn, d, acc, wm, wn, r, gq);
  if (issue) {
    m32_issue_part<NT, 6>(g, m0, n0, k_issue, nxt);
    m32_issue_part<NT, 7>(g, m0, n0, k_issue, nxt);
  }
  __builtin_amdgcn_sched_barrier(0);
  m32_pair<4, NT>(cur, f, q, qn, d, acc, wm, wn, r, gq);
  m32_pair<5, NT>(cur, f, q, qn, d, acc, wm, wn, r, gq);
  m32_pair<6, NT>(cur, f, q, qn, d, acc, wm, wn, r, gq);
  M32Frag<NT> f1;
  m32_mfma<NT>(f, acc);
  m32_unpack<7, 1, NT>(q, d, f1);
  m32_order<0, false, NT>();
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();  // waits for this wave's loads of nxt (vmcnt(0)), then all waves
  __builtin_amdgcn_sched_barrier(0);
  m32_mfma<NT>(f1, acc);
  m32_read_scales<NT>(nxt, wm, wn, r, gq, d);
  m32_read_raw<0, NT>(nxt, wm, wn, r, gq, q);
  m32_unpack<0, 0, NT>(q, d, f);
  m32_order<NT == 4 ? 6 : 5, true, NT>();
  __builtin_amdgcn_sched_barrier(0);
}

// Tiles are numbered in band order: bands of four tile rows, walked column
// by column (u -> tile_mn), so that 32 consecutive tiles form a 4 x 8 block.
// A launch covers tiles tile0 .. tile0 + ntl - 1 of that order.  With NT = 4
// the workgroups are dealt to the eight XCDs in turn and each XCD takes a
// contiguous run, so its 32 concurrent tiles share 4 slices of A and 8 of B
// per K-step in its L2 (instead of about 36 distinct ones); with NT = 2 or 1
// (the last, partial wave) workgroup u computes columns (u % (4 / NT)) * 64 NT
// .. of tile tile0 + u / (4 / NT).
// EX: the epilogue options of nvfp4_gemm_ex (bf16 output, beta, output
// amax); without them the plain fp32 epilogue, compiled on its own so that
// the main loop's register allocation is the same as for nvfp4_gemm.
__device__ __forceinline__ void tile_mn(int64_t u, int64_t ntm, int64_t ntn, int64_t& m0, int64_t& n0) {
  constexpr int64_t kBand = 4;
  const int64_t band = u / (kBand * ntn), rem = u % (kBand * ntn);
  const int64_t band_rows = min<int64_t>(kBand, ntm - band * kBand);
  m0 = (band * kBand + rem % band_rows) * 256;
  n0 = (rem / band_rows) * 256;
}

template <int NT, bool EX>
__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm_m32(GemmArgs g, int64_t tile0, int64_t ntl) {
  using L = M32<NT>;
  __shared__ __align__(16) uint8_t buf0[L::kStage];
  __shared__ __align__(16) uint8_t buf1[L::kStage];
  const int64_t ntm = g.M / 256, ntn = g.N / 256;
  int64_t u;
  if (NT == 4) {
    const int64_t per_xcd = (ntl + 7) / 8;
    u = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (u >= ntl) return;  // the whole workgroup
  } else {
    u = blockIdx.x / (4 / NT);
  }
  int64_t m0, n0;
  tile_mn(tile0 + u, ntm, ntn, m0, n0);
  if (NT < 4) n0 += (blockIdx.x % (4 / NT)) * L::kBN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 31, gq = lane >> 5;

  floatx16 acc[4][NT];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int k = 0; k < 16; ++k) acc[i][j][k] = 0.f;

  const int64_t nk = g.K / kDirBK;  // even
  m32_issue<NT>(g, m0, n0, 0, buf0);
  __syncthreads();
  M32Frag<NT> f;
  M32Raw<NT> q;
  M32Scales<NT> d;
  m32_read_scales<NT>(buf0, wm, wn, r, gq, d);
  m32_read_raw<0, NT>(buf0, wm, wn, r, gq, q);
  m32_unpack<0, 0, NT>(q, d, f);
  for (int64_t kt = 0; kt < nk; kt += 2) {
    m32_stage<NT>(g, m0, n0, true, (kt + 1) * kDirBK, buf0, buf1, f, q, d, acc, wm, wn, r, gq);
    // on the last stage the reads of buf0 at its end are of stale data and unused
    m32_stage<NT>(g, m0, n0, kt + 2 < nk, (kt + 2) * kDirBK, buf1, buf0, f, q, d, acc, wm, wn, r, gq);
  }

  // D layout of the 32 x 32 MFMA: lane l, value k -> column l % 32, row
  // 8 * (k / 4) + 4 * (l / 32) + k % 4
  const float inv_a = __fdiv_rn(1.0f, g.a_ts[0]), inv_b = __fdiv_rn(1.0f, g.b_ts[0]);
  float cmax = 0.0f;
  if (EX && g.c16 && g.beta == 0.0f && ((uintptr_t)g.c16 & 3) == 0) {
    // bf16 output without beta: columns n and n + 1 sit in lanes r and r ^ 1,
    // and values k, k + 1 (k even) in rows m, m + 1.  The lane pair swaps one
    // value, so the even lane stores row m and the odd lane row m + 1 as two
    // bf16 in 4 bytes each (half the store instructions of one bf16 per lane)
    const bool odd = r & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int64_t n = n0 + wn * 32 * NT + j * 32 + (r & ~1);
#pragma unroll
        for (int k = 0; k < 16; k += 2) {
          const int64_t m = m0 + wm * 128 + i * 32 + 8 * (k >> 2) + 4 * gq + (k & 3);
          const uint32_t h0 = bf16_rne((acc[i][j][k] * inv_a) * inv_b);
          const uint32_t h1 = bf16_rne((acc[i][j][k + 1] * inv_a) * inv_b);
          cmax = fmaxf(cmax, fmaxf(fabsf(__uint_as_float(h0 << 16)), fabsf(__uint_as_float(h1 << 16))));
          const uint32_t other =
              (uint32_t)__builtin_amdgcn_mov_dpp((int)(odd ? h0 : h1), 0xB1, 0xF, 0xF, true);
          const uint32_t packed = odd ? (other | (h1 << 16)) : (h0 | (other << 16));
          __builtin_nontemporal_store(packed, reinterpret_cast<uint32_t*>(g.c16 + (odd ? m + 1 : m) * g.N + n));
        }
      }
    }
  } else if (EX && g.beta != 0.0f && g.c16 && ((uintptr_t)g.c16 & 3) == 0) {
    // beta-accumulate into bf16, in the lane-pair form of the bf16 output
    // above: the pair swaps the fp32 values acc / (S_A S_B) over DPP, so the
    // even lane holds row m and the odd lane row m + 1, each for columns n
    // and n + 1; the lane loads that pair's old bf16 word, adds beta * old
    // per value (as store_c computes it), rounds and stores one word.  The
    // eight old words of a lane's MFMA tile are loaded together.
    const bool odd = r & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int64_t n = n0 + wn * 32 * NT + j * 32 + (r & ~1);
        int64_t idx[8];
        uint32_t old[8];
#pragma unroll
        for (int k = 0; k < 16; k += 2) {
          const int64_t m = m0 + wm * 128 + i * 32 + 8 * (k >> 2) + 4 * gq + (k & 3);
          idx[k / 2] = (odd ? m + 1 : m) * g.N + n;
          old[k / 2] = *reinterpret_cast<const uint32_t*>(g.c16 + idx[k / 2]);
        }
#pragma unroll
        for (int k = 0; k < 16; k += 2) {
          const float v0 = (acc[i][j][k] * inv_a) * inv_b, v1 = (acc[i][j][k + 1] * inv_a) * inv_b;
          const float other = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(odd ? v0 : v1), 0xB1, 0xF, 0xF, true));
          const float lo = odd ? other : v0, hi = odd ? v1 : other;  // columns n, n + 1 of the lane's row
          const uint32_t w = old[k / 2];
          const uint32_t hl = bf16_rne(lo + g.beta * __uint_as_float(w << 16));
          const uint32_t hh = bf16_rne(hi + g.beta * __uint_as_float(w & 0xFFFF0000u));
          __builtin_nontemporal_store(hl | (hh << 16), reinterpret_cast<uint32_t*>(g.c16 + idx[k / 2]));
          cmax = fmaxf(cmax, fmaxf(fabsf(__uint_as_float(hl << 16)), fabsf(__uint_as_float(hh << 16))));
        }
      }
    }
  } else if (EX && g.beta != 0.0f) {
    // beta-accumulate, v = acc / (S_A S_B) + beta * C_old (as store_c
    // computes it): the lane's 16 old values of one MFMA tile are loaded
    // together, then computed and stored, so the lane waits once per 16
    // values.  Through store_c, one value at a time, each load also waited
    // for the stores before it: 1.9x the plain GEMM's time (measured).
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int64_t n = n0 + wn * 32 * NT + j * 32 + r;
        int64_t idx[16];
        float old[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          idx[k] = (m0 + wm * 128 + i * 32 + 8 * (k >> 2) + 4 * gq + (k & 3)) * g.N + n;
          old[k] = g.c16 ? __uint_as_float((uint32_t)g.c16[idx[k]] << 16) : g.c[idx[k]];
        }
        if (g.c16) {
#pragma unroll
          for (int k = 0; k < 16; ++k) {
            const uint32_t h = bf16_rne((acc[i][j][k] * inv_a) * inv_b + g.beta * old[k]);
            g.c16[idx[k]] = (uint16_t)h;
            cmax = fmaxf(cmax, fabsf(__uint_as_float(h << 16)));
          }
        } else {
#pragma unroll
          for (int k = 0; k < 16; ++k) {
            const float v = (acc[i][j][k] * inv_a) * inv_b + g.beta * old[k];
            __builtin_nontemporal_store(v, &g.c[idx[k]]);
            cmax = fmaxf(cmax, fabsf(v));
          }
        }
      }
    }
  } else if (EX && !g.c16 && g.beta == 0.0f) {
    // fp32 output without beta (with an amax target): straight stores, as
    // below.  Through store_c, whose per-value branches on beta and the
    // output type the compiler keeps, this took about 15% longer.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int64_t n = n0 + wn * 32 * NT + j * 32 + r;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const int64_t m = m0 + wm * 128 + i * 32 + 8 * (k >> 2) + 4 * gq + (k & 3);
          const float v = (acc[i][j][k] * inv_a) * inv_b;
          cmax = fmaxf(cmax, fabsf(v));
          __builtin_nontemporal_store(v, &g.c[m * g.N + n]);
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int64_t n = n0 + wn * 32 * NT + j * 32 + r;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const int64_t m = m0 + wm * 128 + i * 32 + 8 * (k >> 2) + 4 * gq + (k & 3);
          if (EX)
            store_c(g, m * g.N + n, (acc[i][j][k] * inv_a) * inv_b, cmax, true);
          else  // streaming store: C is written once and not read here (+2.5% measured)
            __builtin_nontemporal_store((acc[i][j][k] * inv_a) * inv_b, &g.c[m * g.N + n]);
        }
      }
    }
  }
  if (EX && g.amax) amax_to(g, cmax);
}

// Whole waves of 256 x 256 tiles (one workgroup per CU); when the last wave
// would be at most half full, its tiles run as 256 x 128 halves instead, and
// when at most a quarter full as 256 x 64 quarters, so that wave spreads over
// the CUs (wgrad's 64 leftover tiles: 128 halves left half the CUs idle).
template <bool EX>
static void launch_m32(const GemmArgs& g, int64_t ntiles, int64_t full, int64_t rem, int64_t c, hipStream_t st) {
  const auto groups = [](int64_t n) { return (unsigned)(((n + 7) / 8) * 8); };
  if (rem == 0 || 2 * rem > c) {
    hipLaunchKernelGGL((k_gemm_m32<4, EX>), dim3(groups(ntiles)), dim3(kGemmThreads), 0, st, g, INT64_C(0),
                       ntiles);
  } else {
    if (full > 0)
      hipLaunchKernelGGL((k_gemm_m32<4, EX>), dim3(groups(full)), dim3(kGemmThreads), 0, st, g, INT64_C(0),
                         full);
    if (4 * rem <= c)
      hipLaunchKernelGGL((k_gemm_m32<1, EX>), dim3((unsigned)(4 * rem)), dim3(kGemmThreads), 0, st, g, full, rem);
    else
      hipLaunchKernelGGL((k_gemm_m32<2, EX>), dim3((unsigned)(2 * rem)), dim3(kGemmThreads), 0, st, g, full, rem);
  }
}

void launch_gemm(const GemmArgs& g, int cus, hipStream_t st) {
  constexpr int BM = 256, BN = 256;
  if (g.amax) hipLaunchKernelGGL(k_zero_amax, dim3(1), dim3(1), 0, st, g.amax);
  const dim3 grid((unsigned)((g.N + BN - 1) / BN), (unsigned)((g.M + BM - 1) / BM));
  const bool aligned = g.K % kBK == 0 && ((uintptr_t)g.a_codes % 16 == 0) &&
                       ((uintptr_t)g.b_codes % 16 == 0) && ((uintptr_t)g.a_scales % 8 == 0) &&
                       ((uintptr_t)g.b_scales % 8 == 0);
  if (aligned && g.M % 256 == 0 && g.N % 256 == 0 && g.K % (2 * kDirBK) == 0 &&
      g.K <= (INT64_C(1) << 24) && (uintptr_t)g.a_scales % 16 == 0 && (uintptr_t)g.b_scales % 16 == 0) {
    // (K <= 2^24 keeps the 32-bit byte offsets of m32_issue, up to 255 rows
    // of K / 2 bytes, below 2^31)
    const int64_t ntiles = (g.M / 256) * (g.N / 256);
    const int64_t c = std::max(cus, 1);
    const int64_t full = (ntiles / c) * c, rem = ntiles - full;
    if (g.c16 || g.beta != 0.0f || g.amax)
      launch_m32<true>(g, ntiles, full, rem, c, st);
    else
      launch_m32<false>(g, ntiles, full, rem, c, st);
  } else if ((int64_t)grid.x * grid.y >= (int64_t)std::max(cus, 1)) {
    if (aligned)
      hipLaunchKernelGGL((k_gemm<BM, BN, true>), grid, dim3(kGemmThreads), 0, st, g);
    else
      hipLaunchKernelGGL((k_gemm<BM, BN, false>), grid, dim3(kGemmThreads), 0, st, g);
  } else {
    // fewer 256 x 256 tiles than CUs: 128 x 128 tiles, four times as many
    // workgroups (a 256 x 256 x 256 product: one workgroup 18 us, four 8 us)
    const dim3 grid128((unsigned)((g.N + 127) / 128), (unsigned)((g.M + 127) / 128));
    if (aligned)
      hipLaunchKernelGGL((k_gemm<128, 128, true>), grid128, dim3(kGemmThreads), 0, st, g);
    else
      hipLaunchKernelGGL((k_gemm<128, 128, false>), grid128, dim3(kGemmThreads), 0, st, g);
  }
}

}  // namespace nvfp4
