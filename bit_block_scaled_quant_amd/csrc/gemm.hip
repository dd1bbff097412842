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

// ---- fast path: direct-to-LDS stages of 256 K-elements -----------------
// For M, N multiples of 256, K a multiple of 512 and aligned operands.
// Same 256x256 tile, 128x128 per wave and exact unpack as k_gemm, but
//  - a stage holds 256 K-elements (128 code bytes and 16 scale bytes per
//    row), halving the barriers per K;
//  - operand bytes go from global memory straight into LDS
//    (global_load_lds_dwordx4 for codes, _dword for scales): no staging
//    registers and no LDS store instructions;
//  - in quarter h of a stage, lane group g of a fragment reads one whole
//    NVFP4 block (K-elements 64g + 16h .. 64g + 16h + 15), so each lane needs
//    one scale per tile and quarter; scales sit in LDS as four dword planes
//    per operand, rows in (wave half, lane row, tile) order, and a lane reads
//    the scales of all its tiles for the whole stage with two 16-byte reads.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

constexpr int kDirBK = 256;                     // K-elements per stage
constexpr int kDirRow = kDirBK / 2;             // 128 code bytes per row
constexpr int kDirCodes = 256 * kDirRow;        // 32 KB per operand
constexpr int kDirScales = 256 * (kDirBK / 16);  // 4 KB per operand
constexpr int kDirOffB = kDirCodes;
constexpr int kDirOffAS = 2 * kDirCodes;
constexpr int kDirOffBS = kDirOffAS + kDirScales;
constexpr int kDirStage = kDirOffBS + kDirScales;  // 72 KB

// physical 16-byte chunk of logical chunk c in row r (8 chunks per row)
__device__ __forceinline__ int dswz(int r, int c) { return r * kDirRow + ((c ^ ((r ^ (r >> 3)) & 7)) << 4); }

// Direct loads of one stage (K-elements [k0, k0 + 256)) into buf.
// Codes: 1 KB block blk = 8 * wave + u holds rows 8 * blk .. 8 * blk + 7;
// lane l writes the 16-byte slot 64 * blk + l, i.e. row 8 * blk + l / 8 at
// physical chunk l % 8, and fetches the logical chunk stored there.
// Scales: dword slot 128 * wave + 64 * v + l (4 per wave... see below) holds
// bytes 4p .. 4p + 3 (block columns 4p .. 4p + 3) of one row.
__device__ __forceinline__ void dir_issue(const GemmArgs& g, int64_t m0, int64_t n0, int64_t k0,
                                          uint8_t* buf) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t kb = g.K / 2, ks = g.K / 16;
  const uint8_t* a0 = g.a_codes + m0 * kb + k0 / 2;
  const uint8_t* b0 = g.b_codes + n0 * kb + k0 / 2;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int blk = 8 * wave + u;
    const int row = 8 * blk + (lane >> 3);
    const int chunk = (lane & 7) ^ ((row ^ (row >> 3)) & 7);
    const uint32_t off = (uint32_t)(row * kb + 16 * chunk);
    __builtin_amdgcn_global_load_lds((glb_void_t*)(a0 + off), (lds_void_t*)(buf + 1024 * blk), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((glb_void_t*)(b0 + off), (lds_void_t*)(buf + kDirOffB + 1024 * blk),
                                     16, 0, 0);
  }
  // 1024 dword slots per operand: slot = 256 * plane + q, q = 128 * half +
  // 8 * li + i for row 128 * half + 16 * i + li; wave w covers slots
  // 256 * w .. 256 * w + 255 (plane w) in four 64-slot pieces
  const uint8_t* as0 = g.a_scales + m0 * ks + k0 / 16 + 4 * wave;
  const uint8_t* bs0 = g.b_scales + n0 * ks + k0 / 16 + 4 * wave;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int q = 64 * v + lane;
    const int r = 128 * (q >> 7) + 16 * (q & 7) + ((q >> 3) & 15);
    const uint32_t off = (uint32_t)(r * ks);
    __builtin_amdgcn_global_load_lds((glb_void_t*)(as0 + off),
                                     (lds_void_t*)(buf + kDirOffAS + 1024 * wave + 256 * v), 4, 0, 0);
    __builtin_amdgcn_global_load_lds((glb_void_t*)(bs0 + off),
                                     (lds_void_t*)(buf + kDirOffBS + 1024 * wave + 256 * v), 4, 0, 0);
  }
}

// one stage of MFMA work from buf: four quarters, each one NVFP4 block per
// lane group (two MFMA slices)
__device__ __forceinline__ void dir_compute(const uint8_t* buf, floatx4 (&acc)[8][8], int wm, int wn,
                                            int li, int lg) {
  // scale dwords of plane lg (block columns 4g .. 4g + 3) for all tiles
  uint32_t da[8], db[8];
  {
    const uint4* pa = reinterpret_cast<const uint4*>(buf + kDirOffAS + 4 * (lg * 256 + wm * 128 + li * 8));
    const uint4* pb = reinterpret_cast<const uint4*>(buf + kDirOffBS + 4 * (lg * 256 + wn * 128 + li * 8));
    const uint4 x0 = pa[0], x1 = pa[1], y0 = pb[0], y1 = pb[1];
    da[0] = x0.x; da[1] = x0.y; da[2] = x0.z; da[3] = x0.w;
    da[4] = x1.x; da[5] = x1.y; da[6] = x1.z; da[7] = x1.w;
    db[0] = y0.x; db[1] = y0.y; db[2] = y0.z; db[3] = y0.w;
    db[4] = y1.x; db[5] = y1.y; db[6] = y1.z; db[7] = y1.w;
  }
#pragma unroll 1
  for (int h = 0; h < 4; ++h) {
    // block 4g + h: 8 bytes at logical chunk 2g + h / 2, byte 8 * (h & 1)
    const int c = 2 * lg + (h >> 1), sub = 8 * (h & 1), sh = 8 * h;
    uint2 qa[8], qb[8];
    half2v sa[8], sb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      qa[i] = *reinterpret_cast<const uint2*>(buf + dswz(wm * 128 + i * 16 + li, c) + sub);
      sa[i] = scale_h2(da[i] >> sh);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      qb[j] = *reinterpret_cast<const uint2*>(buf + kDirOffB + dswz(wn * 128 + j * 16 + li, c) + sub);
      sb[j] = scale_h2(db[j] >> sh);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      half8 fa[8], fb[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) fa[i] = unpack8(s ? qa[i].y : qa[i].x, sa[i]);
#pragma unroll
      for (int j = 0; j < 8; ++j) fb[j] = unpack8(s ? qb[j].y : qb[j].x, sb[j]);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  }
}

__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm_direct(GemmArgs g) {
  __shared__ __align__(16) uint8_t buf0[kDirStage];
  __shared__ __align__(16) uint8_t buf1[kDirStage];
  const int64_t m0 = (int64_t)blockIdx.y * 256, n0 = (int64_t)blockIdx.x * 256;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 15, lg = lane >> 4;

  floatx4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int64_t nk = g.K / kDirBK;  // even
  dir_issue(g, m0, n0, 0, buf0);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt(0) only
  __syncthreads();
  // Unrolled over the two buffers: a stage is computed from one buffer while
  // the next stage streams into the other; the barrier after each stage
  // publishes the streamed stage and frees the buffer just read.
  for (int64_t kt = 0; kt < nk; kt += 2) {
    dir_issue(g, m0, n0, (kt + 1) * kDirBK, buf1);
    dir_compute(buf0, acc, wm, wn, li, lg);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __syncthreads();
    if (kt + 2 < nk) dir_issue(g, m0, n0, (kt + 2) * kDirBK, buf0);
    dir_compute(buf1, acc, wm, wn, li, lg);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __syncthreads();
  }

  const float inv_a = __fdiv_rn(1.0f, g.a_ts[0]), inv_b = __fdiv_rn(1.0f, g.b_ts[0]);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t n = n0 + wn * 128 + j * 16 + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm * 128 + i * 16 + lg * 4 + r;
        g.c[m * g.N + n] = (acc[i][j][r] * inv_a) * inv_b;
      }
    }
  }
}

// ---- 8-wave variant of the fast path ------------------------------------
// Same stages, layouts and unpack as k_gemm_direct, but 512 threads: eight
// waves in a 2 x 4 grid, each owning 128 x 64 of the 256 x 256 tile, two per
// SIMD.  A wave unpacks and multiplies in program order; the other wave on
// the SIMD fills its VALU and LDS phases with matrix work.
constexpr int kThreads8 = 512;

__device__ __forceinline__ void dir8_issue(const GemmArgs& g, int64_t m0, int64_t n0, int64_t k0,
                                           uint8_t* buf) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // 0..7
  const int64_t kb = g.K / 2, ks = g.K / 16;
  const uint8_t* a0 = g.a_codes + m0 * kb + k0 / 2;
  const uint8_t* b0 = g.b_codes + n0 * kb + k0 / 2;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int blk = 4 * wave + u;  // 32 blocks of 1 KB per operand
    const int row = 8 * blk + (lane >> 3);
    const int chunk = (lane & 7) ^ ((row ^ (row >> 3)) & 7);
    const uint32_t off = (uint32_t)(row * kb + 16 * chunk);
    __builtin_amdgcn_global_load_lds((glb_void_t*)(a0 + off), (lds_void_t*)(buf + 1024 * blk), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((glb_void_t*)(b0 + off), (lds_void_t*)(buf + kDirOffB + 1024 * blk),
                                     16, 0, 0);
  }
  // scale planes: wave w fills plane w / 2, slots 128 * (w & 1) .. + 127
  const int plane = wave >> 1;
  const uint8_t* as0 = g.a_scales + m0 * ks + k0 / 16 + 4 * plane;
  const uint8_t* bs0 = g.b_scales + n0 * ks + k0 / 16 + 4 * plane;
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    const int q = 128 * (wave & 1) + 64 * v + lane;
    const int r = 128 * (q >> 7) + 16 * (q & 7) + ((q >> 3) & 15);
    const uint32_t off = (uint32_t)(r * ks);
    const int dst = 1024 * plane + 4 * (128 * (wave & 1) + 64 * v);
    __builtin_amdgcn_global_load_lds((glb_void_t*)(as0 + off), (lds_void_t*)(buf + kDirOffAS + dst), 4, 0, 0);
    __builtin_amdgcn_global_load_lds((glb_void_t*)(bs0 + off), (lds_void_t*)(buf + kDirOffBS + dst), 4, 0, 0);
  }
}

// one stage from buf for a 128 x 64 wave tile at rows wm*128, columns wn*64
__device__ __forceinline__ void dir8_compute(const uint8_t* buf, floatx4 (&acc)[8][4], int wm, int wn,
                                             int li, int lg) {
  uint32_t da[8], db[4];
  {
    const uint4* pa = reinterpret_cast<const uint4*>(buf + kDirOffAS + 4 * (lg * 256 + wm * 128 + li * 8));
    const uint4 x0 = pa[0], x1 = pa[1];
    da[0] = x0.x; da[1] = x0.y; da[2] = x0.z; da[3] = x0.w;
    da[4] = x1.x; da[5] = x1.y; da[6] = x1.z; da[7] = x1.w;
    // B rows wn*64 + j*16 + li: half wn / 2, tile 4 * (wn & 1) + j of that half
    const uint4 y = *reinterpret_cast<const uint4*>(buf + kDirOffBS +
                                                    4 * (lg * 256 + (wn >> 1) * 128 + li * 8 + 4 * (wn & 1)));
    db[0] = y.x; db[1] = y.y; db[2] = y.z; db[3] = y.w;
  }
#pragma unroll 1
  for (int h = 0; h < 4; ++h) {
    const int c = 2 * lg + (h >> 1), sub = 8 * (h & 1), sh = 8 * h;
    uint2 qa[8], qb[4];
    half2v sa[8], sb[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      qa[i] = *reinterpret_cast<const uint2*>(buf + dswz(wm * 128 + i * 16 + li, c) + sub);
      sa[i] = scale_h2(da[i] >> sh);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      qb[j] = *reinterpret_cast<const uint2*>(buf + kDirOffB + dswz(wn * 64 + j * 16 + li, c) + sub);
      sb[j] = scale_h2(db[j] >> sh);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      half8 fa[8], fb[4];
#pragma unroll
      for (int i = 0; i < 8; ++i) fa[i] = unpack8(s ? qa[i].y : qa[i].x, sa[i]);
#pragma unroll
      for (int j = 0; j < 4; ++j) fb[j] = unpack8(s ? qb[j].y : qb[j].x, sb[j]);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  }
}

__global__ __launch_bounds__(kThreads8, 1) void k_gemm_direct8(GemmArgs g) {
  __shared__ __align__(16) uint8_t buf0[kDirStage];
  __shared__ __align__(16) uint8_t buf1[kDirStage];
  const int64_t m0 = (int64_t)blockIdx.y * 256, n0 = (int64_t)blockIdx.x * 256;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int li = lane & 15, lg = lane >> 4;

  floatx4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int64_t nk = g.K / kDirBK;  // even
  dir8_issue(g, m0, n0, 0, buf0);
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __syncthreads();
  for (int64_t kt = 0; kt < nk; kt += 2) {
    dir8_issue(g, m0, n0, (kt + 1) * kDirBK, buf1);
    dir8_compute(buf0, acc, wm, wn, li, lg);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __syncthreads();
    if (kt + 2 < nk) dir8_issue(g, m0, n0, (kt + 2) * kDirBK, buf0);
    dir8_compute(buf1, acc, wm, wn, li, lg);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __syncthreads();
  }

  const float inv_a = __fdiv_rn(1.0f, g.a_ts[0]), inv_b = __fdiv_rn(1.0f, g.b_ts[0]);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + wn * 64 + j * 16 + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm * 128 + i * 16 + lg * 4 + r;
        g.c[m * g.N + n] = (acc[i][j][r] * inv_a) * inv_b;
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
  if (aligned && g.M % 256 == 0 && g.N % 256 == 0 && g.K % (2 * kDirBK) == 0 &&
      g.K <= (INT64_C(1) << 26) && (uintptr_t)g.a_scales % 4 == 0 && (uintptr_t)g.b_scales % 4 == 0)
    hipLaunchKernelGGL(k_gemm_direct8, grid, dim3(kThreads8), 0, st, g);
  else if (aligned)
    hipLaunchKernelGGL((k_gemm<BM, BN, true>), grid, dim3(kGemmThreads), 0, st, g);
  else
    hipLaunchKernelGGL((k_gemm<BM, BN, false>), grid, dim3(kGemmThreads), 0, st, g);
}

}  // namespace nvfp4
