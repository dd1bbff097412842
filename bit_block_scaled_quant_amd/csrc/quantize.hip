// NVFP4 quantizer kernels for CDNA4 (gfx950).
//
// "Pretraining Large Language Models with NVFP4", Technische samenvatting,
// 2A: the FP32 per-tensor scale needs the amax of the whole tensor before any
// block can be encoded, so a quantization is two passes over the input:
//   pass 1  k_amax_plain / k_amax_rht: every thread reduces |x| (after the
//           Hadamard transform of 2B.2 when it is on) over its elements,
//           waves reduce with cross-lane shuffles, one atomic max per
//           workgroup on the float bits (non-negative floats order like
//           their bit patterns);
//   pass 2  encode: the per-tensor scale is derived from the amax by every
//           workgroup; each 16-element block gets its E4M3 scale and E2M1
//           codes (RNE, or SR of 2B.4 with Philox draws).
// Pass 2 comes in three shapes:
//   k_encode_rows   1x16 blocks along rows only: one thread per block,
//                   coalesced 16-byte loads, 8-byte code stores;
//   k_encode_tile1d 1x16 rowwise blocks plus the columnwise copy (blocks of
//                   16 rows, written as rows of the transpose): a 128x128
//                   tile is staged in LDS so that both copies leave in
//                   coalesced 64-byte row segments;
//   k_encode_tile2d 16x16 blocks (2B.3): one scale per tile, each element
//                   encoded once and written both ways, so the transposed
//                   copy is bit-identical to quantizing W^T.
// k_rht writes the transform of 2B.2 alone (fp32 output).
#include "internal.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

constexpr int kThreads = 256;
constexpr int kTile = 128;

// ------------------------------------------------------------ pass 1 -----
__global__ void k_init_amax(float* ts) {
  ts[0] = 0.0f;
  ts[1] = 0.0f;
}

// |x| of the two bf16 in a word as the high halves of fp32 bit patterns is
// order-preserving, so the amax without the transform is an integer max of
// (w & 0x7FFF7FFF) per 16-bit half (v_pk_max_u16), and of (w & 0x7FFFFFFF)
// for fp32; four independent 16-byte loads per lane keep enough bytes in
// flight.
typedef unsigned short ushort2v __attribute__((ext_vector_type(2)));

template <bool BF16>
__device__ __forceinline__ void absmax_vec(const uint4& q, ushort2v& m16, uint32_t& m32) {
  if (BF16) {
    m16 = __builtin_elementwise_max(m16, __builtin_bit_cast(ushort2v, q.x & 0x7FFF7FFFu));
    m16 = __builtin_elementwise_max(m16, __builtin_bit_cast(ushort2v, q.y & 0x7FFF7FFFu));
    m16 = __builtin_elementwise_max(m16, __builtin_bit_cast(ushort2v, q.z & 0x7FFF7FFFu));
    m16 = __builtin_elementwise_max(m16, __builtin_bit_cast(ushort2v, q.w & 0x7FFF7FFFu));
  } else {
    m32 = max(m32, max(max(q.x & 0x7FFFFFFFu, q.y & 0x7FFFFFFFu), max(q.z & 0x7FFFFFFFu, q.w & 0x7FFFFFFFu)));
  }
}

__device__ __forceinline__ void block_max_to(float m, float* ts) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  __shared__ float red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kThreads / 64; ++w) m = fmaxf(m, red[w]);
    // Same-address atomics serialize in L2: issue one only when this block's
    // maximum beats the value already there (read past the L1; a stale
    // value only costs an extra atomic).
    unsigned int* t = reinterpret_cast<unsigned int*>(ts + 1);
    const unsigned int bits = __float_as_uint(m);
    if (bits > __hip_atomic_load(t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(t, bits);
  }
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_amax_plain(const uint4* __restrict__ x, int64_t nvec,
                                                         float* __restrict__ ts) {
  ushort2v m16 = {0, 0};
  uint32_t m32 = 0;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + 3 * stride < nvec; i += 4 * stride) {
    const uint4 a = ld_stream(x + i), b = ld_stream(x + i + stride), c = ld_stream(x + i + 2 * stride),
                d = ld_stream(x + i + 3 * stride);
    absmax_vec<BF16>(a, m16, m32);
    absmax_vec<BF16>(b, m16, m32);
    absmax_vec<BF16>(c, m16, m32);
    absmax_vec<BF16>(d, m16, m32);
  }
  for (; i < nvec; i += stride) absmax_vec<BF16>(ld_stream(x + i), m16, m32);
  const uint32_t bits = BF16 ? ((uint32_t)max(m16.x, m16.y) << 16) : m32;
  block_max_to(__uint_as_float(bits), ts);
}

// amax after the Hadamard transform: 16 contiguous elements per lane, two
// chunks per iteration
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_amax_rht(const void* __restrict__ x, int64_t nchunks,
                                                       uint32_t rht_mask, float* __restrict__ ts) {
  float m = 0.0f;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; c + stride < nchunks; c += 2 * stride) {
    float v[16], u[16];
    load16<BF16>(x, c * 16, v);
    load16<BF16>(x, (c + stride) * 16, u);
    rht16(v, rht_mask);
    rht16(u, rht_mask);
    m = fmaxf(m, fmaxf(amax16(v), amax16(u)));
  }
  for (; c < nchunks; c += stride) {
    float v[16];
    load16<BF16>(x, c * 16, v);
    rht16(v, rht_mask);
    m = fmaxf(m, amax16(v));
  }
  block_max_to(m, ts);
}

// ------------------------------------------------------------ pass 2 -----
template <bool BF16, bool RHT, bool SR>
__global__ __launch_bounds__(kThreads) void k_encode_rows(const void* __restrict__ x, int64_t nblk,
                                                          uint64_t seed, uint32_t rht_mask,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales,
                                                          float* __restrict__ ts) {
  const float s_enc = tensor_scale_from_amax(ts[1]);
  if (blockIdx.x == 0 && threadIdx.x == 0) ts[0] = s_enc;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < nblk; b += stride) {
    float v[16];
    load16<BF16>(x, b * 16, v);
    if (RHT) rht16(v, rht_mask);
    float inv;
    const uint32_t byte = block_scale(amax16(v), s_enc, &inv);
    // rowwise: block b covers elements 16b .. 16b+15 of the row-major tensor
    reinterpret_cast<uint2*>(codes)[b] = encode16<SR>(v, inv, seed, 0u, (uint64_t)b * 16);
    scales[b] = (uint8_t)byte;
  }
}

// LDS tile element: the input's own storage type
template <bool BF16>
struct TileElem {
  using T = float;
  static constexpr int kPad = 4;
  static __device__ __forceinline__ float to_float(T v) { return v; }
};
template <>
struct TileElem<true> {
  using T = uint16_t;
  static constexpr int kPad = 8;
  static __device__ __forceinline__ float to_float(T v) { return __uint_as_float((uint32_t)v << 16); }
};

// Load 16 input elements once: the raw storage goes to row segment `trow`
// of the LDS tile, the fp32 values to v.
template <bool BF16>
__device__ __forceinline__ void load16_stash(const void* __restrict__ x, int64_t e,
                                             typename TileElem<BF16>::T* trow, float v[16]) {
  if (BF16) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + e);
    const uint4 a = ld_stream(p), b = ld_stream(p + 1);
    uint4* d = reinterpret_cast<uint4*>(trow);
    d[0] = a;
    d[1] = b;
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(x) + e);
    uint4* d = reinterpret_cast<uint4*>(trow);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 q = ld_stream(p + i);
      d[i] = q;
      v[4 * i] = __uint_as_float(q.x);
      v[4 * i + 1] = __uint_as_float(q.y);
      v[4 * i + 2] = __uint_as_float(q.z);
      v[4 * i + 3] = __uint_as_float(q.w);
    }
  }
}

// Columnwise (transposed) 1D copy, one thread per (column, 64-row half):
// blocks of 16 consecutive rows of a column, SR stream 1, element index of
// the transposed tensor c * R + r.  Writes 8 bytes of codes per block.
template <bool BF16, bool SR>
__device__ __forceinline__ void columnwise_half(const typename TileElem<BF16>::T* tile, int pitch,
                                                int col, int half, int rows_in, int64_t R,
                                                int64_t r0, int64_t c, float s_enc, uint64_t seed,
                                                uint8_t* __restrict__ codes_t,
                                                uint8_t* __restrict__ scales_t) {
#pragma unroll 1
  for (int rb = half * 4; rb < half * 4 + 4; ++rb) {
    if (rb * 16 >= rows_in) break;
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = TileElem<BF16>::to_float(tile[(rb * 16 + j) * pitch + col]);
    float inv;
    const uint32_t byte = block_scale(amax16(v), s_enc, &inv);
    const int64_t r = r0 + rb * 16;
    const uint2 q = encode16<SR>(v, inv, seed, 1u, (uint64_t)(c * R + r));
    *reinterpret_cast<uint2*>(codes_t + c * (R / 2) + r / 2) = q;
    scales_t[c * (R / 16) + r / 16] = (uint8_t)byte;
  }
}

template <bool BF16, bool SR>
__global__ __launch_bounds__(kThreads) void k_encode_tile1d(
    const void* __restrict__ x, int64_t R, int64_t C, uint64_t seed, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, uint8_t* __restrict__ codes_t, uint8_t* __restrict__ scales_t,
    float* __restrict__ ts) {
  using E = TileElem<BF16>;
  constexpr int pitch = kTile + E::kPad;
  __shared__ __align__(16) typename E::T tile[kTile * pitch];

  const float s_enc = tensor_scale_from_amax(ts[1]);
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) ts[0] = s_enc;
  const int64_t r0 = (int64_t)blockIdx.y * kTile, c0 = (int64_t)blockIdx.x * kTile;
  const int rows_in = (int)(R - r0 < kTile ? R - r0 : kTile);
  const int cols_in = (int)(C - c0 < kTile ? C - c0 : kTile);

  // rowwise blocks straight from registers; the raw values also go to LDS
#pragma unroll 1
  for (int q = threadIdx.x; q < kTile * (kTile / 16); q += kThreads) {
    const int row = q >> 3, cb = q & 7;
    if (row >= rows_in || cb * 16 >= cols_in) continue;
    const int64_t e = (r0 + row) * C + c0 + cb * 16;
    float v[16];
    load16_stash<BF16>(x, e, tile + row * pitch + cb * 16, v);
    float inv;
    const uint32_t byte = block_scale(amax16(v), s_enc, &inv);
    *reinterpret_cast<uint2*>(codes + e / 2) = encode16<SR>(v, inv, seed, 0u, (uint64_t)e);
    scales[e / 16] = (uint8_t)byte;
  }
  __syncthreads();
  const int col = threadIdx.x >> 1, half = threadIdx.x & 1;
  if (col < cols_in)
    columnwise_half<BF16, SR>(tile, pitch, col, half, rows_in, R, r0, c0 + col, s_enc, seed,
                              codes_t, scales_t);
}

template <bool BF16, bool SR>
__global__ __launch_bounds__(kThreads) void k_encode_tile2d(
    const void* __restrict__ x, int64_t R, int64_t C, uint64_t seed, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, uint8_t* __restrict__ codes_t, uint8_t* __restrict__ scales_t,
    float* __restrict__ ts) {
  using E = TileElem<BF16>;
  constexpr int pitch = kTile + E::kPad;
  constexpr int cpitch = kTile + 4;
  __shared__ __align__(16) typename E::T tile[kTile * pitch];
  __shared__ uint8_t qt[kTile * cpitch];  // one code per byte, [row][col]

  const float s_enc = tensor_scale_from_amax(ts[1]);
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) ts[0] = s_enc;
  const int64_t r0 = (int64_t)blockIdx.y * kTile, c0 = (int64_t)blockIdx.x * kTile;
  const int rows_in = (int)(R - r0 < kTile ? R - r0 : kTile);
  const int cols_in = (int)(C - c0 < kTile ? C - c0 : kTile);

#pragma unroll 1
  for (int q = threadIdx.x; q < kTile * (kTile / 16); q += kThreads) {
    const int row = q >> 3, cb = q & 7;
    if (row >= rows_in || cb * 16 >= cols_in) continue;
    float v[16];
    load16_stash<BF16>(x, (r0 + row) * C + c0 + cb * 16, tile + row * pitch + cb * 16, v);
  }
  __syncthreads();

  // four threads per 16x16 block, four rows each
  const int blk = threadIdx.x >> 2, quarter = threadIdx.x & 3;
  const int bi = blk >> 3, bj = blk & 7;
  const bool valid = bi * 16 < rows_in && bj * 16 < cols_in;
  float v[4][16];
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = bi * 16 + quarter * 4 + i;
#pragma unroll
    for (int j = 0; j < 16; ++j) v[i][j] = valid ? E::to_float(tile[row * pitch + bj * 16 + j]) : 0.0f;
    m = fmaxf(m, amax16(v[i]));
  }
  m = fmaxf(m, __shfl_xor(m, 1));
  m = fmaxf(m, __shfl_xor(m, 2));
  if (valid) {
    float inv;
    const uint32_t byte = block_scale(m, s_enc, &inv);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = bi * 16 + quarter * 4 + i;
      const int64_t e = (r0 + row) * C + c0 + bj * 16;
      const uint2 q = encode16<SR>(v[i], inv, seed, 0u, (uint64_t)e);
      *reinterpret_cast<uint2*>(codes + e / 2) = q;
      scales[e / 16] = (uint8_t)byte;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        qt[row * cpitch + bj * 16 + j] = (uint8_t)((q.x >> (4 * j)) & 15u);
        qt[row * cpitch + bj * 16 + 8 + j] = (uint8_t)((q.y >> (4 * j)) & 15u);
      }
    }
    if (codes_t) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int64_t c = c0 + bj * 16 + quarter * 4 + k;
        scales_t[c * (R / 16) + (r0 / 16) + bi] = (uint8_t)byte;
      }
    }
  }
  if (!codes_t) return;
  __syncthreads();
  // transposed codes: thread -> (column, 64-row half), 16 rows per 8 bytes
  const int col = threadIdx.x >> 1, half = threadIdx.x & 1;
  if (col >= cols_in) return;
  const int64_t c = c0 + col;
#pragma unroll 1
  for (int rb = half * 4; rb < half * 4 + 4; ++rb) {
    if (rb * 16 >= rows_in) break;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      lo |= (uint32_t)qt[(rb * 16 + j) * cpitch + col] << (4 * j);
      hi |= (uint32_t)qt[(rb * 16 + 8 + j) * cpitch + col] << (4 * j);
    }
    *reinterpret_cast<uint2*>(codes_t + c * (R / 2) + (r0 + rb * 16) / 2) = make_uint2(lo, hi);
  }
}

// ----------------------------------------------------------- RHT only ----
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_rht(const void* __restrict__ x, int64_t nchunks,
                                                  uint32_t rht_mask, float* __restrict__ y) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x; c < nchunks; c += stride) {
    float v[16];
    load16<BF16>(x, c * 16, v);
    rht16(v, rht_mask);
    float4* d = reinterpret_cast<float4*>(y + c * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) d[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  }
}

// ------------------------------------------------------------ launch -----
static int grid_stride_blocks(int64_t work, int cus, int per_cu = 8) {
  const int64_t want = (work + kThreads - 1) / kThreads;
  return (int)std::max<int64_t>(1, std::min<int64_t>(want, (int64_t)cus * per_cu));
}

template <bool BF16, bool RHT>
static void launch_amax(const QuantArgs& a, int cus, hipStream_t st) {
  const int64_t n = a.rows * a.cols;
  if (RHT) {
    hipLaunchKernelGGL((k_amax_rht<BF16>), dim3(grid_stride_blocks(n / 16, cus, 4)), dim3(kThreads), 0, st,
                       a.x, n / 16, a.rht_mask, a.tensor_scale);
  } else {
    const int64_t nvec = n / (BF16 ? 8 : 4);  // 16-byte vectors (n % 16 == 0)
    hipLaunchKernelGGL((k_amax_plain<BF16>), dim3(grid_stride_blocks(nvec / 4, cus, 2)), dim3(kThreads), 0,
                       st, reinterpret_cast<const uint4*>(a.x), nvec, a.tensor_scale);
  }
}

template <bool BF16, bool RHT, bool SR>
static void launch_rows(const QuantArgs& a, int cus, hipStream_t st) {
  const int64_t nblk = a.rows * a.cols / 16;
  hipLaunchKernelGGL((k_encode_rows<BF16, RHT, SR>), dim3(grid_stride_blocks(nblk, cus)),
                     dim3(kThreads), 0, st, a.x, nblk, a.seed, a.rht_mask, a.codes, a.scales,
                     a.tensor_scale);
}

template <bool BF16, bool SR>
static void launch_tile(const QuantArgs& a, bool two_d, hipStream_t st) {
  const dim3 grid((unsigned)((a.cols + kTile - 1) / kTile), (unsigned)((a.rows + kTile - 1) / kTile));
  if (two_d)
    hipLaunchKernelGGL((k_encode_tile2d<BF16, SR>), grid, dim3(kThreads), 0, st, a.x, a.rows, a.cols,
                       a.seed, a.codes, a.scales, a.codes_t, a.scales_t, a.tensor_scale);
  else
    hipLaunchKernelGGL((k_encode_tile1d<BF16, SR>), grid, dim3(kThreads), 0, st, a.x, a.rows, a.cols,
                       a.seed, a.codes, a.scales, a.codes_t, a.scales_t, a.tensor_scale);
}

template <bool BF16>
static void launch_quantize_t(const QuantArgs& a, int cus, hipStream_t st) {
  hipLaunchKernelGGL(k_init_amax, dim3(1), dim3(1), 0, st, a.tensor_scale);
  if (a.rht)
    launch_amax<BF16, true>(a, cus, st);
  else
    launch_amax<BF16, false>(a, cus, st);
  const bool sr = a.rounding == 1;
  if (a.two_d || a.codes_t) {
    if (sr)
      launch_tile<BF16, true>(a, a.two_d, st);
    else
      launch_tile<BF16, false>(a, a.two_d, st);
  } else if (a.rht) {
    if (sr)
      launch_rows<BF16, true, true>(a, cus, st);
    else
      launch_rows<BF16, true, false>(a, cus, st);
  } else {
    if (sr)
      launch_rows<BF16, false, true>(a, cus, st);
    else
      launch_rows<BF16, false, false>(a, cus, st);
  }
}

void launch_quantize(const QuantArgs& a, int cus, hipStream_t st) {
  if (a.bf16)
    launch_quantize_t<true>(a, cus, st);
  else
    launch_quantize_t<false>(a, cus, st);
}

void launch_rht(const void* x, bool bf16, int64_t rows, int64_t cols, uint32_t mask, float* y, int cus,
                hipStream_t st) {
  const int64_t nchunks = rows * cols / 16;
  if (bf16)
    hipLaunchKernelGGL(k_rht<true>, dim3(grid_stride_blocks(nchunks, cus)), dim3(kThreads), 0, st, x,
                       nchunks, mask, y);
  else
    hipLaunchKernelGGL(k_rht<false>, dim3(grid_stride_blocks(nchunks, cus)), dim3(kThreads), 0, st, x,
                       nchunks, mask, y);
}

}  // namespace nvfp4
