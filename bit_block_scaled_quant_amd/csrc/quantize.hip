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
//   k_encode_ct     1x16 rowwise blocks plus the columnwise copy (blocks of
//                   16 rows, written as rows of the transpose), described
//                   with the cast-transpose below;
//   k_encode_ct<.., TWO_D>  16x16 blocks (2B.3) in the cast-transpose
//                   tiles: one scale per block, each element encoded once
//                   and written both ways, so the transposed copy is the
//                   transpose of the codes and scales.
// The cast-transpose (k_amax_ct, k_encode_ct) makes the rowwise copy and an
// independently scaled columnwise copy (with the transform along columns)
// from one read of x per pass.
// k_rht writes the transform of 2B.2 alone (fp32 output).
#include "internal.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

constexpr int kThreads = 256;
static_assert(kThreads >= kInvTable, "the inverse-scale table is built by one thread per entry");

// codes of eight elements (element index0 .. index0 + 7, index0 % 8 == 0)
template <bool SR>
__device__ __forceinline__ uint32_t encode8(const float v[8], float inv, uint64_t seed, uint32_t stream,
                                            uint64_t index0) {
  float y[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) y[j] = v[j] * inv;
  if (SR) return e2m1_sr8(y, sr_draws(seed, stream, index0 >> 3));
  return e2m1_rne8(y);
}

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

template <bool BF16, bool CACHED>
__global__ __launch_bounds__(kThreads) void k_amax_plain(const uint4* __restrict__ x, int64_t nvec,
                                                         float* __restrict__ ts) {
  ushort2v m16 = {0, 0};
  uint32_t m32 = 0;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + 3 * stride < nvec; i += 4 * stride) {
    const uint4 a = ld16<CACHED>(x + i), b = ld16<CACHED>(x + i + stride),
                c = ld16<CACHED>(x + i + 2 * stride), d = ld16<CACHED>(x + i + 3 * stride);
    absmax_vec<BF16>(a, m16, m32);
    absmax_vec<BF16>(b, m16, m32);
    absmax_vec<BF16>(c, m16, m32);
    absmax_vec<BF16>(d, m16, m32);
  }
  for (; i < nvec; i += stride) absmax_vec<BF16>(ld16<CACHED>(x + i), m16, m32);
  const uint32_t bits = BF16 ? ((uint32_t)max(m16.x, m16.y) << 16) : m32;
  block_max_to(__uint_as_float(bits), ts);
}

// amax after the Hadamard transform.  A wave takes 1024 elements (64
// blocks) at a time as two 512-element halves: lane l holds elements
// 8l .. 8l + 7 of each, so every load instruction reads 1 KB of whole lines,
// and a block sits in lanes 2k, 2k + 1 (rht16_pair).  Two such pieces per
// iteration keep four loads in flight per lane.
template <bool BF16, bool CACHED>
__global__ __launch_bounds__(kThreads) void k_amax_rht(const void* __restrict__ x, int64_t nblk,
                                                       uint32_t rht_mask, float* __restrict__ ts) {
  const int lane = threadIdx.x & 63;
  const bool odd = lane & 1;
  const int64_t npiece = (nblk + 31) / 32;  // 512 elements per piece
  const int64_t wstride = (int64_t)gridDim.x * (kThreads / 64);
  float m = 0.0f;
  for (int64_t pc = ((int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)) * 2; pc < npiece;
       pc += 2 * wstride) {
    Raw8<BF16> r[2];
    bool valid[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t blk = (pc + u) * 32 + (lane >> 1);
      valid[u] = pc + u < npiece && blk < nblk;
      if (valid[u]) r[u] = load8_raw<BF16, CACHED>(x, blk * 16 + 8 * odd);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float v[8];
      if (valid[u]) {
        unpack8<BF16>(r[u], v);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = 0.0f;
      }
      m = max_nonneg(m, rht16_pair_absmax(v, rht_mask, odd));
    }
  }
  // the transform's final 1/4, applied to the maximum: rounding is monotone,
  // so max |fl(v / 4)| = fl(max |v| / 4)
  block_max_to(0.25f * m, ts);
}

// ------------------------------------------------------------ pass 2 -----
// 1x16 blocks along rows (RNE).  A wave takes 1024 elements (64 blocks) at a time
// as two halves: lane l holds elements 8l .. 8l + 7 of each, so loads read
// 1 KB of whole lines per instruction and code stores write 256 contiguous
// bytes; a block sits in lanes 2k, 2k + 1, whose amax is one DPP swap.
template <bool BF16, bool RHT, bool SR>
__global__ __launch_bounds__(kThreads) void k_encode_rows(const void* __restrict__ x, int64_t nblk,
                                                          uint64_t seed, uint32_t rht_mask,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales,
                                                          float* __restrict__ ts) {
  __shared__ float inv_tab[kInvTable];
  const float s_enc = tensor_scale_from_amax(ts[1]);
  if (blockIdx.x == 0 && threadIdx.x == 0) ts[0] = s_enc;
  build_inv_table(inv_tab, s_enc);
  const int lane = threadIdx.x & 63;
  const bool odd = lane & 1;
  const int64_t npiece = (nblk + 31) / 32;  // 512 elements per piece
  const int64_t wstride = (int64_t)gridDim.x * (kThreads / 64);
  for (int64_t pc = ((int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)) * 2; pc < npiece;
       pc += 2 * wstride) {
    Raw8<BF16> r[2];
    bool valid[2];
    int64_t blk[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      blk[u] = (pc + u) * 32 + (lane >> 1);
      valid[u] = pc + u < npiece && blk[u] < nblk;  // a lane pair agrees
      if (valid[u]) r[u] = load8_raw<BF16>(x, blk[u] * 16 + 8 * odd);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float v[8];
      if (valid[u]) {
        unpack8<BF16>(r[u], v);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = 0.0f;
      }
      if (RHT) rht16_pair(v, rht_mask, odd);
      float m = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
      m = pair_max(m);
      float inv;
      const uint32_t byte = block_scale(m, s_enc, inv_tab, &inv);
      if (valid[u]) {
        // rowwise: block b covers elements 16b .. 16b + 15 of the row-major tensor
        const int64_t e = blk[u] * 16 + 8 * odd;
        *reinterpret_cast<uint32_t*>(codes + e / 2) = encode8<SR>(v, inv, seed, 0u, (uint64_t)e);
        if (!odd) scales[blk[u]] = (uint8_t)byte;
      }
    }
  }
}

// One thread per 16-element block, two 16-byte loads each: the layout for
// SR and for the Hadamard transform, whose encodes are bound by vector ALU
// work (Philox, the conversions, the butterfly), so that each block's scale
// and transform are computed by one lane rather than two.
template <bool BF16, bool RHT, bool SR>
__global__ __launch_bounds__(kThreads) void k_encode_rows_blk(const void* __restrict__ x, int64_t nblk,
                                                          uint64_t seed, uint32_t rht_mask,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales,
                                                          float* __restrict__ ts) {
  __shared__ float inv_tab[kInvTable];
  const float s_enc = tensor_scale_from_amax(ts[1]);
  if (blockIdx.x == 0 && threadIdx.x == 0) ts[0] = s_enc;
  build_inv_table(inv_tab, s_enc);
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < nblk; b += stride) {
    float v[16];
    load16<BF16>(x, b * 16, v);
    if (RHT) rht16(v, rht_mask);
    float inv;
    const uint32_t byte = block_scale(amax16(v), s_enc, inv_tab, &inv);
    // rowwise: block b covers elements 16b .. 16b+15 of the row-major tensor
    reinterpret_cast<uint2*>(codes)[b] = encode16<SR>(v, inv, seed, 0u, (uint64_t)b * 16);
    scales[b] = (uint8_t)byte;
  }
}

// ----------------------------------------------------- cast-transpose ----
// Both operands a training step takes from one tensor x [R][C], read in its
// own layout: the rowwise copy (1x16 blocks along rows, as nvfp4_quantize
// makes it) and the columnwise copy (blocks of 16 rows of one column, i.e.
// the rows of x^T, optionally through the transform of 2B.2 first) with a
// tensor scale of its own.  x^T is never formed, and x is read once per
// pass instead of once per copy and pass.
//
// A wave works on a chunk of 16 rows x 512 columns: lane l holds columns
// 8l .. 8l + 7 of all 16 rows (one 16-byte load per row for bf16, two for
// fp32), so a rowwise block sits in lanes 2k, 2k + 1 and a columnwise block
// is one column of one lane.
constexpr int kCtCols = 512;                 // columns of a chunk
constexpr int kCtChunks = 8;                 // chunks per encode workgroup (a 128-row tile)
constexpr int kCtThreads = 64 * kCtChunks;
static_assert(kCtThreads == kCtCols, "the columnwise scale write-out takes one thread per column");

template <bool BF16>
struct Chunk16 {
  uint4 w[16][BF16 ? 1 : 2];  // row j: the lane's eight columns
};

template <bool BF16>
__device__ __forceinline__ void load_chunk(const void* __restrict__ x, int64_t e0, int64_t C,
                                           Chunk16<BF16>& ch) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (BF16) {
      ch.w[j][0] = ld_stream(static_cast<const uint16_t*>(x) + e0 + j * C);
    } else {
      const float* p = static_cast<const float*>(x) + e0 + j * C;
      ch.w[j][0] = ld_stream(p);
      ch.w[j][1] = ld_stream(p + 4);
    }
  }
}

// The transform's sign flips on the raw storage: row j of a chunk is element
// j of every columnwise block, so sign j flips all of row j.
template <bool BF16>
__device__ __forceinline__ void chunk_signs(Chunk16<BF16>& ch, uint32_t mask) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t f = ((mask >> j) & 1u) ? (BF16 ? 0x80008000u : 0x80000000u) : 0u;
#pragma unroll
    for (int h = 0; h < (BF16 ? 1 : 2); ++h) {
      ch.w[j][h].x ^= f;
      ch.w[j][h].y ^= f;
      ch.w[j][h].z ^= f;
      ch.w[j][h].w ^= f;
    }
  }
}

// An empty asm statement that claims to change every register of the chunk:
// the second pass then extracts its fp32 values afresh.  Without it the
// compiler keeps the 128 values the first pass extracted alive for reuse,
// which does not fit in 128 VGPRs and spills.
template <bool BF16>
__device__ __forceinline__ void chunk_opaque(Chunk16<BF16>& ch) {
#pragma unroll
  for (int j = 0; j < 16; ++j)
#pragma unroll
    for (int h = 0; h < (BF16 ? 1 : 2); ++h)
      asm volatile("" : "+v"(ch.w[j][h].x), "+v"(ch.w[j][h].y), "+v"(ch.w[j][h].z), "+v"(ch.w[j][h].w));
}

// element (row j, column k of the lane) as fp32; j and k are compile-time
template <bool BF16>
__device__ __forceinline__ float chunk_elem(const Chunk16<BF16>& ch, int j, int k) {
  const uint4& q = ch.w[j][BF16 ? 0 : (k >> 2)];
  const int wi = BF16 ? (k >> 1) : (k & 3);
  const uint32_t w = wi == 0 ? q.x : wi == 1 ? q.y : wi == 2 ? q.z : q.w;
  if (BF16) return __uint_as_float((k & 1) ? (w & 0xFFFF0000u) : (w << 16));
  return __uint_as_float(w);
}

// r[i] holds nibbles (i, 0..7) of an 8 x 8 nibble matrix; afterwards r[j]
// holds nibbles (0..7, j): 16-bit, 8-bit, then 4-bit block swaps
__device__ __forceinline__ void nib_transpose8(uint32_t r[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a = r[i], b = r[i + 4];
    r[i] = (a & 0x0000FFFFu) | (b << 16);
    r[i + 4] = (a >> 16) | (b & 0xFFFF0000u);
  }
#pragma unroll
  for (int h = 0; h < 8; h += 4)
#pragma unroll
    for (int i = h; i < h + 2; ++i) {
      const uint32_t a = r[i], b = r[i + 2];
      r[i] = (a & 0x00FF00FFu) | ((b & 0x00FF00FFu) << 8);
      r[i + 2] = ((a >> 8) & 0x00FF00FFu) | (b & 0xFF00FF00u);
    }
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const uint32_t a = r[i], b = r[i + 1];
    r[i] = (a & 0x0F0F0F0Fu) | ((b & 0x0F0F0F0Fu) << 4);
    r[i + 1] = ((a >> 4) & 0x0F0F0F0Fu) | (b & 0xF0F0F0F0u);
  }
}

// max |x| over a lane's 16 x 8 elements of a chunk: integer max of the
// magnitudes' bit patterns (order-preserving for non-negative floats), two
// bf16 per word
template <bool BF16>
__device__ __forceinline__ float chunk_absmax(const Chunk16<BF16>& ch) {
  if (BF16) {
    ushort2v m = {0, 0};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint4& q = ch.w[j][0];
      m = __builtin_elementwise_max(m, __builtin_bit_cast(ushort2v, q.x & 0x7FFF7FFFu));
      m = __builtin_elementwise_max(m, __builtin_bit_cast(ushort2v, q.y & 0x7FFF7FFFu));
      m = __builtin_elementwise_max(m, __builtin_bit_cast(ushort2v, q.z & 0x7FFF7FFFu));
      m = __builtin_elementwise_max(m, __builtin_bit_cast(ushort2v, q.w & 0x7FFF7FFFu));
    }
    return __uint_as_float((uint32_t)max(m.x, m.y) << 16);
  }
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j)
#pragma unroll
    for (int h = 0; h < (BF16 ? 1 : 2); ++h) {
      const uint4& q = ch.w[j][h];
      m = max(m, max(max(q.x & 0x7FFFFFFFu, q.y & 0x7FFFFFFFu), max(q.z & 0x7FFFFFFFu, q.w & 0x7FFFFFFFu)));
    }
  return __uint_as_float(m);
}

// block_max_to for two maxima: m into ts[1], mt into ts_t[1]
__device__ __forceinline__ void block_max2_to(float m, float mt, float* ts, float* ts_t) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    m = fmaxf(m, __shfl_xor(m, off));
    mt = fmaxf(mt, __shfl_xor(mt, off));
  }
  __shared__ float red[2][kThreads / 64];
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = m;
    red[1][threadIdx.x >> 6] = mt;
  }
  __syncthreads();
  if (threadIdx.x < 2) {
    float r = red[threadIdx.x][0];
    for (int w = 1; w < kThreads / 64; ++w) r = fmaxf(r, red[threadIdx.x][w]);
    unsigned int* t = reinterpret_cast<unsigned int*>((threadIdx.x == 0 ? ts : ts_t) + 1);
    const unsigned int bits = __float_as_uint(r);
    if (bits > __hip_atomic_load(t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(t, bits);
  }
}

__global__ void k_init_amax2(float* ts, float* ts_t) {
  ts[0] = 0.0f;
  ts[1] = 0.0f;
  ts_t[0] = 0.0f;
  ts_t[1] = 0.0f;
}

// Pass 1 with the transform: the plain amax (rowwise copy) and the amax
// after the transform of every 16-row column block (columnwise copy) from
// one read.  |sigma x| = |x|, so the plain amax is taken after the flips.
//
// A wave takes chunks of 16 rows x 256 columns: lane l holds columns
// 4l .. 4l + 3 of the 16 rows (one 8-byte load per row for bf16, so a load
// instruction reads 512 contiguous bytes), i.e. four whole column blocks.
// Waves walk the chunks grid-stride with the next chunk's loads in flight
// while the current one is transformed.  A lane past the last column reads
// the last four columns instead: a duplicate cannot change a maximum, and
// every lane then loads without a branch.
constexpr int kAmaxCtCols = 256;

template <bool BF16>
struct Col4 {
  uint32_t w[16][BF16 ? 2 : 4];  // row j: the lane's four columns
};

template <bool BF16, bool CACHED>
__device__ __forceinline__ void load_col4(const void* __restrict__ x, int64_t e0, int64_t C, Col4<BF16>& c) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (BF16) {
      const uint2 v = ld8<CACHED>(static_cast<const uint16_t*>(x) + e0 + j * C);
      c.w[j][0] = v.x;
      c.w[j][1] = v.y;
    } else {
      const uint4 v = ld16<CACHED>(static_cast<const float*>(x) + e0 + j * C);
      c.w[j][0] = v.x;
      c.w[j][1] = v.y;
      c.w[j][2] = v.z;
      c.w[j][3] = v.w;
    }
  }
}

// element (row j, column k of the lane) with sign j of the transform
template <bool BF16>
__device__ __forceinline__ float col4_elem(const Col4<BF16>& c, int j, int k, uint32_t mask) {
  const uint32_t w = c.w[j][BF16 ? (k >> 1) : k];
  const uint32_t b = BF16 ? ((k & 1) ? (w & 0xFFFF0000u) : (w << 16)) : w;
  return __uint_as_float(b ^ (((mask >> j) & 1u) << 31));
}

template <bool BF16, bool CACHED>
__global__ __launch_bounds__(kThreads) void k_amax_ct(const void* __restrict__ x, int64_t R, int64_t C,
                                                      uint32_t rht_mask, float* __restrict__ ts,
                                                      float* __restrict__ ts_t) {
  const int lane = threadIdx.x & 63;
  const int64_t cchunks = (C + kAmaxCtCols - 1) / kAmaxCtCols;
  const int64_t nchunks = (R / 16) * cchunks;
  const int64_t wstride = (int64_t)gridDim.x * (kThreads / 64);
  // first element of the lane's columns in chunk q (clamped to the last
  // four columns of the tensor; C % 16 == 0)
  auto elem0 = [&](int64_t q) {
    const int64_t col = min<int64_t>((q % cchunks) * kAmaxCtCols + 4 * lane, C - 4);
    return (q / cchunks) * 16 * C + col;
  };
  float m = 0.0f, mt = 0.0f;
  int64_t q = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  Col4<BF16> cur, nxt;
  if (q < nchunks) load_col4<BF16, CACHED>(x, elem0(q), C, cur);
  for (; q < nchunks; q += wstride) {
    const bool more = q + wstride < nchunks;  // wave-uniform
    if (more) load_col4<BF16, CACHED>(x, elem0(q + wstride), C, nxt);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = col4_elem<BF16>(cur, j, k, rht_mask);
      m = max_nonneg(m, max_abs16(v));
      mt = max_nonneg(mt, hadamard16_absmax(v));
    }
    if (more) cur = nxt;
  }
  // the transform's final 1/4, applied to the maximum (rounding is monotone)
  block_max2_to(m, 0.25f * mt, ts, ts_t);
}

// Pass 2.  A workgroup of eight waves takes a tile of 128 rows x 512 columns
// (wave w: rows 16w .. 16w + 15).  The rowwise codes, the columnwise codes
// (8 bytes per column and chunk), and both scale arrays are gathered in LDS
// and leave after one barrier as 16-byte pieces: sixteen threads per
// 256-byte row segment of the rowwise codes, four threads per 64-byte column
// segment of x^T's codes.  (With the rowwise codes stored from registers
// instead, 4 bytes per lane and row in the middle of the encode, the encode
// of [8192 x 20480] took 128 us instead of 122 us, and 40 us instead of
// 36 us at [8192 x 5120].)  A ragged tile stores its rowwise codes from
// registers, 4 bytes per lane.  Tiles are numbered
// column-major and dealt to the eight XCDs in contiguous runs, so the two
// tiles that complete one 128-byte line of x^T's codes (rows rt and
// rt + 128) are neighbours in the same L2.
// bf16 input: at most 128 VGPRs (four waves per SIMD: two workgroups per CU,
// whose load, encode and write-out phases then overlap); unbounded, the
// compiler takes about 170 and one workgroup per CU runs the phases back to
// back (measured 30% slower).  fp32 input holds twice the register data and
// spilled 57-94 VGPRs under that bound; with two waves per SIMD it takes
// 149-195 without spills and runs 10-22% faster (measured).
//
// TWO_D: the same tiles and write-out for the 16x16 blocks of 2B.3 (no
// transform; ts_t is ts; codes_t may be null).  A block is the 16 x 8
// elements of a lane pair, so its maximum is the lanes' own maxima met by
// one DPP swap; each element is encoded once (SR: the rowwise draws, element
// r * C + c, stream 0), and the transposed codes of a lane are the nibble
// transpose of its sixteen row words, in registers.  (This replaced a
// 16 x 64-strip kernel that moved the codes through LDS for the transpose:
// W [20480 x 5120] took 66 us there, at 11 VALU instructions per element
// and LDS bank-conflict cycles five times its LDS-active cycles.)
template <bool BF16, bool SR, bool RHT, bool TWO_D = false>
__global__ __launch_bounds__(kCtThreads, BF16 ? 4 : 2) void k_encode_ct(
    const void* __restrict__ x, int64_t R, int64_t C, uint64_t seed, uint64_t seed_t, uint32_t stream_t,
    uint32_t rht_mask,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* ts, uint8_t* __restrict__ codes_t,
    uint8_t* __restrict__ scales_t, float* ts_t) {
  // (ts and ts_t are the same two floats when the columnwise copy shares the
  // rowwise tensor scale, so they are not restrict)
  // columnwise codes [chunk][column slot][8 bytes]: lane l's eight columns
  // fill bytes 64l .. 64l + 63 of a chunk row, column 8l + k in slot
  // k ^ (l & 7) (the xor spreads a store instruction over the banks); 16
  // bytes of padding per chunk row spread the write-out reads
  constexpr int kPitch = kCtCols * 8 + 16;
  // One LDS block with the inverse-scale tables first: at offset 0 a
  // block's multiplier is a read at (byte << 2) with no base register.
  struct Smem {
    float inv_tab[2][kInvTable];
    __align__(16) uint8_t tq[kCtChunks * kPitch];
    __align__(16) uint8_t cs[kCtChunks][kCtCols];           // columnwise scales
    __align__(16) uint8_t rs[kCtChunks * 16][kCtCols / 16];  // rowwise scales
    __align__(16) uint32_t rq[kCtChunks * 16][kCtCols / 8];  // rowwise codes (whole tiles)
  };
  __shared__ Smem sm;
  auto& inv_tab = sm.inv_tab;
  auto& tq = sm.tq;
  auto& cs = sm.cs;
  auto& rs = sm.rs;
  auto& rq = sm.rq;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const float amax = ts[1];
  const float amax_t = RHT ? ts_t[1] : amax;
  const float s_enc = tensor_scale_from_amax(amax), s_enc_t = tensor_scale_from_amax(amax_t);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    ts[0] = s_enc;
    ts_t[0] = s_enc_t;
    if (!RHT) ts_t[1] = amax;
  }
  if (threadIdx.x < 2 * kInvTable)
    inv_tab[threadIdx.x / kInvTable][threadIdx.x % kInvTable] =
        inv_table_entry(threadIdx.x % kInvTable, threadIdx.x < kInvTable ? s_enc : s_enc_t);
  __syncthreads();

  const int64_t tiles_r = (R + 127) / 128, tiles_c = (C + kCtCols - 1) / kCtCols;
  const int64_t ntiles = tiles_r * tiles_c, per_xcd = (ntiles + 7) / 8;
  const int64_t tile = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (tile >= ntiles) return;  // the whole workgroup
  const int64_t rt = (tile % tiles_r) * 128, c0 = (tile / tiles_r) * kCtCols;
  const int nch = (int)min<int64_t>(kCtChunks, (R - rt) / 16);  // R % 16 == 0
  const int ncols = (int)min<int64_t>(kCtCols, C - c0);         // C % 16 == 0
  const int cl = 8 * lane;
  const bool lane_ok = cl < ncols;  // the two lanes of a rowwise block agree
  const int64_t r0 = rt + 16 * wv;
  // whole tile with 16-byte aligned rows of rowwise codes: those go through LDS
  const bool stage = nch == kCtChunks && ncols == kCtCols && (C / 2) % 16 == 0 &&
                     ((uintptr_t)codes & 15) == 0;  // workgroup-uniform

  if (TWO_D && wv < nch) {  // wave-uniform
    // a lane past the last column loads the last eight columns instead, with
    // no branch: its values reach only its own blocks (a 16-column block is
    // a whole lane pair), whose outputs are not stored
    Chunk16<BF16> ch;
    load_chunk<BF16>(x, r0 * C + min<int64_t>(c0 + cl, C - 8), C, ch);
    // all sixteen loads leave before any use: the scheduler would otherwise
    // start on row 0 after a few of them, and its wait for that row would
    // hold back the rest for a whole memory latency
    __builtin_amdgcn_sched_barrier(0);
    float m = chunk_absmax<BF16>(ch);
    m = pair_max(m);
    float inv;
    const uint32_t byte = block_scale(m, s_enc, inv_tab[0], &inv);
    uint32_t w[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = chunk_elem<BF16>(ch, j, k);
      const int64_t e = (r0 + j) * C + c0 + cl;
      w[j] = encode8<SR>(v, inv, seed, 0u, (uint64_t)e);
      if (stage)
        rq[16 * wv + j][lane] = w[j];
      else if (lane_ok)
        *reinterpret_cast<uint32_t*>(codes + e / 2) = w[j];
      if (!(lane & 1)) rs[16 * wv + j][lane >> 1] = (uint8_t)byte;
    }
    if (codes_t) {
      nib_transpose8(w);
      nib_transpose8(w + 8);
      uint8_t* tqw = tq + wv * kPitch + 64 * lane;
#pragma unroll
      for (int k = 0; k < 8; ++k)
        *reinterpret_cast<uint2*>(tqw + 8 * (k ^ (lane & 7))) = make_uint2(w[k], w[8 + k]);
      const uint32_t b4 = byte * 0x01010101u;
      *reinterpret_cast<uint2*>(&cs[wv][cl]) = make_uint2(b4, b4);
    }
  }
  if (!TWO_D && wv < nch) {  // wave-uniform: every lane of the wave takes part below
    // a lane past the last column loads the last eight columns instead, with
    // no branch: its values reach only its own blocks (a 16-column block is
    // a whole lane pair), whose outputs are not stored
    Chunk16<BF16> ch;
    load_chunk<BF16>(x, r0 * C + min<int64_t>(c0 + cl, C - 8), C, ch);
    // all sixteen loads leave before any use: the scheduler would otherwise
    // start on row 0 after a few of them, and its wait for that row would
    // hold back the rest for a whole memory latency
    __builtin_amdgcn_sched_barrier(0);
    const bool odd = lane & 1;
    // rowwise copy: SR stream 0 of seed, element index r * C + c
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = chunk_elem<BF16>(ch, j, k);
      float m = max_abs8(v);
      m = pair_max(m);
      float inv;
      const uint32_t byte = block_scale(m, s_enc, inv_tab[0], &inv);
      const int64_t e = (r0 + j) * C + c0 + cl;
      const uint32_t q = encode8<SR>(v, inv, seed, 0u, (uint64_t)e);
      if (stage)
        rq[16 * wv + j][lane] = q;
      else if (lane_ok)
        *reinterpret_cast<uint32_t*>(codes + e / 2) = q;
      if (!odd) rs[16 * wv + j][lane >> 1] = (uint8_t)byte;
    }
    // columnwise copy: the rows of x^T, SR stream stream_t of seed_t (0 for
    // the cast-transpose, 1 for the columnwise copy of one 1D quantization),
    // element index c * R + r (the index in x^T)
    if (RHT)
      chunk_signs<BF16>(ch, rht_mask);
    else
      chunk_opaque<BF16>(ch);
    uint32_t sc_lo = 0u, sc_hi = 0u;
    uint8_t* tqw = tq + wv * kPitch + 64 * lane;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = chunk_elem<BF16>(ch, j, k);
      if (RHT) hadamard16(v);
      float inv;
      const uint32_t byte = block_scale(max_abs16(v), s_enc_t, inv_tab[1], &inv);
      const int64_t c = c0 + cl + k;
      const uint2 q = encode16<SR>(v, inv, seed_t, stream_t, (uint64_t)(c * R + r0));
      *reinterpret_cast<uint2*>(tqw + 8 * (k ^ (lane & 7))) = q;
      if (k < 4)
        sc_lo |= byte << (8 * k);
      else
        sc_hi |= byte << (8 * (k - 4));
    }
    *reinterpret_cast<uint2*>(&cs[wv][cl]) = make_uint2(sc_lo, sc_hi);
  }
  __syncthreads();

  // rowwise codes of a whole tile: 128 rows x 256 bytes, 16 threads per row
  if (stage) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int id = threadIdx.x + kCtThreads * k, row = id >> 4, part = id & 15;
      *reinterpret_cast<uint4*>(codes + (rt + row) * (C / 2) + c0 / 2 + 16 * part) =
          *reinterpret_cast<const uint4*>(&rq[row][4 * part]);
    }
  }
  // rowwise scales: 32 bytes per row of the tile
  const int64_t srow = C / 16;
  if (ncols == kCtCols && srow % 16 == 0 && ((uintptr_t)scales & 15) == 0) {
    if ((int)threadIdx.x < 32 * nch) {
      const int row = threadIdx.x >> 1, p = threadIdx.x & 1;
      *reinterpret_cast<uint4*>(scales + (rt + row) * srow + c0 / 16 + 16 * p) =
          *reinterpret_cast<const uint4*>(&rs[row][16 * p]);
    }
  } else {
    const int nb = ncols / 16;
    for (int i = threadIdx.x; i < 16 * nch * nb; i += kCtThreads) {
      const int row = i / nb, b = i % nb;
      scales[(rt + row) * srow + c0 / 16 + b] = rs[row][b];
    }
  }
  if (TWO_D && !codes_t) return;
  // columnwise codes: four threads per column, 16 bytes (two chunks) each
  const int64_t tpitch = R / 2;
  const bool t16 = tpitch % 16 == 0 && ((uintptr_t)codes_t & 15) == 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int item = threadIdx.x + kCtThreads * i;
    const int cc = item >> 2, p = item & 3;
    if (cc >= ncols || 2 * p >= nch) continue;
    const int slot = 64 * (cc >> 3) + 8 * ((cc & 7) ^ ((cc >> 3) & 7));
    const uint2 a = *reinterpret_cast<const uint2*>(tq + (2 * p) * kPitch + slot);
    uint8_t* dst = codes_t + (c0 + cc) * tpitch + rt / 2 + 16 * p;
    if (2 * p + 1 < nch) {
      const uint2 b = *reinterpret_cast<const uint2*>(tq + (2 * p + 1) * kPitch + slot);
      if (t16) {
        *reinterpret_cast<uint4*>(dst) = make_uint4(a.x, a.y, b.x, b.y);
      } else {
        *reinterpret_cast<uint2*>(dst) = a;
        *reinterpret_cast<uint2*>(dst + 8) = b;
      }
    } else {
      *reinterpret_cast<uint2*>(dst) = a;
    }
  }
  // columnwise scales: one thread per column, one byte per chunk
  const int64_t spitch = R / 16;
  if ((int)threadIdx.x < ncols) {
    const int cc = threadIdx.x;
    uint8_t* dst = scales_t + (c0 + cc) * spitch + rt / 16;
    if (nch == kCtChunks && spitch % 8 == 0 && ((uintptr_t)scales_t & 7) == 0) {
      uint32_t lo = 0u, hi = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo |= (uint32_t)cs[i][cc] << (8 * i);
        hi |= (uint32_t)cs[i + 4][cc] << (8 * i);
      }
      *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
    } else {
      for (int i = 0; i < nch; ++i) dst[i] = cs[i][cc];
    }
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

// The amax pass reads a tensor of at most this many bytes with cached loads,
// so that the encode pass after it finds much of the tensor in the 256 MB
// MALL.  Measured on the layer-step calls: 84 MB 3% and 210 MB 4% faster
// per call; a 335 MB tensor, which does not fit, 7% slower.
constexpr int64_t kMallFitBytes = (int64_t)224 << 20;

static bool amax_cached(int64_t rows, int64_t cols, bool bf16) {
  return rows * cols * (bf16 ? 2 : 4) <= kMallFitBytes;
}

template <bool BF16, bool CACHED>
static void launch_amax_plain(const void* x, int64_t n, float* ts, int cus, hipStream_t st) {
  const int64_t nvec = n / (BF16 ? 8 : 4);  // 16-byte vectors (n % 16 == 0)
  hipLaunchKernelGGL((k_amax_plain<BF16, CACHED>), dim3(grid_stride_blocks(nvec / 4, cus, 2)), dim3(kThreads), 0,
                     st, reinterpret_cast<const uint4*>(x), nvec, ts);
}

template <bool BF16, bool RHT>
static void launch_amax(const QuantArgs& a, int cus, hipStream_t st) {
  const int64_t n = a.rows * a.cols;
  const bool cached = amax_cached(a.rows, a.cols, BF16);
  if (RHT) {
    const dim3 grid(grid_stride_blocks(n / 16, cus, 4));  // n / 16 blocks
    if (cached)
      hipLaunchKernelGGL((k_amax_rht<BF16, true>), grid, dim3(kThreads), 0, st, a.x, n / 16, a.rht_mask,
                         a.tensor_scale);
    else
      hipLaunchKernelGGL((k_amax_rht<BF16, false>), grid, dim3(kThreads), 0, st, a.x, n / 16, a.rht_mask,
                         a.tensor_scale);
  } else if (cached) {
    launch_amax_plain<BF16, true>(a.x, n, a.tensor_scale, cus, st);
  } else {
    launch_amax_plain<BF16, false>(a.x, n, a.tensor_scale, cus, st);
  }
}

template <bool BF16, bool RHT, bool SR>
static void launch_rows(const QuantArgs& a, int cus, hipStream_t st) {
  const int64_t nblk = a.rows * a.cols / 16;
  if (SR || RHT)
    hipLaunchKernelGGL((k_encode_rows_blk<BF16, RHT, SR>), dim3(grid_stride_blocks(nblk, cus)),
                       dim3(kThreads), 0, st, a.x, nblk, a.seed, a.rht_mask, a.codes, a.scales,
                       a.tensor_scale);
  else
    hipLaunchKernelGGL((k_encode_rows<BF16, RHT, SR>), dim3(grid_stride_blocks(nblk, cus)),
                       dim3(kThreads), 0, st, a.x, nblk, a.seed, a.rht_mask, a.codes, a.scales,
                       a.tensor_scale);
}

template <bool BF16, bool SR, bool RHT, bool TWO_D = false>
static void launch_ct_encode(const CastTransposeArgs& a, int cus, hipStream_t st);

template <bool BF16, bool SR>
static void launch_tile(const QuantArgs& a, bool two_d, int cus, hipStream_t st) {
  if (two_d) {
    // the cast-transpose encoder in its 16x16-block mode: one tensor scale,
    // every element encoded once from the rowwise draws
    CastTransposeArgs c{a.x,     a.bf16,   a.rows,         a.cols,  a.rounding, a.seed, a.seed,
                        false,   0u,       a.codes,        a.scales, a.tensor_scale, a.codes_t, a.scales_t,
                        a.tensor_scale, 0u};
    launch_ct_encode<BF16, SR, false, true>(c, cus, st);
  } else {
    // 1D with the columnwise copy: the cast-transpose encoder with one tensor
    // scale for both copies and the columnwise SR draws from stream 1 of seed
    CastTransposeArgs c{a.x,     a.bf16,   a.rows,         a.cols,  a.rounding, a.seed, a.seed,
                        false,   0u,       a.codes,        a.scales, a.tensor_scale, a.codes_t, a.scales_t,
                        a.tensor_scale, 1u};
    launch_ct_encode<BF16, SR, false>(c, cus, st);
  }
}

template <bool BF16>
static void launch_quantize_t(const QuantArgs& a, int cus, hipStream_t st) {
  if (!a.amax_given) {
    hipLaunchKernelGGL(k_init_amax, dim3(1), dim3(1), 0, st, a.tensor_scale);
    if (a.rht)
      launch_amax<BF16, true>(a, cus, st);
    else
      launch_amax<BF16, false>(a, cus, st);
  }
  const bool sr = a.rounding == 1;
  if (a.two_d || a.codes_t) {
    if (sr)
      launch_tile<BF16, true>(a, a.two_d, cus, st);
    else
      launch_tile<BF16, false>(a, a.two_d, cus, st);
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

template <bool BF16, bool SR, bool RHT, bool TWO_D>
static void launch_ct_encode(const CastTransposeArgs& a, int, hipStream_t st) {
  const int64_t tiles = ((a.rows + 127) / 128) * ((a.cols + kCtCols - 1) / kCtCols);
  const int blocks = (int)(((tiles + 7) / 8) * 8);  // tiles <= 2^24 (rows * cols <= 2^40)
  hipLaunchKernelGGL((k_encode_ct<BF16, SR, RHT, TWO_D>), dim3(blocks), dim3(kCtThreads), 0, st, a.x, a.rows, a.cols,
                     a.seed, a.seed_t, a.stream_t, a.rht_mask, a.codes, a.scales, a.tensor_scale, a.codes_t,
                     a.scales_t, a.tensor_scale_t);
}

template <bool BF16>
static void launch_cast_transpose_t(const CastTransposeArgs& a, int cus, hipStream_t st) {
  const bool sr = a.rounding == 1;
  if (a.rht_t) {
    hipLaunchKernelGGL(k_init_amax2, dim3(1), dim3(1), 0, st, a.tensor_scale, a.tensor_scale_t);
    // two workgroups of four waves per CU, each wave walking several chunks
    // with the next one in flight (X [8192 x 5120]: 5 chunks per wave).  In
    // a same-process A/B of whole calls, 1 / 2 / 3 / 4 / 5 workgroups per CU
    // took 60.0 / 56.4 / 59.0 / 61.5 / 63.9 us for X and 263.8 / 247.5 /
    // 249.3 / 252.2 / 254.9 us for dY: with fewer chunks per wave the loads
    // of a wave's first chunk are not hidden.
    const int64_t nchunks = (a.rows / 16) * ((a.cols + kAmaxCtCols - 1) / kAmaxCtCols);
    const int blocks = (int)std::max<int64_t>(
        1, std::min<int64_t>((nchunks + kThreads / 64 - 1) / (kThreads / 64), (int64_t)cus * 2));
    if (amax_cached(a.rows, a.cols, BF16))
      hipLaunchKernelGGL((k_amax_ct<BF16, true>), dim3(blocks), dim3(kThreads), 0, st, a.x, a.rows, a.cols,
                         a.rht_mask, a.tensor_scale, a.tensor_scale_t);
    else
      hipLaunchKernelGGL((k_amax_ct<BF16, false>), dim3(blocks), dim3(kThreads), 0, st, a.x, a.rows, a.cols,
                         a.rht_mask, a.tensor_scale, a.tensor_scale_t);
    if (sr)
      launch_ct_encode<BF16, true, true>(a, cus, st);
    else
      launch_ct_encode<BF16, false, true>(a, cus, st);
  } else {
    hipLaunchKernelGGL(k_init_amax, dim3(1), dim3(1), 0, st, a.tensor_scale);
    if (amax_cached(a.rows, a.cols, BF16))
      launch_amax_plain<BF16, true>(a.x, a.rows * a.cols, a.tensor_scale, cus, st);
    else
      launch_amax_plain<BF16, false>(a.x, a.rows * a.cols, a.tensor_scale, cus, st);
    if (sr)
      launch_ct_encode<BF16, true, false>(a, cus, st);
    else
      launch_ct_encode<BF16, false, false>(a, cus, st);
  }
}

void launch_cast_transpose(const CastTransposeArgs& a, int cus, hipStream_t st) {
  if (a.bf16)
    launch_cast_transpose_t<true>(a, cus, st);
  else
    launch_cast_transpose_t<false>(a, cus, st);
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
