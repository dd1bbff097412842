// MXFP4 for CDNA4 (gfx950): quantizer, dequantizer and GEMM on the native
// scaled FP4 matrix instruction.
//
// MXFP4 is the format "Pretraining Large Language Models with NVFP4",
// Technische samenvatting 2A, measures NVFP4 against: blocks of 32 E2M1
// elements sharing one power-of-two (UE8M0) scale, and no per-tensor scale.
// The conversion follows OCP Microscaling Formats (MX) v1.0, section 6.3: a
// block with absolute maximum amax gets X = 2^(floor(log2 amax) - 2) (2 is
// the exponent of E2M1's largest value, 6 = 1.5 * 2^2), stored as the E8M0
// byte log2(X) + 127 clamped to [0, 254] (an all-zero block takes byte 0);
// each element is x / X rounded to E2M1, nearest-even, saturating at 6.
//
// gfx950's v_mfma_scale_f32_32x32x64_f8f6f4 multiplies exactly this format:
// with FP4 operands (cbsz = blgp = 4) lane l supplies row l % 32 and the 32
// K-elements [32 (l / 32), +32) as 16 bytes (element 2k in the low nibble of
// byte k, the layout the quantizer writes), plus that 32-block's E8M0 byte in
// a scale register (op_sel picks the byte); accumulation is fp32 and the
// output layout is the usual one of the 32 x 32 MFMAs.  (Probed on the
// device against a CPU product: exact on random codes and scales.)  So a
// GEMM operand fragment is a 16-byte read and no unpacking is needed.
#include "internal.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

constexpr int kMxThreads = 256;

// E8M0 byte of a block with absolute maximum m: the biased exponent of m
// is E, floor(log2 m) = E - 127 for a normal m, so the byte is
// (E - 127 - 2) + 127 = E - 2; the clamp at 0 also covers zero and
// subnormal maxima (floor(log2 m) - 2 < -127 there).
__device__ __forceinline__ uint32_t mx_scale_byte(float m) {
  const uint32_t e = __float_as_uint(m) >> 23;  // m >= 0
  return e >= 2u ? e - 2u : 0u;
}

// ---------------------------------------------------------- quantizer ---
// A wave takes 512 elements (16 blocks) at a time: lane l holds elements
// 8l .. 8l + 7, so a block sits in the four lanes of a DPP quad and its
// maximum is two quad swaps.  y = x * 2^(127 - byte) is exact (a power of
// two; results below 2^-126 round once, as in the definition, and encode to
// a signed zero), then the RNE conversion of e2m1_rne8.
template <bool BF16>
__global__ __launch_bounds__(kMxThreads) void k_mx_quantize(const void* __restrict__ x, int64_t nblk,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t npiece = (nblk + 15) / 16;
  const int64_t wstride = (int64_t)gridDim.x * (kMxThreads / 64);
  for (int64_t pc = ((int64_t)blockIdx.x * (kMxThreads / 64) + (threadIdx.x >> 6)) * 2; pc < npiece;
       pc += 2 * wstride) {
    Raw8<BF16> r[2];
    bool valid[2];
    int64_t blk[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      blk[u] = (pc + u) * 16 + (lane >> 2);
      valid[u] = pc + u < npiece && blk[u] < nblk;  // the four lanes of a block agree
      if (valid[u]) r[u] = load8_raw<BF16>(x, blk[u] * 32 + 8 * (lane & 3));
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
      float m = max_abs8(v);
      m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0xB1, 0xF, 0xF, true)));
      m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0x4E, 0xF, 0xF, true)));
      const uint32_t byte = mx_scale_byte(m);
      const float mult = __uint_as_float((254u - byte) << 23);  // 2^(127 - byte), byte <= 252
      float y[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = v[j] * mult;
      if (valid[u]) {
        const int64_t e = blk[u] * 32 + 8 * (lane & 3);
        *reinterpret_cast<uint32_t*>(codes + e / 2) = e2m1_rne8(y);
        if ((lane & 3) == 0) scales[blk[u]] = (uint8_t)byte;
      }
    }
  }
}

// -------------------------------------------------------- dequantizer ---
// value = e2m1(code) * 2^(byte - 127), exact in fp32 for every byte the
// quantizer writes (0 .. 252); a thread takes four consecutive elements.
template <bool BF16OUT>
__global__ __launch_bounds__(kMxThreads) void k_mx_dequantize(const uint8_t* __restrict__ codes,
                                                              const uint8_t* __restrict__ scales, int64_t nquad,
                                                              void* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kMxThreads;
  for (int64_t q = (int64_t)blockIdx.x * kMxThreads + threadIdx.x; q < nquad; q += stride) {
    const uint32_t cw = *reinterpret_cast<const uint16_t*>(codes + 2 * q);
    const int ex = (int)scales[q >> 3] - 127;  // elements 4q .. 4q + 3 lie in block (4q) / 32
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t c = (cw >> (4 * j)) & 15u;
      v[j] = __builtin_amdgcn_ldexpf(e2m1_magnitude(c & 7u), ex);
      v[j] = __uint_as_float(__float_as_uint(v[j]) | ((c & 8u) << 28));
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

// --------------------------------------------------------------- GEMM ---
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void mx_lds_void_t;
typedef __attribute__((address_space(1))) void mx_glb_void_t;

__device__ __forceinline__ floatx16 mx_mfma(const uint4& a, const uint4& b, floatx16 acc, uint32_t sa,
                                            uint32_t sb, int t) {
  const intx8 va = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const intx8 vb = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  // op_sel picks byte t of each scale register
  switch (t) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, vb, acc, 4, 4, 0, (int)sa, 0, (int)sb);
    case 1: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, vb, acc, 4, 4, 1, (int)sa, 1, (int)sb);
    case 2: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, vb, acc, 4, 4, 2, (int)sa, 2, (int)sb);
    default: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, vb, acc, 4, 4, 3, (int)sa, 3, (int)sb);
  }
}

// Fast path: M, N multiples of 256, K a multiple of 256 (at most 2^24, so
// a tile's byte offsets fit in 32 bits), 16-byte aligned codes, 8-byte
// aligned scales.  A 256-thread workgroup owns a 256 x 256
// tile of C; its four waves (2 x 2) own 128 x 128 each as 4 x 4 MFMA tiles
// (256 accumulators per lane).  K advances in stages of 256 elements: 128
// code bytes per row of A and B (32 KB each) and 8 scale bytes per row
// (2 KB each) go from global memory straight into LDS (global_load_lds,
// 16-byte pieces for codes, 4-byte for scales); two stages are double
// buffered (136 KB).  Code rows are eight 16-byte chunks, chunk c of row r
// stored at c ^ ((r ^ (r >> 3)) & 7), so the eight rows a read instruction
// serves at a time hit eight different bank groups.  A stage is four MFMA
// steps of K = 64; step t of lane l reads chunk 2t + l / 32 of its rows.
constexpr int kMxBK = 256;
constexpr int kMxRow = kMxBK / 2;             // code bytes per row per stage
constexpr int kMxOffB = 256 * kMxRow;         // B codes after 32 KB of A codes
constexpr int kMxOffAS = 2 * kMxOffB;         // A scales: 256 rows x 8 bytes
constexpr int kMxOffBS = kMxOffAS + 256 * 8;  // B scales
constexpr int kMxStage = kMxOffBS + 256 * 8;  // 69632 bytes

__device__ __forceinline__ int mx_swz(int r, int c) { return r * kMxRow + ((c ^ ((r ^ (r >> 3)) & 7)) << 4); }

__device__ __forceinline__ void mx_issue(const MxGemmArgs& g, int64_t m0, int64_t n0, int64_t k0, uint8_t* buf) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t kb = g.K / 2, ks = g.K / 32;
  const uint8_t* a0 = g.a_codes + m0 * kb + k0 / 2;
  const uint8_t* b0 = g.b_codes + n0 * kb + k0 / 2;
  // 1 KB LDS blocks of 8 rows: lane l fills physical chunk l & 7 of row l >> 3
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int blk = 8 * wave + u;
    const int row = 8 * blk + (lane >> 3);
    const int chunk = (lane & 7) ^ ((row ^ (row >> 3)) & 7);
    const uint32_t off = (uint32_t)(row * kb + 16 * chunk);  // < 2^31 (K <= 2^24)
    __builtin_amdgcn_global_load_lds((mx_glb_void_t*)(a0 + off), (mx_lds_void_t*)(buf + 1024 * blk), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((mx_glb_void_t*)(b0 + off), (mx_lds_void_t*)(buf + kMxOffB + 1024 * blk),
                                     16, 0, 0);
  }
  // scales: 256 rows x 8 bytes per operand = 512 dwords; slot s = row 2r + half
  const uint8_t* as0 = g.a_scales + m0 * ks + k0 / 32;
  const uint8_t* bs0 = g.b_scales + n0 * ks + k0 / 32;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int slot = 256 * u + 64 * wave + lane;
    const uint32_t off = (uint32_t)((slot >> 1) * ks + 4 * (slot & 1));
    __builtin_amdgcn_global_load_lds((mx_glb_void_t*)(as0 + off),
                                     (mx_lds_void_t*)(buf + kMxOffAS + 1024 * u + 256 * wave), 4, 0, 0);
    __builtin_amdgcn_global_load_lds((mx_glb_void_t*)(bs0 + off),
                                     (mx_lds_void_t*)(buf + kMxOffBS + 1024 * u + 256 * wave), 4, 0, 0);
  }
}

struct MxFrag {
  uint4 a[4], b[4];
};

// fragments of step t: chunk 2t + g of the lane's four A rows and four B rows
__device__ __forceinline__ void mx_read(const uint8_t* buf, int wm, int wn, int r, int g, int t, MxFrag& f) {
  const int c = 2 * t + g;
#pragma unroll
  for (int i = 0; i < 4; ++i) f.a[i] = *reinterpret_cast<const uint4*>(buf + mx_swz(wm * 128 + i * 32 + r, c));
#pragma unroll
  for (int j = 0; j < 4; ++j)
    f.b[j] = *reinterpret_cast<const uint4*>(buf + kMxOffB + mx_swz(wn * 128 + j * 32 + r, c));
}

// the lane's scale bytes of a stage for row `row`: byte t = block 2t + g
__device__ __forceinline__ uint32_t mx_scales(const uint8_t* base, int row, uint32_t sel) {
  const uint2 s = *reinterpret_cast<const uint2*>(base + 8 * row);
  return __builtin_amdgcn_perm(s.y, s.x, sel);
}

__device__ __forceinline__ void mx_read_scales(const uint8_t* buf, int wm, int wn, int r, uint32_t sel,
                                               uint32_t (&sa)[4], uint32_t (&sb)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) sa[i] = mx_scales(buf + kMxOffAS, wm * 128 + i * 32 + r, sel);
#pragma unroll
  for (int j = 0; j < 4; ++j) sb[j] = mx_scales(buf + kMxOffBS, wn * 128 + j * 32 + r, sel);
}

template <int T>
__device__ __forceinline__ void mx_mfmas(const MxFrag& f, const uint32_t (&sa)[4], const uint32_t (&sb)[4],
                                         floatx16 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = mx_mfma(f.a[i], f.b[j], acc[i][j], sa[i], sb[j], T);
}

// Instruction order of one step: the 16 MFMAs, with READS LDS reads (the
// next step's fragments, and at a stage's end the next stage's scales) and
// VALU VALU ops placed one after each of the first MFMAs, so that the matrix
// core stays busy while the reads are in flight (left alone, the compiler
// issues a whole stage of reads, waits, then all 64 MFMAs).
template <int READS, int VALU>
__device__ __forceinline__ void mx_order() {
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (k < READS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (k >= 16 - VALU) __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
  }
}

// One stage from cur.  In: f = step 0 of cur, sa/sb = cur's scales.  Out: the
// same for nxt.  The barrier sits before the last step: by then every wave
// has read all of cur into registers and its loads of nxt have landed; the
// stage after nxt then streams into cur while the last step's MFMAs cover
// the reads of nxt's first step.
__device__ __forceinline__ void mx_stage(const MxGemmArgs& g, int64_t m0, int64_t n0, bool issue, int64_t k_issue,
                                         uint8_t* cur, const uint8_t* nxt, MxFrag& f, uint32_t (&sa)[4],
                                         uint32_t (&sb)[4], floatx16 (&acc)[4][4], int wm, int wn, int r, int gq,
                                         uint32_t sel) {
  MxFrag fn;
  mx_mfmas<0>(f, sa, sb, acc);
  mx_read(cur, wm, wn, r, gq, 1, fn);
  mx_order<8, 0>();
  __builtin_amdgcn_sched_barrier(0);
  mx_mfmas<1>(fn, sa, sb, acc);
  mx_read(cur, wm, wn, r, gq, 2, f);
  mx_order<8, 0>();
  __builtin_amdgcn_sched_barrier(0);
  mx_mfmas<2>(f, sa, sb, acc);
  mx_read(cur, wm, wn, r, gq, 3, fn);
  mx_order<8, 0>();
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();  // waits for this wave's loads of nxt (vmcnt(0)), then every wave
  // Unconditional, so the stage has no branch (with one, the compiler sinks
  // the MFMAs below it and issues the stage's reads first): past the last
  // stage it reloads stage 0 into a buffer no one reads again.
  mx_issue(g, m0, n0, issue ? k_issue : 0, cur);
  __builtin_amdgcn_sched_barrier(0);
  uint32_t na[4], nb[4];
  mx_mfmas<3>(fn, sa, sb, acc);
  mx_read(nxt, wm, wn, r, gq, 0, f);
  mx_read_scales(nxt, wm, wn, r, sel, na, nb);
  mx_order<16, 8>();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sa[i] = na[i];
    sb[i] = nb[i];
  }
}

__global__ __launch_bounds__(kMxThreads, 1) void k_mx_gemm(MxGemmArgs g) {
  __shared__ __align__(16) uint8_t buf0[kMxStage];
  __shared__ __align__(16) uint8_t buf1[kMxStage];
  const int64_t ntm = g.M / 256, ntn = g.N / 256, ntiles = ntm * ntn;
  // Workgroups are dealt to the eight XCDs in turn; each XCD takes a
  // contiguous run u of an order that walks bands of four tile rows column
  // by column, so the 32 tiles an XCD runs at once form a 4 x 8 block: per
  // K-step they need 4 slices of A and 8 of B from its L2 instead of 1 and 32.
  const int64_t per_xcd = (ntiles + 7) / 8;
  const int64_t u = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (u >= ntiles) return;
  constexpr int64_t kBand = 4;
  const int64_t band = u / (kBand * ntn), rem = u % (kBand * ntn);
  const int64_t band_rows = min<int64_t>(kBand, ntm - band * kBand);
  const int64_t m0 = (band * kBand + rem % band_rows) * 256, n0 = (rem / band_rows) * 256;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 31, gq = lane >> 5;
  const uint32_t sel = gq ? 0x07050301u : 0x06040200u;

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int k = 0; k < 16; ++k) acc[i][j][k] = 0.f;

  const int64_t nk = g.K / kMxBK;  // >= 1
  mx_issue(g, m0, n0, 0, buf0);
  __syncthreads();  // waits for this wave's loads (vmcnt(0)), then for every wave
  if (nk > 1) mx_issue(g, m0, n0, kMxBK, buf1);
  MxFrag f;
  uint32_t sa[4], sb[4];
  mx_read(buf0, wm, wn, r, gq, 0, f);
  mx_read_scales(buf0, wm, wn, r, sel, sa, sb);
  int64_t kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    mx_stage(g, m0, n0, kt + 2 < nk, (kt + 2) * kMxBK, buf0, buf1, f, sa, sb, acc, wm, wn, r, gq, sel);
    // on the last stage the reads of buf0 at its end are of stale data and unused
    mx_stage(g, m0, n0, kt + 3 < nk, (kt + 3) * kMxBK, buf1, buf0, f, sa, sb, acc, wm, wn, r, gq, sel);
  }
  if (kt < nk) mx_stage(g, m0, n0, false, 0, buf0, buf1, f, sa, sb, acc, wm, wn, r, gq, sel);

  // D layout of the 32 x 32 MFMA: lane l, value k -> column l % 32, row
  // 8 * (k / 4) + 4 * (l / 32) + k % 4
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + wn * 128 + j * 32 + r;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int64_t m = m0 + wm * 128 + i * 32 + 8 * (k >> 2) + 4 * gq + (k & 3);
        __builtin_nontemporal_store(acc[i][j][k], &g.c[m * g.N + n]);
      }
    }
  }
}

// General path (any M, N >= 1, K % 32 == 0): each wave owns a 32 x 32 tile of
// C and reads its fragments straight from global memory, one MFMA per K =
// 64; rows past M or N are clamped (their results are not stored) and the
// half of a final K step past K is zero codes.
__global__ __launch_bounds__(kMxThreads) void k_mx_gemm_any(MxGemmArgs g) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 31, gq = lane >> 5;
  const int64_t m0 = (int64_t)blockIdx.y * 64 + (wave >> 1) * 32, n0 = (int64_t)blockIdx.x * 64 + (wave & 1) * 32;
  const int64_t am = min<int64_t>(m0 + r, g.M - 1), bn = min<int64_t>(n0 + r, g.N - 1);
  const int64_t kb = g.K / 2, ks = g.K / 32;
  floatx16 acc;
#pragma unroll
  for (int k = 0; k < 16; ++k) acc[k] = 0.f;
  for (int64_t k0 = 0; k0 < g.K; k0 += 64) {
    const int64_t kk = k0 + 32 * gq;
    uint4 a = make_uint4(0u, 0u, 0u, 0u), b = make_uint4(0u, 0u, 0u, 0u);
    uint32_t sa = 127u, sb = 127u;
    if (kk < g.K) {
      a = *reinterpret_cast<const uint4*>(g.a_codes + am * kb + kk / 2);
      b = *reinterpret_cast<const uint4*>(g.b_codes + bn * kb + kk / 2);
      sa = g.a_scales[am * ks + kk / 32];
      sb = g.b_scales[bn * ks + kk / 32];
    }
    acc = mx_mfma(a, b, acc, sa, sb, 0);
  }
  const int64_t n = n0 + r;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int64_t m = m0 + 8 * (k >> 2) + 4 * gq + (k & 3);
    if (m < g.M && n < g.N) g.c[m * g.N + n] = acc[k];
  }
}

// ------------------------------------------------------------ launch ----
void launch_mx_quantize(const void* x, bool bf16, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                        int cus, hipStream_t st) {
  const int64_t nblk = rows * cols / 32;
  const int64_t want = (nblk / 16 + 2 * (kMxThreads / 64) - 1) / (2 * (kMxThreads / 64));  // 2 pieces per wave
  const int blocks = (int)std::max<int64_t>(1, std::min<int64_t>(want, (int64_t)cus * 8));
  if (bf16)
    hipLaunchKernelGGL(k_mx_quantize<true>, dim3(blocks), dim3(kMxThreads), 0, st, x, nblk, codes, scales);
  else
    hipLaunchKernelGGL(k_mx_quantize<false>, dim3(blocks), dim3(kMxThreads), 0, st, x, nblk, codes, scales);
}

void launch_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols, bool bf16_out,
                          void* out, int cus, hipStream_t st) {
  const int64_t nquad = rows * cols / 4;
  const int blocks = (int)std::max<int64_t>(
      1, std::min<int64_t>((nquad + kMxThreads - 1) / kMxThreads, (int64_t)cus * 8));
  if (bf16_out)
    hipLaunchKernelGGL(k_mx_dequantize<true>, dim3(blocks), dim3(kMxThreads), 0, st, codes, scales, nquad, out);
  else
    hipLaunchKernelGGL(k_mx_dequantize<false>, dim3(blocks), dim3(kMxThreads), 0, st, codes, scales, nquad, out);
}

void launch_mx_gemm(const MxGemmArgs& g, hipStream_t st) {
  const bool fast = g.M % 256 == 0 && g.N % 256 == 0 && g.K % kMxBK == 0 && g.K <= (INT64_C(1) << 24) &&
                    (uintptr_t)g.a_codes % 16 == 0 &&
                    (uintptr_t)g.b_codes % 16 == 0 && (uintptr_t)g.a_scales % 8 == 0 &&
                    (uintptr_t)g.b_scales % 8 == 0;
  if (fast) {
    const int64_t ntiles = (g.M / 256) * (g.N / 256);
    const int64_t blocks = ((ntiles + 7) / 8) * 8;
    hipLaunchKernelGGL(k_mx_gemm, dim3((unsigned)blocks), dim3(kMxThreads), 0, st, g);
  } else {
    const dim3 grid((unsigned)((g.N + 63) / 64), (unsigned)((g.M + 63) / 64));
    hipLaunchKernelGGL(k_mx_gemm_any, grid, dim3(kMxThreads), 0, st, g);
  }
}

}  // namespace nvfp4
