// MXFP6 (E2M3, E3M2) quantization for gfx950: row-wise, column-wise and dual.
//
// "EU8M0 FP8" article, MX definition paragraph: the MX family shares the E8M0
// block scale over k = 32 elements; MXFP6 is its 6-bit member.  Scale rule,
// saturation and the NaN/Inf block rule are those of the other formats (the
// FP6 formats have no NaN or Inf: a block holding one gets scale 0xFF and every
// code the largest magnitude with the input's sign).  Codes are packed as a
// little-endian bit stream along the row (element i at bits 6i .. 6i+5), so a
// block is 24 bytes and 8 elements are 6 bytes.
//
// Kernels, flat over the row-wise blocks (contiguous in row-major input):
//   rowwise_bf16_kernel  BF16 input: a lane owns a whole block (64 bytes in, 24
//     out) and converts it with one V_CVT_SCALEF32_PK32_{FP6,BF6}_BF16.  An
//     in-bounds probe over every BF16 value at block scales 2^-124 .. 2^125 found
//     these converts equal to RNE(v / 2^e) on the E2M3 / E3M2 grids, saturating
//     beyond the largest magnitude, elements in bit-stream order.  (The FP32-input
//     converts differ on some values, so FP32 and FP16 inputs do not use them.)
//     All-zero blocks convert at scale 1 (+-0 gives +-0).  Blocks with NaN/Inf,
//     or with a nonzero amax and e = -127 (not a normal FP32 scale), take the
//     integer encoder below.
//   rowwise_kernel  FP32 / FP16 input: a lane owns 8 elements, a quad owns a block
//     and takes its amax with two DPP steps; the cast is the exact integer RNE +
//     saturation encoder on v * 2^-e (a power-of-two multiply, exact wherever the
//     result can matter).
// Tiled kernels, for the column-wise copy (blocks run down the columns):
//   tile_kernel      any input type, column-wise or dual: a tile is staged in
//     LDS and each lane encodes whole 32-element blocks (the BF16 converter or
//     the integer encoder, as above).
//   dual_bf16_kernel BF16 dual, register resident: a lane holds an 8 x 8 patch,
//     so a row block is a quad and a column block is 4 lanes of a DPP row; each
//     lane converts its own 8 values with the 32-element converter (the other
//     slots zero) and keeps its 6 bytes.  Both copies are staged in LDS as
//     96-byte lines (128 elements) and leave as 8-byte pieces.

#include "mx_device.hpp"
#include "mx_launch.hpp"

namespace mxk {

namespace fp6 {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

template <int IN, int F, int R, bool AMAX>
__global__ __launch_bounds__(kThreads) void rowwise_kernel(const void* __restrict__ x, int64_t nchunks,
                                                           uint8_t* __restrict__ q, uint8_t* __restrict__ scales,
                                                           uint32_t* __restrict__ amax_out) {
  const int lane_q = threadIdx.x & 3;
  uint32_t tmax = 0;
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t chunk = (int64_t(blockIdx.x) * kUnroll + u) * kThreads + threadIdx.x;
    // nchunks is a multiple of 4 and quads are aligned: a quad is entirely in or out of range
    if (chunk >= nchunks) continue;
    float v[8];
    load8<IN>(x, chunk * 8, v);
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = umax(m, abs_bits(v[j]));
    if constexpr (AMAX) {
#pragma unroll
      for (int j = 0; j < 8; ++j) tmax = umax(tmax, abs_bits_no_nan(v[j]));
    }
    const uint32_t bmax = quad_max(m);
    const bool nonfinite = bmax >= 0x7F800000u;
    const int e = nonfinite ? 0 : shared_exponent<F, R>(bmax);
    const float mul = pow2_neg(e);
    uint32_t c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t sign = (__float_as_uint(v[j]) >> 31) << 5;
      c[j] = nonfinite ? (Fmt_<F>::kNan | sign) : encode_rne_sat<F>(v[j] * mul);
    }
    // 48 bits: lo = elements 0..4 and the low 2 bits of element 5, hi = the rest
    const uint32_t lo = c[0] | (c[1] << 6) | (c[2] << 12) | (c[3] << 18) | (c[4] << 24) | (c[5] << 30);
    const uint32_t hi = (c[5] >> 2) | (c[6] << 4) | (c[7] << 10);
    uint8_t* dst = q + chunk * 6;                       // 4-byte aligned for even chunks, 2-byte for odd
    if ((chunk & 1) == 0) {
      *reinterpret_cast<uint32_t*>(dst) = lo;
      *reinterpret_cast<uint16_t*>(dst + 4) = uint16_t(hi);
    } else {
      *reinterpret_cast<uint16_t*>(dst) = uint16_t(lo);
      *reinterpret_cast<uint32_t*>(dst + 2) = (lo >> 16) | (hi << 16);
    }
    if (lane_q == 0) scales[chunk >> 2] = uint8_t(nonfinite ? 0xFFu : uint32_t(e + 127));
  }
  if constexpr (AMAX) {
    __shared__ uint32_t red[kThreads / 64];
    tmax = wave_max(tmax);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = tmax;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t mm = red[0];
#pragma unroll
      for (int k = 1; k < kThreads / 64; ++k) mm = umax(mm, red[k]);
      if (mm) atomic_max_u32(amax_out, mm);
    }
  }
}

typedef __bf16 v32bf_t __attribute__((ext_vector_type(32)));
typedef unsigned int v16u_t __attribute__((ext_vector_type(16)));
typedef unsigned int v6u_t __attribute__((ext_vector_type(6)));
constexpr int kUnrollB = 1;   // blocks per thread (BF16 8192 x 4096: 18.4 us against 18.65 with two)

template <int F, int R, bool AMAX>
__global__ __launch_bounds__(kThreads) void rowwise_bf16_kernel(const uint16_t* __restrict__ x, int64_t nblocks,
                                                                uint8_t* __restrict__ q, uint8_t* __restrict__ scales,
                                                                uint32_t* __restrict__ amax_out) {
  uint32_t tmax = 0;
#pragma unroll
  for (int u = 0; u < kUnrollB; ++u) {
    const int64_t blk = (int64_t(blockIdx.x) * kUnrollB + u) * kThreads + threadIdx.x;
    if (blk >= nblocks) continue;
    const uint4* src = reinterpret_cast<const uint4*>(x + blk * 32);
    v16u_t d;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint4 t = src[k];
      d[4 * k] = t.x;
      d[4 * k + 1] = t.y;
      d[4 * k + 2] = t.z;
      d[4 * k + 3] = t.w;
    }
    // block amax of the 32 magnitudes as FP32 bit patterns (NaN > Inf > finite)
    uint32_t mp = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) mp = pk_umax16(mp, d[k] & 0x7FFF7FFFu);
    const uint32_t bmax = umax((mp & 0xFFFFu) << 16, mp & 0xFFFF0000u);
    if constexpr (AMAX) {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        tmax = umax(tmax, abs_bits_no_nan(__uint_as_float(d[k] << 16)));
        tmax = umax(tmax, abs_bits_no_nan(__uint_as_float(d[k] & 0xFFFF0000u)));
      }
    }
    const bool nonfinite = bmax >= 0x7F800000u;
    const int e = nonfinite ? 0 : shared_exponent<F, R>(bmax);
    uint32_t w[6];
    // an all-zero block (e = -127) converts too: +-0 gives +-0 at any scale, and
    // keeping it off the integer encoder keeps its wave off the launch's tail
    if (!nonfinite && (e > -127 || bmax == 0u)) {
      const float scale = bmax == 0u ? 1.0f : __uint_as_float(uint32_t(127 + e) << 23);
      const v32bf_t xv = __builtin_bit_cast(v32bf_t, d);
      v6u_t r;
      if constexpr (F == E2M3) r = __builtin_bit_cast(v6u_t, __builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(xv, scale));
      else r = __builtin_bit_cast(v6u_t, __builtin_amdgcn_cvt_scalef32_pk32_bf6_bf16(xv, scale));
#pragma unroll
      for (int k = 0; k < 6; ++k) w[k] = r[k];
    } else {
      const float mul = pow2_neg(e);
      uint64_t acc = 0;
      int nb = 0, wi = 0;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const uint32_t bits = (i & 1) ? (d[i >> 1] & 0xFFFF0000u) : (d[i >> 1] << 16);
        const uint32_t c = nonfinite ? (Fmt_<F>::kNan | ((bits >> 31) << 5)) : encode_rne_sat<F>(__uint_as_float(bits) * mul);
        acc |= uint64_t(c) << nb;
        nb += 6;
        if (nb >= 32) {
          w[wi++] = uint32_t(acc);
          acc >>= 32;
          nb -= 32;
        }
      }
    }
    // 24 bytes at 24 * blk: 8-byte aligned
    uint2* dst = reinterpret_cast<uint2*>(q + blk * 24);
    dst[0] = make_uint2(w[0], w[1]);
    dst[1] = make_uint2(w[2], w[3]);
    dst[2] = make_uint2(w[4], w[5]);
    scales[blk] = uint8_t(nonfinite ? 0xFFu : uint32_t(e + 127));
  }
  if constexpr (AMAX) {
    __shared__ uint32_t red[kThreads / 64];
    tmax = wave_max(tmax);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = tmax;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t mm = red[0];
#pragma unroll
      for (int k = 1; k < kThreads / 64; ++k) mm = umax(mm, red[k]);
      if (mm) atomic_max_u32(amax_out, mm);
    }
  }
}

template <int F, int R>
static mx_status_t launch_bf16(const void* x, int64_t n, uint8_t* q, uint8_t* s, uint32_t* amax, hipStream_t st) {
  const int64_t nblocks = n / 32;
  const int64_t per = int64_t(kThreads) * kUnrollB;
  const dim3 grid{unsigned((nblocks + per - 1) / per)}, block{unsigned(kThreads)};
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  if (amax)
    hipLaunchKernelGGL((rowwise_bf16_kernel<F, R, true>), grid, block, 0, st, xb, nblocks, q, s, amax);
  else
    hipLaunchKernelGGL((rowwise_bf16_kernel<F, R, false>), grid, block, 0, st, xb, nblocks, q, s, amax);
  return hipGetLastError() == hipSuccess ? MX_OK : MX_ERR_LAUNCH;
}

template <int IN, int F, int R>
static mx_status_t launch(const void* x, int64_t n, uint8_t* q, uint8_t* s, uint32_t* amax, hipStream_t st) {
  const int64_t nchunks = n / 8;
  const int64_t per = int64_t(kThreads) * kUnroll;
  const dim3 grid{unsigned((nchunks + per - 1) / per)}, block{unsigned(kThreads)};
  if (amax)
    hipLaunchKernelGGL((rowwise_kernel<IN, F, R, true>), grid, block, 0, st, x, nchunks, q, s, amax);
  else
    hipLaunchKernelGGL((rowwise_kernel<IN, F, R, false>), grid, block, 0, st, x, nchunks, q, s, amax);
  return hipGetLastError() == hipSuccess ? MX_OK : MX_ERR_LAUNCH;
}

template <int F, int R>
static mx_status_t by_input(mx_dtype_t in, const void* x, int64_t n, uint8_t* q, uint8_t* s, uint32_t* amax,
                            hipStream_t st) {
  if (in == MX_BF16) return launch_bf16<F, R>(x, n, q, s, amax, st);
  if (in == MX_F16) return launch<IN_F16, F, R>(x, n, q, s, amax, st);
  return launch<IN_F32, F, R>(x, n, q, s, amax, st);
}

// ---------------------------------------------------------------------------
// Column-wise and dual MXFP6: a workgroup stages a 128-row x 64-column tile in LDS
// (coalesced 16-byte loads), then each of its 256 threads encodes one column block
// (32 rows of one column; threads 4 c .. 4 c + 3 cover the 4 blocks of column c, so
// they write its 96 contiguous output bytes) and, for the dual layout, one row block
// (32 contiguous values of a staged row).
// ---------------------------------------------------------------------------
constexpr int kTR = 128, kTC = 64;
template <int IN> struct TileWord { using T = uint16_t; };
template <> struct TileWord<IN_F32> { using T = float; };

template <int IN>
__device__ __forceinline__ float tile_value(typename TileWord<IN>::T w) {
  if constexpr (IN == IN_F32) return w;
  else if constexpr (IN == IN_BF16) return __uint_as_float(uint32_t(w) << 16);
  else return f16_bits_to_f32(w);
}

// Encode one block of 32 values (v: the FP32 values; bf: their BF16 bit pairs, used
// only for BF16 input) into 6 code words; returns the scale code.
template <int IN, int F, int R>
__device__ __forceinline__ uint32_t encode_block32(const float (&v)[32], const uint32_t (&bf)[16], uint32_t (&w)[6]) {
  uint32_t bmax = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) bmax = umax(bmax, abs_bits(v[i]));
  const bool nonfinite = bmax >= 0x7F800000u;
  const int e = nonfinite ? 0 : shared_exponent<F, R>(bmax);
  if constexpr (IN == IN_BF16) {
    // an all-zero block converts too (+-0 gives +-0 at any scale)
    if (!nonfinite && (e > -127 || bmax == 0u)) {
      const float scale = bmax == 0u ? 1.0f : __uint_as_float(uint32_t(127 + e) << 23);
      v16u_t d;
#pragma unroll
      for (int k = 0; k < 16; ++k) d[k] = bf[k];
      const v32bf_t xv = __builtin_bit_cast(v32bf_t, d);
      v6u_t r;
      if constexpr (F == E2M3) r = __builtin_bit_cast(v6u_t, __builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(xv, scale));
      else r = __builtin_bit_cast(v6u_t, __builtin_amdgcn_cvt_scalef32_pk32_bf6_bf16(xv, scale));
#pragma unroll
      for (int k = 0; k < 6; ++k) w[k] = r[k];
      return uint32_t(e + 127);
    }
  }
  const float mul = pow2_neg(e);
  uint64_t acc = 0;
  int nb = 0, wi = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t c = nonfinite ? (Fmt_<F>::kNan | ((__float_as_uint(v[i]) >> 31) << 5)) : encode_rne_sat<F>(v[i] * mul);
    acc |= uint64_t(c) << nb;
    nb += 6;
    if (nb >= 32) {
      w[wi++] = uint32_t(acc);
      acc >>= 32;
      nb -= 32;
    }
  }
  return nonfinite ? 0xFFu : uint32_t(e + 127);
}

// 24 code bytes at an 8-byte aligned address
__device__ __forceinline__ void store24(uint8_t* dst, const uint32_t (&w)[6]) {
  uint2* d = reinterpret_cast<uint2*>(dst);
  d[0] = make_uint2(w[0], w[1]);
  d[1] = make_uint2(w[2], w[3]);
  d[2] = make_uint2(w[4], w[5]);
}

template <int IN, int F, int R, bool DUAL, bool AMAX>
__global__ __launch_bounds__(kThreads) void tile_kernel(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                        int tiles_c, uint8_t* __restrict__ q_row,
                                                        uint8_t* __restrict__ s_row, uint8_t* __restrict__ q_col,
                                                        uint8_t* __restrict__ s_col, uint32_t* __restrict__ amax_out) {
  using W = typename TileWord<IN>::T;
  constexpr int kPitch = kTC + 2;   // elements per staged row (an odd number of dwords apart for 2-byte W)
  __shared__ W t[kTR][kPitch];
  const int tid = threadIdx.x;
  const int64_t r0 = int64_t(blockIdx.x / tiles_c) * kTR;
  const int64_t c0 = int64_t(blockIdx.x % tiles_c) * kTC;
  // ---- stage: 16-byte pieces (8 elements of 2-byte input, 4 of FP32), zero outside the matrix
  constexpr int kPer = 16 / int(sizeof(W));
  constexpr int kPieces = kTR * kTC / kPer;
#pragma unroll
  for (int k = 0; k < kPieces / kThreads; ++k) {
    const int id = tid + kThreads * k, row = id / (kTC / kPer), pc = id % (kTC / kPer);
    const int64_t gr = r0 + row, gc = c0 + pc * kPer;
    uint4 d = make_uint4(0, 0, 0, 0);
    if (gr < rows && gc < cols)
      d = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(x) + (gr * cols + gc) * int64_t(sizeof(W)));
    const W* e = reinterpret_cast<const W*>(&d);
#pragma unroll
    for (int j = 0; j < kPer; ++j) t[row][pc * kPer + j] = e[j];
  }
  __syncthreads();
  uint32_t tmax = 0;
  // ---- column block: column c, rows 32 b .. 32 b + 31 of the tile
  {
    const int c = tid >> 2, b = tid & 3;
    const int64_t gc = c0 + c, gr = r0 + 32 * b;
    if (gc < cols && gr < rows) {
      float v[32];
      uint32_t bf[16];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        v[i] = tile_value<IN>(t[32 * b + i][c]);
        tmax = umax(tmax, abs_bits_no_nan(v[i]));
      }
      if constexpr (IN == IN_BF16) {
#pragma unroll
        for (int k = 0; k < 16; ++k) bf[k] = uint32_t(t[32 * b + 2 * k][c]) | (uint32_t(t[32 * b + 2 * k + 1][c]) << 16);
      }
      uint32_t w[6];
      const uint32_t sc = encode_block32<IN, F, R>(v, bf, w);
      store24(q_col + gc * (rows / 32 * 24) + (gr / 32) * 24, w);
      s_col[gc * (rows / 32) + gr / 32] = uint8_t(sc);
    }
  }
  // ---- row block (dual): row r, columns 32 h .. 32 h + 31 of the tile
  if constexpr (DUAL) {
    const int r = tid >> 1, h = tid & 1;
    const int64_t gr = r0 + r, gc = c0 + 32 * h;
    if (gr < rows && gc < cols) {
      float v[32];
      uint32_t bf[16];
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = tile_value<IN>(t[r][32 * h + i]);
      if constexpr (IN == IN_BF16) {
#pragma unroll
        for (int k = 0; k < 16; ++k) bf[k] = uint32_t(t[r][32 * h + 2 * k]) | (uint32_t(t[r][32 * h + 2 * k + 1]) << 16);
      }
      uint32_t w[6];
      const uint32_t sc = encode_block32<IN, F, R>(v, bf, w);
      store24(q_row + gr * (cols / 32 * 24) + (gc / 32) * 24, w);
      s_row[gr * (cols / 32) + gc / 32] = uint8_t(sc);
    }
  }
  if constexpr (AMAX) {
    __shared__ uint32_t red[kThreads / 64];
    tmax = wave_max(tmax);
    if ((tid & 63) == 0) red[tid >> 6] = tmax;
    __syncthreads();
    if (tid == 0) {
      uint32_t mm = red[0];
#pragma unroll
      for (int k = 1; k < kThreads / 64; ++k) mm = umax(mm, red[k]);
      if (mm) atomic_max_u32(amax_out, mm);
    }
  }
}

template <int IN, int F, int R, bool DUAL>
static mx_status_t launch_tiles(const void* x, int64_t rows, int64_t cols, uint8_t* qr, uint8_t* sr, uint8_t* qc,
                                uint8_t* sc, uint32_t* amax, hipStream_t st) {
  const int64_t tr = (rows + kTR - 1) / kTR, tc = (cols + kTC - 1) / kTC;
  const dim3 grid{unsigned(tr * tc)}, block{unsigned(kThreads)};
  if (amax)
    hipLaunchKernelGGL((tile_kernel<IN, F, R, DUAL, true>), grid, block, 0, st, x, rows, cols, int(tc), qr, sr, qc, sc,
                       amax);
  else
    hipLaunchKernelGGL((tile_kernel<IN, F, R, DUAL, false>), grid, block, 0, st, x, rows, cols, int(tc), qr, sr, qc,
                       sc, amax);
  return hipGetLastError() == hipSuccess ? MX_OK : MX_ERR_LAUNCH;
}

template <int F, int R, bool DUAL>
static mx_status_t tiles_by_input(mx_dtype_t in, const void* x, int64_t rows, int64_t cols, uint8_t* qr, uint8_t* sr,
                                  uint8_t* qc, uint8_t* sc, uint32_t* amax, hipStream_t st) {
  if (in == MX_BF16) return launch_tiles<IN_BF16, F, R, DUAL>(x, rows, cols, qr, sr, qc, sc, amax, st);
  if (in == MX_F16) return launch_tiles<IN_F16, F, R, DUAL>(x, rows, cols, qr, sr, qc, sc, amax, st);
  return launch_tiles<IN_F32, F, R, DUAL>(x, rows, cols, qr, sr, qc, sc, amax, st);
}

// ---------------------------------------------------------------------------
// Register-resident MXFP6 dual quantizer for BF16 input
// ---------------------------------------------------------------------------
// The layout of the MXFP8 dual kernel: a workgroup of 4 waves takes a 128 x 128
// tile, each wave a 64 x 64 quarter in which a lane holds rows 8h .. 8h+7 of
// columns 8g .. 8g+7 (8 loads of 16 bytes).  A row block (32 columns) sits in a
// quad and a column block (32 rows) in 4 lanes of one 16-lane DPP row, so both
// block maxima are DPP steps.  The 32-element FP6 converter encodes each element
// from its own value and the block scale, so a lane converts just its 8 values
// (the other 24 inputs zero) and keeps the first 6 bytes of the stream: its 8
// codes, in place in the block's little-endian bit stream.  Codes are staged in
// LDS (96 bytes per tile row / column) and leave as 8-byte pieces of whole
// lines; scales leave as one dword per row and per column.
constexpr int kD6Tile = 128, kD6Wave = 64;
constexpr int kD6Line = kD6Tile * 6 / 8;     // 96 code bytes per tile row / column

__device__ __forceinline__ uint32_t d6_word(const uint4& u, int d) {
  return d == 0 ? u.x : d == 1 ? u.y : d == 2 ? u.z : u.w;
}

// 48 code bits of 8 BF16 values (4 pairs, element order) at the given scale.
template <int F>
__device__ __forceinline__ uint2 d6_convert8(const uint32_t (&p)[4], float scale) {
  v16u_t d;
  d[0] = p[0]; d[1] = p[1]; d[2] = p[2]; d[3] = p[3];
#pragma unroll
  for (int k = 4; k < 16; ++k) d[k] = 0u;
  const v32bf_t xv = __builtin_bit_cast(v32bf_t, d);
  v6u_t r;
  if constexpr (F == E2M3) r = __builtin_bit_cast(v6u_t, __builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(xv, scale));
  else r = __builtin_bit_cast(v6u_t, __builtin_amdgcn_cvt_scalef32_pk32_bf6_bf16(xv, scale));
  return make_uint2(r[0], r[1] & 0xFFFFu);
}

// 48 code bits of 8 BF16 values of a block that is non-finite (largest
// magnitude with each input's sign) or has a subnormal amax (integer encoder
// on v * 2^-e).  Out of line: rare.
template <int F>
__device__ __attribute__((noinline)) uint2 d6_encode8_general(uint4 c, int e, int nonfinite) {
  const uint32_t w4[4] = {c.x, c.y, c.z, c.w};
  const float mul = pow2_neg(e);
  uint64_t acc = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t bits = (i & 1) ? (w4[i >> 1] & 0xFFFF0000u) : (w4[i >> 1] << 16);
    const uint32_t code = nonfinite ? (Fmt_<F>::kNan | ((bits >> 31) << 5))
                                    : encode_rne_sat<F>(__uint_as_float(bits) * mul);
    acc |= uint64_t(code & 0x3Fu) << (6 * i);
  }
  return make_uint2(uint32_t(acc), uint32_t(acc >> 32));
}

template <int F, int R>
__device__ __forceinline__ uint2 d6_encode8(const uint32_t (&p)[4], uint32_t bmax, uint32_t& scale_code) {
  const bool nonfinite = bmax >= 0x7F800000u;
  const int e = nonfinite ? 0 : shared_exponent<F, R>(bmax);
  // the converter saturates: both rules go straight in; an all-zero block
  // converts at scale 1 (+-0 gives +-0)
  if (!nonfinite && (e > -127 || bmax == 0u)) {
    scale_code = uint32_t(e + 127);
    return d6_convert8<F>(p, bmax == 0u ? 1.0f : __uint_as_float(uint32_t(127 + e) << 23));
  }
  scale_code = nonfinite ? 0xFFu : uint32_t(e + 127);
  return d6_encode8_general<F>(make_uint4(p[0], p[1], p[2], p[3]), e, nonfinite ? 1 : 0);
}

// 6 bytes at a 2-byte aligned LDS address
__device__ __forceinline__ void d6_put6(uint8_t* dst, uint2 w) {
  uint16_t* d = reinterpret_cast<uint16_t*>(dst);
  d[0] = uint16_t(w.x);
  d[1] = uint16_t(w.x >> 16);
  d[2] = uint16_t(w.y);
}

__device__ __forceinline__ uint32_t d6_absmax(const uint4& c) {
  const uint32_t k = 0x7FFF7FFFu;
  const uint32_t m = pk_umax16(pk_umax16(c.x & k, c.y & k), pk_umax16(c.z & k, c.w & k));
  return umax(m & 0xFFFFu, m >> 16) << 16;
}

template <int F, int R, bool AMAX>
__global__ __launch_bounds__(256) void dual_bf16_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                        int tiles_c, uint8_t* __restrict__ q_row,
                                                        uint8_t* __restrict__ s_row, uint8_t* __restrict__ q_col,
                                                        uint8_t* __restrict__ s_col, uint32_t* __restrict__ amax_out) {
  __shared__ __attribute__((aligned(16))) uint8_t qr_lds[kD6Tile * kD6Line];   // [tile row][96 B]
  __shared__ __attribute__((aligned(16))) uint8_t qc_lds[kD6Tile * kD6Line];   // [tile column][96 B]
  __shared__ uint32_t srow_lds[kD6Tile], scol_lds[kD6Tile];
  __shared__ uint32_t red[4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // lane bits 0-1 and 4 give g, bits 2-3 and 5 give h
  const int g = (lane & 3) | ((lane >> 2) & 4), h = ((lane >> 2) & 3) | ((lane >> 3) & 4), lane_q = lane & 3;
  const int t = blockIdx.x;
  const int64_t tr = int64_t(t / tiles_c) * kD6Tile, tc = int64_t(t % tiles_c) * kD6Tile;
  const int wro = (wave >> 1) * kD6Wave, wco = (wave & 1) * kD6Wave;
  uint8_t* const srl = reinterpret_cast<uint8_t*>(srow_lds) + wro * 4 + (wave & 1) * 2;
  uint8_t* const scl = reinterpret_cast<uint8_t*>(scol_lds) + wco * 4 + (wave >> 1) * 2;
  // rows and cols are multiples of 32: a quad and the lanes h = 4k .. 4k+3 are in or out together
  const bool ok = tr + wro + 8 * h < rows && tc + wco + 8 * g < cols;
  uint32_t tmax = 0;
  if (ok) {
    // a scalar base plus a 32-bit lane offset (the host keeps 64 * cols * 2 below 2^32)
    const uint8_t* xb = reinterpret_cast<const uint8_t*>(x) + ((tr + wro) * cols + tc + wco) * 2;
    const uint32_t c32 = uint32_t(cols);
    uint4 raw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4_t v = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(xb + (uint32_t(8 * h + i) * c32 + uint32_t(8 * g)) * 2u));
      raw[i] = make_uint4(v[0], v[1], v[2], v[3]);
    }
    // ---- row-wise half: lane q of a quad holds elements 8q .. 8q+7 of the block
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t m = d6_absmax(raw[i]);
      if constexpr (AMAX) {
        if (m <= 0x7F800000u) {
          tmax = umax(tmax, m);
        } else {
          const uint32_t w4[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            tmax = umax(tmax, abs_bits_no_nan(__uint_as_float(w4[j] << 16)));
            tmax = umax(tmax, abs_bits_no_nan(__uint_as_float(w4[j] & 0xFFFF0000u)));
          }
        }
      }
      const uint32_t p[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
      uint32_t sc;
      const uint2 w = d6_encode8<F, R>(p, quad_max(m), sc);
      if (lane_q == 0) srl[(8 * h + i) * 4 + (g >> 2)] = uint8_t(sc);
      d6_put6(qr_lds + (wro + 8 * h + i) * kD6Line + 6 * ((wco >> 3) + g), w);
    }
    // ---- column-wise half: dword d holds columns 2d (low halves) and 2d+1
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t mp = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) mp = pk_umax16(mp, d6_word(raw[i], d) & 0x7FFF7FFFu);
      mp = pk_umax16(mp, dpp_u32<kRowRor4>(mp));
      mp = pk_umax16(mp, dpp_u32<kRowRor8>(mp));
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint32_t sel = k ? 0x07060302u : 0x05040100u;
        uint32_t p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          p[i] = __builtin_amdgcn_perm(d6_word(raw[2 * i + 1], d), d6_word(raw[2 * i], d), sel);
        uint32_t sc;
        const uint2 w = d6_encode8<F, R>(p, k ? (mp & 0xFFFF0000u) : (mp << 16), sc);
        const int c = 8 * g + 2 * d + k;                     // column within the wave quarter
        d6_put6(qc_lds + (wco + c) * kD6Line + 6 * ((wro >> 3) + h), w);
        if ((h & 3) == 0) scl[c * 4 + (h >> 2)] = uint8_t(sc);
      }
    }
  }
  if constexpr (AMAX) {
    const uint32_t wm = wave_max(tmax);
    if (lane == 0) red[wave] = wm;
  }
  __syncthreads();
  // ---- codes: 8-byte pieces, 12 per 96-byte line; 3 pieces are one block, so a
  // ragged edge (whole 32-element blocks) stays exact
  {
    const int64_t row_pitch = cols / 32 * 24, col_pitch = rows / 32 * 24;
#pragma unroll
    for (int it = 0; it < kD6Tile * 12 / 256; ++it) {
      const int item = threadIdx.x + 256 * it;
      const int r = item / 12, pc = item % 12;
      const int64_t e = int64_t(pc / 3) * 32;                        // first element of the piece's block
      if (tr + r < rows && tc + e < cols)
        *reinterpret_cast<uint2*>(q_row + (tr + r) * row_pitch + (tc / 32) * 24 + 8 * pc) =
            *reinterpret_cast<const uint2*>(qr_lds + r * kD6Line + 8 * pc);
      if (tc + r < cols && tr + e < rows)
        *reinterpret_cast<uint2*>(q_col + (tc + r) * col_pitch + (tr / 32) * 24 + 8 * pc) =
            *reinterpret_cast<const uint2*>(qc_lds + r * kD6Line + 8 * pc);
    }
  }
  // ---- scales: thread j < 128 writes tile row j's 4 row scales, thread 128 + j
  // tile column j's 4 column scales (fewer, byte by byte, on a ragged edge)
  {
    const int j = threadIdx.x & (kD6Tile - 1);
    const bool col_side = threadIdx.x >= kD6Tile;
    const int64_t line = col_side ? tc + j : tr + j;
    const int64_t lines = col_side ? cols : rows;
    const int64_t other0 = col_side ? tr : tc, other = col_side ? rows : cols;
    if (line < lines) {
      const uint32_t v = col_side ? scol_lds[j] : srow_lds[j];
      uint8_t* dst = (col_side ? s_col : s_row) + line * (other >> 5) + (other0 >> 5);
      const int64_t nb = (other - other0) >> 5;
      if (nb >= 4 && (reinterpret_cast<uintptr_t>(dst) & 3u) == 0) {
        *reinterpret_cast<uint32_t*>(dst) = v;
      } else {
        for (int b = 0; b < 4 && b < nb; ++b) dst[b] = uint8_t(v >> (8 * b));
      }
    }
  }
  if constexpr (AMAX) {
    if (threadIdx.x == 0) {
      const uint32_t mm = umax(umax(red[0], red[1]), umax(red[2], red[3]));
      if (mm) atomic_max_u32(amax_out, mm);
    }
  }
}

template <int F, int R>
static mx_status_t launch_dual_bf16(const void* x, int64_t rows, int64_t cols, uint8_t* qr, uint8_t* sr,
                                    uint8_t* qc, uint8_t* sc, uint32_t* amax, hipStream_t st) {
  const int64_t tiles_c = (cols + kD6Tile - 1) / kD6Tile;
  const int64_t ntiles = tiles_c * ((rows + kD6Tile - 1) / kD6Tile);
  const dim3 grid{unsigned(ntiles)}, block{256u};
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  if (amax)
    hipLaunchKernelGGL((dual_bf16_kernel<F, R, true>), grid, block, 0, st, xb, rows, cols, int(tiles_c), qr, sr, qc,
                       sc, amax);
  else
    hipLaunchKernelGGL((dual_bf16_kernel<F, R, false>), grid, block, 0, st, xb, rows, cols, int(tiles_c), qr, sr, qc,
                       sc, amax);
  return hipGetLastError() == hipSuccess ? MX_OK : MX_ERR_LAUNCH;
}

template <bool DUAL>
static mx_status_t tiles(mx_elem_t fmt, mx_scale_rule_t rule, mx_dtype_t in, const void* x, int64_t rows,
                         int64_t cols, uint8_t* qr, uint8_t* sr, uint8_t* qc, uint8_t* sc, uint32_t* amax,
                         hipStream_t st) {
  const bool ceil = rule == MX_SCALE_CEIL;
  if (fmt == MX_E2M3)
    return ceil ? tiles_by_input<E2M3, CEIL, DUAL>(in, x, rows, cols, qr, sr, qc, sc, amax, st)
                : tiles_by_input<E2M3, FLOOR, DUAL>(in, x, rows, cols, qr, sr, qc, sc, amax, st);
  return ceil ? tiles_by_input<E3M2, CEIL, DUAL>(in, x, rows, cols, qr, sr, qc, sc, amax, st)
              : tiles_by_input<E3M2, FLOOR, DUAL>(in, x, rows, cols, qr, sr, qc, sc, amax, st);
}

}  // namespace fp6

mx_status_t fp6_quantize_dual(const void* x, mx_dtype_t in, int64_t rows, int64_t cols, int block, mx_elem_t fmt,
                              mx_scale_rule_t rule, uint8_t* q_row, uint8_t* s_row, uint8_t* q_colT,
                              uint8_t* s_colT, float* amax_out, hipStream_t stream) {
  if (in != MX_F32 && in != MX_BF16 && in != MX_F16) return MX_ERR_UNSUPPORTED;
  if (rule != MX_SCALE_FLOOR && rule != MX_SCALE_CEIL) return MX_ERR_UNSUPPORTED;
  if (block != 32) return MX_ERR_UNSUPPORTED;
  if (rows < 0 || cols < 0 || rows > (int64_t(1) << 31) || cols > (int64_t(1) << 31)) return MX_ERR_SHAPE;
  if (rows % 32 != 0 || cols % 32 != 0) return MX_ERR_SHAPE;
  if (rows * cols == 0) return MX_OK;
  if (!x || !q_row || !s_row || !q_colT || !s_colT) return MX_ERR_NULL;
  if (misaligned(x) || misaligned(q_row) || misaligned(q_colT)) return MX_ERR_ALIGN;
  uint32_t* am = reinterpret_cast<uint32_t*>(amax_out);
  const int64_t ntiles = ((cols + fp6::kD6Tile - 1) / fp6::kD6Tile) * ((rows + fp6::kD6Tile - 1) / fp6::kD6Tile);
  if (in == MX_BF16 && ntiles < (int64_t(1) << 31) && cols < (int64_t(1) << 25)) {
    const bool ceil = rule == MX_SCALE_CEIL;
    if (fmt == MX_E2M3)
      return ceil ? fp6::launch_dual_bf16<E2M3, CEIL>(x, rows, cols, q_row, s_row, q_colT, s_colT, am, stream)
                  : fp6::launch_dual_bf16<E2M3, FLOOR>(x, rows, cols, q_row, s_row, q_colT, s_colT, am, stream);
    return ceil ? fp6::launch_dual_bf16<E3M2, CEIL>(x, rows, cols, q_row, s_row, q_colT, s_colT, am, stream)
                : fp6::launch_dual_bf16<E3M2, FLOOR>(x, rows, cols, q_row, s_row, q_colT, s_colT, am, stream);
  }
  return fp6::tiles<true>(fmt, rule, in, x, rows, cols, q_row, s_row, q_colT, s_colT, am, stream);
}

mx_status_t fp6_quantize(const void* x, mx_dtype_t in, int64_t rows, int64_t cols, int block, mx_elem_t fmt,
                         mx_scale_rule_t rule, mx_orient_t orient, int hadamard, uint8_t* q, uint8_t* scales,
                         float* amax_out, hipStream_t stream) {
  if (in != MX_F32 && in != MX_BF16 && in != MX_F16) return MX_ERR_UNSUPPORTED;
  if (rule != MX_SCALE_FLOOR && rule != MX_SCALE_CEIL) return MX_ERR_UNSUPPORTED;
  if (block != 32 || (orient != MX_ROWWISE && orient != MX_COLWISE_T) || hadamard != 0) return MX_ERR_UNSUPPORTED;
  if (rows < 0 || cols < 0 || rows > (int64_t(1) << 31) || cols > (int64_t(1) << 31)) return MX_ERR_SHAPE;
  if (orient == MX_ROWWISE && cols % 32 != 0) return MX_ERR_SHAPE;
  if (orient == MX_COLWISE_T && (rows % 32 != 0 || cols % 8 != 0)) return MX_ERR_SHAPE;
  const int64_t n = rows * cols;
  if (n == 0) return MX_OK;
  if (!x || !q || !scales) return MX_ERR_NULL;
  if (misaligned(x) || misaligned(q)) return MX_ERR_ALIGN;
  uint32_t* am = reinterpret_cast<uint32_t*>(amax_out);
  if (orient == MX_COLWISE_T)
    return fp6::tiles<false>(fmt, rule, in, x, rows, cols, nullptr, nullptr, q, scales, am, stream);
  const bool ceil = rule == MX_SCALE_CEIL;
  if (fmt == MX_E2M3)
    return ceil ? fp6::by_input<E2M3, CEIL>(in, x, n, q, scales, am, stream)
                : fp6::by_input<E2M3, FLOOR>(in, x, n, q, scales, am, stream);
  return ceil ? fp6::by_input<E3M2, CEIL>(in, x, n, q, scales, am, stream)
              : fp6::by_input<E3M2, FLOOR>(in, x, n, q, scales, am, stream);
}

}  // namespace mxk
