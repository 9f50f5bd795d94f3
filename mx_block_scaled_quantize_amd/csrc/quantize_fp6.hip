// Row-wise MXFP6 (E2M3, E3M2) quantization for gfx950.
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
//     Blocks with NaN/Inf, or with e = -127 (not a normal FP32 scale), take the
//     integer encoder below.
//   rowwise_kernel  FP32 / FP16 input: a lane owns 8 elements, a quad owns a block
//     and takes its amax with two DPP steps; the cast is the exact integer RNE +
//     saturation encoder on v * 2^-e (a power-of-two multiply, exact wherever the
//     result can matter).

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
constexpr int kUnrollB = 2;

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
    if (!nonfinite && e > -127) {
      const float scale = __uint_as_float(uint32_t(127 + e) << 23);
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

}  // namespace fp6

mx_status_t fp6_quantize(const void* x, mx_dtype_t in, int64_t rows, int64_t cols, int block, mx_elem_t fmt,
                         mx_scale_rule_t rule, mx_orient_t orient, int hadamard, uint8_t* q, uint8_t* scales,
                         float* amax_out, hipStream_t stream) {
  if (in != MX_F32 && in != MX_BF16 && in != MX_F16) return MX_ERR_UNSUPPORTED;
  if (rule != MX_SCALE_FLOOR && rule != MX_SCALE_CEIL) return MX_ERR_UNSUPPORTED;
  if (block != 32 || orient != MX_ROWWISE || hadamard != 0) return MX_ERR_UNSUPPORTED;
  if (rows < 0 || cols < 0 || rows > (int64_t(1) << 31) || cols > (int64_t(1) << 31)) return MX_ERR_SHAPE;
  if (cols % 32 != 0) return MX_ERR_SHAPE;
  const int64_t n = rows * cols;
  if (n == 0) return MX_OK;
  if (!x || !q || !scales) return MX_ERR_NULL;
  if (misaligned(x) || misaligned(q)) return MX_ERR_ALIGN;
  uint32_t* am = reinterpret_cast<uint32_t*>(amax_out);
  const bool ceil = rule == MX_SCALE_CEIL;
  if (fmt == MX_E2M3)
    return ceil ? fp6::by_input<E2M3, CEIL>(in, x, n, q, scales, am, stream)
                : fp6::by_input<E2M3, FLOOR>(in, x, n, q, scales, am, stream);
  return ceil ? fp6::by_input<E3M2, CEIL>(in, x, n, q, scales, am, stream)
              : fp6::by_input<E3M2, FLOOR>(in, x, n, q, scales, am, stream);
}

}  // namespace mxk
