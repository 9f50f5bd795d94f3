// Stochastic-rounding MXFP4, row-wise, for gfx950.
//
// [FAF] (the configuration that reached 37.2K tokens/s): row gradients are
// quantized to MXFP4 with stochastic rounding.  The page names the technique
// only; the definition implemented here is the plain one, driven by random
// words the caller supplies (one uint32 per element):
//   * the block scale is the ordinary MX scale (same rule as mx_quantize);
//   * the magnitude y = |V| / X is exact; an E2M1 magnitude is kept, y >= 6
//     saturates to 6, and strictly between neighbours lo < hi it becomes hi iff
//     r < floor(2^32 (y - lo) / (hi - lo)), else lo;
//   * the sign is copied; a block holding NaN or Inf gets scale 0xFF and +-6.
//
// Kernel: the flat row-wise layout (row-wise blocks are contiguous): a lane
// owns 8 consecutive elements and their 8 random words, a quad owns a block and
// takes the block amax with two DPP steps.  y is never formed as a float: its
// exponent is the input's exponent minus the block exponent and its significand
// is the input's, so every threshold below is an exact integer.

#include "mx_device.hpp"
#include "mx_launch.hpp"

namespace mxk {

namespace sr {

constexpr int kThreads = 256;
// chunks per thread: one (many small workgroups keep the most loads in flight;
// on a BF16 8192 x 4096 input it measured 41.8 us against 43.6 with two and
// 47.7 with four)
constexpr int kUnroll = 1;

// Exponent (unbiased) and 23-bit fraction of |v| for finite nonzero v, with FP32
// subnormals normalized.
__device__ __forceinline__ void split_f32(uint32_t mag, int& ex, uint32_t& frac) {
  const uint32_t field = mag >> 23;
  if (field != 0) {
    ex = int(field) - 127;
    frac = mag & 0x7FFFFFu;
  } else {
    const int top = 31 - __builtin_clz(mag);        // mag = m * 2^-149, top set bit of m
    ex = top - 149;
    frac = (mag << (23 - top)) & 0x7FFFFFu;
  }
}

// E2M1 magnitude code (0..7) of y = |v| 2^-e with random word r.
__device__ __forceinline__ uint32_t sr_code(uint32_t mag, int e, uint32_t r) {
  if (mag == 0) return 0;
  int ex;
  uint32_t frac;
  split_f32(mag, ex, frac);
  const int ey = ex - e;                             // y in [2^ey, 2^(ey+1))
  if (ey >= 3 || (ey == 2 && frac >= 0x400000u)) return 7;   // y >= 6: saturate
  uint32_t lo, t;
  if (ey >= 0) {
    // y in [1, 6): neighbours 2^ey {1, 1.5, 2}; the code's mantissa bit is frac bit 22
    lo = uint32_t(2 * (ey + 1)) + (frac >> 22);
    t = (frac & 0x3FFFFFu) << 10;                    // 2^32 (y - lo) / 2^(ey-1)
  } else if (ey == -1) {
    lo = 1;                                          // y in [0.5, 1): lo 0.5, hi 1
    t = frac << 9;                                   // 2^32 (y - 0.5) / 0.5
  } else {
    lo = 0;                                          // y < 0.5: lo 0, hi 0.5
    const int s = ey + 10;                           // floor(2^33 y) = (2^23 + frac) 2^(ey + 10)
    const uint32_t sig = 0x800000u | frac;
    t = s >= 0 ? sig << s : (s > -32 ? sig >> -s : 0u);
  }
  return lo + (r < t ? 1u : 0u);
}

template <int IN, int R, bool AMAX>
__global__ __launch_bounds__(kThreads) void sr_rowwise_kernel(const void* __restrict__ x,
                                                              const uint32_t* __restrict__ rand, int64_t nchunks,
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
    const u32x4_t* rp = reinterpret_cast<const u32x4_t*>(rand + chunk * 8);   // read once: streaming
    const u32x4_t r0 = __builtin_nontemporal_load(rp), r1 = __builtin_nontemporal_load(rp + 1);
    const uint32_t r[8] = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = umax(m, abs_bits(v[j]));
    if constexpr (AMAX) {
#pragma unroll
      for (int j = 0; j < 8; ++j) tmax = umax(tmax, abs_bits_no_nan(v[j]));
    }
    const uint32_t bmax = quad_max(m);
    const bool nonfinite = bmax >= 0x7F800000u;
    const int e = nonfinite ? 0 : shared_exponent<E2M1, R>(bmax);
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t bits = __float_as_uint(v[j]);
      const uint32_t code = nonfinite ? 7u : sr_code(bits & 0x7FFFFFFFu, e, r[j]);
      w |= (code | ((bits >> 31) << 3)) << (4 * j);
    }
    *reinterpret_cast<uint32_t*>(q + chunk * 4) = w;
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

template <int IN, int R>
static mx_status_t dispatch(const void* x, const uint32_t* rand, int64_t n, uint8_t* q, uint8_t* s, uint32_t* amax,
                            hipStream_t st) {
  const int64_t nchunks = n / 8;
  const int64_t per = int64_t(kThreads) * kUnroll;
  const dim3 grid{unsigned((nchunks + per - 1) / per)}, block{unsigned(kThreads)};
  if (amax)
    hipLaunchKernelGGL((sr_rowwise_kernel<IN, R, true>), grid, block, 0, st, x, rand, nchunks, q, s, amax);
  else
    hipLaunchKernelGGL((sr_rowwise_kernel<IN, R, false>), grid, block, 0, st, x, rand, nchunks, q, s, amax);
  return hipGetLastError() == hipSuccess ? MX_OK : MX_ERR_LAUNCH;
}

}  // namespace sr
}  // namespace mxk

using namespace mxk;

extern "C" mx_status_t mx_quantize_sr(const void* x, mx_dtype_t in, int64_t rows, int64_t cols, int block,
                                      mx_elem_t fmt, mx_scale_rule_t rule, const uint32_t* rand, uint8_t* q,
                                      uint8_t* scales, float* amax_out, hipStream_t stream) {
  mx_status_t st = check_common_quant(in, rows, cols, block, fmt, rule);
  if (st != MX_OK) return st;
  if (fmt != MX_E2M1) return MX_ERR_UNSUPPORTED;
  if (cols % 32 != 0) return MX_ERR_SHAPE;
  const int64_t n = rows * cols;
  if (n == 0) return MX_OK;
  if (!x || !rand || !q || !scales) return MX_ERR_NULL;
  if (misaligned(x) || misaligned(rand) || misaligned(q)) return MX_ERR_ALIGN;
  uint32_t* am = reinterpret_cast<uint32_t*>(amax_out);
  if (in == MX_BF16)
    return rule == MX_SCALE_CEIL ? sr::dispatch<IN_BF16, CEIL>(x, rand, n, q, scales, am, stream)
                                 : sr::dispatch<IN_BF16, FLOOR>(x, rand, n, q, scales, am, stream);
  if (in == MX_F16)
    return rule == MX_SCALE_CEIL ? sr::dispatch<IN_F16, CEIL>(x, rand, n, q, scales, am, stream)
                                 : sr::dispatch<IN_F16, FLOOR>(x, rand, n, q, scales, am, stream);
  return rule == MX_SCALE_CEIL ? sr::dispatch<IN_F32, CEIL>(x, rand, n, q, scales, am, stream)
                               : sr::dispatch<IN_F32, FLOOR>(x, rand, n, q, scales, am, stream);
}
