// MX dequantization for gfx950: V^_i = Q_i * 2^(c - 127) ("EU8M0 FP8" article,
// first part section 2: decoding an E8M0 scale only shifts the exponent, no
// multiplication or rounding of the element is involved).
//
// Each element code is decoded to an integer significand and an exponent, the
// block's scale exponent is added, and one ldexp produces the exact FP32 value
// (FP32 holds every product for in-range scales: significands have at most 4
// bits and the smallest exponent is 2^-136 > 2^-149).  BF16 output rounds that
// exact value once, to nearest even.
//
//   rowwise_deq_kernel  flat over row-wise blocks: 8 codes per lane.
//   colwise_deq_kernel  transposed storage [cols][rows] -> output [rows][cols]
//                       through a 64 x 64 LDS tile.

#include "mx_device.hpp"
#include "mx_launch.hpp"

namespace mxk {

// Exact value of an element code times 2^sexp (sexp = scale code - 127).
template <int F>
__device__ __forceinline__ float decode_scaled(uint32_t code, int sexp) {
  if constexpr (F == E4M3) {
    const uint32_t ef = (code >> 3) & 0xFu, mf = code & 7u;
    const bool neg = (code & 0x80u) != 0;
    if (ef == 15u && mf == 7u) return __uint_as_float(0x7FC00000u);
    const int sig = ef ? int(8u + mf) : int(mf);
    const int ex = ef ? int(ef) - 10 : -9;     // value = sig * 2^ex
    const float m = ldexpf(float(sig), ex + sexp);
    return neg ? -m : m;
  } else if constexpr (F == E5M2) {
    const uint32_t ef = (code >> 2) & 0x1Fu, mf = code & 3u;
    const bool neg = (code & 0x80u) != 0;
    if (ef == 31u) {
      if (mf) return __uint_as_float(0x7FC00000u);
      return neg ? -__uint_as_float(0x7F800000u) : __uint_as_float(0x7F800000u);
    }
    const int sig = ef ? int(4u + mf) : int(mf);
    const int ex = ef ? int(ef) - 17 : -16;
    const float m = ldexpf(float(sig), ex + sexp);
    return neg ? -m : m;
  } else if constexpr (F == E2M3) {   // bias 1, 3 mantissa bits, no specials
    const uint32_t ef = (code >> 3) & 3u, mf = code & 7u;
    const bool neg = (code & 0x20u) != 0;
    const int sig = ef ? int(8u + mf) : int(mf);
    const int ex = ef ? int(ef) - 4 : -3;
    const float m = ldexpf(float(sig), ex + sexp);
    return neg ? -m : m;
  } else if constexpr (F == E3M2) {   // bias 3, 2 mantissa bits, no specials
    const uint32_t ef = (code >> 2) & 7u, mf = code & 3u;
    const bool neg = (code & 0x20u) != 0;
    const int sig = ef ? int(4u + mf) : int(mf);
    const int ex = ef ? int(ef) - 5 : -4;
    const float m = ldexpf(float(sig), ex + sexp);
    return neg ? -m : m;
  } else {
    const uint32_t ef = (code >> 1) & 3u, mf = code & 1u;
    const bool neg = (code & 0x8u) != 0;
    const int sig = ef ? int(2u + mf) : int(mf);
    const int ex = ef ? int(ef) - 2 : -1;
    const float m = ldexpf(float(sig), ex + sexp);
    return neg ? -m : m;
  }
}

// FP32 -> BF16, nearest even, NaN kept quiet.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  const uint32_t b = __float_as_uint(f);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return ((b >> 16) | 0x40u) & 0xFFFFu;
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

template <int F>
__device__ __forceinline__ void decode8(const uint8_t* __restrict__ q, int64_t elem, uint32_t scale, float (&o)[8]) {
  uint32_t c[8];
  if constexpr (Fmt_<F>::kBits == 8) {
    const uint2 w = *reinterpret_cast<const uint2*>(q + elem);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c[j] = (w.x >> (8 * j)) & 0xFFu;
      c[4 + j] = (w.y >> (8 * j)) & 0xFFu;
    }
  } else if constexpr (Fmt_<F>::kBits == 6) {
    // 6 bytes at elem * 3 / 4: 4-byte aligned for even chunks, 2-byte aligned for odd
    const uint8_t* p = q + elem / 8 * 6;
    uint32_t lo, hi;
    if (((elem / 8) & 1) == 0) {
      lo = *reinterpret_cast<const uint32_t*>(p);
      hi = *reinterpret_cast<const uint16_t*>(p + 4);
    } else {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(p + 2);
      lo = uint32_t(*reinterpret_cast<const uint16_t*>(p)) | (w << 16);
      hi = w >> 16;
    }
#pragma unroll
    for (int j = 0; j < 5; ++j) c[j] = (lo >> (6 * j)) & 0x3Fu;
    c[5] = (lo >> 30) | ((hi & 0xFu) << 2);
    c[6] = (hi >> 4) & 0x3Fu;
    c[7] = (hi >> 10) & 0x3Fu;
  } else {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(q + elem / 2);
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = (w >> (4 * j)) & 0xFu;
  }
  if (scale == 0xFFu) {
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = __uint_as_float(0x7FC00000u);
    return;
  }
  const int sexp = int(scale) - 127;
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = decode_scaled<F>(c[j], sexp);
}

template <bool BF16OUT>
__device__ __forceinline__ void store8(void* __restrict__ out, int64_t elem, const float (&o)[8]) {
  if constexpr (BF16OUT) {
    uint4 w;
    w.x = f32_to_bf16(o[0]) | (f32_to_bf16(o[1]) << 16);
    w.y = f32_to_bf16(o[2]) | (f32_to_bf16(o[3]) << 16);
    w.z = f32_to_bf16(o[4]) | (f32_to_bf16(o[5]) << 16);
    w.w = f32_to_bf16(o[6]) | (f32_to_bf16(o[7]) << 16);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + elem) = w;
  } else {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(out) + elem);
    p[0] = make_float4(o[0], o[1], o[2], o[3]);
    p[1] = make_float4(o[4], o[5], o[6], o[7]);
  }
}

constexpr int kDeqThreads = 256;

template <int F, bool BF16OUT>
__global__ __launch_bounds__(kDeqThreads) void rowwise_deq_kernel(const uint8_t* __restrict__ q,
                                                                  const uint8_t* __restrict__ scales,
                                                                  int64_t nchunks, void* __restrict__ out,
                                                                  int64_t lines, int64_t gemm_kblocks) {
  const int64_t chunk = int64_t(blockIdx.x) * kDeqThreads + threadIdx.x;
  if (chunk >= nchunks) return;
  // block index chunk / 4 = line * kblocks + kb; gemm_kblocks != 0 selects the GEMM scale layout
  const int64_t blk = chunk >> 2;
  const uint8_t sc =
      scales[gemm_kblocks ? scale_offset(blk / gemm_kblocks, blk % gemm_kblocks, lines, gemm_kblocks, true) : blk];
  float o[8];
  decode8<F>(q, chunk * 8, sc, o);
  store8<BF16OUT>(out, chunk * 8, o);
}

// Transposed storage: codes [cols][rows] (rows contiguous), scales [cols][rows/32].
// A workgroup owns 64 stored rows (output columns) x 64 stored columns (output rows).
constexpr int kDT = 64;

template <int F, bool BF16OUT>
__global__ __launch_bounds__(kDeqThreads) void colwise_deq_kernel(const uint8_t* __restrict__ q,
                                                                  const uint8_t* __restrict__ scales,
                                                                  int64_t rows, int64_t cols, int tiles_r,
                                                                  void* __restrict__ out, bool gemm_scales) {
  __shared__ float t[kDT][kDT + 1];
  const int tid = threadIdx.x;
  const int64_t oc0 = int64_t(blockIdx.x / tiles_r) * kDT;   // output column = stored row
  const int64_t or0 = int64_t(blockIdx.x % tiles_r) * kDT;   // output row = stored column
  // read: 64 stored rows x 8 chunks of 8 codes
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int item = tid + k * kDeqThreads;
    const int sr = item >> 3, ch = (item & 7) * 8;
    const int64_t c = oc0 + sr, r = or0 + ch;
    float o[8];
    if (c < cols && r < rows) {
      decode8<F>(q, c * rows + r, scales[scale_offset(c, r >> 5, cols, rows >> 5, gemm_scales)], o);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) t[ch + j][sr] = o[j];
  }
  __syncthreads();
  // write: 64 output rows x 8 chunks of 8 values
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int item = tid + k * kDeqThreads;
    const int orow = item >> 3, ch = (item & 7) * 8;
    const int64_t r = or0 + orow, c = oc0 + ch;
    if (r < rows && c < cols) {
      float o[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] = t[orow][ch + j];
      store8<BF16OUT>(out, r * cols + c, o);
    }
  }
}

template <typename K, typename... Args>
static mx_status_t launch_k(K kernel, dim3 grid, dim3 block, hipStream_t s, Args... args) {
  hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
  return hipGetLastError() == hipSuccess ? MX_OK : MX_ERR_LAUNCH;
}

template <int F, bool BF>
static mx_status_t deq_dispatch(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t cols, bool colwise,
                                bool gemm_scales, void* out, hipStream_t st) {
  if (!colwise) {
    const int64_t nchunks = rows * cols / 8;
    return launch_k(rowwise_deq_kernel<F, BF>, dim3(unsigned((nchunks + kDeqThreads - 1) / kDeqThreads)),
                    dim3(kDeqThreads), st, q, s, nchunks, out, rows, gemm_scales ? cols / 32 : int64_t(0));
  }
  const int64_t tr = (rows + kDT - 1) / kDT, tc = (cols + kDT - 1) / kDT;
  return launch_k(colwise_deq_kernel<F, BF>, dim3(unsigned(tr * tc)), dim3(kDeqThreads), st, q, s, rows, cols,
                  int(tr), out, gemm_scales);
}

}  // namespace mxk

using namespace mxk;

extern "C" mx_status_t mx_dequantize(const uint8_t* q, const uint8_t* scales, int64_t rows, int64_t cols, int block,
                                     mx_elem_t fmt, mx_orient_t orient, mx_scale_layout_t scale_layout, void* out,
                                     mx_dtype_t out_dtype, hipStream_t stream) {
  const bool fp6 = fmt == MX_E2M3 || fmt == MX_E3M2;
  if (fmt != MX_E4M3 && fmt != MX_E5M2 && fmt != MX_E2M1 && !fp6) return MX_ERR_UNSUPPORTED;
  if (out_dtype != MX_F32 && out_dtype != MX_BF16) return MX_ERR_UNSUPPORTED;
  if (orient != MX_ROWWISE && orient != MX_COLWISE_T) return MX_ERR_UNSUPPORTED;
  if (block != 32) return MX_ERR_UNSUPPORTED;
  if (rows < 0 || cols < 0 || rows > (int64_t(1) << 31) || cols > (int64_t(1) << 31)) return MX_ERR_SHAPE;
  if (orient == MX_ROWWISE && cols % 32 != 0) return MX_ERR_SHAPE;
  if (orient == MX_COLWISE_T && (rows % 32 != 0 || cols % 8 != 0)) return MX_ERR_SHAPE;
  if (scale_layout != MX_SCALES_ROW_MAJOR && scale_layout != MX_SCALES_GEMM) return MX_ERR_UNSUPPORTED;
  const bool gemm_scales = scale_layout == MX_SCALES_GEMM;
  if (gemm_scales && (orient == MX_ROWWISE ? cols : rows) % 512 != 0) return MX_ERR_SHAPE;
  if (rows * cols == 0) return MX_OK;
  if (!q || !scales || !out) return MX_ERR_NULL;
  if (misaligned(q) || misaligned(out)) return MX_ERR_ALIGN;
  const bool col = orient == MX_COLWISE_T;
  const bool bf = out_dtype == MX_BF16;
  switch (fmt) {
    case MX_E4M3: return bf ? deq_dispatch<E4M3, true>(q, scales, rows, cols, col, gemm_scales, out, stream)
                            : deq_dispatch<E4M3, false>(q, scales, rows, cols, col, gemm_scales, out, stream);
    case MX_E5M2: return bf ? deq_dispatch<E5M2, true>(q, scales, rows, cols, col, gemm_scales, out, stream)
                            : deq_dispatch<E5M2, false>(q, scales, rows, cols, col, gemm_scales, out, stream);
    case MX_E2M3: return bf ? deq_dispatch<E2M3, true>(q, scales, rows, cols, col, gemm_scales, out, stream)
                            : deq_dispatch<E2M3, false>(q, scales, rows, cols, col, gemm_scales, out, stream);
    case MX_E3M2: return bf ? deq_dispatch<E3M2, true>(q, scales, rows, cols, col, gemm_scales, out, stream)
                            : deq_dispatch<E3M2, false>(q, scales, rows, cols, col, gemm_scales, out, stream);
    default: return bf ? deq_dispatch<E2M1, true>(q, scales, rows, cols, col, gemm_scales, out, stream)
                       : deq_dispatch<E2M1, false>(q, scales, rows, cols, col, gemm_scales, out, stream);
  }
}

extern "C" const char* mx_status_str(mx_status_t s) {
  switch (s) {
    case MX_OK: return "MX_OK";
    case MX_ERR_NULL: return "MX_ERR_NULL: a required pointer is NULL";
    case MX_ERR_SHAPE: return "MX_ERR_SHAPE: size not supported by the layout";
    case MX_ERR_ALIGN: return "MX_ERR_ALIGN: tensor pointer not 16-byte aligned";
    case MX_ERR_UNSUPPORTED: return "MX_ERR_UNSUPPORTED: format/rule/layout/block combination";
    case MX_ERR_LAUNCH: return "MX_ERR_LAUNCH: kernel launch failed";
    case MX_ERR_ARG: return "MX_ERR_ARG: scalar argument out of range";
  }
  return "unknown mx_status_t";
}

extern "C" int mx_abi_version(void) { return 200; }
