// MX block quantizers and the per-tensor delayed-scaling FP8 quantizer for gfx950.
//
// Method: "EU8M0 FP8" article, MX definition paragraph (blocks of k = 32 values
// sharing an E8M0 scale X with Q_i * X ~ V_i) and section 4 of the first part
// (amax -> exponent, rounding that avoids overflow, saturating element cast);
// second part, section 2 (row-wise and column-wise copies, a transposed MX copy
// re-quantized from the source).  Per-tensor path: AstrAI fp8.py page
// (quantize / quantize_dual with fused amax and the in-kernel ring fold).
//
// Kernels
//   rowwise_kernel   row-wise MX blocks.  Row-wise blocks are contiguous in
//                    memory, so the tensor is treated as a flat array: each
//                    lane owns 8 consecutive elements (one 16-byte load for
//                    2-byte inputs), a quad of lanes owns one block, and the
//                    block amax is a 2-step DPP max inside the quad.
//   tile_kernel      128 x 128 tiles through LDS: the row-wise half is done
//                    from registers right after the coalesced loads, the tile
//                    is staged in LDS in the input type, and each lane then
//                    walks 32 rows of 2 adjacent columns (conflict-free dword
//                    reads) for the column-wise half, written transposed as
//                    16-byte stores.  Used for MX dual, MX column-wise
//                    (optionally with the in-lane Hadamard transform) and the
//                    per-tensor FP8 path (row / transposed / dual) whose last
//                    workgroup folds the amax ring (atomic ticket).

#include "mx_device.hpp"
#include "mx_launch.hpp"

namespace mxk {

// ---------------------------------------------------------------------------
// Packing helpers
// ---------------------------------------------------------------------------
template <int F>
__device__ __forceinline__ void store_codes8(uint8_t* __restrict__ q, int64_t elem, const uint32_t (&c)[8]) {
  if constexpr (Fmt_<F>::kBits == 8) {
    uint2 w;
    w.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
    w.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
    *reinterpret_cast<uint2*>(q + elem) = w;
  } else {
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) w |= (c[j] & 0xFu) << (4 * j);
    *reinterpret_cast<uint32_t*>(q + elem / 2) = w;
  }
}

// 32 codes of one column segment -> 32 bytes (FP8) or 16 bytes (FP4) at dst.
template <int F>
__device__ __forceinline__ void store_codes32(uint8_t* __restrict__ dst, const uint32_t (&c)[32]) {
  if constexpr (Fmt_<F>::kBits == 8) {
    uint4 w0, w1;
    w0.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
    w0.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
    w0.z = c[8] | (c[9] << 8) | (c[10] << 16) | (c[11] << 24);
    w0.w = c[12] | (c[13] << 8) | (c[14] << 16) | (c[15] << 24);
    w1.x = c[16] | (c[17] << 8) | (c[18] << 16) | (c[19] << 24);
    w1.y = c[20] | (c[21] << 8) | (c[22] << 16) | (c[23] << 24);
    w1.z = c[24] | (c[25] << 8) | (c[26] << 16) | (c[27] << 24);
    w1.w = c[28] | (c[29] << 8) | (c[30] << 16) | (c[31] << 24);
    reinterpret_cast<uint4*>(dst)[0] = w0;
    reinterpret_cast<uint4*>(dst)[1] = w1;
  } else {
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 32; ++j) w[j / 8] |= (c[j] & 0xFu) << (4 * (j % 8));
    *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Quantize N values that form one MX block (or, for the row path, this lane's
// share of it): given the block-wide max |.| bits, produce codes and the scale.
template <int F, int R, int N>
__device__ __forceinline__ uint32_t mx_encode(const float (&v)[N], uint32_t bmax, uint32_t (&c)[N]) {
  if (bmax >= 0x7F800000u) {                       // NaN or Inf in the block
#pragma unroll
    for (int j = 0; j < N; ++j)
      c[j] = Fmt_<F>::kNan | ((__float_as_uint(v[j]) >> 31) << (Fmt_<F>::kBits - 1));
    return 0xFFu;
  }
  const int e = shared_exponent<F, R>(bmax);
  const float mul = pow2_neg(e);
#pragma unroll
  for (int j = 0; j < N; ++j) c[j] = encode_rne_sat<F>(v[j] * mul);
  return uint32_t(e + 127);
}

// ---------------------------------------------------------------------------
// Row-wise MX quantization (flat)
// ---------------------------------------------------------------------------
constexpr int kRowThreads = 256;
constexpr int kRowUnroll = 4;

template <int IN, int F, int R, bool HAD, bool AMAX>
__global__ __launch_bounds__(kRowThreads) void rowwise_kernel(const void* __restrict__ x, int64_t nchunks,
                                                               uint8_t* __restrict__ q, uint8_t* __restrict__ scales,
                                                               uint32_t* __restrict__ amax_out, uint32_t had_mask) {
  const int lane_q = threadIdx.x & 3;
  uint32_t tmax = 0;
  float v[kRowUnroll][8];
  int64_t chunk[kRowUnroll];
#pragma unroll
  for (int u = 0; u < kRowUnroll; ++u) {
    chunk[u] = (int64_t(blockIdx.x) * kRowUnroll + u) * kRowThreads + threadIdx.x;
    if (chunk[u] < nchunks) load8<IN>(x, chunk[u] * 8, v[u]);
  }
#pragma unroll
  for (int u = 0; u < kRowUnroll; ++u) {
    // nchunks is a multiple of 4 and quads are aligned, so a quad is either
    // entirely in range or entirely out of range
    if (chunk[u] >= nchunks) continue;
    if constexpr (AMAX) {
#pragma unroll
      for (int j = 0; j < 8; ++j) tmax = umax(tmax, abs_bits_no_nan(v[u][j]));
    }
    if constexpr (HAD) hadamard32_quad(v[u], had_mask, lane_q);
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = umax(m, abs_bits(v[u][j]));
    m = quad_max(m);
    uint32_t c[8];
    const uint32_t sc = mx_encode<F, R, 8>(v[u], m, c);
    store_codes8<F>(q, chunk[u] * 8, c);
    if (lane_q == 0) scales[chunk[u] >> 2] = uint8_t(sc);
  }
  if constexpr (AMAX) {
    __shared__ uint32_t red[kRowThreads / 64];
    tmax = wave_max(tmax);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = tmax;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t m = red[0];
#pragma unroll
      for (int w = 1; w < kRowThreads / 64; ++w) m = umax(m, red[w]);
      atomic_max_u32(amax_out, m);
    }
  }
}

// ---------------------------------------------------------------------------
// Tile kernel: MX dual / MX column-wise / per-tensor FP8 (row, transposed, dual)
// ---------------------------------------------------------------------------
constexpr int kTile = 128;          // rows and columns per tile
constexpr int kTileThreads = 256;
constexpr int kPasses = kTile * kTile / 8 / kTileThreads;   // 8 chunk loads per lane

enum TileMode : int {
  MX_DUAL = 0,     // MX row-wise + column-wise (transposed)
  MX_COL = 1,      // MX column-wise (transposed) only
  PT_ROW = 2,      // per-tensor FP8, row-major output
  PT_COL = 3,      // per-tensor FP8, transposed output
  PT_DUAL = 4,     // per-tensor FP8, both
};

struct TileArgs {
  const void* x;
  int64_t rows, cols;
  uint8_t* q_row;       // MX_DUAL / PT_ROW / PT_DUAL
  uint8_t* s_row;       // MX_DUAL
  uint8_t* q_col;       // transposed codes
  uint8_t* s_col;       // MX column scales
  uint32_t* amax_out;   // MX modes: max-accumulator (bit pattern of a non-negative float), may be null
  float* ring;          // PT modes
  int hist_len, hist_idx;
  float fp8_max, margin;
  float* pt_amax_out;   // PT modes: optional copy of this call's amax
  uint32_t had_mask;
  int tiles_c;          // tiles along the column axis
};

template <int IN> struct LdsWord;   // element storage in LDS
template <> struct LdsWord<IN_BF16> { using T = uint16_t; };
template <> struct LdsWord<IN_F16> { using T = uint16_t; };
template <> struct LdsWord<IN_F32> { using T = float; };

// Raw 8-element chunk as loaded from global memory: one 16-byte word for 2-byte
// types, two for FP32.
template <int IN> struct ChunkWords { static constexpr int kN = IN == IN_F32 ? 2 : 1; };

template <int IN>
__device__ __forceinline__ void load_chunk(const void* __restrict__ base, int64_t i, uint4 (&w)[ChunkWords<IN>::kN]) {
  const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(base) + i * (IN == IN_F32 ? 4 : 2));
#pragma unroll
  for (int k = 0; k < ChunkWords<IN>::kN; ++k) w[k] = p[k];
}

template <int IN>
__device__ __forceinline__ void widen_chunk(const uint4 (&c)[ChunkWords<IN>::kN], float (&v)[8]) {
  if constexpr (IN == IN_F32) {
    v[0] = __uint_as_float(c[0].x); v[1] = __uint_as_float(c[0].y);
    v[2] = __uint_as_float(c[0].z); v[3] = __uint_as_float(c[0].w);
    v[4] = __uint_as_float(c[1].x); v[5] = __uint_as_float(c[1].y);
    v[6] = __uint_as_float(c[1].z); v[7] = __uint_as_float(c[1].w);
  } else {
    const uint32_t w[4] = {c[0].x, c[0].y, c[0].z, c[0].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (IN == IN_BF16) {
        v[2 * j] = __uint_as_float(w[j] << 16);
        v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
      } else {
        v[2 * j] = f16_bits_to_f32(w[j] & 0xFFFFu);
        v[2 * j + 1] = f16_bits_to_f32(w[j] >> 16);
      }
    }
  }
}

// Two adjacent LDS elements (columns 2l, 2l+1 of one row) widened to FP32.
template <int IN>
__device__ __forceinline__ void lds_pair(const typename LdsWord<IN>::T* p, float& lo, float& hi) {
  if constexpr (IN == IN_F32) {
    const float2 d = *reinterpret_cast<const float2*>(p);
    lo = d.x;
    hi = d.y;
  } else {
    const uint32_t d = *reinterpret_cast<const uint32_t*>(p);
    if constexpr (IN == IN_BF16) {
      lo = __uint_as_float(d << 16);
      hi = __uint_as_float(d & 0xFFFF0000u);
    } else {
      lo = f16_bits_to_f32(d & 0xFFFFu);
      hi = f16_bits_to_f32(d >> 16);
    }
  }
}

template <int IN, int F, int R, int MODE, bool HAD, bool AMAX>
__global__ __launch_bounds__(kTileThreads) void tile_kernel(TileArgs a) {
  using W = typename LdsWord<IN>::T;
  constexpr bool kRowOut = MODE == MX_DUAL || MODE == PT_ROW || MODE == PT_DUAL;
  constexpr bool kColOut = MODE != PT_ROW;
  constexpr bool kPT = MODE >= PT_ROW;
  constexpr int kPad = 16 / sizeof(W);      // 16 bytes per LDS row keeps 16-byte alignment
  constexpr int kPitch = kTile + kPad;
  __shared__ W tile[kColOut ? kTile * kPitch : 1];
  __shared__ uint32_t red[kTileThreads / 64];

  const int tid = threadIdx.x;
  const int tr = blockIdx.x / a.tiles_c, tc = blockIdx.x % a.tiles_c;
  const int64_t r0 = int64_t(tr) * kTile, c0 = int64_t(tc) * kTile;
  const int lane_q = tid & 3;
  float mult = 1.0f;
  if constexpr (kPT) mult = a.ring[a.hist_len + 1];
  uint32_t tmax = 0;

  // ---- load the tile: pass p covers row p*16 + tid/16, 8 columns per lane
  const int lrow = tid >> 4, lcol = (tid & 15) * 8;
  const bool col_ok = c0 + lcol < a.cols;
  constexpr int kW = ChunkWords<IN>::kN;
  uint4 raw[kPasses][kW];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int64_t r = r0 + p * 16 + lrow;
#pragma unroll
    for (int k = 0; k < kW; ++k) raw[p][k] = make_uint4(0, 0, 0, 0);
    if (r < a.rows && col_ok) load_chunk<IN>(a.x, r * a.cols + c0 + lcol, raw[p]);
  }
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int64_t r = r0 + p * 16 + lrow;
    const bool ok = r < a.rows && col_ok;
    if constexpr (kColOut) {
      // stage the raw input (zeros outside the matrix) for the column pass
      uint4* lds = reinterpret_cast<uint4*>(&tile[(p * 16 + lrow) * kPitch + lcol]);
#pragma unroll
      for (int k = 0; k < kW; ++k) lds[k] = raw[p][k];
    }
    if (!ok) continue;
    if constexpr (AMAX || kPT || kRowOut) {
      float v[8];
      widen_chunk<IN>(raw[p], v);
      if constexpr (AMAX || kPT) {
#pragma unroll
        for (int j = 0; j < 8; ++j) tmax = umax(tmax, abs_bits_no_nan(v[j]));
      }
      if constexpr (kRowOut) {
        const int64_t e0 = r * a.cols + c0 + lcol;
        uint32_t c[8];
        if constexpr (MODE == MX_DUAL) {
          uint32_t m = 0;
#pragma unroll
          for (int j = 0; j < 8; ++j) m = umax(m, abs_bits(v[j]));
          m = quad_max(m);
          const uint32_t sc = mx_encode<F, R, 8>(v, m, c);
          if (lane_q == 0) a.s_row[e0 >> 5] = uint8_t(sc);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) c[j] = encode_rne_sat<F>(v[j] * mult);
        }
        store_codes8<F>(a.q_row, e0, c);
      }
    }
  }

  if constexpr (kColOut) {
    __syncthreads();
    // ---- column pass: wave w takes rows 32w..32w+31, lane l columns 2l, 2l+1
    const int wv = tid >> 6, ln = tid & 63;
    const int64_t rs = r0 + 32 * wv;
    const int64_t cc = c0 + 2 * ln;
    // cols is even, so columns cc and cc+1 are in range together
    if (rs < a.rows && cc < a.cols) {
      float cv[2][32];
#pragma unroll
      for (int i = 0; i < 32; ++i) lds_pair<IN>(&tile[(32 * wv + i) * kPitch + 2 * ln], cv[0][i], cv[1][i]);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t col = cc + h;
        uint32_t c[32];
        if constexpr (MODE == MX_DUAL || MODE == MX_COL) {
          if constexpr (HAD) hadamard32_inlane(cv[h], a.had_mask);
          uint32_t m = 0;
#pragma unroll
          for (int i = 0; i < 32; ++i) m = umax(m, abs_bits(cv[h][i]));
          const uint32_t sc = mx_encode<F, R, 32>(cv[h], m, c);
          a.s_col[col * (a.rows >> 5) + (rs >> 5)] = uint8_t(sc);
        } else {
#pragma unroll
          for (int i = 0; i < 32; ++i) c[i] = encode_rne_sat<F>(cv[h][i] * mult);
        }
        constexpr int kPerByte = Fmt_<F>::kBits == 8 ? 1 : 2;
        store_codes32<F>(a.q_col + (col * a.rows + rs) / kPerByte, c);
      }
    }
  }

  // ---- per-tensor amax
  if constexpr (AMAX || kPT) {
    tmax = wave_max(tmax);
    if ((tid & 63) == 0) red[tid >> 6] = tmax;
    __syncthreads();
    if (tid == 0) {
      uint32_t m = red[0];
#pragma unroll
      for (int w = 1; w < kTileThreads / 64; ++w) m = umax(m, red[w]);
      if constexpr (!kPT) {
        atomic_max_u32(a.amax_out, m);
      } else {
        // in-kernel delayed-scaling fold by the last workgroup (atomic ticket)
        uint32_t* amax_slot = reinterpret_cast<uint32_t*>(a.ring + a.hist_len + 2);
        uint32_t* ticket = reinterpret_cast<uint32_t*>(a.ring + a.hist_len + 3);
        __hip_atomic_fetch_max(amax_slot, m, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t t = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (t == gridDim.x - 1) {
          const uint32_t ab = __hip_atomic_load(amax_slot, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
          const float amax = __uint_as_float(ab);
          float* hist = a.ring;
          hist[a.hist_idx] = amax;
          float h = 0.0f;
          for (int i = 0; i < a.hist_len; ++i) h = fmaxf(h, hist[i]);
          if (h > 0.0f && h < __uint_as_float(0x7F800000u)) {
            const float s = (h / a.fp8_max) / a.margin;   // correctly rounded FP32 divisions
            a.ring[a.hist_len] = s;
            a.ring[a.hist_len + 1] = 1.0f / s;
          }
          if (a.pt_amax_out) *a.pt_amax_out = amax;
          __hip_atomic_store(amax_slot, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host-side dispatch
// ---------------------------------------------------------------------------
template <typename K, typename... Args>
static mx_status_t launch(K kernel, dim3 grid, dim3 block, hipStream_t s, Args... args) {
  hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
  return hipGetLastError() == hipSuccess ? MX_OK : MX_ERR_LAUNCH;
}

template <int IN, int F, int R>
static mx_status_t rowwise_dispatch(const void* x, int64_t n, uint8_t* q, uint8_t* s, uint32_t* amax, bool had,
                                    uint32_t mask, hipStream_t st) {
  const int64_t nchunks = n / 8;
  const int64_t per = int64_t(kRowThreads) * kRowUnroll;
  const dim3 grid{unsigned((nchunks + per - 1) / per)}, block{unsigned(kRowThreads)};
  if (had) {
    return amax ? launch(rowwise_kernel<IN, F, R, true, true>, grid, block, st, x, nchunks, q, s, amax, mask)
                : launch(rowwise_kernel<IN, F, R, true, false>, grid, block, st, x, nchunks, q, s, amax, mask);
  }
  return amax ? launch(rowwise_kernel<IN, F, R, false, true>, grid, block, st, x, nchunks, q, s, amax, mask)
              : launch(rowwise_kernel<IN, F, R, false, false>, grid, block, st, x, nchunks, q, s, amax, mask);
}

template <int IN, int F, int R, int MODE>
static mx_status_t tile_dispatch(TileArgs& a, bool had, bool amax, hipStream_t st) {
  const int64_t tr = (a.rows + kTile - 1) / kTile, tcn = (a.cols + kTile - 1) / kTile;
  a.tiles_c = int(tcn > 0 ? tcn : 1);
  int64_t nt = tr * tcn;
  if (nt == 0) nt = 1;   // per-tensor mode still folds an empty input
  const dim3 grid{unsigned(nt)}, block{unsigned(kTileThreads)};
  if constexpr (MODE == MX_COL) {
    if (had) {
      return amax ? launch(tile_kernel<IN, F, R, MODE, true, true>, grid, block, st, a)
                  : launch(tile_kernel<IN, F, R, MODE, true, false>, grid, block, st, a);
    }
  }
  return amax ? launch(tile_kernel<IN, F, R, MODE, false, true>, grid, block, st, a)
              : launch(tile_kernel<IN, F, R, MODE, false, false>, grid, block, st, a);
}

// Expand runtime (in, fmt, rule) into template instances.
template <template <int, int, int> class Op, typename... Args>
static mx_status_t expand(int in, int fmt, int rule, Args&&... args) {
#define MXK_CASE(I, F, R) \
  if (in == I && fmt == F && rule == R) return Op<I, F, R>::run(args...);
#define MXK_RULES(I, F) MXK_CASE(I, F, FLOOR) MXK_CASE(I, F, CEIL)
#define MXK_FMTS(I) MXK_RULES(I, E4M3) MXK_RULES(I, E5M2) MXK_RULES(I, E2M1)
  MXK_FMTS(IN_F32) MXK_FMTS(IN_BF16) MXK_FMTS(IN_F16)
#undef MXK_FMTS
#undef MXK_RULES
#undef MXK_CASE
  return MX_ERR_UNSUPPORTED;
}

template <int IN, int F, int R> struct RowOp {
  static mx_status_t run(const void* x, int64_t n, uint8_t* q, uint8_t* s, uint32_t* amax, bool had, uint32_t mask,
                         hipStream_t st) {
    return rowwise_dispatch<IN, F, R>(x, n, q, s, amax, had, mask, st);
  }
};
template <int IN, int F, int R> struct ColOp {
  static mx_status_t run(TileArgs& a, bool had, bool amax, hipStream_t st) {
    return tile_dispatch<IN, F, R, MX_COL>(a, had, amax, st);
  }
};
template <int IN, int F, int R> struct DualOp {
  static mx_status_t run(TileArgs& a, bool amax, hipStream_t st) {
    return tile_dispatch<IN, F, R, MX_DUAL>(a, false, amax, st);
  }
};
template <int IN, int F, int R> struct PtOp {
  static mx_status_t run(TileArgs& a, int layout, hipStream_t st) {
    if constexpr (F == E2M1 || R != FLOOR) {
      return MX_ERR_UNSUPPORTED;
    } else {
      if (layout == FP8_ROW) return tile_dispatch<IN, F, R, PT_ROW>(a, false, false, st);
      if (layout == FP8_TRANSPOSED) return tile_dispatch<IN, F, R, PT_COL>(a, false, false, st);
      return tile_dispatch<IN, F, R, PT_DUAL>(a, false, false, st);
    }
  }
};

}  // namespace mxk

using namespace mxk;

extern "C" mx_status_t mx_quantize(const void* x, mx_dtype_t in, int64_t rows, int64_t cols, int block,
                                   mx_elem_t fmt, mx_scale_rule_t rule, mx_orient_t orient, int hadamard,
                                   uint32_t hadamard_sign_mask, uint8_t* q, uint8_t* scales, float* amax_out,
                                   hipStream_t stream) {
  if (mx_status_t st = check_common_quant(in, rows, cols, block, fmt, rule); st != MX_OK) return st;
  if (orient != MX_ROWWISE && orient != MX_COLWISE_T) return MX_ERR_UNSUPPORTED;
  const int64_t n = rows * cols;
  if (n > 0 && (!x || !q || !scales)) return MX_ERR_NULL;
  if (orient == MX_ROWWISE && cols % 32 != 0) return MX_ERR_SHAPE;
  if (orient == MX_COLWISE_T && (rows % 32 != 0 || cols % 8 != 0)) return MX_ERR_SHAPE;
  if (n > 0 && (misaligned(x) || misaligned(q))) return MX_ERR_ALIGN;
  // amax_out is a max-accumulator the caller initialises; nothing to do when empty
  uint32_t* amax = reinterpret_cast<uint32_t*>(amax_out);
  if (n == 0) return MX_OK;
  if (orient == MX_ROWWISE)
    return expand<RowOp>(in, fmt, rule, x, n, q, scales, amax, hadamard != 0, hadamard_sign_mask, stream);
  TileArgs a{};
  a.x = x; a.rows = rows; a.cols = cols; a.q_col = q; a.s_col = scales; a.amax_out = amax;
  a.had_mask = hadamard_sign_mask;
  return expand<ColOp>(in, fmt, rule, a, hadamard != 0, amax != nullptr, stream);
}

extern "C" mx_status_t mx_quantize_dual(const void* x, mx_dtype_t in, int64_t rows, int64_t cols, int block,
                                        mx_elem_t fmt, mx_scale_rule_t rule, uint8_t* q_row, uint8_t* s_row,
                                        uint8_t* q_colT, uint8_t* s_colT, float* amax_out, hipStream_t stream) {
  if (mx_status_t st = check_common_quant(in, rows, cols, block, fmt, rule); st != MX_OK) return st;
  const int64_t n = rows * cols;
  if (n > 0 && (!x || !q_row || !s_row || !q_colT || !s_colT)) return MX_ERR_NULL;
  if (rows % 32 != 0 || cols % 32 != 0) return MX_ERR_SHAPE;
  if (n > 0 && (misaligned(x) || misaligned(q_row) || misaligned(q_colT))) return MX_ERR_ALIGN;
  // amax_out is a max-accumulator the caller initialises; nothing to do when empty
  uint32_t* amax = reinterpret_cast<uint32_t*>(amax_out);
  if (n == 0) return MX_OK;
  TileArgs a{};
  a.x = x; a.rows = rows; a.cols = cols; a.q_row = q_row; a.s_row = s_row; a.q_col = q_colT; a.s_col = s_colT;
  a.amax_out = amax;
  return expand<DualOp>(in, fmt, rule, a, amax != nullptr, stream);
}

extern "C" mx_status_t fp8_quantize_delayed(const void* x, mx_dtype_t in, int64_t rows, int64_t cols,
                                            mx_elem_t fmt, fp8_layout_t layout, uint8_t* q, uint8_t* qT,
                                            float* ring, int hist_len, int hist_idx, float fp8_max, float margin,
                                            float* amax_out, hipStream_t stream) {
  if (in != MX_F32 && in != MX_BF16 && in != MX_F16) return MX_ERR_UNSUPPORTED;
  if (fmt != MX_E4M3 && fmt != MX_E5M2) return MX_ERR_UNSUPPORTED;
  if (layout != FP8_ROW && layout != FP8_TRANSPOSED && layout != FP8_DUAL) return MX_ERR_UNSUPPORTED;
  if (rows < 0 || cols < 0) return MX_ERR_SHAPE;
  if (!ring) return MX_ERR_NULL;
  if (hist_len < 1 || hist_len > 4096 || hist_idx < 0 || hist_idx >= hist_len) return MX_ERR_ARG;
  if (!(fp8_max > 0.0f) || !(fp8_max < 3.4e38f) || !(margin > 0.0f) || !(margin < 3.4e38f)) return MX_ERR_ARG;
  const int64_t n = rows * cols;
  const bool need_q = layout != FP8_TRANSPOSED, need_qT = layout != FP8_ROW;
  if (n > 0 && (!x || (need_q && !q) || (need_qT && !qT))) return MX_ERR_NULL;
  if (cols % 8 != 0 || (need_qT && rows % 32 != 0)) return MX_ERR_SHAPE;
  if (n > 0 && (misaligned(x) || (need_q && misaligned(q)) || (need_qT && misaligned(qT)))) return MX_ERR_ALIGN;
  TileArgs a{};
  a.x = x; a.rows = rows; a.cols = cols; a.q_row = q; a.q_col = qT; a.ring = ring; a.hist_len = hist_len;
  a.hist_idx = hist_idx; a.fp8_max = fp8_max; a.margin = margin; a.pt_amax_out = amax_out;
  return expand<PtOp>(in, fmt, MX_SCALE_FLOOR, a, int(layout), stream);
}
