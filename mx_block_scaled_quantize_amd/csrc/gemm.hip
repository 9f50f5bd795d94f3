// Block-scaled (MX) GEMM on gfx950 scaled MFMA.
//
// "EU8M0 FP8" article, MX definition paragraph: the matrix unit consumes the
// E8M0 scale X and the element codes Q_i of both operands, with FP32
// accumulation.  gfx950's V_MFMA_SCALE_F32_32X32X64_F8F6F4 does exactly that for
// one 32 x 32 x 64 step: every lane feeds 32 consecutive K-codes of one row of A
// (or of one row of B^T) together with the E8M0 scale of those 32 codes, so an
// MX block (k = 32) maps onto one lane's operand and its scale register.
//
// Operand layouts (K-contiguous "NT"): A [M][K] codes, sa [M][K/32];
// B^T [N][K] codes, sb [N][K/32]; FP4 codes are packed two per byte.
//
// gemm_kernel: 128 x 128 output tile per workgroup, 4 waves in a 2 x 2 grid
// with a 64 x 64 sub-tile (2 x 2 MFMA tiles) each, K-steps of 128 staged in LDS
// (rows padded by 16 bytes so that the 8 lanes of a ds_read_b128 phase hit
// distinct banks), scales staged next to the codes.  Rows / K-blocks beyond
// the matrix are filled with code 0 and scale 2^0, which contribute nothing.

#include "mx_device.hpp"
#include "mx_launch.hpp"

namespace mxk {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kBM = 128, kBN = 128, kBK = 128;
constexpr int kGemmThreads = 256;

template <int FA> struct OpBytes { static constexpr int kRow = FA == E2M1 ? kBK / 2 : kBK; };

// Operand-format field of the scaled MFMA: 0 FP8 E4M3, 1 FP8 E5M2, 2 FP6 E2M3,
// 3 FP6 E3M2, 4 FP4 E2M1.
template <int F> struct MfmaFmt { static constexpr int kCode = F == E4M3 ? 0 : F == E5M2 ? 1 : 4; };

// One lane's operand for K-step kk (64 K-values) of a row staged in LDS; h = lane / 32.
//   FP4: the lane holds the 32 codes of K-block 2*kk + h (16 contiguous bytes).
//   FP8: the lane holds K = 16h .. 16h+15 of the step in bytes 0..15 and
//        K = 32 + 16h .. 32 + 16h + 15 in bytes 16..31, i.e. half of each of the
//        step's two K-blocks; the scale register of lane (row + 32 kb) still
//        carries the scale of K-block kb.
template <int F>
__device__ __forceinline__ v8i load_operand(const uint8_t* row, int kk, int h) {
  if constexpr (F == E2M1) {
    const uint4 x = *reinterpret_cast<const uint4*>(row + kk * 32 + h * 16);
    return v8i{int(x.x), int(x.y), int(x.z), int(x.w), 0, 0, 0, 0};
  } else {
    const uint4 x = *reinterpret_cast<const uint4*>(row + kk * 64 + h * 16);
    const uint4 y = *reinterpret_cast<const uint4*>(row + kk * 64 + 32 + h * 16);
    return v8i{int(x.x), int(x.y), int(x.z), int(x.w), int(y.x), int(y.y), int(y.z), int(y.w)};
  }
}

template <int FA, int FB, bool BF16OUT>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA,
                                                            const uint8_t* __restrict__ B, const uint8_t* __restrict__ SB,
                                                            int64_t M, int64_t N, int64_t K, float alpha,
                                                            void* __restrict__ C, int64_t ldc, int tiles_n) {
  constexpr int kRowA = OpBytes<FA>::kRow, kRowB = OpBytes<FB>::kRow;
  constexpr int kPitchA = kRowA + 16, kPitchB = kRowB + 16;
  __shared__ __attribute__((aligned(16))) uint8_t sA[kBM * kPitchA];
  __shared__ __attribute__((aligned(16))) uint8_t sB[kBN * kPitchB];
  __shared__ uint8_t sSA[kBM * 4];
  __shared__ uint8_t sSB[kBN * 4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = int64_t(blockIdx.x / tiles_n) * kBM;
  const int64_t n0 = int64_t(blockIdx.x % tiles_n) * kBN;
  const int64_t kbytesA = FA == E2M1 ? K / 2 : K, kbytesB = FB == E2M1 ? K / 2 : K;
  const int64_t kblocks = K / 32;

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  for (int64_t k0 = 0; k0 < K; k0 += kBK) {
    // ---- stage codes: 16-byte chunks, zero past the matrix
    constexpr int kChA = kRowA / 16, kChB = kRowB / 16;
    for (int i = tid; i < kBM * kChA; i += kGemmThreads) {
      const int r = i / kChA, ch = i % kChA;
      const int64_t gr = m0 + r;
      const int64_t kb = (FA == E2M1 ? k0 / 2 : k0) + ch * 16;
      uint4 d = make_uint4(0, 0, 0, 0);
      if (gr < M && kb < kbytesA) d = *reinterpret_cast<const uint4*>(A + gr * kbytesA + kb);
      *reinterpret_cast<uint4*>(&sA[r * kPitchA + ch * 16]) = d;
    }
    for (int i = tid; i < kBN * kChB; i += kGemmThreads) {
      const int r = i / kChB, ch = i % kChB;
      const int64_t gr = n0 + r;
      const int64_t kb = (FB == E2M1 ? k0 / 2 : k0) + ch * 16;
      uint4 d = make_uint4(0, 0, 0, 0);
      if (gr < N && kb < kbytesB) d = *reinterpret_cast<const uint4*>(B + gr * kbytesB + kb);
      *reinterpret_cast<uint4*>(&sB[r * kPitchB + ch * 16]) = d;
    }
    // ---- stage scales: 4 K-blocks per row, 2^0 (code 127) past the matrix
    for (int i = tid; i < kBM * 4; i += kGemmThreads) {
      const int r = i >> 2, kb = i & 3;
      const int64_t gr = m0 + r, gk = k0 / 32 + kb;
      sSA[i] = (gr < M && gk < kblocks) ? SA[gr * kblocks + gk] : uint8_t(127);
    }
    for (int i = tid; i < kBN * 4; i += kGemmThreads) {
      const int r = i >> 2, kb = i & 3;
      const int64_t gr = n0 + r, gk = k0 / 32 + kb;
      sSB[i] = (gr < N && gk < kblocks) ? SB[gr * kblocks + gk] : uint8_t(127);
    }
    __syncthreads();

    // ---- two MFMA K-steps of 64; lane l feeds row l%32, K-block (2*kk + l/32)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int kblk = 2 * kk + (lane >> 5);
      v8i a[2], b[2];
      int sa[2], sb[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int ra = wm * 64 + t * 32 + (lane & 31);
        const int rb = wn * 64 + t * 32 + (lane & 31);
        a[t] = load_operand<FA>(&sA[ra * kPitchA], kk, lane >> 5);
        b[t] = load_operand<FB>(&sB[rb * kPitchB], kk, lane >> 5);
        sa[t] = sSA[ra * 4 + kblk];
        sb[t] = sSB[rb * 4 + kblk];
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], MfmaFmt<FA>::kCode,
                                                                       MfmaFmt<FB>::kCode, 0, sa[i], 0, sb[j]);
    }
    __syncthreads();
  }

  // ---- epilogue: D[8*(v/4) + 4*(l/32) + v%4][l%32] of each 32 x 32 tile
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
        if (row < M && col < N) {
          const float o = alpha * acc[i][j][v];
          if constexpr (BF16OUT) {
            const uint32_t bits = __float_as_uint(o);
            const uint32_t r = (bits & 0x7FFFFFFFu) > 0x7F800000u ? ((bits >> 16) | 0x40u)
                                                                   : (bits + 0x7FFFu + ((bits >> 16) & 1u)) >> 16;
            static_cast<uint16_t*>(C)[row * ldc + col] = uint16_t(r);
          } else {
            static_cast<float*>(C)[row * ldc + col] = o;
          }
        }
      }
}

template <int FA, int FB, bool BF>
static mx_status_t gemm_dispatch(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb, int64_t M,
                                 int64_t N, int64_t K, float alpha, void* c, int64_t ldc, hipStream_t st) {
  const int64_t tm = (M + kBM - 1) / kBM, tn = (N + kBN - 1) / kBN;
  hipLaunchKernelGGL((gemm_kernel<FA, FB, BF>), dim3(unsigned(tm * tn)), dim3(kGemmThreads), 0, st, a, sa, b, sb, M,
                     N, K, alpha, c, ldc, int(tn));
  return hipGetLastError() == hipSuccess ? MX_OK : MX_ERR_LAUNCH;
}

template <bool BF>
static mx_status_t gemm_formats(int fa, int fb, const uint8_t* a, const uint8_t* sa, const uint8_t* b,
                                const uint8_t* sb, int64_t M, int64_t N, int64_t K, float alpha, void* c, int64_t ldc,
                                hipStream_t st) {
  if (fa == E4M3 && fb == E4M3) return gemm_dispatch<E4M3, E4M3, BF>(a, sa, b, sb, M, N, K, alpha, c, ldc, st);
  if (fa == E4M3 && fb == E5M2) return gemm_dispatch<E4M3, E5M2, BF>(a, sa, b, sb, M, N, K, alpha, c, ldc, st);
  if (fa == E5M2 && fb == E4M3) return gemm_dispatch<E5M2, E4M3, BF>(a, sa, b, sb, M, N, K, alpha, c, ldc, st);
  if (fa == E5M2 && fb == E5M2) return gemm_dispatch<E5M2, E5M2, BF>(a, sa, b, sb, M, N, K, alpha, c, ldc, st);
  if (fa == E2M1 && fb == E2M1) return gemm_dispatch<E2M1, E2M1, BF>(a, sa, b, sb, M, N, K, alpha, c, ldc, st);
  return MX_ERR_UNSUPPORTED;
}

}  // namespace mxk

using namespace mxk;

extern "C" mx_status_t mx_gemm(const uint8_t* a, const uint8_t* sa, mx_elem_t fmt_a, const uint8_t* b,
                               const uint8_t* sb, mx_elem_t fmt_b, int64_t M, int64_t N, int64_t K, float alpha,
                               void* c, mx_dtype_t c_dtype, int64_t ldc, hipStream_t stream) {
  const bool f8a = fmt_a == MX_E4M3 || fmt_a == MX_E5M2, f8b = fmt_b == MX_E4M3 || fmt_b == MX_E5M2;
  if (!((f8a && f8b) || (fmt_a == MX_E2M1 && fmt_b == MX_E2M1))) return MX_ERR_UNSUPPORTED;
  if (c_dtype != MX_BF16 && c_dtype != MX_F32) return MX_ERR_UNSUPPORTED;
  if (M < 0 || N < 0 || K < 0 || K % 32 != 0) return MX_ERR_SHAPE;
  if (M > (int64_t(1) << 31) || N > (int64_t(1) << 31) || K > (int64_t(1) << 31)) return MX_ERR_SHAPE;
  if (ldc < N) return MX_ERR_SHAPE;
  if (M == 0 || N == 0) return MX_OK;
  if (!c || (K > 0 && (!a || !sa || !b || !sb))) return MX_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(c) & (c_dtype == MX_BF16 ? 1u : 3u)) != 0) return MX_ERR_ALIGN;
  if (K > 0 && (misaligned(a) || misaligned(b))) return MX_ERR_ALIGN;
  return c_dtype == MX_BF16 ? gemm_formats<true>(fmt_a, fmt_b, a, sa, b, sb, M, N, K, alpha, c, ldc, stream)
                            : gemm_formats<false>(fmt_a, fmt_b, a, sa, b, sb, M, N, K, alpha, c, ldc, stream);
}
