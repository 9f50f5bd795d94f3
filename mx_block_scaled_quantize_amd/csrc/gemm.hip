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
// B^T [N][K] codes, sb [N][K/32]; FP4 codes are packed two per byte, FP6 codes
// as a little-endian 6-bit stream along the row (24 bytes per block).
//
// The same kernels serve the per-tensor FP8 GEMM of the AstrAI fp8.py page
// (mm_fp8: C = op(a) op(b) * scale + bias, BF16 out): every block scale is
// 2^0, the device-resident scale and the BF16 bias are applied in the FP32
// epilogue, the batch index is the grid's y, and an operand stored with M (or
// N) contiguous is handled in the kernel (no transposed copy).
//
// gemm_kernel: 128 x 128 output tile per workgroup, 4 waves in a 2 x 2 grid
// with a 64 x 64 sub-tile (2 x 2 MFMA tiles) each, K-steps of 128 (256 for
// FP6 x FP6) staged in LDS (rows padded by 16 bytes so that the 8 lanes of a
// ds_read_b128 phase hit distinct banks), scales staged next to the codes.  Rows / K-blocks beyond
// the matrix are filled with code 0 and scale 2^0, which contribute nothing.
// The next K-step's codes and scales are loaded into registers right after a
// step is staged, so the loads run under that step's MFMAs.  This kernel serves
// every shape the 256 x 256 kernel below does not take (for FP6 x FP6: K not a
// multiple of 512).

#include "mx_device.hpp"
#include "mx_launch.hpp"

#include <utility>

namespace mxk {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kBM = 128, kBN = 128, kBK = 128;
constexpr int kGemmThreads = 256;

// Code bytes of k elements: FP4 two per byte, FP6 four per three bytes.
template <int F> constexpr bool kIsFp6 = F == E2M3 || F == E3M2;
template <int F>
__host__ __device__ constexpr int64_t code_bytes(int64_t k) {
  return F == E2M1 ? k / 2 : kIsFp6<F> ? k / 4 * 3 : k;
}

// Arguments of both GEMM kernels.  C[p] = alpha op(A[p]) op(B[p])^T where A is
// [M][K] and B is [N][K] as the MFMA consumes them.  An operand is stored either
// K-contiguous ([M][lda] / [N][ldb] bytes) or, per-tensor FP8 only, M- / N-
// contiguous ([K][lda] / [K][ldb]).  Batch strides are in bytes for A and B (0
// broadcasts one matrix) and in elements for C.
struct GemmArgs {
  const uint8_t* a;
  const uint8_t* sa;            // MX scales of A [M][K/32] (unused per-tensor)
  const uint8_t* b;
  const uint8_t* sb;
  void* c;
  const float* alpha_ptr;       // per-tensor: the device-resident combined scale
  const uint16_t* bias;         // per-tensor: BF16 [N] or null
  int64_t M, N, K;
  int64_t lda, ldb, ldc;
  int64_t batch_a, batch_b, batch_c;
  float alpha;                  // MX: the host scalar
  int tiles_m, tiles_n;
  // MX re-quantization of the FP32 result (row-wise, k = 32): codes [M][N] (E2M1
  // packed [M][N/2]), E8M0 scales [M][N/32], optional max-accumulator
  uint8_t* qc;
  uint8_t* sc;
  uint32_t* amax;
  int fc, rc;                   // element format and scale rule of the re-quantization
  bool gemm_scales;             // sa / sb in the GEMM scale layout ([K/512][rows][16]) instead of row-major
};

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Operand-format field of the scaled MFMA: 0 FP8 E4M3, 1 FP8 E5M2, 2 FP6 E2M3,
// 3 FP6 E3M2, 4 FP4 E2M1.
template <int F> struct MfmaFmt {
  static constexpr int kCode = F == E4M3 ? 0 : F == E5M2 ? 1 : F == E2M3 ? 2 : F == E3M2 ? 3 : 4;
};

// One lane's operand for K-step kk (64 K-values) of a row staged in LDS; h = lane / 32.
//   FP4: the lane holds the 32 codes of K-block 2*kk + h (16 contiguous bytes).
//   FP6: likewise, the 24 bytes of K-block 2*kk + h (its codes as a little-endian
//        bit stream, element i at bits 6i .. 6i+5) in dwords 0..5.
//   FP8: the lane holds K = 16h .. 16h+15 of the step in bytes 0..15 and
//        K = 32 + 16h .. 32 + 16h + 15 in bytes 16..31, i.e. half of each of the
//        step's two K-blocks; the scale register of lane (row + 32 kb) still
//        carries the scale of K-block kb.
template <int F>
__device__ __forceinline__ v8i load_operand(const uint8_t* row, int kk, int h) {
  if constexpr (F == E2M1) {
    const uint4 x = *reinterpret_cast<const uint4*>(row + kk * 32 + h * 16);
    return v8i{int(x.x), int(x.y), int(x.z), int(x.w), 0, 0, 0, 0};
  } else if constexpr (kIsFp6<F>) {
    const uint2* p = reinterpret_cast<const uint2*>(row + kk * 48 + h * 24);
    const uint2 x = p[0], y = p[1], z = p[2];
    return v8i{int(x.x), int(x.y), int(y.x), int(y.y), int(z.x), int(z.y), 0, 0};
  } else {
    const uint4 x = *reinterpret_cast<const uint4*>(row + kk * 64 + h * 16);
    const uint4 y = *reinterpret_cast<const uint4*>(row + kk * 64 + 32 + h * 16);
    return v8i{int(x.x), int(x.y), int(x.z), int(x.w), int(y.x), int(y.y), int(y.z), int(y.w)};
  }
}

// Row-wise MX encoding of one 32-value block of the FP32 result, then its stores:
// 32 (FP8) or 16 (E2M1) code bytes at qrow, the scale byte at *srow.
template <int FC, int RC>
__device__ __forceinline__ void requant_block32(const float (&v)[32], uint8_t* __restrict__ qrow,
                                                uint8_t* __restrict__ srow) {
  uint32_t bmax = 0;
#pragma unroll
  for (int k = 0; k < 32; ++k) bmax = umax(bmax, abs_bits(v[k]));
  uint32_t w[Words<FC, 32>::kN];
  *srow = uint8_t(mx_encode_f32<FC, RC, 32>(v, bmax, w));
#pragma unroll
  for (int k = 0; k < Words<FC, 32>::kN / 4; ++k)
    reinterpret_cast<uint4*>(qrow)[k] = make_uint4(w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]);
}

template <int FA, int FB, bool BF16OUT, bool PT, bool TA, bool TB, bool RQ = false>
__global__ __launch_bounds__(kGemmThreads)
__attribute__((amdgpu_waves_per_eu((kIsFp6<FA> && kIsFp6<FB>) ? 2 : 1))) void gemm_kernel(const GemmArgs g) {
  // FP6 x FP6 takes K-steps of 256 (four MFMA steps per pair of barriers; a
  // 128-step stages only 96 bytes per row); every other pair 128
  constexpr int kStep = (kIsFp6<FA> && kIsFp6<FB>) ? 2 * kBK : kBK;
  constexpr int kSB = kStep / 32;                                   // scales per row and step
  constexpr int kRowA = int(code_bytes<FA>(kStep)), kRowB = int(code_bytes<FB>(kStep));
  constexpr int kPitchA = kRowA + 16, kPitchB = kRowB + 16;
  static_assert(!(TA || TB) || (PT && FA != E2M1 && FB != E2M1), "M/N-contiguous operands: per-tensor FP8 only");
  __shared__ __attribute__((aligned(16))) uint8_t sA[kBM * kPitchA];
  __shared__ __attribute__((aligned(16))) uint8_t sB[kBN * kPitchB];
  __shared__ uint8_t sSA[kBM * kSB];
  __shared__ uint8_t sSB[kBN * kSB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = int64_t(blockIdx.x / g.tiles_n) * kBM;
  const int64_t n0 = int64_t(blockIdx.x % g.tiles_n) * kBN;
  const int64_t M = g.M, N = g.N, K = g.K;
  const uint8_t* __restrict__ A = g.a + int64_t(blockIdx.y) * g.batch_a;
  const uint8_t* __restrict__ B = g.b + int64_t(blockIdx.y) * g.batch_b;
  const uint8_t* __restrict__ SA = g.sa;
  const uint8_t* __restrict__ SB = g.sb;
  const int64_t kbytesA = code_bytes<FA>(K), kbytesB = code_bytes<FB>(K);
  const int64_t kblocks = K / 32;

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // K-contiguous operands (the MX GEMM and per-tensor NT): the next K-step's
  // codes and scales are loaded into registers while the current step's MFMAs
  // run, then written to LDS between the two barriers
  constexpr int kChA = kRowA / 16, kChB = kRowB / 16;
  constexpr int kNA = (kBM * kChA + kGemmThreads - 1) / kGemmThreads;
  constexpr int kNB = (kBN * kChB + kGemmThreads - 1) / kGemmThreads;
  constexpr int kNS = (kBM * kSB + kGemmThreads - 1) / kGemmThreads;
  uint4 ra[kNA], rb[kNB];
  uint8_t rsa[kNS], rsb[kNS];
  auto fetch = [&](int64_t k0) {
    if constexpr (!TA) {
#pragma unroll
      for (int u = 0; u < kNA; ++u) {
        const int i = tid + u * kGemmThreads, r = i / kChA, ch = i % kChA;
        const int64_t gr = m0 + r, kb = code_bytes<FA>(k0) + ch * 16;
        ra[u] = make_uint4(0, 0, 0, 0);
        if (i < kBM * kChA && gr < M && kb < kbytesA) ra[u] = *reinterpret_cast<const uint4*>(A + gr * g.lda + kb);
      }
    }
    if constexpr (!TB) {
#pragma unroll
      for (int u = 0; u < kNB; ++u) {
        const int i = tid + u * kGemmThreads, r = i / kChB, ch = i % kChB;
        const int64_t gr = n0 + r, kb = code_bytes<FB>(k0) + ch * 16;
        rb[u] = make_uint4(0, 0, 0, 0);
        if (i < kBN * kChB && gr < N && kb < kbytesB) rb[u] = *reinterpret_cast<const uint4*>(B + gr * g.ldb + kb);
      }
    }
    if constexpr (!PT) {
#pragma unroll
      for (int u = 0; u < kNS; ++u) {
        const int i = tid + u * kGemmThreads, r = i / kSB, kb = i % kSB;
        const int64_t gk = k0 / 32 + kb;
        rsa[u] = (m0 + r < M && gk < kblocks) ? SA[scale_offset(m0 + r, gk, M, kblocks, g.gemm_scales)] : uint8_t(127);
        rsb[u] = (n0 + r < N && gk < kblocks) ? SB[scale_offset(n0 + r, gk, N, kblocks, g.gemm_scales)] : uint8_t(127);
      }
    }
  };
  if (K > 0) fetch(0);

  for (int64_t k0 = 0; k0 < K; k0 += kStep) {
    // ---- stage codes: the prefetched 16-byte chunks (zero past the matrix:
    // K-contiguous rows are whole 16-byte chunks, K being a multiple of 16); an
    // M- / N-contiguous operand is gathered byte by byte, consecutive lanes on
    // consecutive rows of the tile
    if constexpr (TA) {
      for (int i = tid; i < kBM * kStep; i += kGemmThreads) {
        const int r = i % kBM, kk = i / kBM;
        const int64_t gr = m0 + r, gk = k0 + kk;
        sA[r * kPitchA + kk] = (gr < M && gk < K) ? A[gk * g.lda + gr] : uint8_t(0);
      }
    } else {
#pragma unroll
      for (int u = 0; u < kNA; ++u) {
        const int i = tid + u * kGemmThreads;
        if (i < kBM * kChA) *reinterpret_cast<uint4*>(&sA[(i / kChA) * kPitchA + (i % kChA) * 16]) = ra[u];
      }
    }
    if constexpr (TB) {
      for (int i = tid; i < kBN * kStep; i += kGemmThreads) {
        const int r = i % kBN, kk = i / kBN;
        const int64_t gr = n0 + r, gk = k0 + kk;
        sB[r * kPitchB + kk] = (gr < N && gk < K) ? B[gk * g.ldb + gr] : uint8_t(0);
      }
    } else {
#pragma unroll
      for (int u = 0; u < kNB; ++u) {
        const int i = tid + u * kGemmThreads;
        if (i < kBN * kChB) *reinterpret_cast<uint4*>(&sB[(i / kChB) * kPitchB + (i % kChB) * 16]) = rb[u];
      }
    }
    // ---- scales: kSB K-blocks per row, 2^0 (code 127) past the matrix
    if constexpr (!PT) {
#pragma unroll
      for (int u = 0; u < kNS; ++u) {
        const int i = tid + u * kGemmThreads;
        if (i < kBM * kSB) {
          sSA[i] = rsa[u];
          sSB[i] = rsb[u];
        }
      }
    }
    __syncthreads();
    if (k0 + kStep < K) fetch(k0 + kStep);

    // ---- MFMA K-steps of 64; lane l feeds row l%32, K-block (2*kk + l/32)
#pragma unroll
    for (int kk = 0; kk < kStep / 64; ++kk) {
      const int kblk = 2 * kk + (lane >> 5);
      v8i a[2], b[2];
      int sa[2], sb[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int ra = wm * 64 + t * 32 + (lane & 31);
        const int rb = wn * 64 + t * 32 + (lane & 31);
        a[t] = load_operand<FA>(&sA[ra * kPitchA], kk, lane >> 5);
        b[t] = load_operand<FB>(&sB[rb * kPitchB], kk, lane >> 5);
        sa[t] = PT ? 127 : sSA[ra * kSB + kblk];
        sb[t] = PT ? 127 : sSB[rb * kSB + kblk];
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
  const float alpha = PT ? *g.alpha_ptr : g.alpha;
  if constexpr (RQ) {
    // MX re-quantization: the FP32 tile passes through LDS in two halves of 64 rows
    // (the two wave rows), then each thread encodes one 32-column block of a row
    __shared__ float sC[64][kBN + 1];
    uint32_t tmax = 0;
    const int lr = tid >> 2, blk = tid & 3;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      __syncthreads();
      if (wm == half) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v)
              sC[i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3)][wn * 64 + j * 32 + (lane & 31)] = alpha * acc[i][j][v];
      }
      __syncthreads();
      const int64_t row = m0 + 64 * half + lr, col = n0 + 32 * blk;
      if (row < M && col < N) {
        float v[32];
#pragma unroll
        for (int k = 0; k < 32; ++k) {
          v[k] = sC[lr][32 * blk + k];
          tmax = umax(tmax, abs_bits_no_nan(v[k]));
        }
        const int64_t nb = N / 32;
        uint8_t* srow = g.sc + row * nb + col / 32;
        const int bits = g.fc == E2M1 ? 4 : 8;
        uint8_t* qrow = g.qc + (row * N + col) * bits / 8;
        const int sel = g.fc * 2 + g.rc;
        if (sel == E4M3 * 2 + FLOOR) requant_block32<E4M3, FLOOR>(v, qrow, srow);
        else if (sel == E4M3 * 2 + CEIL) requant_block32<E4M3, CEIL>(v, qrow, srow);
        else if (sel == E5M2 * 2 + FLOOR) requant_block32<E5M2, FLOOR>(v, qrow, srow);
        else if (sel == E5M2 * 2 + CEIL) requant_block32<E5M2, CEIL>(v, qrow, srow);
        else if (sel == E2M1 * 2 + FLOOR) requant_block32<E2M1, FLOOR>(v, qrow, srow);
        else requant_block32<E2M1, CEIL>(v, qrow, srow);
      }
    }
    if (g.amax) {
      const uint32_t m = wave_max(tmax);
      if (lane == 0 && m) atomic_max_u32(g.amax, m);
    }
    return;
  }
  const int64_t ldc = g.ldc;
  void* __restrict__ C = static_cast<uint8_t*>(g.c) + int64_t(blockIdx.y) * g.batch_c * (BF16OUT ? 2 : 4);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
        if (row < M && col < N) {
          float o = alpha * acc[i][j][v];
          if (PT && g.bias) o = __builtin_fmaf(alpha, acc[i][j][v], bf16_to_f32(g.bias[col]));
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

// ---------------------------------------------------------------------------
// gemm256_kernel: the large-shape path (K a multiple of 512, or of 128 per-tensor; any M, N, a partial last
// tile row / column reading zeros past the matrix and storing only inside it).
//
// One workgroup of 8 waves (two per SIMD) owns a 256 x 256 output tile; each
// wave owns a 128 x 64 eighth held as 4 x 2 MFMA accumulators (128 FP32 per
// lane), which leaves each wave half of the SIMD's registers.  K advances in
// stages of 64 code bytes per row (two K-blocks of FP8, four of FP4, i.e. one or
// two 32 x 32 x 64 MFMA steps).  An FP6 stage is one MFMA step (two 24-byte
// K-blocks) in a 64-byte slot: a stage pair is 96 bytes of the row, which the DMA
// lanes place in 6 of the row's 8 LDS chunks (the lanes of the other two load
// nothing and write zeros).  Stages go straight from memory into LDS with
// gfx950's LDS-DMA loads (no register staging), four deep: a stage's loads are
// issued three stages before it is consumed.  The LDS-DMA rate of a CU grows
// with the number of waves issuing (measured on L2-resident data: about 84 GB/s
// with 4 waves, 128 GB/s with 8), and the second wave of a SIMD keeps the matrix
// unit busy while the first waits, which is why the tile is split 8 ways rather
// than 4 (bit-identical results, 4-6% faster on every path).
//
// Every buffer the loop reads is its own __shared__ object, written only by
// LDS-DMA, and the loop is unrolled so that each access names its object
// statically: the compiler can then tell which in-flight DMA an LDS read may
// alias and waits for that one alone instead of draining every load.
//
// Codes: stages 2m and 2m + 1 share one __shared__ object (a stage pair), so
// that one DMA instruction fetches 8 whole 128-byte lines (a K-contiguous row of
// the pair holds stage 2m in its first 64 bytes and stage 2m + 1 in the second).
// 16-byte chunk c (0..7) of row r sits at position c ^ swz(r), so the lanes of
// one ds_read_b128 phase hit distinct banks; the DMA side applies the
// permutation by choosing which global chunk each lane fetches.
//
// Scales: a scale stage is 16 K-blocks = one 16-byte group per row, fetched by
// 16-byte LDS-DMA (64 rows per instruction) into [row][16 bytes]; two scale
// stages are resident.  (4-byte loads of one word per row cost the address
// unit as many cache-line lookups as all the code loads together.)
//
// The MFMA is fed with B as its first operand: the accumulator then holds
// C^T fragments, i.e. each lane owns 4 consecutive columns of one row of C,
// which makes the epilogue's stores 8 (BF16) or 16 (FP32) bytes wide.
//
// An M- (or N-) contiguous FP8 operand keeps its storage order in LDS: a stage
// is 64 K-rows of the tile's 256 columns (256 bytes each), 16-byte chunk c of
// K-row k at position c ^ 2 (k % 8).  gfx950's ds_read_b64_tr_b8 turns it into
// MFMA operands: within each group of 16 lanes, output lane i gets byte i % 8
// of the 8 bytes addressed by lanes 2 b + i / 8 (b = 0..7), so lanes pointing
// at K-row k0 + j / 2, columns m0 + 8 (j % 2) deliver column m0 + i, K-rows
// k0 .. k0 + 7 to lane i -- one quarter of an FP8 operand.  With the XOR every
// 32-lane half of such a read touches 16 distinct 16-byte bank groups.  Per-
// tensor mode issues no scale loads and feeds every MFMA the scale 2^0.
// ---------------------------------------------------------------------------

namespace t256 {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));

constexpr int kTile = 256, kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kRow = 64;                      // code bytes per tile row per stage
constexpr int kStages = 4;
constexpr int kOpBytes = kTile * kRow;        // one operand of one stage: 16 KiB
constexpr int kPairOp = 2 * kOpBytes;         // one operand of a stage pair: 32 KiB
constexpr int kPairRow = 2 * kRow;            // K-contiguous row of a stage pair: one 128-byte line
constexpr int kPairLoads = kPairOp / 1024 / kWaves;   // 1 KiB DMA instructions per wave per operand per pair
constexpr int kCodeGroup = kPairLoads;        // vector-memory instructions per wave per stage (both operands)
constexpr int kKbPerScale = 16;               // K-blocks per scale stage
constexpr int kMxK = 512;                     // K granule with MX scales: whole scale stages (16 K-blocks)
constexpr int kPtK = 128;                     // K granule of the per-tensor mode: whole stage pairs
constexpr int kMnPitch = kTile;               // M/N-contiguous stage: bytes per K-row
constexpr int kEpBytes = 16384;               // a wave's epilogue staging area inside the stage buffers

__shared__ __attribute__((aligned(1024))) uint8_t g_pair0[2 * kPairOp];   // stages 4n, 4n + 1: [A | B]
__shared__ __attribute__((aligned(1024))) uint8_t g_pair1[2 * kPairOp];   // stages 4n + 2, 4n + 3
__shared__ __attribute__((aligned(1024))) uint32_t g_scale0[2][kTile][4];   // [A/B][row][word]
__shared__ __attribute__((aligned(1024))) uint32_t g_scale1[2][kTile][4];

// The object holding stage buffer I (0..3): stage pair I / 2; stage I is its half I % 2.
template <int I>
__device__ __forceinline__ uint8_t* stage() {
  static_assert(I >= 0 && I < kStages, "four stage buffers in two pairs");
  if constexpr (I / 2 == 0) return g_pair0;
  else return g_pair1;
}

template <int I>
__device__ __forceinline__ uint32_t (*scales())[kTile][4] {
  static_assert(I == 0 || I == 1, "two scale buffers");
  if constexpr (I == 0) return g_scale0;
  else return g_scale1;
}

template <bool FP4>
struct Geo {
  static constexpr int kSub = FP4 ? 2 : 1;           // MFMA steps per stage
  static constexpr int kKb = FP4 ? 4 : 2;            // K-blocks per stage
  static constexpr int kPerScale = kKbPerScale / kKb;  // stages per scale stage (8 or 4)
  static constexpr int kUnroll = 2 * kPerScale;      // stages per unrolled loop body
};

// Chunk permutation of a 128-byte row r (measured on gfx950: rows read as row = lane % 32,
// chunk = lane / 32 (^ a uniform XOR) make ds_read_b128 conflict-free with this choice,
// i.e. four active LDS cycles per instruction, the 256 B/clock peak).
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// s_waitcnt vmcnt(vm) expcnt(7) lgkmcnt(0) (gfx9 encoding)
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | ((VM >> 4) << 14));
}

// Workgroup barrier that nothing is scheduled across (MFMAs have no memory
// dependence and would otherwise drift past it).
__device__ __forceinline__ void barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Raw buffer resource over [base, base + bytes): loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}

// Cache policy of the operand loads: SC0 (measured ~7% faster than the default here;
// SC1 2-3% slower, SC0 + SC1 the same as SC0, NT 3-25% slower: the lines are re-read
// by the other tiles of their row or column and must stay in L2)
constexpr int kPolicySc0 = 1;

// LDS-DMA: lane i's 16 bytes at rsrc + voff + soff land at lds_dst + 16 i
// (lds_dst wave-uniform).  soff is uniform and lives in an SGPR.
__device__ __forceinline__ void dma(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff, void* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds_dst, 16, voff, soff, 0,
                                           kPolicySc0);
}

// Workgroups are dealt to the 8 XCDs round-robin; give every XCD a contiguous
// run of the tile order, and walk tiles in groups of 4 tile-rows so that the
// tiles running together on one XCD (4 x 8 of them) share their A and B panels
// in its L2 (groups of 4 measured 1% faster than 8, groups of 16 3% slower).
__device__ __forceinline__ void map_tile(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int ntiles = tiles_m * tiles_n;
  int idx = bid;
  if ((ntiles & 7) == 0) idx = (bid & 7) * (ntiles >> 3) + (bid >> 3);
  constexpr int kGroupM = 4;
  const int group = idx / (kGroupM * tiles_n);
  const int first = group * kGroupM;
  const int gm = min(tiles_m - first, kGroupM);
  const int in = idx - group * kGroupM * tiles_n;
  tm = first + in % gm;
  tn = in / gm;
}


struct Ctx {
  __amdgpu_buffer_rsrc_t a, b;     // the tile's code rows (K-contiguous) or columns (M/N-contiguous) of A / B
  __amdgpu_buffer_rsrc_t sa, sb;   // the tile's 256 scale rows of A / B
  __amdgpu_buffer_rsrc_t ss;       // this wave's scale operand (A for waves 0..3, B for 4..7)
  __amdgpu_buffer_rsrc_t z;        // empty range: loads return 0 and touch no memory (any base will do)
  uint32_t off_a[2];               // lane's byte offset in the tile: K-contiguous, for DMA instructions of
                                   // parity j % 2; M/N-contiguous, for instruction jj of a stage
  uint32_t off_b[2];               // same for B
  uint32_t js_a, js_b;             // K-contiguous: bytes between the rows of DMA instructions j and j + 1
  uint32_t step_a, step_b;         // bytes between consecutive stages (M/N-contiguous operands)
  uint32_t sc_off;                 // lane's byte offset of its scale row (row 64 wave + lane)
  uint32_t sc_step_a, sc_step_b;   // bytes between consecutive scale stages of a row
  uint32_t sc_step;                // the same for this wave's scale operand
  int rd_a, rd_b;                  // lane's read base inside a stage object (row-tile 0)
  int c0, c1;                      // lane's swizzled chunk offsets: chunk h and chunk h + 2
  int tp_a, tp_b;                  // M/N-contiguous: lane's swizzled chunk byte offset (row-tile 0)
  int sc_row_a, sc_row_b;          // lane's scale row (row-tile 0)
  int h8;                          // 8 * (lane / 32): the second K-block of an MFMA step is one byte up
  uint32_t kstep;                  // K-contiguous: global bytes per stage (64; FP6 48)
  int f6[2];                       // FP6: lane's 16-byte and 8-byte pieces in a stage-pair row (stage half 0)
};

// Stage pair (t, t + 1) (t even) into stage buffers SA_, SB_ (= SA_ + 1): for each
// operand 4 instructions per wave, each 1 KiB.  K-contiguous: 8 rows x one 128-byte
// line holding both stages (FP6: the pair's 96 bytes of each row, whose stage
// halves take 48 of their 64 bytes).  M/N-contiguous: 4 K-rows x 256 bytes, instructions
// 0, 1 for stage t, 2, 3 for stage t + 1.  A dead stage (past the end of K) issues
// the same loads on the empty resource (zeros, no memory traffic), which keeps the
// vmcnt bookkeeping uniform and the loop free of branches.
template <int SA_, int SB_, bool TA, bool TB>
__device__ __forceinline__ void issue_pair(const Ctx& c, int t, int wave, bool live0, bool live1) {
  static_assert(SA_ % 2 == 0 && SB_ == SA_ + 1, "a pair starts at an even stage");
  uint8_t* dst = stage<SA_>();
#pragma unroll
  for (int j = 0; j < kPairLoads; ++j) {
    const int e = j / 2, jj = j % 2;   // M/N-contiguous: stage t + e, instruction jj of that stage
    const bool live = e == 0 ? live0 : live1;
    if constexpr (TA)
      dma(live ? c.a : c.z, c.off_a[jj], uint32_t(t + e) * c.step_a, dst + e * kOpBytes + (wave * 2 + jj) * 1024);
    else
      dma(live0 ? c.a : c.z, c.off_a[jj], uint32_t(t) * c.kstep + uint32_t(j) * c.js_a,
          dst + (wave * kPairLoads + j) * 1024);
    if constexpr (TB)
      dma(live ? c.b : c.z, c.off_b[jj], uint32_t(t + e) * c.step_b,
          dst + kPairOp + e * kOpBytes + (wave * 2 + jj) * 1024);
    else
      dma(live0 ? c.b : c.z, c.off_b[jj], uint32_t(t) * c.kstep + uint32_t(j) * c.js_b,
          dst + kPairOp + (wave * kPairLoads + j) * 1024);
  }
}

// Scale stage u (K-blocks 16 u .. 16 u + 15): one instruction per wave, waves 0..3
// fetching rows 64 (wave % 4) .. + 63 of A, waves 4..7 the same rows of B.
constexpr int kScaleOps = 1;
template <int U>
__device__ __forceinline__ void issue_scales(const Ctx& c, int u, int wave, bool live) {
  dma(live ? c.ss : c.z, c.sc_off, uint32_t(u) * c.sc_step, &scales<U>()[wave >> 2][64 * (wave & 3)][0]);
}

typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i lds_v2i;

// FP8 operand from an M/N-contiguous stage: p is the lane's transpose-read address
// for K-rows 16 h .. 16 h + 7; the other quarters sit 8, 32 and 40 K-rows down.
__device__ __forceinline__ v8i mn_operand(const uint8_t* p) {
  uint8_t* q = const_cast<uint8_t*>(p);
  const v2i x0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(q));
  const v2i x1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(q + 8 * kMnPitch));
  const v2i x2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(q + 32 * kMnPitch));
  const v2i x3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(q + 40 * kMnPitch));
  return v8i{x0[0], x0[1], x1[0], x1[1], x2[0], x2[1], x3[0], x3[1]};
}

// Operand kinds of the K-contiguous stages: FP8, FP4, FP6
constexpr int kOkFp8 = 0, kOkFp4 = 1, kOkFp6 = 2;
template <int F> constexpr int kOperandKind = F == E2M1 ? kOkFp4 : kIsFp6<F> ? kOkFp6 : kOkFp8;

// Operand from a K-contiguous stage-pair row p (the lane's row start); HALF is the
// stage's half of the row (chunks 4 HALF .. 4 HALF + 3, before the permutation).
template <int OK, int KK, int HALF>
__device__ __forceinline__ v8i km_operand(const Ctx& c, const uint8_t* p) {
  if constexpr (OK == kOkFp6) {
    // the 24 bytes of K-block h: h = 0, chunk 0 then the low half of chunk 1; h = 1, the
    // high half of chunk 1 then chunk 2 -- one 16-byte and one 8-byte read, put in order
    const uint4 q = *reinterpret_cast<const uint4*>(p + (c.f6[0] ^ (64 * HALF)));
    const uint2 d = *reinterpret_cast<const uint2*>(p + (c.f6[1] ^ (64 * HALF)));
    return c.h8 ? v8i{int(d.x), int(d.y), int(q.x), int(q.y), int(q.z), int(q.w), 0, 0}
                : v8i{int(q.x), int(q.y), int(q.z), int(q.w), int(d.x), int(d.y), 0, 0};
  } else if constexpr (OK == kOkFp4) {   // the 32 codes of K-block 2 kk + h: chunk 2 kk + h
    const int ch = (KK == 0 ? c.c0 : c.c1) ^ (64 * HALF);
    const uint4 x = *reinterpret_cast<const uint4*>(p + ch);
    return v8i{int(x.x), int(x.y), int(x.z), int(x.w), 0, 0, 0, 0};
  } else {               // FP8: K = 16 h + [0, 16) and 32 + 16 h + [0, 16): chunks h and h + 2
    const uint4 x0 = *reinterpret_cast<const uint4*>(p + (c.c0 ^ (64 * HALF)));
    const uint4 x1 = *reinterpret_cast<const uint4*>(p + (c.c1 ^ (64 * HALF)));
    return v8i{int(x0.x), int(x0.y), int(x0.z), int(x0.w), int(x1.x), int(x1.y), int(x1.z), int(x1.w)};
  }
}

// Operands of MFMA step kk of stage t (stage buffer SI, scale buffer U).  With
// FRESH false the step's scale words are those of the step before (one word
// holds 4 K-blocks: two FP8 stages, or both MFMA steps of an FP4 stage) and are
// left to the caller to carry over.
template <int OK, int SI, int U, int KK, bool PT, bool TA, bool TB, bool FRESH = true>
__device__ __forceinline__ void read_step(const Ctx& c, int t, int lane, v8i (&a)[4], v8i (&b)[2], int (&sa)[4],
                                          int (&sb)[2]) {
  using G = Geo<OK == kOkFp4>;
  constexpr int kHalf = SI % 2;   // stage SI is this half of its pair
  const uint8_t* base = stage<SI>();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (TA) a[i] = mn_operand(base + kHalf * kOpBytes + c.rd_a + (c.tp_a ^ (32 * i)));
    else a[i] = km_operand<OK, KK, kHalf>(c, base + c.rd_a + i * 32 * kPairRow);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if constexpr (TB) b[j] = mn_operand(base + kHalf * kOpBytes + c.rd_b + (c.tp_b ^ (32 * j)));
    else b[j] = km_operand<OK, KK, kHalf>(c, base + c.rd_b + j * 32 * kPairRow);
  }
  if constexpr (!PT && FRESH) {
    // the word holding the lane's K-block (t * kKb) % 16 + 2 kk + h; the byte is
    // picked by the consumer (scale_byte), after the read has surely landed
    const int word = ((t * G::kKb) % kKbPerScale + 2 * KK) >> 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) sa[i] = scales<U>()[0][c.sc_row_a + 32 * i][word];
#pragma unroll
    for (int j = 0; j < 2; ++j) sb[j] = scales<U>()[1][c.sc_row_b + 32 * j][word];
  }
}

// Byte of a scale word for MFMA step kk of stage t: K-block (t * kKb + 2 kk + h) % 4.
template <bool FP4, int KK>
__device__ __forceinline__ int scale_byte(uint32_t word, int t, int h8) {
  return (word >> (8 * ((t * Geo<FP4>::kKb + 2 * KK) & 3) + h8)) & 0xFF;
}

template <int FA, int FB, int KK, bool PT>
__device__ __forceinline__ void mfma_all(v16f (&acc)[4][2], const v8i (&a)[4], const v8i (&b)[2], const int (&swa)[4],
                                         const int (&swb)[2], int t, int h8) {
  constexpr bool kFp4 = FA == E2M1;
  int sa[4], sb[2];
  // per-tensor: every block scale is 2^0
#pragma unroll
  for (int i = 0; i < 4; ++i) sa[i] = PT ? 127 : scale_byte<kFp4, KK>(swa[i], t, h8);
#pragma unroll
  for (int j = 0; j < 2; ++j) sb[j] = PT ? 127 : scale_byte<kFp4, KK>(swb[j], t, h8);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[j], a[i], acc[i][j], MfmaFmt<FB>::kCode,
                                                                   MfmaFmt<FA>::kCode, 0, sb[j], 0, sa[i]);
}

// Scheduling masks of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x008, kSchedVmemRead = 0x020, kSchedDsRead = 0x100;

// Interleave one MFMA step (8 MFMAs) with the memory instructions issued in
// the same region -- VM LDS-DMA loads and DS operand reads for the next step --
// so the LDS reads run in the shadow of the matrix unit instead of after it.
// (the VM loads spread over all 8 MFMAs: over the first 4 measured up to 1.5% slower,
// all before the first MFMA 2-3% slower -- the earlier issue does not pay, the burst
// of LDS-DMA writes against the step's LDS reads costs)
template <int VM, int DS, int K>
__device__ __forceinline__ void interleave_slot() {
  __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
  constexpr int kVm = VM * (K + 1) / 8 - VM * K / 8;
  if constexpr (kVm > 0) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, kVm, 0);
  constexpr int kDs = K < 7 ? DS * (K + 1) / 7 - DS * K / 7 : 0;   // all DS reads within the first 7 MFMAs
  if constexpr (kDs > 0) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kDs, 0);
}

template <int VM, int DS, int... K>
__device__ __forceinline__ void interleave_slots(std::integer_sequence<int, K...>) {
  (interleave_slot<VM, DS, K>(), ...);
}

template <int VM, int DS>
__device__ __forceinline__ void interleave() {
  static_assert(VM <= 12 && DS <= 24, "one step's worth");
  interleave_slots<VM, DS>(std::make_integer_sequence<int, 8>{});
}

struct Regs {
  v8i a[2][4], b[2][2];
  int sa[2][4], sb[2][2];
};

// Stage t = t0 + P (P static inside the unrolled body).  The operands of its
// first MFMA step are already in register set (P * kSub) & 1.
// Stage groups are issued in pairs (2m + 4, 2m + 5) after odd stage 2m + 1: the
// two DMA instructions for the same rows fetch the two 64-byte halves of the
// same 128-byte lines back to back, so each line is fetched from L2 once.  A pair
// issued after stage q also brings the next scale stage when q closes a scale stage.
template <bool FP4>
constexpr bool pair_has_scales(int q) {   // q: the (odd) stage after which the pair is issued
  return ((q % Geo<FP4>::kPerScale) + Geo<FP4>::kPerScale) % Geo<FP4>::kPerScale == Geo<FP4>::kPerScale - 1;
}

// Vector-memory instructions issued after group t + 1 by the time the boundary
// after stage t waits for it (t = P modulo the unrolled body, which is a
// multiple of the scale stage, so the pattern is static).  Only odd P waits.
template <bool FP4, int P, bool PT>
constexpr int later_ops() {
  constexpr int kSO = PT ? 0 : kScaleOps;   // per-tensor mode issues no scale loads
  // both stages of a pair arrive with every one of its instructions, so the first
  // stage of a pair is complete only once the whole pair is; every pair is followed
  // by its scale stage (if any)
  if constexpr (P % 2 == 1)   // group t + 1 opens the pair issued after stage t - 2
    return pair_has_scales<FP4>(P - 2) ? kSO : 0;
  else                         // group t + 1 closes the pair issued after stage t - 3
    return (pair_has_scales<FP4>(P - 3) ? kSO : 0) + 2 * kCodeGroup + (pair_has_scales<FP4>(P - 1) ? kSO : 0);
}

// LDS reads of one operand step: A's 4 row tiles and B's 2 (FP8 two ds_read_b128
// per tile K-contiguous, four transpose reads M/N-contiguous; FP4 one
// ds_read_b128), plus one scale word per tile in MX mode when the words change
template <int OK, bool PT, bool TA, bool TB, bool FRESH = true>
constexpr int kDsReads() {
  // FP6: a ds_read_b128 and a ds_read_b64 per tile
  return PT ? (TA ? 16 : 8) + (TB ? 8 : 4) : (OK == kOkFp4 ? 6 : 12) + (FRESH ? 6 : 0);
}

// Scale words of the next step are those of the current one
__device__ __forceinline__ void carry_scales(Regs& r, int from, int to) {
#pragma unroll
  for (int i = 0; i < 4; ++i) r.sa[to][i] = r.sa[from][i];
#pragma unroll
  for (int j = 0; j < 2; ++j) r.sb[to][j] = r.sb[from][j];
}

// CARRY: FP8 stages reuse the scale words of the stage before when they hold the
// same K-blocks (off where the re-quantizing epilogue leaves no registers for it)
template <int FA, int FB, int P, bool PT, bool TA, bool TB, bool CARRY>
__device__ __forceinline__ void stage_steps(const Ctx& c, int t, int T, int nsuper, int lane, int wave, Regs& r,
                                            v16f (&acc)[4][2]) {
  constexpr bool kFp4 = FA == E2M1;
  constexpr int kOk = kOperandKind<FA>;
  using G = Geo<kFp4>;
  constexpr int SI = P % kStages;                          // this stage's buffer
  constexpr int U = (P / G::kPerScale) & 1;                // this stage's scale buffer
  constexpr int SIn = (P + 1) % kStages;                   // next stage's buffer
  constexpr int Un = ((P + 1) / G::kPerScale) & 1;
#pragma unroll
  for (int kk = 0; kk < G::kSub; ++kk) {
    const int cur = (P * G::kSub + kk) & 1, nxt = cur ^ 1;
    if (kk + 1 < G::kSub) {
      // next MFMA step is in this stage, already visible
      // (FP4) the stage's second step: same scale words as its first
      read_step<kOk, SI, U, 1, PT, TA, TB, false>(c, t, lane, r.a[nxt], r.b[nxt], r.sa[nxt], r.sb[nxt]);
      if constexpr (!PT) carry_scales(r, cur, nxt);
      mfma_all<FA, FB, 0, PT>(acc, r.a[cur], r.b[cur], r.sa[cur], r.sb[cur], t, c.h8);
      interleave<0, kDsReads<kOk, PT, TA, TB, false>()>();
    } else {
      // Only a boundary into a new stage pair (odd P) synchronizes: stage t + 1 of an
      // even P arrived with stage t, in the same pair, and is visible since the
      // barrier that opened the pair.
      constexpr bool kIssue = P % 2 == 1;
      constexpr bool kScales = kIssue && !PT && pair_has_scales<kFp4>(P);
      if constexpr (kIssue) {
        // own DMA of the next pair landed and own LDS reads done, then everybody's
        wait_vm_lgkm0<later_ops<kFp4, P, PT>()>();
        barrier();
        // stages t - 1 and t are fully read into registers: refill their buffers
        // with stages t + 3 and t + 4, the two halves of the same lines
        issue_pair<(P + 3) % kStages, (P + 4) % kStages, TA, TB>(c, t + 3, wave, t + 3 < T, t + 4 < T);
        if constexpr (kScales) {
          const int un = (t + 1) / G::kPerScale + 1;
          issue_scales<((P + 1) / G::kPerScale + 1) & 1>(c, un, wave, un < nsuper);
        }
      }
      // after the last stage this reads stale (in-bounds) LDS that no MFMA consumes; an
      // unconditional read keeps the operand registers free of merge copies
      // FP8 stage t + 1 takes a new scale word only when it is even (P odd)
      constexpr bool kFresh = kFp4 || P % 2 == 1 || !CARRY;
      read_step<kOk, SIn, Un, 0, PT, TA, TB, kFresh>(c, t + 1, lane, r.a[nxt], r.b[nxt], r.sa[nxt], r.sb[nxt]);
      if constexpr (!PT && !kFresh) carry_scales(r, cur, nxt);
      mfma_all<FA, FB, G::kSub - 1, PT>(acc, r.a[cur], r.b[cur], r.sa[cur], r.sb[cur], t, c.h8);
      interleave<(kIssue ? 2 * kCodeGroup : 0) + (kScales ? kScaleOps : 0), kDsReads<kOk, PT, TA, TB, kFresh>()>();
    }
  }
}

template <int FA, int FB, bool PT, bool TA, bool TB, bool CARRY, int... P>
__device__ __forceinline__ void unrolled_body(const Ctx& c, int t0, int T, int nsuper, int lane, int wave, Regs& r,
                                              v16f (&acc)[4][2], std::integer_sequence<int, P...>) {
  (stage_steps<FA, FB, P, PT, TA, TB, CARRY>(c, t0 + P, T, nsuper, lane, wave, r, acc), ...);
}

// MX re-quantization of a wave's 128 x 64 eighth of C (row-wise blocks of 32
// columns), one 32-row tile at a time: the wave stages the tile's FP32 values in
// its LDS region ([32][68] floats; lane (rr, h) holds row rr, columns
// 32 j + 8 q + 4 h + [0, 4)), then each lane encodes one whole block (two
// consecutive lanes cover the two blocks of a row, so the code stores of a row
// are contiguous).
constexpr int kRqPitch = 68;   // floats per staged row (16-byte aligned, rows 4 banks apart)
template <int FC, int RC>
__device__ __forceinline__ void requant_eighth(const v16f (&acc)[4][2], float alpha, int lane, uint8_t* ep,
                                               const GemmArgs& g, int64_t row0, int64_t col0, uint32_t& tmax) {
  constexpr int kBits = Fmt_<FC>::kBits;
  const int rr = lane & 31, h = lane >> 5;
  const int64_t nb = g.N / 32, qpitch = g.N * kBits / 8;
  float* t = reinterpret_cast<float*>(ep);
  // the register tile is picked statically (accumulators cannot be indexed at run
  // time); the encoding below is shared by the four tiles
  auto stage_tile = [&](const v16f (&ai)[2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(t + rr * kRqPitch + 32 * j + 8 * q + 4 * h) =
            make_float4(alpha * ai[j][4 * q], alpha * ai[j][4 * q + 1], alpha * ai[j][4 * q + 2],
                        alpha * ai[j][4 * q + 3]);
  };
#pragma unroll 1
  for (int i = 0; i < 4; ++i) {
    if (i == 0) stage_tile(acc[0]);
    else if (i == 1) stage_tile(acc[1]);
    else if (i == 2) stage_tile(acc[2]);
    else stage_tile(acc[3]);
    wave_lds_fence();
    {
      const int row = lane >> 1, blk = lane & 1;
      float v[32];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float4 x = *reinterpret_cast<const float4*>(t + row * kRqPitch + 32 * blk + 4 * c);
        v[4 * c] = x.x;
        v[4 * c + 1] = x.y;
        v[4 * c + 2] = x.z;
        v[4 * c + 3] = x.w;
      }
      const int64_t r = row0 + 32 * i + row;
      if (r < g.M && col0 + 32 * blk < g.N) {   // partial last tile row / column
#pragma unroll
        for (int c = 0; c < 32; ++c) tmax = umax(tmax, abs_bits_no_nan(v[c]));
        requant_block32<FC, RC>(v, g.qc + r * qpitch + (col0 + 32 * blk) * kBits / 8, g.sc + r * nb + col0 / 32 + blk);
      }
    }
    wave_lds_fence();   // the tile is read before the next one overwrites it
  }
}

template <int FA, int FB, bool BF16OUT, bool PT, bool TA, bool TB, bool RQ = false>
__global__ __launch_bounds__(kThreads, 1) void gemm256_kernel(const GemmArgs g) {
  constexpr bool kFp4 = FA == E2M1;
  constexpr bool kFp6 = kIsFp6<FA>;
  static_assert(!(TA || TB) || (PT && !kFp4 && BF16OUT), "M/N-contiguous operands: per-tensor FP8, BF16 out");
  static_assert(kIsFp6<FA> == kIsFp6<FB> && !(kFp6 && (PT || RQ)), "FP6 operands: both, MX scales, plain output");
  using G = Geo<kFp4>;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;   // wave's 128 rows x 64 columns of the tile
  int tm, tn;
  map_tile(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
  const int K = int(g.K);
  // code bytes per row; stages of 64 code bytes (FP8 64, FP4 128 K-values), FP6 of 64
  // K-values (48 bytes, in a 64-byte stage slot)
  const int kbytes = kFp4 ? K / 2 : kFp6 ? K / 4 * 3 : K, kblocks = K / 32;
  const int T = kFp4 ? K / 128 : K / 64, nsuper = kblocks / kKbPerScale;
  // row pitch of the stored operands: K bytes when K-contiguous
  const int lda = TA ? int(g.lda) : kbytes, ldb = TB ? int(g.ldb) : kbytes;
  const uint8_t* A = g.a + int64_t(blockIdx.y) * g.batch_a;
  const uint8_t* B = g.b + int64_t(blockIdx.y) * g.batch_b;

  // rows (columns) of the tile inside the matrix: the last tile row / column may be
  // partial; the resources end there, so loads beyond return zeros (K-contiguous) or,
  // M/N-contiguous, the next K-row's leading codes (which only reach outputs beyond
  // M / N, never stored) and zeros past the end of the matrix
  const int rows_a = int(min(int64_t(kTile), g.M - int64_t(tm) * kTile));
  const int rows_b = int(min(int64_t(kTile), g.N - int64_t(tn) * kTile));
  Ctx c;
  if constexpr (TA)   // columns tm * 256 .. + 255 of every K-row
    c.a = make_rsrc(A + int64_t(tm) * kTile, uint32_t(int64_t(K - 1) * lda + rows_a));
  else
    c.a = make_rsrc(A + int64_t(tm) * kTile * kbytes, uint32_t(rows_a * kbytes));
  if constexpr (TB)
    c.b = make_rsrc(B + int64_t(tn) * kTile, uint32_t(int64_t(K - 1) * ldb + rows_b));
  else
    c.b = make_rsrc(B + int64_t(tn) * kTile * kbytes, uint32_t(rows_b * kbytes));
  c.z = make_rsrc(A, 0);
  if constexpr (!PT) {
    if (g.gemm_scales) {
      // [K/512][rows][16]: the tile's 16-byte rows of scale stage u start u * rows * 16 bytes in
      // (the host keeps rows * K / 32 below 2^31); rows past the tile's last one read other rows'
      // scales, which only meet zero codes and reach outputs that are never stored
      const int64_t oa = int64_t(tm) * kTile * 16, ob = int64_t(tn) * kTile * 16;
      c.sa = make_rsrc(g.sa + oa, uint32_t(g.M * kblocks - oa));
      c.sb = make_rsrc(g.sb + ob, uint32_t(g.N * kblocks - ob));
      c.sc_step_a = uint32_t(g.M) * 16u;
      c.sc_step_b = uint32_t(g.N) * 16u;
    } else {
      c.sa = make_rsrc(g.sa + int64_t(tm) * kTile * kblocks, uint32_t(rows_a * kblocks));
      c.sb = make_rsrc(g.sb + int64_t(tn) * kTile * kblocks, uint32_t(rows_b * kblocks));
      c.sc_step_a = c.sc_step_b = 16u;
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    // K-contiguous: instruction j of a wave covers rows 32 wave + 8 j + [0, 8), one 128-byte
    // line each; swz of those rows depends on j only through j % 2 (the 8 j term moves it by 4 j)
    const int row = 32 * wave + 8 * j + (lane >> 3);
    uint32_t km = uint32_t(32 * wave + (lane >> 3)) * uint32_t(kbytes) + 16u * uint32_t((lane & 7) ^ swz(row));
    if constexpr (kFp6) {
      // the lane's LDS chunk holds stage half e, chunk cc of the slot; global chunk 3 e + cc
      // of the pair's 96 bytes, and nothing for the unused chunk 3 (an offset past any
      // buffer's end: the load writes zeros and touches no memory)
      const int sc = (lane & 7) ^ swz(row), e = sc >> 2, cc = sc & 3;
      km = cc == 3 ? 0xF0000000u : uint32_t(32 * wave + (lane >> 3)) * uint32_t(kbytes) + 16u * uint32_t(3 * e + cc);
    }
    // M/N-contiguous: instruction j of a stage covers K-rows 8 wave + 4 j + [0, 4), 256 bytes each
    const int kr = 8 * wave + 4 * j + (lane >> 4);
    const uint32_t mn_chunk = 16u * uint32_t((lane & 15) ^ (2 * (kr & 7)));
    c.off_a[j] = TA ? uint32_t(kr) * uint32_t(lda) + mn_chunk : km;
    c.off_b[j] = TB ? uint32_t(kr) * uint32_t(ldb) + mn_chunk : km;
  }
  c.js_a = uint32_t(8 * kbytes);
  c.js_b = uint32_t(8 * kbytes);
  c.step_a = uint32_t(kRow) * uint32_t(TA ? lda : 1);
  c.step_b = uint32_t(kRow) * uint32_t(TB ? ldb : 1);
  c.sc_off = uint32_t(64 * (wave & 3) + lane) * uint32_t(g.gemm_scales ? 16 : kblocks);
  if constexpr (!PT) {
    c.ss = wave < 4 ? c.sa : c.sb;
    c.sc_step = wave < 4 ? c.sc_step_a : c.sc_step_b;
  }
  const int rr = lane & 31, h = lane >> 5;
  // K-contiguous: rows 32 i + rr of a wave's half share swz(rr): 32 i only changes higher row bits;
  // chunk h (stage half 0) at h ^ swz, chunk h + 2 at that ^ 2
  // M/N-contiguous: transpose-read lane j = lane % 16 of group lane / 16 points at K-row
  // 16 h + j / 2 (+ 8, 32, 40), byte 8 (j % 2) of the group's 16-column chunk
  const int tr_base = (16 * h + ((lane & 15) >> 1)) * kMnPitch + 8 * (lane & 1);
  c.rd_a = TA ? tr_base : (wm * 128 + rr) * kPairRow;
  c.rd_b = kPairOp + (TB ? tr_base : (wn * 64 + rr) * kPairRow);
  c.tp_a = 16 * ((8 * wm) ^ (lane & 14) ^ ((lane >> 4) & 1));
  c.tp_b = 16 * ((4 * wn) ^ (lane & 14) ^ ((lane >> 4) & 1));
  c.c0 = 16 * (h ^ swz(rr));
  c.c1 = c.c0 ^ 32;
  c.sc_row_a = wm * 128 + rr;
  c.sc_row_b = wn * 64 + rr;
  c.h8 = 8 * h;
  c.kstep = kFp6 ? 48u : uint32_t(kRow);
  // FP6: chunk 2 h of the stage slot, and bytes 16 + 8 h (the half of chunk 1 that belongs to block h)
  c.f6[0] = 16 * ((2 * h) ^ swz(rr));
  c.f6[1] = 16 * (1 ^ swz(rr)) + 8 * h;

  v16f acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  Regs r;

  // prologue: code stages 0..3, scale stages 0 and 1 (T >= 2 and even, nsuper >= 1); stages
  // and scale stages past the end of K load zeros from the empty resource, and so do the
  // dead stages of the last unrolled body, so their MFMAs add nothing
  // same op pattern as the loop (pair, then its scale stage if any) so that the
  // first boundaries' wait counts hold
  if constexpr (!PT) issue_scales<0>(c, 0, wave, true);
  issue_pair<0, 1, TA, TB>(c, 0, wave, true, true);   // T >= 2
  issue_pair<2, 3, TA, TB>(c, 2, wave, 2 < T, 3 < T);
  if constexpr (!PT) issue_scales<1>(c, 1, wave, 1 < nsuper);
  // scale stage 0 and code stage 0 landed; the pair order interleaves stages 0 and 1
  // instruction by instruction, so wait for both: what may stay in flight is stages
  // 2 and 3 and scale stage 1
  wait_vm_lgkm0<2 * kCodeGroup + (PT ? 0 : kScaleOps)>();
  barrier();
  read_step<kOperandKind<FA>, 0, 0, 0, PT, TA, TB>(c, 0, lane, r.a[0], r.b[0], r.sa[0], r.sb[0]);

  for (int t0 = 0; t0 < T; t0 += G::kUnroll)
    unrolled_body<FA, FB, PT, TA, TB, !RQ>(c, t0, T, nsuper, lane, wave, r, acc,
                                      std::make_integer_sequence<int, G::kUnroll>{});

  // the last groups (empty-range loads) still write LDS: drain them before the
  // workgroup reuses its LDS or retires and hands it to another one
  wait_vm_lgkm0<0>();

  // epilogue: accumulator (i, j) holds C^T fragments -- lane (rr, h) owns row
  // 32 i + rr and columns 32 j + 8 q + 4 h + [0, 4) in registers 4 q + [0, 4)
  const float alpha = PT ? *g.alpha_ptr : g.alpha;
  const int64_t ldc = g.ldc;
  const int64_t row0 = int64_t(tm) * kTile + wm * 128;
  const int64_t col0 = int64_t(tn) * kTile + wn * 64;
  if constexpr (RQ) {
    barrier();   // every wave is done with the stage buffers
    uint8_t* ep = (wave < 4 ? stage<0>() : stage<2>()) + (wave & 3) * kEpBytes;
    uint32_t tmax = 0;
    const int sel = g.fc * 2 + g.rc;
    if (sel == E4M3 * 2 + FLOOR) requant_eighth<E4M3, FLOOR>(acc, alpha, lane, ep, g, row0, col0, tmax);
    else if (sel == E4M3 * 2 + CEIL) requant_eighth<E4M3, CEIL>(acc, alpha, lane, ep, g, row0, col0, tmax);
    else if (sel == E5M2 * 2 + FLOOR) requant_eighth<E5M2, FLOOR>(acc, alpha, lane, ep, g, row0, col0, tmax);
    else if (sel == E5M2 * 2 + CEIL) requant_eighth<E5M2, CEIL>(acc, alpha, lane, ep, g, row0, col0, tmax);
    else if (sel == E2M1 * 2 + FLOOR) requant_eighth<E2M1, FLOOR>(acc, alpha, lane, ep, g, row0, col0, tmax);
    else requant_eighth<E2M1, CEIL>(acc, alpha, lane, ep, g, row0, col0, tmax);
    if (g.amax) {
      const uint32_t m = wave_max(tmax);
      if (lane == 0 && m) atomic_max_u32(g.amax, m);
    }
    return;
  }
  if constexpr (BF16OUT) {
    uint16_t* C = static_cast<uint16_t*>(g.c) + int64_t(blockIdx.y) * g.batch_c;
    // per-tensor bias of the lane's 64 columns, added to alpha * acc with one rounding
    float bias[2][4][4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint2 bw = make_uint2(0, 0);
        if (PT && g.bias && col0 + 32 * j + 8 * q + 4 * h < g.N)
          bw = *reinterpret_cast<const uint2*>(g.bias + col0 + 32 * j + 8 * q + 4 * h);
        bias[j][q][0] = __uint_as_float(bw.x << 16);
        bias[j][q][1] = __uint_as_float(bw.x & 0xFFFF0000u);
        bias[j][q][2] = __uint_as_float(bw.y << 16);
        bias[j][q][3] = __uint_as_float(bw.y & 0xFFFF0000u);
      }
    const bool has_bias = PT && g.bias;
    // BF16: each wave stages its 128 x 64 eighth in 16 KiB of the stage buffers (row
    // pitch 128 B, 16-byte unit u of row r at u ^ (r % 8)), then writes whole
    // 128-byte row segments: 8 lanes per row, 16 bytes per lane.
    barrier();   // every wave is done with the stage buffers
    uint8_t* ep = (wave < 4 ? stage<0>() : stage<2>()) + (wave & 3) * kEpBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = 32 * i + rr, u = 4 * j + q;
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            o[e] = has_bias ? __builtin_fmaf(alpha, acc[i][j][4 * q + e], bias[j][q][e]) : alpha * acc[i][j][4 * q + e];
          const bf16x2 lo = __builtin_convertvector(f2{o[0], o[1]}, bf16x2);
          const bf16x2 hi = __builtin_convertvector(f2{o[2], o[3]}, bf16x2);
          *reinterpret_cast<uint2*>(ep + row * 128 + 16 * (u ^ (row & 7)) + 8 * h) =
              make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
        }
    barrier();
    const int u = lane & 7;
#pragma unroll 8
    for (int it = 0; it < 16; ++it) {
      const int row = 8 * it + (lane >> 3);
      const uint4 v = *reinterpret_cast<const uint4*>(ep + row * 128 + 16 * (u ^ (row & 7)));
      if (row0 + row < g.M && col0 + 8 * u < g.N)   // N % 8 == 0: a piece is wholly in or out
        *reinterpret_cast<uint4*>(C + (row0 + row) * ldc + col0 + 8 * u) = v;
    }
  } else {
    float* C = static_cast<float*>(g.c) + int64_t(blockIdx.y) * g.batch_c;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t off = (row0 + 32 * i + rr) * ldc + col0 + 32 * j + 8 * q + 4 * h;
          if (row0 + 32 * i + rr < g.M && col0 + 32 * j + 8 * q + 4 * h < g.N)   // N % 4 == 0
          *reinterpret_cast<float4*>(C + off) =
              make_float4(alpha * acc[i][j][4 * q], alpha * acc[i][j][4 * q + 1], alpha * acc[i][j][4 * q + 2],
                          alpha * acc[i][j][4 * q + 3]);
        }
  }
}

}  // namespace t256

template <int FA, int FB, bool BF>
static mx_status_t gemm_dispatch(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb, int64_t M,
                                 int64_t N, int64_t K, float alpha, void* c, int64_t ldc, bool gemm_scales,
                                 hipStream_t st) {
  const int esize = BF ? 2 : 4;
  GemmArgs g{};
  g.gemm_scales = gemm_scales;
  g.a = a;
  g.sa = sa;
  g.b = b;
  g.sb = sb;
  g.c = c;
  g.M = M;
  g.N = N;
  g.K = K;
  g.lda = code_bytes<FA>(K);
  g.ldb = code_bytes<FB>(K);
  g.ldc = ldc;
  g.alpha = alpha;
  {
    const int64_t tm256 = (M + t256::kTile - 1) / t256::kTile, tn256 = (N + t256::kTile - 1) / t256::kTile;
    const bool big = N % (BF ? 8 : 4) == 0 && K % t256::kMxK == 0 && K > 0 && K <= (int64_t(1) << 22) &&
                     tm256 * tn256 < (int64_t(1) << 31) && !misaligned(a) && !misaligned(b) && !misaligned(sa) &&
                     !misaligned(sb) && !misaligned(c) && (ldc * esize) % 16 == 0;
    if (big) {
      g.tiles_m = int(tm256);
      g.tiles_n = int(tn256);
      hipLaunchKernelGGL((t256::gemm256_kernel<FA, FB, BF, false, false, false>),
                         dim3(unsigned(g.tiles_m * g.tiles_n)), dim3(t256::kThreads), 0, st, g);
      return hipGetLastError() == hipSuccess ? MX_OK : MX_ERR_LAUNCH;
    }
  }
  g.tiles_m = int((M + kBM - 1) / kBM);
  g.tiles_n = int((N + kBN - 1) / kBN);
  hipLaunchKernelGGL((gemm_kernel<FA, FB, BF, false, false, false>), dim3(unsigned(g.tiles_m * g.tiles_n)),
                     dim3(kGemmThreads), 0, st, g);
  return hipGetLastError() == hipSuccess ? MX_OK : MX_ERR_LAUNCH;
}

// Per-tensor FP8: TA / TB say that the MFMA's A ([M][K]) / B ([N][K]) is stored
// M- / N-contiguous.
template <int F, bool TA, bool TB>
static mx_status_t mm_launch(GemmArgs g, int64_t batch, hipStream_t st) {
  constexpr int64_t kTile = t256::kTile;
  const int64_t tm256 = (g.M + kTile - 1) / kTile, tn256 = (g.N + kTile - 1) / kTile;
  // M/N-contiguous operands are fetched in 16-byte chunks of each K-row: rows must stay 16-byte aligned
  const bool big = g.N % 8 == 0 && (!TA || g.M % 16 == 0) && (!TB || g.N % 16 == 0) && g.K % t256::kPtK == 0 &&
                   g.K > 0 && g.K <= (int64_t(1) << 22) && tm256 * tn256 < (int64_t(1) << 31) &&
                   g.K * g.lda < (int64_t(1) << 31) && g.K * g.ldb < (int64_t(1) << 31) && !misaligned(g.a) &&
                   !misaligned(g.b) && !misaligned(g.c) && (g.batch_a % 16) == 0 && (g.batch_b % 16) == 0 &&
                   (reinterpret_cast<uintptr_t>(g.bias) & 7u) == 0;
  if (big) {
    g.tiles_m = int(tm256);
    g.tiles_n = int(tn256);
    hipLaunchKernelGGL((t256::gemm256_kernel<F, F, true, true, TA, TB>),
                       dim3(unsigned(g.tiles_m * g.tiles_n), unsigned(batch)), dim3(t256::kThreads), 0, st, g);
    return hipGetLastError() == hipSuccess ? MX_OK : MX_ERR_LAUNCH;
  }
  g.tiles_m = int((g.M + kBM - 1) / kBM);
  g.tiles_n = int((g.N + kBN - 1) / kBN);
  hipLaunchKernelGGL((gemm_kernel<F, F, true, true, TA, TB>), dim3(unsigned(g.tiles_m * g.tiles_n), unsigned(batch)),
                     dim3(kGemmThreads), 0, st, g);
  return hipGetLastError() == hipSuccess ? MX_OK : MX_ERR_LAUNCH;
}

template <int F>
static mx_status_t mm_layouts(const GemmArgs& g, bool ta, bool tb, int64_t batch, hipStream_t st) {
  if (ta) return tb ? mm_launch<F, true, true>(g, batch, st) : mm_launch<F, true, false>(g, batch, st);
  return tb ? mm_launch<F, false, true>(g, batch, st) : mm_launch<F, false, false>(g, batch, st);
}

template <int FA, int FB>
static mx_status_t requant_dispatch(GemmArgs g, hipStream_t st) {
  const int64_t M = g.M, N = g.N, K = g.K;
  const int64_t tm256 = (M + t256::kTile - 1) / t256::kTile, tn256 = (N + t256::kTile - 1) / t256::kTile;
  const bool big = K % t256::kMxK == 0 && K > 0 && K <= (int64_t(1) << 22) && tm256 * tn256 < (int64_t(1) << 31) &&
                   !misaligned(g.a) && !misaligned(g.b) && !misaligned(g.sa) && !misaligned(g.sb);
  if (big) {
    g.tiles_m = int(tm256);
    g.tiles_n = int(tn256);
    hipLaunchKernelGGL((t256::gemm256_kernel<FA, FB, true, false, false, false, true>),
                       dim3(unsigned(g.tiles_m * g.tiles_n)), dim3(t256::kThreads), 0, st, g);
    return hipGetLastError() == hipSuccess ? MX_OK : MX_ERR_LAUNCH;
  }
  g.tiles_m = int((M + kBM - 1) / kBM);
  g.tiles_n = int((N + kBN - 1) / kBN);
  hipLaunchKernelGGL((gemm_kernel<FA, FB, true, false, false, false, true>), dim3(unsigned(g.tiles_m * g.tiles_n)),
                     dim3(kGemmThreads), 0, st, g);
  return hipGetLastError() == hipSuccess ? MX_OK : MX_ERR_LAUNCH;
}

template <bool BF>
static mx_status_t gemm_formats(int fa, int fb, const uint8_t* a, const uint8_t* sa, const uint8_t* b,
                                const uint8_t* sb, int64_t M, int64_t N, int64_t K, float alpha, void* c, int64_t ldc,
                                bool gs, hipStream_t st) {
  if (fa == E4M3 && fb == E4M3) return gemm_dispatch<E4M3, E4M3, BF>(a, sa, b, sb, M, N, K, alpha, c, ldc, gs, st);
  if (fa == E4M3 && fb == E5M2) return gemm_dispatch<E4M3, E5M2, BF>(a, sa, b, sb, M, N, K, alpha, c, ldc, gs, st);
  if (fa == E5M2 && fb == E4M3) return gemm_dispatch<E5M2, E4M3, BF>(a, sa, b, sb, M, N, K, alpha, c, ldc, gs, st);
  if (fa == E5M2 && fb == E5M2) return gemm_dispatch<E5M2, E5M2, BF>(a, sa, b, sb, M, N, K, alpha, c, ldc, gs, st);
  if (fa == E2M1 && fb == E2M1) return gemm_dispatch<E2M1, E2M1, BF>(a, sa, b, sb, M, N, K, alpha, c, ldc, gs, st);
  if (fa == E2M3 && fb == E2M3) return gemm_dispatch<E2M3, E2M3, BF>(a, sa, b, sb, M, N, K, alpha, c, ldc, gs, st);
  if (fa == E2M3 && fb == E3M2) return gemm_dispatch<E2M3, E3M2, BF>(a, sa, b, sb, M, N, K, alpha, c, ldc, gs, st);
  if (fa == E3M2 && fb == E2M3) return gemm_dispatch<E3M2, E2M3, BF>(a, sa, b, sb, M, N, K, alpha, c, ldc, gs, st);
  if (fa == E3M2 && fb == E3M2) return gemm_dispatch<E3M2, E3M2, BF>(a, sa, b, sb, M, N, K, alpha, c, ldc, gs, st);
  return MX_ERR_UNSUPPORTED;
}

}  // namespace mxk

using namespace mxk;

// The GEMM scale layout groups 16 K-blocks (K % 512 == 0) and its stage offsets
// are 32-bit (rows * K / 32 below 2^31 for both operands).
static mx_status_t check_scale_layout(mx_scale_layout_t layout, int64_t M, int64_t N, int64_t K) {
  if (layout != MX_SCALES_ROW_MAJOR && layout != MX_SCALES_GEMM) return MX_ERR_UNSUPPORTED;
  if (layout == MX_SCALES_GEMM &&
      (K % 512 != 0 || M * (K / 32) >= (int64_t(1) << 31) || N * (K / 32) >= (int64_t(1) << 31)))
    return MX_ERR_SHAPE;
  return MX_OK;
}

extern "C" mx_status_t mx_gemm(const uint8_t* a, const uint8_t* sa, mx_elem_t fmt_a, const uint8_t* b,
                               const uint8_t* sb, mx_elem_t fmt_b, mx_scale_layout_t scale_layout, int64_t M,
                               int64_t N, int64_t K, float alpha, void* c, mx_dtype_t c_dtype, int64_t ldc,
                               hipStream_t stream) {
  const bool f8a = fmt_a == MX_E4M3 || fmt_a == MX_E5M2, f8b = fmt_b == MX_E4M3 || fmt_b == MX_E5M2;
  const bool f6a = fmt_a == MX_E2M3 || fmt_a == MX_E3M2, f6b = fmt_b == MX_E2M3 || fmt_b == MX_E3M2;
  if (!((f8a && f8b) || (f6a && f6b) || (fmt_a == MX_E2M1 && fmt_b == MX_E2M1))) return MX_ERR_UNSUPPORTED;
  if (c_dtype != MX_BF16 && c_dtype != MX_F32) return MX_ERR_UNSUPPORTED;
  if (M < 0 || N < 0 || K < 0 || K % 32 != 0) return MX_ERR_SHAPE;
  // FP6 rows of K codes are K * 3 / 4 bytes, read in 16-byte chunks
  if (f6a && K % 64 != 0) return MX_ERR_SHAPE;
  if (M > (int64_t(1) << 31) || N > (int64_t(1) << 31) || K > (int64_t(1) << 31)) return MX_ERR_SHAPE;
  if (ldc < N) return MX_ERR_SHAPE;
  if (mx_status_t st = check_scale_layout(scale_layout, M, N, K); st != MX_OK) return st;
  if (M == 0 || N == 0) return MX_OK;
  if (!c || (K > 0 && (!a || !sa || !b || !sb))) return MX_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(c) & (c_dtype == MX_BF16 ? 1u : 3u)) != 0) return MX_ERR_ALIGN;
  if (K > 0 && (misaligned(a) || misaligned(b))) return MX_ERR_ALIGN;
  const bool gs = scale_layout == MX_SCALES_GEMM;
  return c_dtype == MX_BF16 ? gemm_formats<true>(fmt_a, fmt_b, a, sa, b, sb, M, N, K, alpha, c, ldc, gs, stream)
                            : gemm_formats<false>(fmt_a, fmt_b, a, sa, b, sb, M, N, K, alpha, c, ldc, gs, stream);
}

extern "C" mx_status_t mm_fp8(const uint8_t* a, const uint8_t* b, mx_elem_t fmt, int64_t batch, int64_t M, int64_t N,
                              int64_t K, int a_batched, int b_batched, int trans_a, int trans_b, const float* scale,
                              const uint16_t* bias, uint16_t* c, hipStream_t stream) {
  if (fmt != MX_E4M3 && fmt != MX_E5M2) return MX_ERR_UNSUPPORTED;
  if (batch < 0 || M < 0 || N < 0 || K < 0 || K % 16 != 0) return MX_ERR_SHAPE;
  if (batch > 65535 || M > (int64_t(1) << 31) || N > (int64_t(1) << 31) || K > (int64_t(1) << 31)) return MX_ERR_SHAPE;
  if (batch == 0 || M == 0 || N == 0) return MX_OK;
  if (!c || !scale || (K > 0 && (!a || !b))) return MX_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(c) & 1u) || (reinterpret_cast<uintptr_t>(bias) & 1u)) return MX_ERR_ALIGN;
  if (K > 0 && (misaligned(a) || misaligned(b))) return MX_ERR_ALIGN;
  GemmArgs g{};
  g.a = a;
  g.b = b;
  g.c = c;
  g.alpha_ptr = scale;
  g.bias = bias;
  g.M = M;
  g.N = N;
  g.K = K;
  g.lda = trans_a ? M : K;         // a stored [K][M] when transposed, else [M][K]
  g.ldb = trans_b ? K : N;         // b stored [N][K] when transposed, else [K][N]
  g.ldc = N;
  g.batch_a = a_batched ? M * K : 0;
  g.batch_b = b_batched ? K * N : 0;
  g.batch_c = M * N;
  if (!trans_a && a_batched && !b_batched && batch * M <= (int64_t(1) << 31)) {   // one GEMM with M' = batch M
    g.M = batch * M;
    g.batch_a = g.batch_c = 0;
    batch = 1;
  }
  // the MFMA's B is op(b)^T: N-contiguous exactly when b is not transposed
  return fmt == MX_E4M3 ? mm_layouts<E4M3>(g, trans_a != 0, trans_b == 0, batch, stream)
                        : mm_layouts<E5M2>(g, trans_a != 0, trans_b == 0, batch, stream);
}

extern "C" mx_status_t mx_gemm_requant(const uint8_t* a, const uint8_t* sa, mx_elem_t fmt_a, const uint8_t* b,
                                       const uint8_t* sb, mx_elem_t fmt_b, mx_scale_layout_t scale_layout, int64_t M,
                                       int64_t N, int64_t K, float alpha, mx_elem_t fmt_c, mx_scale_rule_t rule_c,
                                       uint8_t* qc,
                                       uint8_t* sc, float* amax_out, hipStream_t stream) {
  const bool f8a = fmt_a == MX_E4M3 || fmt_a == MX_E5M2, f8b = fmt_b == MX_E4M3 || fmt_b == MX_E5M2;
  if (!((f8a && f8b) || (fmt_a == MX_E2M1 && fmt_b == MX_E2M1))) return MX_ERR_UNSUPPORTED;
  if (fmt_c != MX_E4M3 && fmt_c != MX_E5M2 && fmt_c != MX_E2M1) return MX_ERR_UNSUPPORTED;
  if (rule_c != MX_SCALE_FLOOR && rule_c != MX_SCALE_CEIL) return MX_ERR_UNSUPPORTED;
  if (M < 0 || N < 0 || K < 0 || K % 32 != 0 || N % 32 != 0) return MX_ERR_SHAPE;
  if (M > (int64_t(1) << 31) || N > (int64_t(1) << 31) || K > (int64_t(1) << 31)) return MX_ERR_SHAPE;
  if (mx_status_t st = check_scale_layout(scale_layout, M, N, K); st != MX_OK) return st;
  if (M == 0 || N == 0) return MX_OK;
  if (!qc || !sc || (K > 0 && (!a || !sa || !b || !sb))) return MX_ERR_NULL;
  if (misaligned(qc) || (K > 0 && (misaligned(a) || misaligned(b)))) return MX_ERR_ALIGN;
  GemmArgs g{};
  g.a = a;
  g.sa = sa;
  g.b = b;
  g.sb = sb;
  g.M = M;
  g.N = N;
  g.K = K;
  g.lda = fmt_a == MX_E2M1 ? K / 2 : K;
  g.ldb = fmt_b == MX_E2M1 ? K / 2 : K;
  g.alpha = alpha;
  g.qc = qc;
  g.sc = sc;
  g.amax = reinterpret_cast<uint32_t*>(amax_out);
  g.fc = int(fmt_c);
  g.rc = int(rule_c);
  g.gemm_scales = scale_layout == MX_SCALES_GEMM;
  if (fmt_a == MX_E4M3 && fmt_b == MX_E4M3) return requant_dispatch<E4M3, E4M3>(g, stream);
  if (fmt_a == MX_E4M3 && fmt_b == MX_E5M2) return requant_dispatch<E4M3, E5M2>(g, stream);
  if (fmt_a == MX_E5M2 && fmt_b == MX_E4M3) return requant_dispatch<E5M2, E4M3>(g, stream);
  if (fmt_a == MX_E5M2 && fmt_b == MX_E5M2) return requant_dispatch<E5M2, E5M2>(g, stream);
  return requant_dispatch<E2M1, E2M1>(g, stream);
}
