// Device-side building blocks of libmx for gfx950 (CDNA4): element encoders,
// E8M0 shared-exponent rules, input widening and wavefront reductions.
//
// Formats ("EU8M0 FP8" article, glossary 'FP8 (E4M3/E5M2)', 'EU8M0', 'MXFP8'):
//   E4M3  bias 7,  3 mantissa bits, max 448,   no Inf, NaN = S.1111.111
//   E5M2  bias 15, 2 mantissa bits, max 57344, IEEE Inf/NaN
//   E2M1  bias 1,  1 mantissa bit,  max 6,     no specials
//   E8M0  code c -> 2^(c-127), 255 = NaN
// Casts round to nearest even and saturate (same article, section 4 of the
// first part: values beyond the format's upper limit are clamped).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxk {

enum Fmt : int { E4M3 = 0, E5M2 = 1, E2M1 = 2, E2M3 = 3, E3M2 = 4 };
enum InType : int { IN_F32 = 0, IN_BF16 = 1, IN_F16 = 2 };
enum Rule : int { FLOOR = 0, CEIL = 1 };

// Per-format constants, all as FP32 bit patterns so the encoder is integer work
// plus one FP32 addition.
template <int F> struct Fmt_;
template <> struct Fmt_<E4M3> {
  static constexpr int kBits = 8;
  static constexpr int kEmax = 8;                    // 448 = 1.75 * 2^8
  static constexpr uint32_t kMaxFrac = 0x600000u;    // FP32 fraction of 1.75
  static constexpr uint32_t kMaxBits = 0x43E00000u;  // 448.0f
  static constexpr uint32_t kMinNormBits = 0x3C800000u;  // 2^-6
  static constexpr uint32_t kSubMagicBits = 0x46800000u; // 2^14: its FP32 ulp is 2^-9
  static constexpr int kShift = 20;                  // 23 - 3 mantissa bits
  static constexpr uint32_t kRebias = (127u - 7u) << 3;
  static constexpr uint32_t kNan = 0x7Fu;
};
template <> struct Fmt_<E5M2> {
  static constexpr int kBits = 8;
  static constexpr int kEmax = 15;                   // 57344 = 1.75 * 2^15
  static constexpr uint32_t kMaxFrac = 0x600000u;
  static constexpr uint32_t kMaxBits = 0x47600000u;  // 57344.0f
  static constexpr uint32_t kMinNormBits = 0x38800000u;  // 2^-14
  static constexpr uint32_t kSubMagicBits = 0x43000000u; // 2^7: ulp 2^-16
  static constexpr int kShift = 21;
  static constexpr uint32_t kRebias = (127u - 15u) << 2;
  static constexpr uint32_t kNan = 0x7Fu;
};
template <> struct Fmt_<E2M1> {
  static constexpr int kBits = 4;
  static constexpr int kEmax = 2;                    // 6 = 1.5 * 2^2
  static constexpr uint32_t kMaxFrac = 0x400000u;    // fraction of 1.5
  static constexpr uint32_t kMaxBits = 0x40C00000u;  // 6.0f
  static constexpr uint32_t kMinNormBits = 0x3F800000u;  // 1.0
  static constexpr uint32_t kSubMagicBits = 0x4A800000u; // 2^22: ulp 2^-1
  static constexpr int kShift = 22;
  static constexpr uint32_t kRebias = (127u - 1u) << 1;
  static constexpr uint32_t kNan = 0x7u;             // no NaN: largest magnitude
};
template <> struct Fmt_<E2M3> {
  static constexpr int kBits = 6;
  static constexpr int kEmax = 2;                    // 7.5 = 1.875 * 2^2
  static constexpr uint32_t kMaxFrac = 0x700000u;    // fraction of 1.875
  static constexpr uint32_t kMaxBits = 0x40F00000u;  // 7.5f
  static constexpr uint32_t kMinNormBits = 0x3F800000u;  // 1.0
  static constexpr uint32_t kSubMagicBits = 0x49800000u; // 2^20: ulp 2^-3
  static constexpr int kShift = 20;
  static constexpr uint32_t kRebias = (127u - 1u) << 3;
  static constexpr uint32_t kNan = 0x1Fu;            // no NaN: largest magnitude
};
template <> struct Fmt_<E3M2> {
  static constexpr int kBits = 6;
  static constexpr int kEmax = 4;                    // 28 = 1.75 * 2^4
  static constexpr uint32_t kMaxFrac = 0x600000u;
  static constexpr uint32_t kMaxBits = 0x41E00000u;  // 28.0f
  static constexpr uint32_t kMinNormBits = 0x3E800000u;  // 2^-2
  static constexpr uint32_t kSubMagicBits = 0x49000000u; // 2^19: ulp 2^-4
  static constexpr int kShift = 21;
  static constexpr uint32_t kRebias = (127u - 3u) << 2;
  static constexpr uint32_t kNan = 0x1Fu;
};

// Round-to-nearest-even, saturating cast of an FP32 value to format F.
// Returns the code in the low kBits bits (sign in the top one of them).
//   |v| below the smallest normal: adding 2^(emin - mbits + 23) makes the FP32
//   adder round |v| to a multiple of the subnormal quantum (one RNE), and the
//   integer difference of the bit patterns is the quantum count (a count equal
//   to 2^mbits is the smallest normal's code, so the carry is free);
//   otherwise: the usual add-half-minus-one-plus-lsb rounding of the FP32
//   fraction down to mbits bits, then re-biasing of the exponent field.
template <int F>
__device__ __forceinline__ uint32_t encode_rne_sat(float v) {
  using T = Fmt_<F>;
  const uint32_t b = __float_as_uint(v);
  const uint32_t sign = (b >> 31) << (T::kBits - 1);
  uint32_t a = b & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return T::kNan | sign;       // NaN in, NaN out
  a = a < T::kMaxBits ? a : T::kMaxBits;            // saturate (also +-Inf)
  uint32_t code;
  if (a < T::kMinNormBits) {
    const float t = __uint_as_float(a) + __uint_as_float(T::kSubMagicBits);
    code = __float_as_uint(t) - T::kSubMagicBits;
  } else {
    a += ((1u << (T::kShift - 1)) - 1u) + ((a >> T::kShift) & 1u);
    code = (a >> T::kShift) - T::kRebias;
  }
  return code | sign;
}

// Shared block exponent e (scale code = e + 127) from the block amax, given as
// the bit pattern of a finite non-negative FP32 value.
//   FLOOR: e = floor(log2 amax) - emax
//   CEIL:  smallest e with amax <= max * 2^e, which is FLOOR + 1 exactly when
//          amax's significand exceeds the format maximum's significand.
// Clamped to [-127, 127]; amax == 0 gives -127 (scale code 0).
template <int F, int R>
__device__ __forceinline__ int shared_exponent(uint32_t abits) {
  using T = Fmt_<F>;
  if (abits >= 0x00800000u) {
    // normal amax: the exponent field does it, one compare for the round-up rule
    const int e = int(abits >> 23) - 127 - T::kEmax + ((R == CEIL && (abits & 0x7FFFFFu) > T::kMaxFrac) ? 1 : 0);
    return e < -127 ? -127 : e;      // e <= 127 - kEmax + 1 < 127 always
  }
  if (abits == 0u) return -127;
  // FP32 subnormal amax: e is far below -127 for every format
  return -127;
}

// 2^-e as FP32 (exact; e never exceeds 126 for FP32 inputs, 2^-127 is kept as
// the subnormal for completeness).
__device__ __forceinline__ float pow2_neg(int e) {
  return e <= 126 ? __uint_as_float(uint32_t(127 - e) << 23) : __uint_as_float(0x00400000u);
}

// Byte offset of the E8M0 scale of K-block kb of line `line` (an operand row) in
// a scale array of `lines` lines and `kblocks` K-blocks per line:
//   row-major      [lines][kblocks]
//   GEMM layout    [kblocks / 16][lines][16]: the 16 scales a GEMM stage of 16
//                  K-blocks needs are contiguous per line, and the lines of a
//                  stage are contiguous (kblocks % 16 == 0)
__host__ __device__ __forceinline__ int64_t scale_offset(int64_t line, int64_t kb, int64_t lines, int64_t kblocks,
                                                         bool gemm_layout) {
  return gemm_layout ? (((kb >> 4) * lines + line) << 4) + (kb & 15) : line * kblocks + kb;
}

// ---------------------------------------------------------------------------
// Input widening: 8 consecutive elements starting at element index `i`
// (16-byte aligned for 2-byte types, 32-byte aligned for FP32).
// ---------------------------------------------------------------------------
// FP16 bit pattern -> FP32 (exact).
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return float(__builtin_bit_cast(_Float16, uint16_t(h)));
}

template <int IN>
__device__ __forceinline__ void load8(const void* __restrict__ base, int64_t i, float (&v)[8]);

template <>
__device__ __forceinline__ void load8<IN_BF16>(const void* __restrict__ base, int64_t i, float (&v)[8]) {
  const uint4 d = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + i);
  const uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = __uint_as_float(w[j] << 16);
    v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
  }
}

template <>
__device__ __forceinline__ void load8<IN_F16>(const void* __restrict__ base, int64_t i, float (&v)[8]) {
  const uint4 d = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + i);
  const uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = f16_bits_to_f32(w[j] & 0xFFFFu);
    v[2 * j + 1] = f16_bits_to_f32(w[j] >> 16);
  }
}

template <>
__device__ __forceinline__ void load8<IN_F32>(const void* __restrict__ base, int64_t i, float (&v)[8]) {
  const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + i);
  const float4 a = p[0], b = p[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <int IN> struct InSize { static constexpr int kBytes = IN == IN_F32 ? 4 : 2; };

// Bit pattern of |v|.
__device__ __forceinline__ uint32_t abs_bits(float v) { return __float_as_uint(v) & 0x7FFFFFFFu; }
// |v| for the per-tensor amax: NaN counts as 0 (ignored).
__device__ __forceinline__ uint32_t abs_bits_no_nan(float v) {
  const uint32_t a = __float_as_uint(v) & 0x7FFFFFFFu;
  return a > 0x7F800000u ? 0u : a;
}

// ---------------------------------------------------------------------------
// Cross-lane helpers (wave64)
// ---------------------------------------------------------------------------
// DPP quad permutations: [1,0,3,2] and [2,3,0,1].
constexpr int kQuadXor1 = 0xB1;
constexpr int kQuadXor2 = 0x4E;
// DPP rotations by 4 and 8 lanes within each 16-lane row (row_ror).
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return uint32_t(__builtin_amdgcn_mov_dpp(int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// max over the 4 lanes of each quad
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  v = umax(v, dpp_u32<kQuadXor1>(v));
  v = umax(v, dpp_u32<kQuadXor2>(v));
  return v;
}

// max over the whole wavefront (uniform result)
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = umax(v, uint32_t(__shfl_xor(int(v), off, 64)));
  return v;
}

// Agent-scope atomics on the amax / ticket words (multi-XCD coherent).
// Same-address atomics serialize at the memory side, so the max is only sent
// when it can change the word: the word only grows, so a value not above what
// an (atomic) read returns can never be the final maximum.
__device__ __forceinline__ void atomic_max_u32(uint32_t* p, uint32_t v) {
  if (v > __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
    __hip_atomic_fetch_max(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Fixed-sign 32-point Walsh-Hadamard transform on 32 values held by one lane
// ("Format-aware fusion" article, MXFP4 recipe): negate element j when bit j
// of the mask is set, then butterflies of span 1, 2, 4, 8, 16, each pair
// (i, i+h) with (i & h) == 0 becoming (v_i + v_{i+h}, v_i - v_{i+h}).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void hadamard32_inlane(float (&v)[32], uint32_t mask) {
#pragma unroll
  for (int j = 0; j < 32; ++j) v[j] = ((mask >> j) & 1u) ? -v[j] : v[j];
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
}

// The same transform on a block spread over a quad: lane q of the quad holds
// elements 8q .. 8q+7.  Spans 1, 2, 4 stay in the lane; spans 8 and 16 pair lane
// q with lane q^1 and q^2, where the lower lane keeps a + b and the upper lane
// computes a - b with a = the lower lane's value (the same FP32 operations).
__device__ __forceinline__ void hadamard32_quad(float (&v)[8], uint32_t mask, int q) {
  const uint32_t lm = mask >> (8 * q);
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = __uint_as_float(__float_as_uint(v[j]) ^ (((lm >> j) & 1u) << 31));
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
  // the upper lane adds its own value negated: p + (-v) is p - v exactly
  {
    const uint32_t neg = (q & 1) ? 0x80000000u : 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = dpp_f32<kQuadXor1>(v[i]);
      v[i] = p + __uint_as_float(__float_as_uint(v[i]) ^ neg);
    }
  }
  {
    const uint32_t neg = (q & 2) ? 0x80000000u : 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = dpp_f32<kQuadXor2>(v[i]);
      v[i] = p + __uint_as_float(__float_as_uint(v[i]) ^ neg);
    }
  }
}


// A NaN made by the transform's additions has no sign that IEEE 754 fixes (the
// FP32 adders here and other hardware may differ), so the Hadamard paths clear
// the sign bit of every NaN they encode; Inf and finite values keep theirs.
// Only called on blocks already known to hold a non-finite value.
template <int N>
__device__ __forceinline__ void clear_nan_signs(float (&v)[N]) {
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] = abs_bits(v[j]) > 0x7F800000u ? __uint_as_float(abs_bits(v[j])) : v[j];
}


// ---------------------------------------------------------------------------
// gfx950 scaled pair converts (V_CVT_SCALEF32_PK_{FP8,BF8,FP4}_{F32,BF16}).
// Measured against the CPU oracle on every BF16 value at several scales: for
// |v / scale| within the format's range the result is exactly RNE(v / scale)
// (subnormals included), the first operand lands in the low byte (FP4: low
// nibble) and SEL picks the 16-bit word (FP8) or the byte (FP4) written.  Out of
// range, FP8 gives NaN / Inf instead of saturating and NaN inputs lose their
// sign, so callers only use them on finite blocks whose scaled values are in
// range (round-up rule, or after an explicit clamp) and override the rest.
// ---------------------------------------------------------------------------
typedef short v2s_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// Orders one wave's LDS writes before its later LDS reads of other lanes' data:
// LDS instructions of a wave execute in order, so only the compiler has to be
// kept from moving memory operations across this point.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
typedef unsigned short v2u16_t __attribute__((ext_vector_type(2)));

template <int F, int SEL>
__device__ __forceinline__ uint32_t cvt_pair_f32(uint32_t old, float a, float b, float scale) {
  if constexpr (F == E4M3) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(__builtin_bit_cast(v2s_t, old), a, b,
                                                                                 scale, SEL != 0));
  } else if constexpr (F == E5M2) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(__builtin_bit_cast(v2s_t, old), a, b,
                                                                                 scale, SEL != 0));
  } else {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, scale, SEL);
  }
}

// Same on two BF16 values packed in one dword (element 0 in the low half).
template <int F, int SEL>
__device__ __forceinline__ uint32_t cvt_pair_bf16(uint32_t old, uint32_t ab, float scale) {
  const v2bf_t v = __builtin_bit_cast(v2bf_t, ab);
  if constexpr (F == E4M3) {
    return __builtin_bit_cast(uint32_t,
                              __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(__builtin_bit_cast(v2s_t, old), v, scale, SEL != 0));
  } else if constexpr (F == E5M2) {
    return __builtin_bit_cast(uint32_t,
                              __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(__builtin_bit_cast(v2s_t, old), v, scale, SEL != 0));
  } else {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(old, v, scale, SEL);
  }
}

// Dwords holding N codes of format F.
template <int F, int N> struct Words { static constexpr int kN = N * Fmt_<F>::kBits / 32; };

// Pack N codes (low bits of c[j]) into dwords, element 0 lowest.
template <int F, int N>
__device__ __forceinline__ void pack_codes(const uint32_t (&c)[N], uint32_t (&w)[Words<F, N>::kN]) {
  constexpr int kPer = 32 / Fmt_<F>::kBits;
  constexpr uint32_t kMask = (1u << Fmt_<F>::kBits) - 1u;
#pragma unroll
  for (int i = 0; i < Words<F, N>::kN; ++i) {
    uint32_t x = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) x |= (c[i * kPer + j] & kMask) << (Fmt_<F>::kBits * j);
    w[i] = x;
  }
}

// N values (pairs in element order) through the pair converter with one scale.
template <int F, int N>
__device__ __forceinline__ void cvt_values_f32(const float (&v)[N], float scale, uint32_t (&w)[Words<F, N>::kN]) {
  if constexpr (Fmt_<F>::kBits == 8) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      uint32_t x = cvt_pair_f32<F, 0>(0u, v[4 * i], v[4 * i + 1], scale);
      w[i] = cvt_pair_f32<F, 1>(x, v[4 * i + 2], v[4 * i + 3], scale);
    }
  } else {
#pragma unroll
    for (int i = 0; i < N / 8; ++i) {
      uint32_t x = cvt_pair_f32<F, 0>(0u, v[8 * i], v[8 * i + 1], scale);
      x = cvt_pair_f32<F, 1>(x, v[8 * i + 2], v[8 * i + 3], scale);
      x = cvt_pair_f32<F, 2>(x, v[8 * i + 4], v[8 * i + 5], scale);
      w[i] = cvt_pair_f32<F, 3>(x, v[8 * i + 6], v[8 * i + 7], scale);
    }
  }
}

// N BF16 values given as N/2 packed pairs.
template <int F, int N>
__device__ __forceinline__ void cvt_values_bf16(const uint32_t (&p)[N / 2], float scale,
                                                uint32_t (&w)[Words<F, N>::kN]) {
  if constexpr (Fmt_<F>::kBits == 8) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) w[i] = cvt_pair_bf16<F, 1>(cvt_pair_bf16<F, 0>(0u, p[2 * i], scale), p[2 * i + 1], scale);
  } else {
#pragma unroll
    for (int i = 0; i < N / 8; ++i) {
      uint32_t x = cvt_pair_bf16<F, 0>(0u, p[4 * i], scale);
      x = cvt_pair_bf16<F, 1>(x, p[4 * i + 1], scale);
      x = cvt_pair_bf16<F, 2>(x, p[4 * i + 2], scale);
      w[i] = cvt_pair_bf16<F, 3>(x, p[4 * i + 3], scale);
    }
  }
}

// Codes of a block whose max |.| bit pattern is NaN / Inf: the format's NaN
// (E2M1: largest magnitude) with each input's sign.
template <int F, int N>
__device__ __forceinline__ void nan_block_words(const float (&v)[N], uint32_t (&w)[Words<F, N>::kN]) {
  uint32_t c[N];
#pragma unroll
  for (int j = 0; j < N; ++j) c[j] = Fmt_<F>::kNan | ((__float_as_uint(v[j]) >> 31) << (Fmt_<F>::kBits - 1));
  pack_codes<F, N>(c, w);
}

// MX-encode N FP32 values of one block (or a part of it) whose shared exponent
// e is already known (`nonfinite`: the block holds NaN / Inf).
template <int F, int R, int N>
__device__ __forceinline__ void mx_encode_given(const float (&v)[N], bool nonfinite, int e,
                                                uint32_t (&w)[Words<F, N>::kN]) {
  if (nonfinite) {
    nan_block_words<F, N>(v, w);
  } else if (e > -127) {
    const float scale = __uint_as_float(uint32_t(127 + e) << 23);
    if constexpr (R == FLOOR && F != E2M1) {
      // the round-down rule can put |v| / 2^e above the format maximum: saturate first
      const float lim = __uint_as_float(Fmt_<F>::kMaxBits + (uint32_t(e) << 23));
      float c[N];
#pragma unroll
      for (int j = 0; j < N; ++j) c[j] = fminf(fmaxf(v[j], -lim), lim);
      cvt_values_f32<F, N>(c, scale, w);
    } else {
      cvt_values_f32<F, N>(v, scale, w);
    }
  } else {
    // e = -127: an all-zero group converts at scale 1 (+-0 gives +-0 codes at
    // any scale), which keeps its wave off the slow integer encoder
    uint32_t any = 0;
#pragma unroll
    for (int j = 0; j < N; ++j) any |= abs_bits(v[j]);
    if (any == 0u) {
      cvt_values_f32<F, N>(v, 1.0f, w);
      return;
    }
    // otherwise 2^-127 is not a normal FP32 scale operand; use the integer encoder
    const float mul = pow2_neg(e);
    uint32_t c[N];
#pragma unroll
    for (int j = 0; j < N; ++j) c[j] = encode_rne_sat<F>(v[j] * mul);
    pack_codes<F, N>(c, w);
  }
}

// MX-encode N FP32 values of one block (or this lane's share of it) given the
// block's max |.| bit pattern; returns the E8M0 scale code.
template <int F, int R, int N>
__device__ __forceinline__ uint32_t mx_encode_f32(const float (&v)[N], uint32_t bmax, uint32_t (&w)[Words<F, N>::kN]) {
  const bool nonfinite = bmax >= 0x7F800000u;
  const int e = nonfinite ? 0 : shared_exponent<F, R>(bmax);
  mx_encode_given<F, R, N>(v, nonfinite, e, w);
  return nonfinite ? 0xFFu : uint32_t(e + 127);
}

// Per-tensor cast of N FP32 values: y = fl32(v * m), saturating RNE, NaN -> NaN
// with the input's sign.  `chunk_max` is the max |v| bit pattern of the values.
template <int F, int N>
__device__ __forceinline__ void pt_encode_f32(const float (&v)[N], float m, uint32_t chunk_max,
                                              uint32_t (&w)[Words<F, N>::kN]) {
  float y[N];
#pragma unroll
  for (int j = 0; j < N; ++j) y[j] = v[j] * m;
  if (chunk_max > 0x7F800000u) {               // a NaN among them: integer encoder
    uint32_t c[N];
#pragma unroll
    for (int j = 0; j < N; ++j) c[j] = encode_rne_sat<F>(y[j]);
    pack_codes<F, N>(c, w);
    return;
  }
  const float mx = __uint_as_float(Fmt_<F>::kMaxBits);
#pragma unroll
  for (int j = 0; j < N; ++j) y[j] = fminf(fmaxf(y[j], -mx), mx);   // also maps +-Inf to +-max
  cvt_values_f32<F, N>(y, 1.0f, w);
}

// max over the two halves of a packed pair of 16-bit magnitudes
__device__ __forceinline__ uint32_t pk_umax16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(v2u16_t, a),
                                                                __builtin_bit_cast(v2u16_t, b)));
}

// min of the two halves of packed pairs of 16-bit magnitudes
__device__ __forceinline__ uint32_t pk_umin16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(v2u16_t, a),
                                                                __builtin_bit_cast(v2u16_t, b)));
}

}  // namespace mxk
