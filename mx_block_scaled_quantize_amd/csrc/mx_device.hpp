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

enum Fmt : int { E4M3 = 0, E5M2 = 1, E2M1 = 2 };
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
  if (abits == 0u) return -127;
  int E;
  uint32_t frac;
  if (abits >= 0x00800000u) {
    E = int(abits >> 23) - 127;
    frac = abits & 0x7FFFFFu;
  } else {                                        // FP32 subnormal amax
    const int p = 31 - __clz(abits);
    E = p - 149;
    frac = (abits << (23 - p)) & 0x7FFFFFu;
  }
  int e = E - T::kEmax;
  if (R == CEIL && frac > T::kMaxFrac) e += 1;
  e = e < -127 ? -127 : e;
  return e > 127 ? 127 : e;
}

// 2^-e as FP32 (exact; e never exceeds 126 for FP32 inputs, 2^-127 is kept as
// the subnormal for completeness).
__device__ __forceinline__ float pow2_neg(int e) {
  return e <= 126 ? __uint_as_float(uint32_t(127 - e) << 23) : __uint_as_float(0x00400000u);
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
__device__ __forceinline__ void atomic_max_u32(uint32_t* p, uint32_t v) {
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
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = ((mask >> (8 * q + j)) & 1u) ? -v[j] : v[j];
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
  {
    const bool upper = (q & 1) != 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = dpp_f32<kQuadXor1>(v[i]);
      v[i] = upper ? (p - v[i]) : (v[i] + p);
    }
  }
  {
    const bool upper = (q & 2) != 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = dpp_f32<kQuadXor2>(v[i]);
      v[i] = upper ? (p - v[i]) : (v[i] + p);
    }
  }
}

}  // namespace mxk
