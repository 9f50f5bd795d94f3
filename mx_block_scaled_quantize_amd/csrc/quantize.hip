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
//   rowwise_kernel  row-wise MX blocks.  Row-wise blocks are contiguous in
//                   memory, so the tensor is treated as a flat array: each lane
//                   owns 8 consecutive elements (one 16-byte load for 2-byte
//                   inputs), a quad of lanes owns one block, and the block amax
//                   is a 2-step DPP max inside the quad.
//   pt_row_kernel   per-tensor FP8 cast with row-major output, flat the same way,
//                   ending with the ring fold.
//   strip_kernel    one wavefront per 32-row x 128-column strip: coalesced
//                   16-byte loads (4 rows of 256 bytes per instruction), the
//                   row-wise half straight from registers, the strip staged in
//                   LDS in the input type, then each lane walks the 32 rows of
//                   2 adjacent columns (conflict-free dword reads) for the
//                   column-wise half, stored transposed with 16-byte stores.
//                   A single wave needs no cross-wave barrier and keeps ~16
//                   independent strips in flight per CU.  Workgroup ids are
//                   mapped so that the 4 strips that share the 128-byte lines of
//                   the transposed output run on the same XCD (ids are handed
//                   to the 8 XCDs round-robin).  Used for FP32 / FP16 inputs
//                   (MX dual, MX column-wise with or without the Hadamard
//                   transform, per-tensor transposed / dual outputs) and for
//                   BF16 tensors too large for the tiled kernels below.
//   BF16 input has register-resident kernels that never stage the input in LDS:
//   dual_bf16_kernel    MX dual.  A 256-thread workgroup takes a 128 x 128 tile;
//                       each lane holds an 8 x 8 patch, so a row block is one
//                       quad of lanes (DPP max) and a column block is 4 lanes
//                       of a DPP row (row_ror max).  Both code copies are
//                       staged in LDS and leave as 16-byte pieces of whole
//                       128-byte lines; the scales leave as dwords.  Two
//                       workgroups per CU walk the tiles; for FP8 each loads
//                       its next tile's input while the current one converts.
//   col_bf16_kernel     MX column-wise (optionally after the 32-point Hadamard
//                       transform, butterflies across the quad), same staging
//                       of the transposed codes; 256-row tiles for FP4 so that
//                       a column's output line is whole.
//   pt_col_bf16_kernel  per-tensor FP8 cast, transposed output only.
//   The per-tensor kernels end with the delayed-scaling fold, done by the last
//   workgroup to finish (two-level ring ticket: a ticket per group of
//   workgroups, then one over the groups).

#include <mutex>

#include "mx_device.hpp"
#include "mx_launch.hpp"

namespace mxk {

// ---------------------------------------------------------------------------
// Stores
// ---------------------------------------------------------------------------
// 8 codes of a row chunk starting at element `elem` (2 dwords FP8, 1 dword FP4); streaming stores.
template <int F>
__device__ __forceinline__ void store_row8(uint8_t* __restrict__ q, int64_t elem, const uint32_t (&w)[Words<F, 8>::kN]) {
  if constexpr (Fmt_<F>::kBits == 8) {
    __builtin_nontemporal_store(u32x2_t{w[0], w[1]}, reinterpret_cast<u32x2_t*>(q + elem));
  } else {
    __builtin_nontemporal_store(w[0], reinterpret_cast<uint32_t*>(q + elem / 2));
  }
}

// ---------------------------------------------------------------------------
// Input chunks: 8 consecutive elements = one 16-byte word (2-byte types) or two (FP32)
// ---------------------------------------------------------------------------
template <int IN> struct ChunkWords { static constexpr int kN = IN == IN_F32 ? 2 : 1; };

template <int IN>
__device__ __forceinline__ void load_chunk(const void* __restrict__ base, int64_t i, uint4 (&w)[ChunkWords<IN>::kN]) {
  const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(base) + i * (IN == IN_F32 ? 4 : 2));
#pragma unroll
  for (int k = 0; k < ChunkWords<IN>::kN; ++k) w[k] = p[k];
}

// Same, with the streaming (non-temporal) hint: the input is read exactly once.
template <int IN>
__device__ __forceinline__ void load_chunk_nt(const void* __restrict__ base, int64_t i,
                                              uint4 (&w)[ChunkWords<IN>::kN]) {
  const u32x4_t* p = reinterpret_cast<const u32x4_t*>(static_cast<const uint8_t*>(base) + i * (IN == IN_F32 ? 4 : 2));
#pragma unroll
  for (int k = 0; k < ChunkWords<IN>::kN; ++k) {
    const u32x4_t v = __builtin_nontemporal_load(p + k);
    w[k] = make_uint4(v[0], v[1], v[2], v[3]);
  }
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

// Max |x| of a chunk as an FP32 bit pattern (a NaN element makes it > 0x7F800000).
template <int IN>
__device__ __forceinline__ uint32_t chunk_absmax(const uint4 (&c)[ChunkWords<IN>::kN], const float (&v)[8]) {
  if constexpr (IN == IN_BF16) {
    const uint32_t k = 0x7FFF7FFFu;
    const uint32_t m = pk_umax16(pk_umax16(c[0].x & k, c[0].y & k), pk_umax16(c[0].z & k, c[0].w & k));
    return umax(m & 0xFFFFu, m >> 16) << 16;
  } else {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = umax(m, abs_bits(v[j]));
    return m;
  }
}

// Per-tensor amax contribution of a chunk with max-bits m (NaN entries ignored).
__device__ __forceinline__ uint32_t amax_update(uint32_t tmax, uint32_t m, const float (&v)[8]) {
  if (m <= 0x7F800000u) return umax(tmax, m);
#pragma unroll
  for (int j = 0; j < 8; ++j) tmax = umax(tmax, abs_bits_no_nan(v[j]));
  return tmax;
}

// ---------------------------------------------------------------------------
// Row-wise MX quantization of one 8-element chunk held by a lane of a quad
// (the quad holds one 32-element block).  Returns the scale code.
// ---------------------------------------------------------------------------
template <int IN, int F, int R, bool HAD>
__device__ __forceinline__ uint32_t row_chunk_mx(const uint4 (&c)[ChunkWords<IN>::kN], float (&v)[8], uint32_t m,
                                                 uint32_t had_mask, int lane_q, uint32_t (&w)[Words<F, 8>::kN]) {
  if constexpr (HAD) {
    hadamard32_quad(v, had_mask, lane_q);
    m = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = umax(m, abs_bits(v[j]));
  }
  const uint32_t bmax = quad_max(m);
  if constexpr (HAD) {
    if (bmax >= 0x7F800000u) clear_nan_signs(v);
  }
  if constexpr (IN == IN_BF16 && R == CEIL && !HAD) {
    // no element exceeds the format maximum under the round-up rule: convert the
    // BF16 pairs directly
    if (bmax < 0x7F800000u) {
      const int e = shared_exponent<F, R>(bmax);
      if (e > -127) {
        const uint32_t p[4] = {c[0].x, c[0].y, c[0].z, c[0].w};
        cvt_values_bf16<F, 8>(p, __uint_as_float(uint32_t(127 + e) << 23), w);
        return uint32_t(e + 127);
      }
    }
  }
  return mx_encode_f32<F, R, 8>(v, bmax, w);
}

// ---------------------------------------------------------------------------
// Row-wise MX quantization (flat): row-wise blocks are contiguous in memory
// ---------------------------------------------------------------------------
constexpr int kRowThreads = 256;
// chunks per thread, loaded before any is encoded: two for the MX row-wise
// kernel (BF16 8192 x 4096 to E4M3: 18.8 us against 19.7 with four), four for
// the per-tensor row-wise cast (23.8 us against 24.4 with two)
constexpr int kRowUnroll = 2;
constexpr int kPtRowUnroll = 4;

template <int IN, int F, int R, bool HAD, bool AMAX>
__global__ __launch_bounds__(kRowThreads) void rowwise_kernel(const void* __restrict__ x, int64_t nchunks,
                                                               uint8_t* __restrict__ q, uint8_t* __restrict__ scales,
                                                               uint32_t* __restrict__ amax_out, uint32_t had_mask,
                                                               int64_t lines, int64_t gemm_kblocks) {
  constexpr int kW = ChunkWords<IN>::kN;
  const int lane_q = threadIdx.x & 3;
  uint32_t tmax = 0;
  uint4 raw[kRowUnroll][kW];
  int64_t chunk[kRowUnroll];
#pragma unroll
  for (int u = 0; u < kRowUnroll; ++u) {
    chunk[u] = (int64_t(blockIdx.x) * kRowUnroll + u) * kRowThreads + threadIdx.x;
#pragma unroll
    for (int k = 0; k < kW; ++k) raw[u][k] = make_uint4(0, 0, 0, 0);
    if (chunk[u] < nchunks) load_chunk<IN>(x, chunk[u] * 8, raw[u]);
  }
#pragma unroll
  for (int u = 0; u < kRowUnroll; ++u) {
    // nchunks is a multiple of 4 and quads are aligned: a quad is entirely in or out of range
    if (chunk[u] >= nchunks) continue;
    float v[8];
    widen_chunk<IN>(raw[u], v);
    const uint32_t m = chunk_absmax<IN>(raw[u], v);
    if constexpr (AMAX) tmax = amax_update(tmax, m, v);
    uint32_t w[Words<F, 8>::kN];
    const uint32_t sc = row_chunk_mx<IN, F, R, HAD>(raw[u], v, m, had_mask, lane_q, w);
    store_row8<F>(q, chunk[u] * 8, w);
    if (lane_q == 0) {
      // block index chunk / 4 = line * kblocks + kb; gemm_kblocks != 0 selects the GEMM scale layout
      const int64_t blk = chunk[u] >> 2;
      scales[gemm_kblocks ? scale_offset(blk / gemm_kblocks, blk % gemm_kblocks, lines, gemm_kblocks, true) : blk] =
          uint8_t(sc);
    }
  }
  if constexpr (AMAX) {
    __shared__ uint32_t red[kRowThreads / 64];
    tmax = wave_max(tmax);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = tmax;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t mm = red[0];
#pragma unroll
      for (int w = 1; w < kRowThreads / 64; ++w) mm = umax(mm, red[w]);
      atomic_max_u32(amax_out, mm);
    }
  }
}

// ---------------------------------------------------------------------------
// Delayed-scaling ring fold, run by the last workgroup of a per-tensor kernel
// ---------------------------------------------------------------------------
struct RingArgs {
  float* ring;          // [hist | s | m | amax | ticket], hist_len + 4 words
  uint32_t* tickets;    // optional spread-ticket scratch (MX_TICKET_WORDS words), or null
  int hist_len, hist_idx;
  float fp8_max, margin;
  float* amax_out;      // optional copy of this call's amax
};

// The fold is reached through a ticket taken by every workgroup (thread 0).
// With ticket scratch it is two-level:
//   1. as soon as the workgroup knows its max |x|, it posts it to the max word
//      of its group (workgroup id modulo 128) -- an atomic max, sent only when
//      an atomic read shows that it can raise the word (the word only grows);
//   2. it increments its group's ticket, an increment whose operand depends on
//      the value step 1 returned and on the multiplier the workgroup read, so
//      it is issued only after that max has been performed (or found to be
//      covered) and after the multiplier has been read;
//   3. the group's last arrival reads the group max (an RMW), clears the group
//      words, posts the group max to the top amax word and takes a top ticket
//      (again dependent RMWs);
//   4. the last top ticket reads the overall max, folds it into the history,
//      publishes s and m = 1/s and clears the top words.
// Posting every workgroup's max straight to the top word (one RMW fewer for the
// last arrival) measured 14-56% slower on inputs of 500+ workgroups: even reads
// of one word queue up at that rate.  Reading the history together with the
// overall max (one round trip fewer) measured no different.
// Without scratch, and for grids of at most kSingleLevelGrid workgroups, steps
// 1-2 use the ring's own amax and ticket words and the arrival at step 2 that
// completes the count goes straight to step 4.  A grid of one workgroup takes no
// ticket: it folds its own max (step 4) with no atomic at all.
// Atomics on one cache line serialize (about 12 ns each on MI355X, more under
// load) while different lines proceed in parallel, so every group sits on a
// 128-byte line of its own; the single-word mode is kept to few workgroups by
// the launch (persistent grids, see kNullTicketGrid).
constexpr unsigned kTicketGroups = 128;
constexpr unsigned kTicketStride = MX_TICKET_WORDS / kTicketGroups;   // 32 words = 128 bytes
static_assert(kTicketStride >= 2, "a group needs a max and a ticket word");
// Grid cap of the per-tensor kernels when the caller passes no ticket scratch:
// every workgroup then takes its ticket on one word.
constexpr int64_t kNullTicketGrid = 512;
// Grid cap of the transposed per-tensor kernel with ticket scratch: about four
// resident workgroups per CU, each taking two or more tiles and one ticket
// (measured 3.6% faster than one workgroup per tile on a BF16 8192 x 4096 input).
constexpr int64_t kTicketGrid = 1024;
// Grids up to this size take a single-level ticket on the ring's words even with
// scratch: two dependent round trips fewer for the last arrival, and at most
// 2 x 16 atomics queued on the line (well under a microsecond).  This is the
// launch-bound regime of small tensors, where the round trips are the call's cost.
constexpr unsigned kSingleLevelGrid = 16;

struct RingTicket {
  uint32_t* gmax;
  uint32_t* gctr;
  unsigned members;    // workgroups in this group
  bool two_level;
  bool solo;           // the grid's only workgroup: no ticket, it folds its own max
};

__device__ __forceinline__ RingTicket ring_ticket(const RingArgs& r, unsigned wg, unsigned num_wg) {
  if (num_wg == 1) return RingTicket{nullptr, nullptr, 1u, false, true};
  if (r.tickets == nullptr || num_wg <= kSingleLevelGrid) {
    uint32_t* top = reinterpret_cast<uint32_t*>(r.ring + r.hist_len + 2);
    return RingTicket{top, top + 1, num_wg, false, false};
  }
  const unsigned g = wg % kTicketGroups;
  return RingTicket{r.tickets + g * kTicketStride, r.tickets + g * kTicketStride + 1,
                    num_wg / kTicketGroups + (g < num_wg % kTicketGroups ? 1u : 0u), true, false};
}

// step 1: returns the value the ticket increment will depend on (for the only
// workgroup of the grid: its own max, the value the fold takes)
__device__ __forceinline__ uint32_t ring_post_max(const RingTicket& t, uint32_t wg_max) {
  if (t.solo) return wg_max;
  // a few workgroups on one word: post directly (the read below saves atomics
  // only where many workgroups share the word, and costs a round trip)
  if (!t.two_level && t.members <= kSingleLevelGrid)
    return __hip_atomic_fetch_max(t.gmax, wg_max, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t seen = __hip_atomic_load(t.gmax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (wg_max <= seen) return seen;
  return __hip_atomic_fetch_max(t.gmax, wg_max, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 0, produced by an instruction that reads v: an operand built from it makes the
// consumer wait until v's load has returned (a data dependency the compiler cannot fold).
__device__ __forceinline__ uint32_t zero_after(uint32_t v) {
  uint32_t z;
  asm volatile("v_and_b32 %0, 0, %1" : "=v"(z) : "v"(v));
  return z;
}

// Ticket increment of a posted value (never 0xFFFFFFFF, a NaN-free magnitude:
// the increment is always 1) that also depends on the multiplier bits.
__device__ __forceinline__ uint32_t ticket_inc(uint32_t posted, float mult) {
  return (posted == 0xFFFFFFFFu ? 2u : 1u) + zero_after(__float_as_uint(mult));
}

// Max of the history without slot hist_idx (and 0).  The loads go out sixteen
// at a time, independent of each other (a plain loop waits for each load before
// the next).  Issuing them before the ticket, to overlap its round trips, measured
// slower on small grids: the atomics queue behind them.
__device__ __forceinline__ float hist_rest_max(const RingArgs& r) {
  const float* hist = r.ring;
  float h = 0.0f;
  int i = 0;
  for (; i + 16 <= r.hist_len; i += 16) {
    float v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = hist[i + k];
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (i + k != r.hist_idx) h = fmaxf(h, v[k]);
  }
  for (; i < r.hist_len; ++i)
    if (i != r.hist_idx) h = fmaxf(h, hist[i]);
  return h;
}

// step 4: this call's amax (FP32 bits) enters the history at hist_idx; s and
// m = 1/s follow from the history's max h (max is exact, so its order does not
// matter) when h is finite and non-zero.
__device__ __forceinline__ void ring_fold(const RingArgs& r, uint32_t amax_bits, float hist_rest) {
  const float amax = __uint_as_float(amax_bits);
  r.ring[r.hist_idx] = amax;
  const float h = fmaxf(hist_rest, amax);
  if (h > 0.0f && h < __uint_as_float(0x7F800000u)) {
    const float s = (h / r.fp8_max) / r.margin;   // correctly rounded FP32 divisions
    r.ring[r.hist_len] = s;
    r.ring[r.hist_len + 1] = 1.0f / s;
  }
  if (r.amax_out) *r.amax_out = amax;
}

// steps 2-4 (mult: the multiplier this workgroup read from the ring).  The only
// workgroup of a grid goes straight to step 4 with its own max: every lane that
// read the multiplier used it before the workgroup's last barrier, so the fold
// cannot overtake those reads, and the ring's amax and ticket words stay zero.
__device__ __forceinline__ void ring_finish(const RingArgs& r, const RingTicket& t, uint32_t posted, float mult,
                                            unsigned num_wg) {
  uint32_t* amax_slot = reinterpret_cast<uint32_t*>(r.ring + r.hist_len + 2);
  uint32_t* ticket = reinterpret_cast<uint32_t*>(r.ring + r.hist_len + 3);
  if (t.solo) {
    ring_fold(r, posted, hist_rest_max(r));
    return;
  }
  const uint32_t tg = __hip_atomic_fetch_add(t.gctr, ticket_inc(posted, mult), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
  if (tg != t.members - 1) return;
  if (t.two_level) {
    const uint32_t gm = __hip_atomic_fetch_or(t.gmax, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(t.gmax, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(t.gctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t tm = __hip_atomic_fetch_max(amax_slot, gm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned ngroups = num_wg < kTicketGroups ? num_wg : kTicketGroups;
    const uint32_t tt = __hip_atomic_fetch_add(ticket, tm == 0xFFFFFFFFu ? 2u : 1u, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
    if (tt != ngroups - 1) return;
  }
  const uint32_t ab = __hip_atomic_fetch_or(amax_slot, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  ring_fold(r, ab, hist_rest_max(r));
  __hip_atomic_store(amax_slot, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The multiplier of a per-tensor call; not-finite values (a degenerate ring)
// are handled by the integer encoder.
__device__ __forceinline__ float ring_multiplier(const RingArgs& r, bool& slow) {
  const float m = r.ring[r.hist_len + 1];
  slow = !(fabsf(m) < __uint_as_float(0x7F800000u));
  return m;
}

// Workgroup max of a per-lane value, result valid in thread 0.
template <int THREADS>
__device__ __forceinline__ uint32_t block_max(uint32_t v) {
  v = wave_max(v);
  if constexpr (THREADS == 64) {
    return v;
  } else {
    __shared__ uint32_t red[THREADS / 64];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    uint32_t m = red[0];
#pragma unroll
    for (int w = 1; w < THREADS / 64; ++w) m = umax(m, red[w]);
    return m;
  }
}

// ---------------------------------------------------------------------------
// Per-tensor cast with row-major output (flat), then the fold
// ---------------------------------------------------------------------------
// 1024 threads x 4 chunks = 64 KiB of input per workgroup: one ticket per 64 KiB.
constexpr int kPtRowThreads = 1024;

template <int IN, int F>
__global__ __launch_bounds__(kPtRowThreads) void pt_row_kernel(const void* __restrict__ x, int64_t nchunks,
                                                                uint8_t* __restrict__ q, RingArgs r) {
  constexpr int kW = ChunkWords<IN>::kN;
  bool slow;
  const float mult = ring_multiplier(r, slow);
  uint32_t tmax = 0;
  const RingTicket tk = ring_ticket(r, blockIdx.x, gridDim.x);
  // one block of kPtRowThreads * kPtRowUnroll chunks per iteration; the grid covers
  // the input in one pass unless the launch caps it (no ticket scratch)
  for (int64_t b = int64_t(blockIdx.x) * kPtRowThreads * kPtRowUnroll; b < nchunks;
       b += int64_t(gridDim.x) * kPtRowThreads * kPtRowUnroll) {
    uint4 raw[kPtRowUnroll][kW];
#pragma unroll
    for (int u = 0; u < kPtRowUnroll; ++u) {
      const int64_t c = b + u * kPtRowThreads + threadIdx.x;
#pragma unroll
      for (int k = 0; k < kW; ++k) raw[u][k] = make_uint4(0, 0, 0, 0);
      if (c < nchunks) load_chunk_nt<IN>(x, c * 8, raw[u]);
    }
    uint32_t w[kPtRowUnroll][Words<F, 8>::kN];
#pragma unroll
    for (int u = 0; u < kPtRowUnroll; ++u) {
      float v[8];
      widen_chunk<IN>(raw[u], v);
      const uint32_t m = chunk_absmax<IN>(raw[u], v);
      tmax = amax_update(tmax, m, v);
      pt_encode_f32<F, 8>(v, mult, slow ? 0x7FFFFFFFu : m, w[u]);
    }
#pragma unroll
    for (int u = 0; u < kPtRowUnroll; ++u) {
      const int64_t c = b + u * kPtRowThreads + threadIdx.x;
      if (c < nchunks) store_row8<F>(q, c * 8, w[u]);
    }
  }
  const uint32_t bm = block_max<kPtRowThreads>(tmax);
  if (threadIdx.x == 0) ring_finish(r, tk, ring_post_max(tk, bm), mult, gridDim.x);
}

// ---------------------------------------------------------------------------
// Strip kernel: MX dual / MX column-wise / per-tensor transposed or dual
// ---------------------------------------------------------------------------
constexpr int kStripRows = 32;
constexpr int kStripCols = 128;
constexpr int kStripLoads = kStripRows * kStripCols / 8 / 64;   // 8 chunk loads per lane

enum StripMode : int {
  MX_DUAL = 0,     // MX row-wise + column-wise (transposed)
  MX_COL = 1,      // MX column-wise (transposed) only
  PT_COL = 3,      // per-tensor FP8, transposed output
  PT_DUAL = 4,     // per-tensor FP8, both
};

struct StripArgs {
  const void* x;
  int64_t rows, cols;
  uint8_t* q_row;       // MX_DUAL / PT_DUAL
  uint8_t* s_row;       // MX_DUAL
  uint8_t* q_col;       // transposed codes
  uint8_t* s_col;       // MX column scales
  uint32_t* amax_out;   // MX modes: max-accumulator (bit pattern of a non-negative float), may be null
  RingArgs ring;        // PT modes
  uint32_t had_mask;
  bool gemm_scales;     // MX scales in the GEMM layout (16-block groups outermost) instead of row-major
  int strips_c;         // strips along the column axis
  int bands;            // 128-row bands (4 strips each)
  int supertiles;       // bands * strips_c
};

template <int IN> struct LdsWord;   // element storage in LDS
template <> struct LdsWord<IN_BF16> { using T = uint16_t; };
template <> struct LdsWord<IN_F16> { using T = uint16_t; };
template <> struct LdsWord<IN_F32> { using T = float; };

// Column pass of one lane: columns c, c+1 of a 32-row segment of the LDS strip.
// Element (i, h) = row i, column c + h.  The LDS strip is re-read per column
// instead of holding both columns in registers (LDS bandwidth is plentiful,
// registers are not).
template <int IN>
__device__ __forceinline__ float lds_elem(const typename LdsWord<IN>::T* t, int pitch, int i, int h) {
  if constexpr (IN == IN_F32) {
    return t[i * pitch + h];
  } else {
    const uint32_t d = *reinterpret_cast<const uint32_t*>(t + i * pitch);
    const uint32_t bits = h ? (d >> 16) : (d & 0xFFFFu);
    if constexpr (IN == IN_BF16) return __uint_as_float(bits << 16);
    else return f16_bits_to_f32(bits);
  }
}

// Max |x| bit patterns of both columns (NaN > Inf).
template <int IN>
__device__ __forceinline__ void col_absmax(const typename LdsWord<IN>::T* t, int pitch, uint32_t (&cmax)[2]) {
  if constexpr (IN == IN_BF16) {
    uint32_t mp = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) mp = pk_umax16(mp, *reinterpret_cast<const uint32_t*>(t + i * pitch) & 0x7FFF7FFFu);
    cmax[0] = (mp & 0xFFFFu) << 16;
    cmax[1] = mp & 0xFFFF0000u;
  } else {
    cmax[0] = cmax[1] = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      cmax[0] = umax(cmax[0], abs_bits(lds_elem<IN>(t, pitch, i, 0)));
      cmax[1] = umax(cmax[1], abs_bits(lds_elem<IN>(t, pitch, i, 1)));
    }
  }
}

// Codes (and MX scale) of column h.
template <int IN, int F, int R, int MODE, bool HAD>
__device__ __forceinline__ uint32_t col_encode(const typename LdsWord<IN>::T* __restrict__ t, int pitch, int h,
                                               uint32_t cmax, float mult, bool pt_slow, uint32_t had_mask,
                                               uint32_t (&w)[Words<F, 32>::kN]) {
  constexpr bool kMX = MODE == MX_DUAL || MODE == MX_COL;
  if constexpr (IN == IN_BF16 && kMX && R == CEIL && !HAD) {
    // BF16 pairs of consecutive rows of the column straight into the converter
    if (cmax < 0x7F800000u) {
      const int e = shared_exponent<F, R>(cmax);
      if (e > -127) {
        const float scale = __uint_as_float(uint32_t(127 + e) << 23);
        const uint32_t sel = h ? 0x07060302u : 0x05040100u;
        uint32_t p[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t d0 = *reinterpret_cast<const uint32_t*>(t + (2 * i) * pitch);
          const uint32_t d1 = *reinterpret_cast<const uint32_t*>(t + (2 * i + 1) * pitch);
          p[i] = __builtin_amdgcn_perm(d1, d0, sel);
        }
        cvt_values_bf16<F, 32>(p, scale, w);
        return uint32_t(e + 127);
      }
    }
  }
  if constexpr (kMX && HAD) {
    float cv[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) cv[i] = lds_elem<IN>(t, pitch, i, h);
    hadamard32_inlane(cv, had_mask);
    cmax = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) cmax = umax(cmax, abs_bits(cv[i]));
    if (cmax >= 0x7F800000u) clear_nan_signs(cv);
    return mx_encode_f32<F, R, 32>(cv, cmax, w);
  } else {
    // the scale (or the per-tensor multiplier) is known: convert 16 values at a time
    const bool nonfinite = cmax >= 0x7F800000u;
    int e = 0;
    if constexpr (kMX) e = nonfinite ? 0 : shared_exponent<F, R>(cmax);
    constexpr int kHalfW = Words<F, 16>::kN;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      float cv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) cv[i] = lds_elem<IN>(t, pitch, 16 * half + i, h);
      uint32_t wh[kHalfW];
      if constexpr (kMX) {
        mx_encode_given<F, R, 16>(cv, nonfinite, e, wh);
      } else {
        pt_encode_f32<F, 16>(cv, mult, pt_slow ? 0x7FFFFFFFu : cmax, wh);
      }
#pragma unroll
      for (int k = 0; k < kHalfW; ++k) w[half * kHalfW + k] = wh[k];
    }
    if constexpr (kMX) return nonfinite ? 0xFFu : uint32_t(e + 127);
    return 0;
  }
}

// A workgroup of four waves quantizes one 128 x 128 supertile: wave j takes the
// 32-row strip j.  Each wave loads its strip, does the row-wise half from
// registers, stages the strip in its own LDS region and converts its column
// blocks, leaving the transposed codes in that region.  After one workgroup
// barrier all 256 threads write the supertile's transposed output so that 8
// consecutive lanes fill each 128-byte line (a lane-per-column store pattern
// would touch 64 lines per instruction), and the 4 column scales of each
// column go out as one store.
constexpr int kStripWaves = 4;

template <int IN, int F, int R, int MODE, bool HAD, bool AMAX>
__global__ __launch_bounds__(64 * kStripWaves) void strip_kernel(StripArgs a) {
  using W = typename LdsWord<IN>::T;
  constexpr bool kRowOut = MODE == MX_DUAL || MODE == PT_DUAL;
  constexpr bool kPT = MODE == PT_COL || MODE == PT_DUAL;
  constexpr bool kMXCol = MODE == MX_DUAL || MODE == MX_COL;
  constexpr int kW = ChunkWords<IN>::kN;
  constexpr int kPitch = kStripCols + 16 / int(sizeof(W));   // 16 bytes of padding keep 16-byte alignment
  constexpr int kRegion = kStripRows * kPitch * int(sizeof(W));  // bytes of LDS per wave
  constexpr int kColBytes = kStripRows * Fmt_<F>::kBits / 8;     // codes of one column of a strip: 32 or 16
  static_assert(kStripCols * kColBytes <= kRegion, "transposed codes must fit the strip region");
  __shared__ __attribute__((aligned(16))) uint8_t lds_all[kStripWaves][kRegion];
  __shared__ uint8_t sc_lds[kStripWaves][kStripCols];
  __shared__ uint32_t red[kStripWaves];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  W* const tile = reinterpret_cast<W*>(lds_all[wave]);
  const int lane_q = lane & 3;
  float mult = 1.0f;
  bool pt_slow = false;
  if constexpr (kPT) mult = ring_multiplier(a.ring, pt_slow);
  uint32_t tmax = 0;
  const int lrow = lane >> 4, lcol = (lane & 15) * 8;
  const int64_t scale_pitch = a.rows >> 5;        // column scales per column
  // per-tensor modes: one ticket per workgroup
  RingTicket tk{};
  uint32_t posted = 0;
  if constexpr (kPT) tk = ring_ticket(a.ring, blockIdx.x, gridDim.x);

  for (int T = blockIdx.x; T < a.supertiles; T += gridDim.x) {
    const int64_t rb = int64_t(T / a.strips_c) * 128;      // band origin
    const int64_t r0 = rb + 32 * wave;
    const int64_t c0 = int64_t(T % a.strips_c) * kStripCols;
    const bool strip_ok = r0 < a.rows;                      // ragged bottom band
    const bool col_ok = strip_ok && c0 + lcol < a.cols;

    if (strip_ok) {
      // ---- load: instruction i covers rows 4i .. 4i+3, 16 lanes (256 bytes) per row
      const uint8_t* xs = static_cast<const uint8_t*>(a.x) + (r0 * a.cols + c0) * int64_t(sizeof(W));
      uint4 raw[kStripLoads][kW];
#pragma unroll
      for (int i = 0; i < kStripLoads; ++i) {
#pragma unroll
        for (int kk = 0; kk < kW; ++kk) raw[i][kk] = make_uint4(0, 0, 0, 0);
        if (col_ok) load_chunk_nt<IN>(xs, (4 * i + lrow) * a.cols + lcol, raw[i]);
      }
#pragma unroll
      for (int i = 0; i < kStripLoads; ++i) {
        uint4* l = reinterpret_cast<uint4*>(&tile[(4 * i + lrow) * kPitch + lcol]);
#pragma unroll
        for (int kk = 0; kk < kW; ++kk) l[kk] = raw[i][kk];
        if (!col_ok) continue;
        if constexpr (AMAX || kPT || kRowOut) {
          float v[8];
          widen_chunk<IN>(raw[i], v);
          const uint32_t m = chunk_absmax<IN>(raw[i], v);
          if constexpr (AMAX || kPT) tmax = amax_update(tmax, m, v);
          if constexpr (kRowOut) {
            const int64_t e0 = (r0 + 4 * i + lrow) * a.cols + c0 + lcol;
            uint32_t w[Words<F, 8>::kN];
            if constexpr (MODE == MX_DUAL) {
              const uint32_t sc = row_chunk_mx<IN, F, R, false>(raw[i], v, m, 0u, lane_q, w);
              if (lane_q == 0)
                a.s_row[scale_offset(r0 + 4 * i + lrow, (c0 + lcol) >> 5, a.rows, a.cols >> 5, a.gemm_scales)] =
                    uint8_t(sc);
            } else {
              pt_encode_f32<F, 8>(v, mult, pt_slow ? 0x7FFFFFFFu : m, w);
            }
            store_row8<F>(a.q_row, e0, w);
          }
        }
      }
      // LDS accesses of one wave execute in order; keep the compiler from
      // moving the reads above the writes
      wave_lds_fence();
      // ---- column pass: lane l converts columns 2l, 2l+1 (cols is even: both or neither in range)
      uint32_t w[2][Words<F, 32>::kN];
      uint32_t sc[2] = {0, 0};
      const bool cc_ok = c0 + 2 * lane < a.cols;
      if (cc_ok) {
        const W* t = &tile[2 * lane];
        uint32_t cmax[2];
        col_absmax<IN>(t, kPitch, cmax);
#pragma unroll
        for (int h = 0; h < 2; ++h)
          sc[h] = col_encode<IN, F, R, MODE, HAD>(t, kPitch, h, cmax[h], mult, pt_slow, a.had_mask, w[h]);
      }
      wave_lds_fence();   // every lane has read the strip before it is overwritten
      if (cc_ok) {
        // transposed codes of this strip: column c at byte c * kColBytes of the region
        uint4* dst = reinterpret_cast<uint4*>(lds_all[wave] + 2 * lane * kColBytes);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int k = 0; k < kColBytes / 16; ++k)
            dst[h * (kColBytes / 16) + k] = make_uint4(w[h][4 * k], w[h][4 * k + 1], w[h][4 * k + 2], w[h][4 * k + 3]);
        }
        if constexpr (kMXCol) {
          sc_lds[wave][2 * lane] = uint8_t(sc[0]);
          sc_lds[wave][2 * lane + 1] = uint8_t(sc[1]);
        }
      }
    }
    if constexpr (kPT) {
      const uint32_t wm = wave_max(tmax);
      if (lane == 0) red[wave] = wm;
    }
    __syncthreads();
    if constexpr (kPT) {
      // post the workgroup's max now; the dependent ticket is taken after the stores
      if (threadIdx.x == 0) {
        uint32_t mm = red[0];
#pragma unroll
        for (int k = 1; k < kStripWaves; ++k) mm = umax(mm, red[k]);
        posted = ring_post_max(tk, mm);
      }
    }

    // ---- coalesced transposed stores: output line (column c, 128 rows of the band)
    {
      constexpr int kPieces = 128 * Fmt_<F>::kBits / 8 / 16;    // 16-byte pieces per column: 8 (FP8) or 4 (FP4)
      constexpr int kPerPiece = kPieces / kStripWaves;           // pieces per strip: 2 or 1
      constexpr int kPerByte = Fmt_<F>::kBits == 8 ? 1 : 2;
#pragma unroll
      for (int it = 0; it < kStripCols * kPieces / 256; ++it) {
        const int item = threadIdx.x + 256 * it;
        const int c = item / kPieces, pc = item % kPieces;
        const int sw = pc / kPerPiece;                           // strip (wave region) holding the piece
        const int64_t col = c0 + c, row = rb + 32 * sw;
        if (col < a.cols && row < a.rows) {
          const uint4 v = *reinterpret_cast<const uint4*>(lds_all[sw] + c * kColBytes + (pc % kPerPiece) * 16);
          *reinterpret_cast<uint4*>(a.q_col + (col * a.rows + rb) / kPerByte + pc * 16) = v;
        }
      }
      if constexpr (kMXCol) {
        if (threadIdx.x < kStripCols) {
          const int c = threadIdx.x;
          const int64_t col = c0 + c;
          if (col < a.cols) {
            uint8_t* sp = a.s_col + scale_offset(col, rb >> 5, a.cols, scale_pitch, a.gemm_scales);
            const int nst = a.rows - rb >= 128 ? 4 : int((a.rows - rb) >> 5);
            if (nst == 4 && (reinterpret_cast<uintptr_t>(sp) & 3u) == 0) {
              *reinterpret_cast<uint32_t*>(sp) = uint32_t(sc_lds[0][c]) | (uint32_t(sc_lds[1][c]) << 8) |
                                                 (uint32_t(sc_lds[2][c]) << 16) | (uint32_t(sc_lds[3][c]) << 24);
            } else {
              for (int k = 0; k < nst; ++k) sp[k] = sc_lds[k][c];
            }
          }
        }
      }
    }
    if (T + int(gridDim.x) < a.supertiles) __syncthreads();   // LDS is reused by the next supertile
  }

  if constexpr (kPT) {
    // an empty input runs no supertile: post nothing, still take the ticket
    if (threadIdx.x == 0) ring_finish(a.ring, tk, posted, mult, gridDim.x);
  } else if constexpr (AMAX) {
    // ---- per-tensor amax: one (conditional) atomic per workgroup
    const uint32_t m = wave_max(tmax);
    if (lane == 0) red[wave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t mm = red[0];
#pragma unroll
      for (int w = 1; w < kStripWaves; ++w) mm = umax(mm, red[w]);
      if (mm) atomic_max_u32(a.amax_out, mm);
    }
  }
}

__device__ __forceinline__ uint32_t u4_word(const uint4& u, int d) {
  return d == 0 ? u.x : d == 1 ? u.y : d == 2 ? u.z : u.w;
}

// Max |x| of 8 BF16 values as an FP32 bit pattern (a NaN makes it > 0x7F800000).
__device__ __forceinline__ uint32_t bf16_chunk_absmax(const uint4& c) {
  const uint32_t k = 0x7FFF7FFFu;
  const uint32_t m = pk_umax16(pk_umax16(c.x & k, c.y & k), pk_umax16(c.z & k, c.w & k));
  return umax(m & 0xFFFFu, m >> 16) << 16;
}

// ---------------------------------------------------------------------------
// Register-resident MX dual quantizer for BF16 input
// ---------------------------------------------------------------------------
// A workgroup of 4 waves takes a 128 x 128 tile, each wave a 64 x 64 quarter in
// which a lane holds rows 8h .. 8h+7 of columns 8g .. 8g+7 (8 loads of 16
// bytes, each load instruction reading 8 rows x 128 bytes; the input never goes
// through LDS).  A row-wise block (32 columns) sits in a quad and a column-wise
// block (32 rows) in 4 lanes of one 16-lane row, so both block maxima are DPP
// steps.  Both code outputs are staged in LDS and leave as 16-byte pieces of
// whole 128-byte lines; the scales are gathered in LDS and leave as one dword
// per row and per column.  The converter handles the round-up rule on finite
// blocks inline; every other block (non-finite, round-down rule, e = -127) goes
// through an out-of-line general encoder, which keeps the register count of the
// common path at 4 waves per SIMD.  (Waves that take the general encoder are
// slow: it is kept for non-finite blocks and blocks with a subnormal amax.)  The
// launch holds two workgroups per CU, each walking its share of the tiles.
constexpr int kDualTile = 128, kDualWave = 64;

// General MX encoding of 8 BF16 values of one block (element order, pairs
// low half first) whose max |x| bit pattern is bmax.  Out of line: rare.
template <int F, int R>
__device__ __attribute__((noinline)) uint2 dual_encode8_general(uint4 c, uint32_t bmax) {
  float v[8];
  const uint32_t w4[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = __uint_as_float(w4[j] << 16);
    v[2 * j + 1] = __uint_as_float(w4[j] & 0xFFFF0000u);
  }
  uint32_t w[Words<F, 8>::kN];
  mx_encode_f32<F, R, 8>(v, bmax, w);
  if constexpr (Words<F, 8>::kN == 2) return make_uint2(w[0], w[1]);
  else return make_uint2(w[0], 0u);
}

// Per-tensor amax of a BF16 chunk holding a NaN (which the amax ignores).  Out of line: rare.
__device__ __attribute__((noinline)) uint32_t dual_amax_nan_chunk(uint4 c) {
  const uint32_t w4[4] = {c.x, c.y, c.z, c.w};
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    m = umax(m, abs_bits_no_nan(__uint_as_float(w4[j] << 16)));
    m = umax(m, abs_bits_no_nan(__uint_as_float(w4[j] & 0xFFFF0000u)));
  }
  return m;
}

// Codes of 8 BF16 values (4 pairs, element order) of a block with max bmax; sets the scale code.
// Inline: finite blocks with e > -127 under either rule (the round-down rule
// first clamps each magnitude to max_elem * 2^e, exact in BF16 since every
// format maximum is a BF16 value, so the converter cannot overflow:
// sat(RNE(v)) = RNE(clamp(v))), and all-zero blocks (+-0 codes, scale 0).  A
// wave that leaves the inline path costs several microseconds of tail, so only
// non-finite blocks and blocks with a subnormal amax take the general encoder.
template <int F, int R>
__device__ __forceinline__ uint2 dual_encode8(const uint32_t (&p)[4], uint32_t bmax, uint32_t& scale_code) {
  constexpr int kB = Fmt_<F>::kBits;
  const int e = shared_exponent<F, R>(bmax);
  if (bmax < 0x7F800000u && e > -127) {
    uint32_t q[4] = {p[0], p[1], p[2], p[3]};
    if constexpr (R == FLOOR) {
      const uint32_t lim = (Fmt_<F>::kMaxBits >> 16) + (uint32_t(e) << 7);     // BF16 bits of max * 2^e
      const uint32_t limp = (lim & 0xFFFFu) * 0x10001u;
#pragma unroll
      for (int i = 0; i < 4; ++i) q[i] = (p[i] & 0x80008000u) | pk_umin16(p[i] & 0x7FFF7FFFu, limp);
    }
    uint32_t w[Words<F, 8>::kN];
    cvt_values_bf16<F, 8>(q, __uint_as_float(uint32_t(127 + e) << 23), w);
    scale_code = uint32_t(e + 127);
    if constexpr (Words<F, 8>::kN == 2) return make_uint2(w[0], w[1]);
    else return make_uint2(w[0], 0u);
  }
  if (bmax == 0u) {
    // +-0 codes: each element's sign bit in the top bit of its code
    scale_code = 0;
    if constexpr (kB == 8) {
      uint32_t b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) b[i] = ((p[i] >> 8) & 0x80u) | ((p[i] >> 16) & 0x8000u);
      return make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
    } else {
      uint32_t x = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) x |= (((p[i] >> 12) & 0x8u) | ((p[i] >> 24) & 0x80u)) << (8 * i);
      return make_uint2(x, 0u);
    }
  }
  scale_code = bmax >= 0x7F800000u ? 0xFFu : uint32_t(e + 127);
  return dual_encode8_general<F, R>(make_uint4(p[0], p[1], p[2], p[3]), bmax);
}

template <int F, int R, bool AMAX>
__global__ __launch_bounds__(256) void dual_bf16_kernel(StripArgs a, int tiles_c, int ntiles) {
  constexpr int kB = Fmt_<F>::kBits;
  constexpr int kLine = kDualTile * kB / 8;                          // code bytes per tile row / column
  __shared__ __attribute__((aligned(16))) uint8_t qr_lds[kDualTile * kLine];   // [tile row][tile column]
  __shared__ __attribute__((aligned(16))) uint8_t qc_lds[kDualTile * kLine];   // [tile column][tile row]
  __shared__ uint32_t srow_lds[kDualTile], scol_lds[kDualTile];                 // 4 scale codes per row / column
  __shared__ uint32_t red[4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // lane bits 0-1 and 4 give g, bits 2-3 and 5 give h
  const int g = (lane & 3) | ((lane >> 2) & 4), h = ((lane >> 2) & 3) | ((lane >> 3) & 4), lane_q = lane & 3;
  const int wro = (wave >> 1) * kDualWave, wco = (wave & 1) * kDualWave;
  uint8_t* const srl = reinterpret_cast<uint8_t*>(srow_lds) + wro * 4 + (wave & 1) * 2;
  uint8_t* const scl = reinterpret_cast<uint8_t*>(scol_lds) + wco * 4 + (wave >> 1) * 2;
  uint32_t tmax = 0;
  const uint32_t cols = uint32_t(a.cols);
  // whether the lane's 8 x 8 patch of tile t is in the matrix (rows and cols are
  // multiples of 32: a quad (row blocks) and the lanes h = 4k .. 4k+3 (column
  // blocks) are entirely in or out of range)
  auto patch_ok = [&](int t) {
    const int64_t tr = int64_t(t / tiles_c) * kDualTile, tc = int64_t(t % tiles_c) * kDualTile;
    return t < ntiles && tr + wro + 8 * h < a.rows && tc + wco + 8 * g < a.cols;
  };
  auto load_patch = [&](int t, uint4 (&dst)[8]) {
    const int64_t tr = int64_t(t / tiles_c) * kDualTile, tc = int64_t(t % tiles_c) * kDualTile;
    // the wave's origin is uniform: a scalar base plus a 32-bit lane offset
    // (the host keeps 64 * cols * 2 below 2^32)
    const uint8_t* xb = static_cast<const uint8_t*>(a.x) + ((tr + wro) * a.cols + tc + wco) * 2;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4_t v = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(xb + (uint32_t(8 * h + i) * cols + uint32_t(8 * g)) * 2u));
      dst[i] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  };
  // FP8: the next tile's input is loaded while this one converts and stores (32 more
  // VGPRs, within the two waves per SIMD of the launch).  On a BF16 8192 x 4096
  // input that measured 3% faster for FP8 and 4% slower for FP4, whose stores are
  // half as large.
  constexpr bool kPrefetch = kB == 8;
  uint4 raw[8];
  if constexpr (kPrefetch) {
    if (patch_ok(blockIdx.x)) load_patch(blockIdx.x, raw);
  }
  // one tile per workgroup, or several when the launch caps the grid
  for (int t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t tr = int64_t(t / tiles_c) * kDualTile, tc = int64_t(t % tiles_c) * kDualTile;
    const bool ok = patch_ok(t);
    uint4 nxt[8];
    if constexpr (kPrefetch) {
      if (patch_ok(t + int(gridDim.x))) load_patch(t + int(gridDim.x), nxt);
    } else if (ok) {
      load_patch(t, raw);
    }
    if (ok) {
      // ---- row-wise half
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t m = bf16_chunk_absmax(raw[i]);
        if constexpr (AMAX) tmax = umax(tmax, m <= 0x7F800000u ? m : dual_amax_nan_chunk(raw[i]));
        const uint32_t p[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
        uint32_t sc;
        const uint2 w = dual_encode8<F, R>(p, quad_max(m), sc);
        if (lane_q == 0) srl[(8 * h + i) * 4 + (g >> 2)] = uint8_t(sc);
        uint8_t* const d = qr_lds + (wro + 8 * h + i) * kLine + (wco + 8 * g) * kB / 8;
        if constexpr (kB == 8) *reinterpret_cast<u32x2_t*>(d) = u32x2_t{w.x, w.y};
        else *reinterpret_cast<uint32_t*>(d) = w.x;
      }
      // ---- column-wise half: dword d holds columns 2d (low halves) and 2d+1
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        uint32_t mp = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) mp = pk_umax16(mp, u4_word(raw[i], d) & 0x7FFF7FFFu);
        mp = pk_umax16(mp, dpp_u32<kRowRor4>(mp));
        mp = pk_umax16(mp, dpp_u32<kRowRor8>(mp));
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const uint32_t sel = k ? 0x07060302u : 0x05040100u;
          uint32_t p[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            p[i] = __builtin_amdgcn_perm(u4_word(raw[2 * i + 1], d), u4_word(raw[2 * i], d), sel);
          uint32_t sc;
          const uint2 w = dual_encode8<F, R>(p, k ? (mp & 0xFFFF0000u) : (mp << 16), sc);
          const int c = 8 * g + 2 * d + k;                     // column within the wave quarter
          uint8_t* const dst = qc_lds + (wco + c) * kLine + (wro + 8 * h) * kB / 8;
          if constexpr (kB == 8) *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{w.x, w.y};
          else *reinterpret_cast<uint32_t*>(dst) = w.x;
          if ((h & 3) == 0) scl[c * 4 + (h >> 2)] = uint8_t(sc);
        }
      }
    }
    __syncthreads();
    // ---- codes: 16-byte pieces, kLine / 16 consecutive threads per line; a piece
    // (16 FP8 or 32 FP4 codes) is entirely in or out of range
#pragma unroll
    for (int it = 0; it < kDualTile * kLine / 16 / 256; ++it) {
      const int item = threadIdx.x + 256 * it;
      const int r = item / (kLine / 16), pc = item % (kLine / 16);
      const int64_t e = pc * 16 * 8 / kB;                              // first element of the piece
      if (tr + r < a.rows && tc + e < a.cols) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(qr_lds + r * kLine + pc * 16);
        __builtin_nontemporal_store(v,
                                    reinterpret_cast<u32x4_t*>(a.q_row + ((tr + r) * a.cols + tc) * kB / 8 + pc * 16));
      }
      if (tc + r < a.cols && tr + e < a.rows) {
        const uint4 v = *reinterpret_cast<const uint4*>(qc_lds + r * kLine + pc * 16);
        *reinterpret_cast<uint4*>(a.q_col + ((tc + r) * a.rows + tr) * kB / 8 + pc * 16) = v;
      }
    }
    // ---- scales: thread j < 128 writes tile row j's 4 row scales, thread 128 + j
    // tile column j's 4 column scales (fewer, byte by byte, on a ragged edge)
    {
      const int j = threadIdx.x & (kDualTile - 1);
      const bool col_side = threadIdx.x >= kDualTile;
      const int64_t line = col_side ? tc + j : tr + j;
      const int64_t lines = col_side ? a.cols : a.rows;
      const int64_t other0 = col_side ? tr : tc, other = col_side ? a.rows : a.cols;
      if (line < lines) {
        const uint32_t v = col_side ? scol_lds[j] : srow_lds[j];
        uint8_t* dst =
            (col_side ? a.s_col : a.s_row) + scale_offset(line, other0 >> 5, lines, other >> 5, a.gemm_scales);
        const int64_t nb = (other - other0) >> 5;
        if (nb >= 4 && (reinterpret_cast<uintptr_t>(dst) & 3u) == 0) {
          *reinterpret_cast<uint32_t*>(dst) = v;
        } else {
          for (int b = 0; b < 4 && b < nb; ++b) dst[b] = uint8_t(v >> (8 * b));
        }
      }
    }
    if (t + int(gridDim.x) < ntiles) __syncthreads();   // the staging buffers are reused by the next tile
    if constexpr (kPrefetch) {
#pragma unroll
      for (int i = 0; i < 8; ++i) raw[i] = nxt[i];
    }
  }
  if constexpr (AMAX) {
    const uint32_t wm = wave_max(tmax);
    if (lane == 0) red[wave] = wm;
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t mm = umax(umax(red[0], red[1]), umax(red[2], red[3]));
      if (mm) atomic_max_u32(a.amax_out, mm);
    }
  }
}

// ---------------------------------------------------------------------------
// Register-resident MX column-wise quantizer for BF16 input (optionally with the
// fixed-sign 32-point Hadamard transform along each column block)
// ---------------------------------------------------------------------------
// A workgroup takes 32 * W rows x 128 columns, wave w the 32-row strip w (W = 4
// for FP8, 8 for FP4, so that a tile column is one 128-byte line of codes).  A
// lane holds rows 8q .. 8q+7 (q = lane & 3) of columns 8g .. 8g+7 (g = lane / 4):
// 8 loads of 16 bytes, each load instruction reading 4 rows x 256 bytes.  A
// column block (32 rows) is a quad, so its maximum is two DPP steps and the
// Hadamard transform is the quad butterfly (spans 1, 2, 4 in the lane, 8 and 16
// across it).  The transposed codes are staged in LDS and leave as 16-byte
// pieces of whole column lines; the W scales of a column leave as one store.

// General MX encoding of 8 FP32 values of one transformed block (non-finite or
// subnormal amax; NaNs made by the transform get a clear sign bit).  Out of line: rare.
template <int F, int R>
__device__ __attribute__((noinline)) uint2 col_encode8_general(float4 lo, float4 hi, uint32_t bmax) {
  float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  if (bmax >= 0x7F800000u) clear_nan_signs(v);
  uint32_t w[Words<F, 8>::kN];
  mx_encode_f32<F, R, 8>(v, bmax, w);
  if constexpr (Words<F, 8>::kN == 2) return make_uint2(w[0], w[1]);
  else return make_uint2(w[0], 0u);
}

// Codes of 8 FP32 values of a block with max |.| bit pattern bmax; sets the scale code.
template <int F, int R>
__device__ __forceinline__ uint2 col_encode8_f32(const float (&v)[8], uint32_t bmax, uint32_t& scale_code) {
  const int e = shared_exponent<F, R>(bmax);
  if (bmax < 0x7F800000u && e > -127) {
    uint32_t w[Words<F, 8>::kN];
    mx_encode_given<F, R, 8>(v, false, e, w);
    scale_code = uint32_t(e + 127);
    if constexpr (Words<F, 8>::kN == 2) return make_uint2(w[0], w[1]);
    else return make_uint2(w[0], 0u);
  }
  if (bmax == 0u) {
    // +-0 codes: each element's sign bit in the top bit of its code
    scale_code = 0;
    uint32_t c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = (__float_as_uint(v[j]) >> 31) << (Fmt_<F>::kBits - 1);
    uint32_t w[Words<F, 8>::kN];
    pack_codes<F, 8>(c, w);
    if constexpr (Words<F, 8>::kN == 2) return make_uint2(w[0], w[1]);
    else return make_uint2(w[0], 0u);
  }
  scale_code = bmax >= 0x7F800000u ? 0xFFu : uint32_t(e + 127);
  return col_encode8_general<F, R>(make_float4(v[0], v[1], v[2], v[3]), make_float4(v[4], v[5], v[6], v[7]), bmax);
}

template <int F> struct ColTile { static constexpr int kWaves = Fmt_<F>::kBits == 4 ? 8 : 4; };

template <int F, int R, bool HAD, bool AMAX>
__global__ __launch_bounds__(64 * ColTile<F>::kWaves) void col_bf16_kernel(StripArgs a, int tiles_c) {
  constexpr int kB = Fmt_<F>::kBits;
  constexpr int kW = ColTile<F>::kWaves;
  constexpr int kRows = 32 * kW;                                     // tile rows
  constexpr int kLine = kRows * kB / 8;                              // code bytes per tile column: 128
  constexpr int kThreads = 64 * kW;
  __shared__ __attribute__((aligned(16))) uint8_t qc_lds[kDualTile * kLine];   // [tile column][tile row]
  __shared__ __attribute__((aligned(8))) uint8_t scol_lds[kDualTile * kW];      // W scale codes per column
  __shared__ uint32_t red[kW];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane & 3, g = lane >> 2;
  const int t = blockIdx.x;
  const int64_t tr = int64_t(t / tiles_c) * kRows, tc = int64_t(t % tiles_c) * kDualTile;
  const int wro = wave * 32;
  uint8_t* const scl = scol_lds + wave;
  // rows are a multiple of 32 and cols of 8: a quad (a column block) and a
  // lane's 8 columns are entirely in or out of range
  const bool ok = tr + wro < a.rows && tc + 8 * g < a.cols;
  uint32_t tmax = 0;
  if (ok) {
    // the wave's origin is uniform: a scalar base plus a 32-bit lane offset
    // (the host keeps 32 * cols * 2 below 2^32)
    const uint8_t* xb = static_cast<const uint8_t*>(a.x) + ((tr + wro) * a.cols + tc) * 2;
    const uint32_t cols = uint32_t(a.cols);
    uint4 raw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4_t v = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(xb + (uint32_t(8 * q + i) * cols + uint32_t(8 * g)) * 2u));
      raw[i] = make_uint4(v[0], v[1], v[2], v[3]);
    }
    // dword d holds columns 2d (low halves) and 2d+1
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t mp = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) mp = pk_umax16(mp, u4_word(raw[i], d) & 0x7FFF7FFFu);
      if constexpr (AMAX) {
        const uint32_t m2 = umax(mp << 16, mp & 0xFFFF0000u);
        if (m2 <= 0x7F800000u) {
          tmax = umax(tmax, m2);
        } else {
#pragma unroll
          for (int i = 0; i < 8; i += 4)
            tmax = umax(tmax, dual_amax_nan_chunk(make_uint4(u4_word(raw[i], d), u4_word(raw[i + 1], d),
                                                             u4_word(raw[i + 2], d), u4_word(raw[i + 3], d))));
        }
      }
      if constexpr (!HAD) {
        mp = pk_umax16(mp, dpp_u32<kQuadXor1>(mp));
        mp = pk_umax16(mp, dpp_u32<kQuadXor2>(mp));
      }
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        uint32_t sc;
        uint2 w;
        if constexpr (HAD) {
          float v[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint32_t x = u4_word(raw[i], d);
            v[i] = __uint_as_float(k ? (x & 0xFFFF0000u) : (x << 16));
          }
          hadamard32_quad(v, a.had_mask, q);
          uint32_t m = 0;
#pragma unroll
          for (int i = 0; i < 8; ++i) m = umax(m, abs_bits(v[i]));
          w = col_encode8_f32<F, R>(v, quad_max(m), sc);
        } else {
          const uint32_t sel = k ? 0x07060302u : 0x05040100u;
          uint32_t p[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_perm(u4_word(raw[2 * i + 1], d), u4_word(raw[2 * i], d), sel);
          w = dual_encode8<F, R>(p, k ? (mp & 0xFFFF0000u) : (mp << 16), sc);
        }
        const int c = 8 * g + 2 * d + k;                     // column within the tile
        uint8_t* const dst = qc_lds + c * kLine + (wro + 8 * q) * kB / 8;
        if constexpr (kB == 8) *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{w.x, w.y};
        else *reinterpret_cast<uint32_t*>(dst) = w.x;
        if (q == 0) scl[c * kW] = uint8_t(sc);
      }
    }
  }
  if constexpr (AMAX) {
    const uint32_t wm = wave_max(tmax);
    if (lane == 0) red[wave] = wm;
  }
  __syncthreads();
  // ---- transposed codes: 16-byte pieces (16 FP8 or 32 FP4 codes of one column),
  // each entirely in or out of range
#pragma unroll
  for (int it = 0; it < kDualTile * kLine / 16 / kThreads; ++it) {
    const int item = threadIdx.x + kThreads * it;
    const int c = item / (kLine / 16), pc = item % (kLine / 16);
    if (tc + c < a.cols && tr + pc * 16 * 8 / kB < a.rows) {
      const uint4 v = *reinterpret_cast<const uint4*>(qc_lds + c * kLine + pc * 16);
      *reinterpret_cast<uint4*>(a.q_col + ((tc + c) * a.rows + tr) * kB / 8 + pc * 16) = v;
    }
  }
  // ---- column scales: thread j < 128 writes tile column j's W scales (fewer,
  // byte by byte, on a ragged bottom edge)
  if (threadIdx.x < kDualTile) {
    const int j = threadIdx.x;
    if (tc + j < a.cols) {
      uint8_t* dst = a.s_col + scale_offset(tc + j, tr >> 5, a.cols, a.rows >> 5, a.gemm_scales);
      const int64_t nb = (a.rows - tr) >> 5;
      if (nb >= kW && (reinterpret_cast<uintptr_t>(dst) & (kW - 1)) == 0) {
        if constexpr (kW == 8) *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(scol_lds + j * kW);
        else *reinterpret_cast<uint32_t*>(dst) = *reinterpret_cast<const uint32_t*>(scol_lds + j * kW);
      } else {
        for (int b = 0; b < kW && b < nb; ++b) dst[b] = scol_lds[j * kW + b];
      }
    }
  }
  if constexpr (AMAX) {
    if (threadIdx.x == 0) {
      uint32_t mm = red[0];
#pragma unroll
      for (int w = 1; w < kW; ++w) mm = umax(mm, red[w]);
      if (mm) atomic_max_u32(a.amax_out, mm);
    }
  }
}

// ---------------------------------------------------------------------------
// Per-tensor FP8 cast of a BF16 tensor, transposed output only
// ---------------------------------------------------------------------------
// A workgroup of 4 waves takes a 128 x 128 tile, each wave a 64 x 64 quarter in
// which lane (g, h) holds rows 8h .. 8h+7 of columns 8g .. 8g+7 (8 loads of 16
// bytes, each load instruction reading 8 rows x 128 bytes).  A lane's 8 rows of
// a column convert to 8 contiguous bytes of the transposed output; they are
// staged in LDS so that the tile leaves as 16-byte pieces of whole 128-byte
// lines (a 64-byte piece per column and wave would cost ~15% of the write
// bandwidth).  The input never goes through LDS.  Every workgroup then takes
// the two-level ring ticket; the last one folds the history.
constexpr int kPtTile = 128, kPtWave = 64;

template <int F>
__global__ __launch_bounds__(256) void pt_col_bf16_kernel(StripArgs a, int tiles_c, int ntiles) {
  __shared__ __attribute__((aligned(16))) uint8_t qc_lds[kPtTile * kPtTile];   // [tile column][tile row]
  __shared__ uint32_t red[4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane & 7, h = lane >> 3;
  bool pt_slow;
  const float mult = ring_multiplier(a.ring, pt_slow);
  const RingTicket tk = ring_ticket(a.ring, blockIdx.x, gridDim.x);
  const int wro = (wave >> 1) * kPtWave, wco = (wave & 1) * kPtWave;       // wave offset in the tile
  uint32_t tmax = 0, posted = 0;
  // one tile per workgroup, unless the launch caps the grid (loading the next
  // tile's input while this one converts and stores, as the FP8 dual does,
  // measured 5% slower on a BF16 8192 x 4096 input)
  for (int t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t tr = int64_t(t / tiles_c) * kPtTile, tc = int64_t(t % tiles_c) * kPtTile;
    // rows are a multiple of 32 and cols of 8: a lane's 8 x 8 block is in or out
    const bool ok = tr + wro + 8 * h < a.rows && tc + wco + 8 * g < a.cols;
    if (ok) {
      // the wave's origin is uniform: a scalar base plus a 32-bit lane offset
      // (the host keeps 64 * cols * 2 below 2^32)
      const uint8_t* xb = static_cast<const uint8_t*>(a.x) + ((tr + wro) * a.cols + tc + wco) * 2;
      const uint32_t cols = uint32_t(a.cols);
      uint4 raw[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const u32x4_t v = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4_t*>(xb + (uint32_t(8 * h + i) * cols + uint32_t(8 * g)) * 2u));
        raw[i] = make_uint4(v[0], v[1], v[2], v[3]);
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        // max |x| of columns 2d (low half) and 2d+1 (high half) over the lane's 8 rows
        uint32_t mp = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) mp = pk_umax16(mp, u4_word(raw[i], d) & 0x7FFF7FFFu);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const uint32_t cmax = k ? (mp & 0xFFFF0000u) : (mp << 16);
          float v[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint32_t x = u4_word(raw[i], d);
            v[i] = __uint_as_float(k ? (x & 0xFFFF0000u) : (x << 16));
          }
          if (cmax <= 0x7F800000u) {
            tmax = umax(tmax, cmax);
          } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) tmax = umax(tmax, abs_bits_no_nan(v[i]));
          }
          uint32_t w[2];
          pt_encode_f32<F, 8>(v, mult, pt_slow ? 0x7FFFFFFFu : cmax, w);
          *reinterpret_cast<u32x2_t*>(qc_lds + (wco + 8 * g + 2 * d + k) * kPtTile + wro + 8 * h) =
              u32x2_t{w[0], w[1]};
        }
      }
    }
    const bool last = t + int(gridDim.x) >= ntiles;
    if (last) {
      const uint32_t wm = wave_max(tmax);
      if (lane == 0) red[wave] = wm;
    }
    __syncthreads();
    // post the workgroup's max now; the dependent ticket is taken after the stores
    if (last && threadIdx.x == 0) posted = ring_post_max(tk, umax(umax(red[0], red[1]), umax(red[2], red[3])));
    // transposed codes: 8 consecutive threads per 128-byte line (column c, 128 rows)
    auto store_piece = [&](int item) {
      const int c = item >> 3, pc = item & 7;
      if (tc + c < a.cols && tr + 16 * pc < a.rows) {
        const uint4 v = *reinterpret_cast<const uint4*>(qc_lds + c * kPtTile + 16 * pc);
        *reinterpret_cast<uint4*>(a.q_col + (tc + c) * a.rows + tr + 16 * pc) = v;
      }
    };
    if (!last) {
#pragma unroll
      for (int it = 0; it < kPtTile * kPtTile / 16 / 256; ++it) store_piece(threadIdx.x + 256 * it);
      __syncthreads();   // the staging buffer is reused by the next tile
    } else if (wave != 0) {
      // the last tile's pieces go out from waves 1-3, so that wave 0 takes the ticket
      // at once: a wave's atomics return only after its own earlier stores complete
      for (int item = threadIdx.x - 64; item < kPtTile * kPtTile / 16; item += 192) store_piece(item);
    }
  }
  if (threadIdx.x == 0) ring_finish(a.ring, tk, posted, mult, gridDim.x);
}

template <typename K, typename... Args>
static mx_status_t launch(K kernel, dim3 grid, dim3 block, hipStream_t s, Args... args) {
  hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
  return hipGetLastError() == hipSuccess ? MX_OK : MX_ERR_LAUNCH;
}

template <int IN, int F, int R>
static mx_status_t rowwise_dispatch(const void* x, int64_t n, uint8_t* q, uint8_t* s, uint32_t* amax, bool had,
                                    uint32_t mask, int64_t lines, int64_t gemm_kblocks, hipStream_t st) {
  const int64_t nchunks = n / 8;
  const int64_t per = int64_t(kRowThreads) * kRowUnroll;
  const dim3 grid{unsigned((nchunks + per - 1) / per)}, block{unsigned(kRowThreads)};
  if (had) {
    return amax ? launch(rowwise_kernel<IN, F, R, true, true>, grid, block, st, x, nchunks, q, s, amax, mask, lines,
                                     gemm_kblocks)
                : launch(rowwise_kernel<IN, F, R, true, false>, grid, block, st, x, nchunks, q, s, amax, mask, lines,
                                     gemm_kblocks);
  }
  return amax ? launch(rowwise_kernel<IN, F, R, false, true>, grid, block, st, x, nchunks, q, s, amax, mask, lines,
                                     gemm_kblocks)
              : launch(rowwise_kernel<IN, F, R, false, false>, grid, block, st, x, nchunks, q, s, amax, mask, lines,
                                     gemm_kblocks);
}

// Workgroups of `kernel` resident at once on the current device (cached per
// kernel and device): the strip kernels run as one such wave of persistent
// workgroups that walk the supertiles (measured ~6-10% faster than one
// workgroup per supertile, whose launch rounds load and compute in lockstep).
// The cache is keyed by the kernel's address: instances of one kernel template
// share a signature but not their register and LDS footprints.
template <typename K>
static int64_t resident_workgroups(K kernel, int threads) {
  struct Entry { const void* fn; int dev; int64_t n; };
  static Entry cache[64];
  static int used = 0;
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  const void* fn = reinterpret_cast<const void*>(kernel);
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < used; ++i)
    if (cache[i].fn == fn && cache[i].dev == dev) return cache[i].n;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess || cus <= 0 ||
      per_cu <= 0)
    return 0;
  const int64_t n = int64_t(cus) * per_cu;
  if (used < 64) cache[used++] = Entry{fn, dev, n};
  return n;
}

template <typename K>
static mx_status_t launch_strips(K kernel, const StripArgs& a, hipStream_t st) {
  const int threads = 64 * kStripWaves;
  int64_t g = a.supertiles;
  const int64_t resident = resident_workgroups(kernel, threads);
  if (resident > 0 && g > resident) g = resident;
  if (a.ring.ring && !a.ring.tickets && g > kNullTicketGrid) g = kNullTicketGrid;
  if (g == 0) g = 1;   // an empty per-tensor input still folds
  return launch(kernel, dim3{unsigned(g)}, dim3{unsigned(threads)}, st, a);
}

template <int IN, int F, int R, int MODE>
static mx_status_t strip_dispatch(StripArgs& a, bool had, bool amax, hipStream_t st) {
  a.strips_c = int((a.cols + kStripCols - 1) / kStripCols);
  a.bands = int((a.rows + 127) / 128);
  a.supertiles = a.strips_c * a.bands;
  if constexpr (MODE == MX_COL) {
    if (had) {
      return amax ? launch_strips(strip_kernel<IN, F, R, MODE, true, true>, a, st)
                  : launch_strips(strip_kernel<IN, F, R, MODE, true, false>, a, st);
    }
  }
  return amax ? launch_strips(strip_kernel<IN, F, R, MODE, false, true>, a, st)
              : launch_strips(strip_kernel<IN, F, R, MODE, false, false>, a, st);
}

template <int IN, int F>
static mx_status_t pt_row_dispatch(const void* x, int64_t n, uint8_t* q, const RingArgs& r, hipStream_t st) {
  const int64_t nchunks = n / 8;
  const int64_t per = int64_t(kPtRowThreads) * kPtRowUnroll;
  int64_t g = (nchunks + per - 1) / per;
  if (!r.tickets && g > kNullTicketGrid / 2) g = kNullTicketGrid / 2;   // 1024-thread workgroups
  if (g == 0) g = 1;   // an empty input still folds
  return launch(pt_row_kernel<IN, F>, dim3{unsigned(g)}, dim3{unsigned(kPtRowThreads)}, st, x, nchunks, q, r);
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
                         int64_t lines, int64_t gemm_kblocks, hipStream_t st) {
    return rowwise_dispatch<IN, F, R>(x, n, q, s, amax, had, mask, lines, gemm_kblocks, st);
  }
};
template <int IN, int F, int R> struct ColOp {
  static mx_status_t run(StripArgs& a, bool had, bool amax, hipStream_t st) {
    if constexpr (IN == IN_BF16) {
      constexpr int kRows = 32 * ColTile<F>::kWaves;
      const int64_t tiles_c = (a.cols + kDualTile - 1) / kDualTile;
      const int64_t ntiles = tiles_c * ((a.rows + kRows - 1) / kRows);
      if (ntiles > 0 && ntiles < (int64_t(1) << 31) && a.cols < (int64_t(1) << 25)) {
        const dim3 grid{unsigned(ntiles)}, block{unsigned(64 * ColTile<F>::kWaves)};
        if (had)
          return amax ? launch(col_bf16_kernel<F, R, true, true>, grid, block, st, a, int(tiles_c))
                      : launch(col_bf16_kernel<F, R, true, false>, grid, block, st, a, int(tiles_c));
        return amax ? launch(col_bf16_kernel<F, R, false, true>, grid, block, st, a, int(tiles_c))
                    : launch(col_bf16_kernel<F, R, false, false>, grid, block, st, a, int(tiles_c));
      }
    }
    return strip_dispatch<IN, F, R, MX_COL>(a, had, amax, st);
  }
};
template <int IN, int F, int R> struct DualOp {
  static mx_status_t run(StripArgs& a, bool amax, hipStream_t st) {
    if constexpr (IN == IN_BF16) {
      const int64_t tiles_c = (a.cols + kDualTile - 1) / kDualTile;
      const int64_t ntiles = tiles_c * ((a.rows + kDualTile - 1) / kDualTile);
      if (ntiles > 0 && ntiles < (int64_t(1) << 31) && a.cols < (int64_t(1) << 25)) {
        // two workgroups per CU, each walking several tiles: on a BF16 8192 x 4096 input
        // (2048 tiles) 512 workgroups measured 3.8% faster than one per tile, while
        // 256, 384 and 640 were slower (too few waves, or unequal tile counts)
        const int64_t cus = device_cus();
        const int64_t cap = cus > 0 ? 2 * cus : ntiles;
        const dim3 grid{unsigned(ntiles < cap ? ntiles : cap)}, block{256u};
        return amax ? launch(dual_bf16_kernel<F, R, true>, grid, block, st, a, int(tiles_c), int(ntiles))
                    : launch(dual_bf16_kernel<F, R, false>, grid, block, st, a, int(tiles_c), int(ntiles));
      }
    }
    return strip_dispatch<IN, F, R, MX_DUAL>(a, false, amax, st);
  }
};
template <int IN, int F, int R> struct PtOp {
  static mx_status_t run(StripArgs& a, int layout, hipStream_t st) {
    if constexpr (F == E2M1 || R != FLOOR) {
      return MX_ERR_UNSUPPORTED;
    } else {
      if (layout == FP8_ROW) return pt_row_dispatch<IN, F>(a.x, a.rows * a.cols, a.q_row, a.ring, st);
      if (layout == FP8_TRANSPOSED) {
        const int64_t tiles_c = (a.cols + kPtTile - 1) / kPtTile;
        const int64_t ntiles = tiles_c * ((a.rows + kPtTile - 1) / kPtTile);
        if (IN == IN_BF16 && ntiles > 0 && ntiles < (int64_t(1) << 31) && a.cols < (int64_t(1) << 25)) {
          const int64_t cap = a.ring.tickets ? kTicketGrid : kNullTicketGrid;
          const int64_t g = ntiles <= cap ? ntiles : cap;
          return launch(pt_col_bf16_kernel<F>, dim3{unsigned(g)}, dim3{256u}, st, a, int(tiles_c), int(ntiles));
        }
        return strip_dispatch<IN, F, R, PT_COL>(a, false, false, st);
      }
      return strip_dispatch<IN, F, R, PT_DUAL>(a, false, false, st);
    }
  }
};

}  // namespace mxk

using namespace mxk;

extern "C" mx_status_t mx_quantize(const void* x, mx_dtype_t in, int64_t rows, int64_t cols, int block,
                                   mx_elem_t fmt, mx_scale_rule_t rule, mx_orient_t orient, int hadamard,
                                   uint32_t hadamard_sign_mask, uint8_t* q, uint8_t* scales,
                                   mx_scale_layout_t scale_layout, float* amax_out, hipStream_t stream) {
  if (scale_layout != MX_SCALES_ROW_MAJOR && scale_layout != MX_SCALES_GEMM) return MX_ERR_UNSUPPORTED;
  const bool gemm_scales = scale_layout == MX_SCALES_GEMM;
  if (fmt == MX_E2M3 || fmt == MX_E3M2) {
    if (gemm_scales) return MX_ERR_UNSUPPORTED;
    return fp6_quantize(x, in, rows, cols, block, fmt, rule, orient, hadamard, q, scales, amax_out, stream);
  }
  if (mx_status_t st = check_common_quant(in, rows, cols, block, fmt, rule); st != MX_OK) return st;
  if (orient != MX_ROWWISE && orient != MX_COLWISE_T) return MX_ERR_UNSUPPORTED;
  // the GEMM layout groups 16 K-blocks: the blocked axis is a multiple of 512
  if (gemm_scales && (orient == MX_ROWWISE ? cols : rows) % 512 != 0) return MX_ERR_SHAPE;
  const int64_t n = rows * cols;
  if (n > 0 && (!x || !q || !scales)) return MX_ERR_NULL;
  if (orient == MX_ROWWISE && cols % 32 != 0) return MX_ERR_SHAPE;
  if (orient == MX_COLWISE_T && (rows % 32 != 0 || cols % 8 != 0)) return MX_ERR_SHAPE;
  if (n > 0 && (misaligned(x) || misaligned(q))) return MX_ERR_ALIGN;
  // amax_out is a max-accumulator the caller initialises; nothing to do when empty
  uint32_t* amax = reinterpret_cast<uint32_t*>(amax_out);
  if (n == 0) return MX_OK;
  if (orient == MX_ROWWISE)
    return expand<RowOp>(in, fmt, rule, x, n, q, scales, amax, hadamard != 0, hadamard_sign_mask, rows,
                         gemm_scales ? cols / 32 : int64_t(0), stream);
  StripArgs a{};
  a.x = x; a.rows = rows; a.cols = cols; a.q_col = q; a.s_col = scales; a.amax_out = amax;
  a.had_mask = hadamard_sign_mask;
  a.gemm_scales = gemm_scales;
  return expand<ColOp>(in, fmt, rule, a, hadamard != 0, amax != nullptr, stream);
}

extern "C" mx_status_t mx_quantize_dual(const void* x, mx_dtype_t in, int64_t rows, int64_t cols, int block,
                                        mx_elem_t fmt, mx_scale_rule_t rule, uint8_t* q_row, uint8_t* s_row,
                                        uint8_t* q_colT, uint8_t* s_colT, mx_scale_layout_t scale_layout,
                                        float* amax_out, hipStream_t stream) {
  if (scale_layout != MX_SCALES_ROW_MAJOR && scale_layout != MX_SCALES_GEMM) return MX_ERR_UNSUPPORTED;
  const bool gemm_scales = scale_layout == MX_SCALES_GEMM;
  if (fmt == MX_E2M3 || fmt == MX_E3M2) {
    if (gemm_scales) return MX_ERR_UNSUPPORTED;
    return fp6_quantize_dual(x, in, rows, cols, block, fmt, rule, q_row, s_row, q_colT, s_colT, amax_out, stream);
  }
  if (mx_status_t st = check_common_quant(in, rows, cols, block, fmt, rule); st != MX_OK) return st;
  const int64_t n = rows * cols;
  if (n > 0 && (!x || !q_row || !s_row || !q_colT || !s_colT)) return MX_ERR_NULL;
  if (rows % 32 != 0 || cols % 32 != 0) return MX_ERR_SHAPE;
  if (gemm_scales && (rows % 512 != 0 || cols % 512 != 0)) return MX_ERR_SHAPE;
  if (n > 0 && (misaligned(x) || misaligned(q_row) || misaligned(q_colT))) return MX_ERR_ALIGN;
  // amax_out is a max-accumulator the caller initialises; nothing to do when empty
  uint32_t* amax = reinterpret_cast<uint32_t*>(amax_out);
  if (n == 0) return MX_OK;
  StripArgs a{};
  a.x = x; a.rows = rows; a.cols = cols; a.q_row = q_row; a.s_row = s_row; a.q_col = q_colT; a.s_col = s_colT;
  a.amax_out = amax;
  a.gemm_scales = gemm_scales;
  return expand<DualOp>(in, fmt, rule, a, amax != nullptr, stream);
}

// Argument checks of the delayed-scaling entry points (nothing is enqueued on failure).
static mx_status_t check_delayed(const void* x, mx_dtype_t in, int64_t rows, int64_t cols, mx_elem_t fmt,
                                 fp8_layout_t layout, const uint8_t* q, const uint8_t* qT, const float* ring,
                                 int hist_len, int hist_idx, float fp8_max, float margin) {
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
  if (reinterpret_cast<uintptr_t>(ring) & 3u) return MX_ERR_ALIGN;
  return MX_OK;
}

extern "C" mx_status_t fp8_quantize_delayed(const void* x, mx_dtype_t in, int64_t rows, int64_t cols,
                                            mx_elem_t fmt, fp8_layout_t layout, uint8_t* q, uint8_t* qT,
                                            float* ring, int hist_len, int hist_idx, float fp8_max, float margin,
                                            float* amax_out, uint32_t* ticket_scratch, hipStream_t stream) {
  if (mx_status_t st = check_delayed(x, in, rows, cols, fmt, layout, q, qT, ring, hist_len, hist_idx, fp8_max, margin);
      st != MX_OK)
    return st;
  if (reinterpret_cast<uintptr_t>(ticket_scratch) & 3u) return MX_ERR_ALIGN;
  StripArgs a{};
  a.x = x; a.rows = rows; a.cols = cols; a.q_row = q; a.q_col = qT;
  a.ring = RingArgs{ring, ticket_scratch, hist_len, hist_idx, fp8_max, margin, amax_out};
  return expand<PtOp>(in, fmt, MX_SCALE_FLOOR, a, int(layout), stream);
}

// ---------------------------------------------------------------------------
// Allocation-free variant: the ticket scratch lives in the library
// ---------------------------------------------------------------------------
// One array per device (each GPU the library runs on holds its own copy until
// the process ends).  It is zero when the code object loads and every call
// leaves it zero again (the last workgroup of each ticket group clears its
// words, the folding workgroup the top words), so each call finds it cleared.
// In host code `scratch` names a host-side stand-in: only the address that
// hipGetSymbolAddress returns for the current device is passed to kernels.
static __device__ __align__(256) uint32_t scratch[MX_TICKET_WORDS];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
uint32_t* scratch_dev_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up once per device.
uint32_t* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_dev_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    scratch_dev_ptr[dev] = static_cast<uint32_t*>(p);
  }
  return scratch_dev_ptr[dev];
}
}  // namespace

extern "C" mx_status_t fp8_quantize_delayed_static(const void* x, mx_dtype_t in, int64_t rows, int64_t cols,
                                                   mx_elem_t fmt, fp8_layout_t layout, uint8_t* q, uint8_t* qT,
                                                   float* ring, int hist_len, int hist_idx, float fp8_max,
                                                   float margin, float* amax_out, hipStream_t stream) {
  if (mx_status_t st = check_delayed(x, in, rows, cols, fmt, layout, q, qT, ring, hist_len, hist_idx, fp8_max, margin);
      st != MX_OK)
    return st;
  uint32_t* t = device_scratch();
  if (t == nullptr) return MX_ERR_LAUNCH;
  return fp8_quantize_delayed(x, in, rows, cols, fmt, layout, q, qT, ring, hist_len, hist_idx, fp8_max, margin,
                              amax_out, t, stream);
}
