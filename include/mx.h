/*
 * mx.h - C ABI of libmx, OCP microscaling (MX) block quantization and
 * block-scaled GEMM for AMD Instinct MI355X (gfx950).
 *
 * Sources the operations follow (cited by page and passage):
 *   [UE8M0] "EU8M0 FP8 ... domestic compute chips" article (ag-981.com, news 240):
 *           MX definition paragraph (k = 32, shared E8M0 scale X, Q_i * X ~ V_i),
 *           glossary entries FP8 / MX / EU8M0 / MXFP8, section 4 of the first part
 *           (amax-derived exponent, rounding that avoids overflow, saturation),
 *           second part section 1 (OCP round-down vs. round-up of log2(amax/destmax))
 *           and section 2 (transposes force re-quantization; dual row/column copies).
 *   [FP8PY] AstrAI astrai/extension/ops/fp8.py page (commit 432dfec): per-tensor
 *           quantize / quantize_dual with fused amax, transposed (K-contiguous)
 *           output, ring-state delayed scaling folded in-kernel by the last block,
 *           and the pre-quantized per-tensor FP8 GEMM mm_fp8.
 *   [FAF]   "Format-aware fusion" FP4 article (theaicronicle.com): MXFP4 with a
 *           fixed-sign 32-point Hadamard transform on the weight-gradient GEMM.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or synchronizes; each call validates its arguments
 *     on the host, enqueues its kernels on `stream` and returns.
 *   - Matrices are dense row-major with no padding: element (r, c) of a
 *     [rows][cols] tensor is at index r * cols + c.
 *   - Element codes are one byte each for E4M3 / E5M2.  E2M1 (FP4) codes are
 *     packed two per byte along the contiguous axis, element 2j in the low nibble.
 *   - Scales are E8M0 bytes: code c in [0, 254] means 2^(c - 127); 255 is NaN.
 *   - Pointers to tensors read or written with vector accesses (x, q, q_row,
 *     q_colT, qT, out, a, b) must be 16-byte aligned; scales and scalars have
 *     no alignment requirement.
 *   - Errors in the arguments return a status other than MX_OK before anything
 *     is enqueued.  MX_ERR_LAUNCH reports a failed kernel launch
 *     (hipGetLastError after the launch).  Device faults surface, as usual in
 *     HIP, at the caller's next synchronization.
 *   - Calls are reentrant; calls on different streams may overlap, except that
 *     two in-flight calls must not share an output or a ring buffer.
 */
#ifndef MX_BLOCK_SCALED_QUANTIZE_MX_H
#define MX_BLOCK_SCALED_QUANTIZE_MX_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element formats ([UE8M0] glossary 'FP8 (E4M3/E5M2)' and 'MXFP8'; values 0 and 1
 * as the format table of [FP8PY]).  E4M3 is OCP E4M3 (no Inf, NaN = S.1111.111,
 * max 448); E5M2 is OCP E5M2 (IEEE specials, max 57344); E2M1 has no specials
 * (max 6).  E2M3 (max 7.5) and E3M2 (max 28) are the FP6 members of the MX family
 * ([UE8M0] names MXFP8/6/4); they have no specials and are stored as a
 * little-endian bit stream along the row (element i at bits 6i .. 6i+5: 32
 * elements in 24 bytes).  FP6 is offered by mx_quantize (no Hadamard),
 * mx_quantize_dual, mx_dequantize and mx_gemm (as both operands); the other
 * entry points return MX_ERR_UNSUPPORTED for it. */
typedef enum { MX_E4M3 = 0, MX_E5M2 = 1, MX_E2M1 = 2, MX_E2M3 = 3, MX_E3M2 = 4 } mx_elem_t;

/* Storage type of a floating-point tensor argument. */
typedef enum { MX_F32 = 0, MX_BF16 = 1, MX_F16 = 2 } mx_dtype_t;

/* Shared-exponent rule for a block with amax > 0 ([UE8M0] second part, section 1):
 *   MX_SCALE_FLOOR: e = floor(log2 amax) - emax_elem  (OCP v1.0 round-down;
 *                   elements above the format maximum saturate);
 *   MX_SCALE_CEIL:  e = smallest integer with amax <= max_elem * 2^e
 *                   (round-up of log2(amax / destmax); never saturates).
 * e is clamped to [-127, 127].  A block whose values are all zero gets code 0. */
typedef enum { MX_SCALE_FLOOR = 0, MX_SCALE_CEIL = 1 } mx_scale_rule_t;

/* Block orientation of an MX quantization ([UE8M0] second part, section 2):
 *   MX_ROWWISE:   blocks are 32 consecutive elements of a row; codes [rows][cols]
 *                 (E2M1: [rows][cols/2]), scales [rows][cols/32].
 *   MX_COLWISE_T: blocks are 32 consecutive rows of a column, stored transposed
 *                 (the K-contiguous operand layout of an NT GEMM): codes
 *                 [cols][rows] (E2M1: [cols][rows/2]), scales [cols][rows/32]. */
typedef enum { MX_ROWWISE = 0, MX_COLWISE_T = 1 } mx_orient_t;

/* Layout of an E8M0 scale array of an operand with `lines` lines (rows of the
 * stored codes) and kblocks = K / 32 K-blocks per line ("format-aware fusion" FP4
 * article, section on the engineering of efficiency: quantizing producers
 * co-designed with the scale fields and layouts their consumers read):
 *   MX_SCALES_ROW_MAJOR: [lines][kblocks], byte (line, kb) at line * kblocks + kb;
 *   MX_SCALES_GEMM:      [kblocks / 16][lines][16], byte (line, kb) at
 *                        ((kb / 16) * lines + line) * 16 + kb % 16 -- the 16 scales
 *                        one GEMM stage of 16 K-blocks needs are contiguous per
 *                        line and the lines of a stage are contiguous, so mx_gemm
 *                        fetches a tile's stage of scales as whole cache lines.
 *                        Needs kblocks % 16 == 0 (K a multiple of 512). */
typedef enum { MX_SCALES_ROW_MAJOR = 0, MX_SCALES_GEMM = 1 } mx_scale_layout_t;

/* Output layout of the per-tensor FP8 quantizer ([FP8PY] quantize(transposed),
 * quantize_dual): q [rows][cols], qT [cols][rows], or both from one read. */
typedef enum { FP8_ROW = 0, FP8_TRANSPOSED = 1, FP8_DUAL = 2 } fp8_layout_t;

/* Size of the delayed-scaling ring state of fp8_quantize_delayed, in FP32 words
 * ([FP8PY] quantize() docstring: ring_state is [hist n | scale | legacy | amax | done]). */
#define MX_RING_WORDS(hist_len) ((hist_len) + 4)
/* Size of the optional ticket scratch of fp8_quantize_delayed, in uint32 words. */
#define MX_TICKET_WORDS 4096

typedef enum {
  MX_OK = 0,
  MX_ERR_NULL = 1,         /* a required pointer is NULL                         */
  MX_ERR_SHAPE = 2,        /* negative size or a size the layout cannot cut up   */
  MX_ERR_ALIGN = 3,        /* a vector-accessed pointer is not 16-byte aligned   */
  MX_ERR_UNSUPPORTED = 4,  /* format / rule / layout / block-size combination    */
  MX_ERR_LAUNCH = 5,       /* the HIP runtime rejected a kernel launch           */
  MX_ERR_ARG = 6           /* an out-of-range scalar argument                    */
} mx_status_t;

/* MX block quantization ([UE8M0] MX definition paragraph and section 4).
 *
 * For every block of 32 values V_i (orientation `orient`): amax = max |V_i|,
 * e = rule(amax) clamped to [-127, 127], scale code = e + 127, and
 * Q_i = RNE + saturating cast of V_i / 2^e to `fmt`.  A block holding NaN or
 * +-Inf gets scale code 255 and every Q_i set to the format's NaN with the
 * input's sign (E2M1, E2M3 and E3M2, having no NaN: the largest magnitude, +-6,
 * +-7.5, +-28).  -0 keeps its sign.  E2M3 / E3M2 (MXFP6): hadamard == 0; q is
 * [rows][cols * 3 / 4] (MX_ROWWISE) or [cols][rows * 3 / 4] (MX_COLWISE_T).
 *
 * hadamard != 0 first replaces each block by H32 * diag(s) * V, where s_j = -1
 * when bit j of `hadamard_sign_mask` is set and H32 is the unnormalised
 * Sylvester Hadamard matrix, evaluated as the in-place fast transform with
 * butterfly spans 1, 2, 4, 8, 16, every addition one FP32 operation ([FAF],
 * MXFP4 recipe).  A GEMM of two operands transformed with the same mask along
 * its reduction axis recovers the plain product with alpha = 1/32.
 *
 *   x        [rows][cols] input of type `in` (F32, BF16 or F16).
 *   block    must be 32 (MX defines k = 32 for every element type).
 *   q, scales  outputs, layouts as described at mx_orient_t; with
 *            scale_layout == MX_SCALES_GEMM the scales are stored in the GEMM
 *            layout (lines = rows, kblocks = cols / 32 for MX_ROWWISE; lines =
 *            cols, kblocks = rows / 32 for MX_COLWISE_T), which needs the blocked
 *            axis to be a multiple of 512 (MX_ERR_SHAPE otherwise) and is not
 *            offered for E2M3 / E3M2 (MX_ERR_UNSUPPORTED).
 *   amax_out optional (NULL to skip) in/out max-accumulator: on completion it
 *            holds max(*amax_out, max |x|) over the whole input, NaN entries
 *            ignored.  It must hold a non-negative FP32 value on entry: 0 gives
 *            this tensor's amax, an earlier result gives a running amax (e.g.
 *            over micro-batches).  An empty input leaves it unchanged.
 * Shapes: MX_ROWWISE needs cols % 32 == 0; MX_COLWISE_T needs rows % 32 == 0
 * and cols % 8 == 0.  rows == 0 or cols == 0 is valid (nothing is enqueued). */
mx_status_t mx_quantize(const void* x, mx_dtype_t in, int64_t rows, int64_t cols, int block,
                        mx_elem_t fmt, mx_scale_rule_t rule, mx_orient_t orient,
                        int hadamard, uint32_t hadamard_sign_mask,
                        uint8_t* q, uint8_t* scales, mx_scale_layout_t scale_layout,
                        float* amax_out, hipStream_t stream);

/* Dual-orientation MX quantization from a single read of x ([UE8M0] second part,
 * section 2: training keeps a row-wise and a column-wise quantized copy, and a
 * transposed MX copy must be re-quantized, not re-laid-out).  Produces exactly
 * what mx_quantize gives for MX_ROWWISE (q_row, s_row) and for MX_COLWISE_T
 * (q_colT, s_colT), plus the optional per-tensor amax (a max-accumulator, as
 * for mx_quantize).  scale_layout applies to both scale outputs (MX_SCALES_GEMM:
 * rows % 512 == 0 and cols % 512 == 0, FP8 / FP4 only).
 * Shapes: rows % 32 == 0 and cols % 32 == 0. */
mx_status_t mx_quantize_dual(const void* x, mx_dtype_t in, int64_t rows, int64_t cols, int block,
                             mx_elem_t fmt, mx_scale_rule_t rule,
                             uint8_t* q_row, uint8_t* s_row, uint8_t* q_colT, uint8_t* s_colT,
                             mx_scale_layout_t scale_layout, float* amax_out, hipStream_t stream);

/* Per-tensor FP8 quantization with delayed scaling ([FP8PY] quantize /
 * quantize_dual with ring_state, and its commit message).
 *
 * ring: caller-owned FP32 device buffer of MX_RING_WORDS(hist_len) = hist_len + 4
 *   words, the page's [hist n | scale | legacy | amax | done]:
 *     hist[0 .. hist_len-1]  the amax history (amaxes: non-negative, never NaN;
 *             a NaN placed there by the caller is passed over by the max);
 *     s       the dequantization scale (x ~ q * s);
 *     m       ("legacy") the multiplier the cast uses, m = 1 / s;
 *     amax    scratch that must read 0 before the first call;
 *     ticket  (uint32 bits) scratch that must read 0 before the first call.
 *   Initialise it to hist = 0, s = m = 1, amax = ticket = 0; every call leaves the
 *   amax and ticket words 0 again.  4-byte aligned.
 * ticket_scratch: optional (NULL allowed) caller-owned uint32 device buffer of
 *   MX_TICKET_WORDS words, all 0 before the first call and left 0 by every call.
 *   It holds 128 groups of (max, ticket) pairs, one group per 128-byte line,
 *   that spread the per-workgroup ticket over many cache lines, because atomics
 *   on one line serialize.  With NULL every workgroup takes its ticket on the
 *   ring's own amax and ticket words, and the launch caps the grid at a few
 *   hundred persistent workgroups to bound that queue; the codes and the ring
 *   are the same either way, only the time differs.  Small inputs (a grid of
 *   at most 16 workgroups) use the ring's words even when scratch is given, and
 *   a grid of one workgroup takes no ticket at all; the scratch is then left
 *   untouched.  4-byte aligned (128-byte alignment keeps each group on one
 *   line).  One scratch buffer may serve many rings, but not two calls in flight
 *   at once.
 *
 * Each call: y = fl32(x * m) with the m the ring holds at launch, q = RNE +
 * saturating cast of y to `fmt` (Inf saturates, NaN gives NaN), written as
 * `layout` says; a = max |x| (NaN ignored).  The last workgroup to finish (an
 * atomic ticket) then sets hist[hist_idx] = a, h = max(hist), and when
 * 0 < h < Inf publishes s = fl32(fl32(h / fp8_max) / margin), m = fl32(1 / s)
 * (correctly rounded FP32 divisions); otherwise s and m stay.  The next call on
 * the same ring sees the new m.  Calls sharing a ring (or a ticket scratch)
 * must be ordered (same stream or explicit events).
 *
 *   fmt      MX_E4M3 or MX_E5M2.
 *   q, qT    outputs: q [rows][cols] for FP8_ROW, qT [cols][rows] for
 *            FP8_TRANSPOSED, both for FP8_DUAL (the unused one may be NULL).
 *   hist_len 1..4096; 0 <= hist_idx < hist_len; fp8_max and margin finite > 0.
 *   amax_out optional: receives a.
 * Shapes: FP8_ROW needs cols % 8 == 0; FP8_TRANSPOSED and FP8_DUAL need
 * rows % 32 == 0 and cols % 8 == 0.  An empty input still folds (a = 0).
 * Errors, returned before any launch: MX_ERR_UNSUPPORTED (in, fmt, layout),
 * MX_ERR_SHAPE, MX_ERR_NULL (ring, or an output or x the layout needs),
 * MX_ERR_ARG (hist_len, hist_idx, fp8_max, margin), MX_ERR_ALIGN (x, q, qT not
 * 16-byte aligned; ring or ticket_scratch not 4-byte aligned); MX_ERR_LAUNCH. */
mx_status_t fp8_quantize_delayed(const void* x, mx_dtype_t in, int64_t rows, int64_t cols,
                                 mx_elem_t fmt, fp8_layout_t layout, uint8_t* q, uint8_t* qT,
                                 float* ring, int hist_len, int hist_idx, float fp8_max,
                                 float margin, float* amax_out, uint32_t* ticket_scratch,
                                 hipStream_t stream);

/* fp8_quantize_delayed for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same operation, arguments and results as
 * fp8_quantize_delayed, with the ticket scratch taken from a fixed array inside
 * the library (MX_TICKET_WORDS uint32 words = 16 KiB per device, held by each
 * GPU the library runs on until the process ends) instead of a caller buffer.
 * The call allocates nothing: the array's device address is looked up once per
 * device (hipGetSymbolAddress) on the first call made with that device current.
 * The array is zero at load and every call leaves it zero.  Its size does not
 * depend on the input (128 ticket groups serve any number of workgroups), so
 * no input is rejected for its size.  All calls on one GPU share the array:
 * calls that overlap on one GPU (different streams without ordering) race on
 * it and must not be issued; calls ordered on one stream are safe.
 * Errors: those of fp8_quantize_delayed, and MX_ERR_LAUNCH when the array's
 * device address cannot be obtained. */
mx_status_t fp8_quantize_delayed_static(const void* x, mx_dtype_t in, int64_t rows, int64_t cols,
                                        mx_elem_t fmt, fp8_layout_t layout, uint8_t* q, uint8_t* qT,
                                        float* ring, int hist_len, int hist_idx, float fp8_max,
                                        float margin, float* amax_out, hipStream_t stream);

/* MX dequantization ([UE8M0] first part, section 2: decoding an E8M0 scale is an
 * exponent shift): out = Q_i * 2^(c - 127), computed exactly and rounded once to
 * `out_dtype` (F32 or BF16; overflow gives +-Inf, scale 255 or a NaN code gives
 * NaN).  `rows`, `cols` describe the dequantized tensor [rows][cols]:
 *   MX_ROWWISE:   q [rows][cols] (E2M1 [rows][cols/2]), scales [rows][cols/32];
 *   MX_COLWISE_T: q [cols][rows] (E2M1 [cols][rows/2]), scales [cols][rows/32],
 *                 and out is still [rows][cols] (the transpose is undone).
 * scale_layout: how `scales` is stored (MX_SCALES_GEMM: lines and kblocks as for
 * mx_quantize; the blocked axis a multiple of 512).
 * Shapes: the blocked axis must be a multiple of 32. */
mx_status_t mx_dequantize(const uint8_t* q, const uint8_t* scales, int64_t rows, int64_t cols,
                          int block, mx_elem_t fmt, mx_orient_t orient, mx_scale_layout_t scale_layout,
                          void* out, mx_dtype_t out_dtype, hipStream_t stream);

/* Row-wise MXFP4 with stochastic rounding ([FAF], the 37.2K tokens/s
 * configuration: row gradients quantized to MXFP4 with stochastic rounding; the
 * page names the technique without defining it).  Definition implemented:
 *   - the block scale X is the ordinary MX scale of `rule` (as mx_quantize);
 *   - each element V_i has its own random word rand[i]; the magnitude
 *     y = |V_i| / X is exact; an E2M1 magnitude is kept, y >= 6 saturates to 6,
 *     and strictly between adjacent magnitudes lo < hi the code is hi iff
 *     rand[i] < floor(2^32 (y - lo) / (hi - lo)), else lo (up with probability
 *     (y - lo) / (hi - lo) to within 2^-32);
 *   - the sign bit is copied (-0 stays -0); a block holding NaN or +-Inf gets
 *     scale 255 and every code +-6 with the input's sign.
 *
 *   x        [rows][cols] input of type `in` (F32, BF16 or F16), 16-byte aligned.
 *   rand     [rows][cols] uint32 random words (device), 16-byte aligned; the
 *            caller draws them (any generator); the same words give the same codes.
 *   fmt      must be MX_E2M1; block must be 32.
 *   q        [rows][cols/2] packed codes (element 2j in the low nibble), 16-byte aligned.
 *   scales   [rows][cols/32] E8M0 codes.
 *   amax_out optional max-accumulator, as for mx_quantize.
 * Shapes: cols % 32 == 0; rows == 0 or cols == 0 enqueues nothing.  Errors:
 * MX_ERR_UNSUPPORTED (fmt, in, rule or block), MX_ERR_SHAPE, MX_ERR_NULL,
 * MX_ERR_ALIGN, returned without a launch; MX_ERR_LAUNCH. */
mx_status_t mx_quantize_sr(const void* x, mx_dtype_t in, int64_t rows, int64_t cols, int block,
                           mx_elem_t fmt, mx_scale_rule_t rule, const uint32_t* rand,
                           uint8_t* q, uint8_t* scales, float* amax_out, hipStream_t stream);

/* Block-scaled GEMM ([UE8M0] MX definition paragraph: the matrix unit consumes the
 * codes and scales of both operands and accumulates in FP32):
 *   C[m][n] = alpha * sum_k (Qa[m][k] 2^(sa[m][k/32]-127)) (Qb[n][k] 2^(sb[n][k/32]-127))
 * with FP32 accumulation, then one rounding to `c_dtype` (BF16 or F32).
 *   a  [M][K] codes (E2M1: [M][K/2]; E2M3 / E3M2: [M][3K/4] bit streams), sa [M][K/32];
 *   b  [N][K] codes (likewise), sb [N][K/32]  -- B^T, K-contiguous ("NT");
 *   c  [M][ldc] output rows, ldc >= N; c needs only the alignment of its element
 *      type (it may be a column slice of a wider matrix).
 * fmt_a / fmt_b: both FP8 (E4M3 / E5M2, any mix), both FP6 (E2M3 / E3M2, any mix;
 * packed as mx_quantize writes them) or both E2M1.
 * scale_layout: how sa and sb are stored; MX_SCALES_GEMM (sa with lines = M, sb
 * with lines = N, kblocks = K / 32) needs K % 512 == 0.
 * Shapes: K % 32 == 0, and K % 64 == 0 for FP6 (K == 0 writes zeros); any M, N >= 0.
 * Accumulation: the matrix unit sums the FP8 products of each MFMA step with a
 * fixed-point alignment of limited width, not with IEEE FP32 rounding after
 * every product; the FP32 result is within a few 2^-12 of the largest product
 * of each 64-long K-step of the exact sum. */
mx_status_t mx_gemm(const uint8_t* a, const uint8_t* sa, mx_elem_t fmt_a,
                    const uint8_t* b, const uint8_t* sb, mx_elem_t fmt_b, mx_scale_layout_t scale_layout,
                    int64_t M, int64_t N, int64_t K, float alpha,
                    void* c, mx_dtype_t c_dtype, int64_t ldc, hipStream_t stream);

/* Block-scaled GEMM with the result re-quantized to MX in the epilogue ([UE8M0]
 * MX definition paragraph: the accumulated FP32 output is quantized to MX when the
 * next operator needs MX; [FAF], format-aware fusion: the quantizing producer is
 * fused with the GEMM that feeds it).  The FP32 result
 *   C32[m][n] = fl32(alpha * acc[m][n])     (acc and alpha exactly as mx_gemm with F32 out)
 * is never written; its row-wise MX quantization (k = 32 along n, `fmt_c`, `rule_c`,
 * the mx_quantize rules: amax, shared E8M0 scale, RNE + saturation, NaN/Inf blocks)
 * is, byte for byte what mx_quantize(C32, fmt_c, rule_c, MX_ROWWISE) would give:
 *   qc        [M][N] codes (E2M1: [M][N/2] packed), 16-byte aligned;
 *   sc        [M][N/32] E8M0 scales;
 *   amax_out  optional max-accumulator of |C32| (NaN excluded), as for mx_quantize.
 * Operands (and scale_layout, which applies to sa and sb; sc is row-major) as
 * mx_gemm, FP8 or FP4 only.  Shapes: K % 32 == 0, N % 32 == 0, any M.
 * Errors: as mx_gemm, plus MX_ERR_UNSUPPORTED for FP6 operands and for fmt_c / rule_c,
 * and MX_ERR_NULL for qc / sc. */
mx_status_t mx_gemm_requant(const uint8_t* a, const uint8_t* sa, mx_elem_t fmt_a,
                            const uint8_t* b, const uint8_t* sb, mx_elem_t fmt_b,
                            mx_scale_layout_t scale_layout, int64_t M, int64_t N, int64_t K, float alpha,
                            mx_elem_t fmt_c, mx_scale_rule_t rule_c, uint8_t* qc, uint8_t* sc,
                            float* amax_out, hipStream_t stream);

/* Per-tensor FP8 GEMM ([FP8PY], mm_fp8: pre-quantized FP8 operands of one format,
 * 2-D or 3-D with the batch broadcast as in matmul, inner-transposed operands
 * folded into the layout, the combined dequantization scale, an optional BF16
 * bias added in the FP32 epilogue, BF16 result):
 *   C[p] = op(a[p]) op(b[p]) * scale (+ bias),   p = 0 .. batch-1
 * where op(x) is x transposed when the matching trans flag is set.
 *   a      trans_a == 0: [batch_a][M][K] codes; trans_a != 0: [batch_a][K][M].
 *   b      trans_b == 0: [batch_b][K][N] codes; trans_b != 0: [batch_b][N][K].
 *          batch_a = batch when a_batched != 0, else 1 (the one matrix is used for
 *          every p); likewise b.  Both 16-byte aligned.
 *   fmt    MX_E4M3 or MX_E5M2 (both operands).
 *   scale  device pointer to one float: the combined dequantization scale (for
 *          the delayed-scaling ring, the product of the two operands' s).  Read by
 *          the kernel, so it may be produced on the stream without a host sync.
 *   bias   device BF16 [N] or NULL; 2-byte aligned.
 *   c      [batch][M][N] BF16, 2-byte aligned.
 * Each output is fl32(acc * scale + bias) (one FMA; acc * scale without a bias),
 * rounded once to BF16 (RNE); acc is the FP32 accumulation of the exact FP8
 * products, with the matrix unit's accumulation described under mx_gemm.
 * Shapes: K % 16 == 0 (K == 0 writes the bias or zeros); batch <= 65535; any M, N.
 * Errors: MX_ERR_UNSUPPORTED (fmt), MX_ERR_SHAPE, MX_ERR_NULL (c, scale, or a / b
 * when K > 0), MX_ERR_ALIGN; MX_ERR_LAUNCH. */
mx_status_t mm_fp8(const uint8_t* a, const uint8_t* b, mx_elem_t fmt, int64_t batch,
                   int64_t M, int64_t N, int64_t K, int a_batched, int b_batched,
                   int trans_a, int trans_b, const float* scale, const uint16_t* bias,
                   uint16_t* c, hipStream_t stream);

/* Human-readable name of a status code (static storage). */
const char* mx_status_str(mx_status_t status);

/* Library ABI version (major * 100 + minor). */
int mx_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MX_BLOCK_SCALED_QUANTIZE_MX_H */
