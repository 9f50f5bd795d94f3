"""MX block quantization, dequantization and per-tensor amax (CPU oracle).

Test infrastructure only (see ``oracle/__init__``).

Method ([UE8M0] MX definition paragraph and section 4): a tensor is cut into
blocks of k = 32 values that share one scale X, an unsigned power of two stored
as E8M0; each value V_i is stored as an element code Q_i with Q_i * X ~ V_i.
The scale exponent comes from the block's amax; the elements are cast with
round-to-nearest-even and saturation.

Two rules for the shared exponent ([UE8M0] section 1 of the second part, on
rounding to a power of two, and the MXFP8 recipe paragraph):

* ``floor`` - OCP v1.0 round-down: e = floor(log2 amax) - emax_elem.
* ``ceil``  - overflow-safe round-up: e = ceil(log2(amax / destmax)), i.e. the
  smallest integer e with amax <= destmax * 2^e.

Readings of points the pages leave open:
* the exponent is clamped to [-127, 127], the E8M0 range;
* an all-zero block gets scale code 0 and +-0 codes;
* a block holding NaN or +-Inf gets the E8M0 NaN scale (0xFF) and every element
  code is the element format's NaN with the input's sign (E2M1, having no NaN,
  gets +-6);
* -0 keeps its sign bit;
* column-wise blocks are 32 consecutive rows of one column, and the column-wise
  result is stored transposed: codes [cols][rows], scales [cols][rows/32];
* FP4 codes are packed two per byte, element 2j in the low nibble.
"""

import numpy as np

from .formats import E8M0_NAN, encode, decode, e8m0_decode, fmt_of

BLOCK = 32
SCALE_RULES = ("floor", "ceil")


def _floor_log2(a: np.ndarray) -> np.ndarray:
    """floor(log2 a) for finite a > 0, exact (frexp is exact in float64)."""
    return np.frexp(a)[1].astype(np.int64) - 1


def scale_exponent(amax, fmt, rule) -> np.ndarray:
    """Shared exponent e of each block (before the E8M0 bias), clamped to [-127, 127].

    ``amax`` are finite non-negative values (float64 holds them exactly).
    """
    f = fmt_of(fmt)
    a = np.asarray(amax, dtype=np.float64)
    pos = a > 0
    safe = np.where(pos, a, 1.0)
    if rule == "floor":
        e = _floor_log2(safe) - f.emax
    elif rule == "ceil":
        # smallest e with amax <= destmax * 2^e; it lies within one of
        # floor(log2 amax) - emax, every product below is exact in float64
        e0 = _floor_log2(safe) - f.emax
        e = np.where(safe <= np.ldexp(f.max_value, (e0 - 1).astype(np.int32)), e0 - 1,
                     np.where(safe <= np.ldexp(f.max_value, e0.astype(np.int32)), e0, e0 + 1))
    else:
        raise ValueError(f"unknown scale rule {rule!r}")
    e = np.clip(e, -127, 127)
    return np.where(pos, e, -127)


def quantize_blocks(blocks, fmt, rule):
    """Quantize an array [..., 32] of FP32 values, one MX block per last-axis row.

    Returns (codes uint8 [..., 32], scales uint8 [...]).
    """
    f = fmt_of(fmt)
    x = np.asarray(blocks, dtype=np.float32).astype(np.float64)
    assert x.shape[-1] == BLOCK
    finite = np.all(np.isfinite(x), axis=-1)
    amax = np.max(np.abs(np.where(np.isfinite(x), x, 0.0)), axis=-1)
    e = scale_exponent(amax, f, rule)
    scale = (e + 127).astype(np.int64)
    scale = np.where(finite, scale, E8M0_NAN)
    # V_i / X, exact in float64
    v = np.ldexp(np.where(np.isfinite(x), x, 0.0), (-e)[..., None].astype(np.int32))
    codes = encode(v, f).astype(np.int64)
    nan_codes = f.nan_code | np.where(np.signbit(x), f.sign_bit, 0)
    codes = np.where(finite[..., None], codes, nan_codes)
    return codes.astype(np.uint8), scale.astype(np.uint8)


def pack_fp4(codes) -> np.ndarray:
    """Pack 4-bit codes along the last axis, element 2j in the low nibble of byte j."""
    c = np.asarray(codes).astype(np.uint8)
    assert c.shape[-1] % 2 == 0
    return ((c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)).astype(np.uint8)


def unpack_fp4(packed) -> np.ndarray:
    p = np.asarray(packed).astype(np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def pack_fp6(codes) -> np.ndarray:
    """Pack 6-bit codes along the last axis as a little-endian bit stream: element i
    occupies bits 6i .. 6i+5 of the row, so 4 elements fill 3 bytes (the FP4 nibble
    order, element 2j in the low nibble, is the same rule at 4 bits)."""
    c = np.asarray(codes).astype(np.uint32) & 0x3F
    assert c.shape[-1] % 4 == 0
    g = c.reshape(c.shape[:-1] + (c.shape[-1] // 4, 4))
    word = g[..., 0] | (g[..., 1] << 6) | (g[..., 2] << 12) | (g[..., 3] << 18)     # 24 bits
    out = np.stack([word & 0xFF, (word >> 8) & 0xFF, (word >> 16) & 0xFF], axis=-1)
    return out.reshape(c.shape[:-1] + (c.shape[-1] * 3 // 4,)).astype(np.uint8)


def unpack_fp6(packed) -> np.ndarray:
    p = np.asarray(packed).astype(np.uint32)
    assert p.shape[-1] % 3 == 0
    g = p.reshape(p.shape[:-1] + (p.shape[-1] // 3, 3))
    word = g[..., 0] | (g[..., 1] << 8) | (g[..., 2] << 16)
    out = np.stack([(word >> (6 * k)) & 0x3F for k in range(4)], axis=-1)
    return out.reshape(p.shape[:-1] + (p.shape[-1] * 4 // 3,)).astype(np.uint8)


def pack_codes(codes, fmt) -> np.ndarray:
    """Storage form of a code array: FP4 and FP6 packed along the last axis, FP8 as is."""
    f = fmt_of(fmt)
    if f.bits == 4:
        return pack_fp4(codes)
    if f.bits == 6:
        return pack_fp6(codes)
    return np.asarray(codes).astype(np.uint8)


def unpack_codes(packed, fmt) -> np.ndarray:
    f = fmt_of(fmt)
    if f.bits == 4:
        return unpack_fp4(packed)
    if f.bits == 6:
        return unpack_fp6(packed)
    return np.asarray(packed).astype(np.uint8)


def scales_to_gemm_layout(scales) -> np.ndarray:
    """E8M0 scales of an operand, [lines][kblocks] row-major, rearranged into the
    GEMM layout [kblocks / 16][lines][16]: byte (line, kb) moves to
    ((kb // 16) * lines + line) * 16 + kb % 16.  A pure permutation: K-blocks in
    groups of 16 (one GEMM stage), each group's lines contiguous ("format-aware
    fusion" FP4 article: the quantizer writes the scale layout its consumer reads;
    the layout itself is this library's reading, defined in its header)."""
    s = np.asarray(scales, dtype=np.uint8)
    lines, kblocks = s.shape
    assert kblocks % 16 == 0, "the GEMM layout needs kblocks % 16 == 0"
    out = np.empty((kblocks // 16, lines, 16), dtype=np.uint8)
    for kb in range(kblocks):
        out[kb // 16, :, kb % 16] = s[:, kb]
    return out


def scales_from_gemm_layout(gemm_scales, lines, kblocks) -> np.ndarray:
    """Inverse of scales_to_gemm_layout: back to [lines][kblocks]."""
    g = np.asarray(gemm_scales, dtype=np.uint8).reshape(kblocks // 16, lines, 16)
    out = np.empty((lines, kblocks), dtype=np.uint8)
    for kb in range(kblocks):
        out[:, kb] = g[kb // 16, :, kb % 16]
    return out


def quantize_rowwise(x, fmt, rule, hadamard_mask=None):
    """Row-wise MX quantization of a 2-D FP32 array [R][C], blocks of 32 along C.

    Returns (codes [R][C] uint8 - or [R][C/2] packed for E2M1, [R][3C/4] for FP6 -,
    scales [R][C/32]).
    With ``hadamard_mask`` (a 32-bit int), each block is first passed through the
    fixed-sign 32-point Hadamard transform of ``oracle.hadamard``.
    """
    f = fmt_of(fmt)
    x = np.asarray(x, dtype=np.float32)
    R, C = x.shape
    assert C % BLOCK == 0
    blocks = x.reshape(R, C // BLOCK, BLOCK)
    if hadamard_mask is not None:
        from .hadamard import hadamard32
        blocks = hadamard32(blocks, hadamard_mask)
    codes, scales = quantize_blocks(blocks, f, rule)
    return pack_codes(codes.reshape(R, C), f), scales


def quantize_colwise_t(x, fmt, rule, hadamard_mask=None):
    """Column-wise MX quantization of [R][C], blocks of 32 consecutive rows.

    The result is stored transposed: codes [C][R] (packed [C][R/2] for E2M1),
    scales [C][R/32].  By definition this is the row-wise quantization of x^T.
    """
    xt = np.ascontiguousarray(np.asarray(x, dtype=np.float32).T)
    return quantize_rowwise(xt, fmt, rule, hadamard_mask)


def quantize_dual(x, fmt, rule):
    """Both orientations of the same input ([UE8M0] second part, section 2, on
    keeping a row-wise and a column-wise quantized copy): (q_row, s_row, q_colT, s_colT)."""
    q_row, s_row = quantize_rowwise(x, fmt, rule)
    q_col, s_col = quantize_colwise_t(x, fmt, rule)
    return q_row, s_row, q_col, s_col


def tensor_amax(x) -> np.float32:
    """max |x| over the whole tensor as FP32, NaN entries ignored (0 if none)."""
    a = np.abs(np.asarray(x, dtype=np.float32))
    a = a[~np.isnan(a)]
    return np.float32(a.max()) if a.size else np.float32(0.0)


def dequantize_exact(codes, scales, fmt, packed_fp4=True) -> np.ndarray:
    """Exact dequantized values V^_i = Q_i * X as float64 ([UE8M0] section 2 of the
    first part: decoding an E8M0 scale is an exponent shift).

    ``codes`` are [R][C] (or packed: [R][C/2] E2M1, [R][3C/4] FP6), ``scales`` [R][C/32].
    """
    f = fmt_of(fmt)
    c = np.asarray(codes)
    if f.bits < 8 and packed_fp4:
        c = unpack_codes(c, f)
    R, C = c.shape
    vals = decode(c, f).reshape(R, C // BLOCK, BLOCK)
    sc = e8m0_decode(scales).reshape(R, C // BLOCK, 1)
    with np.errstate(invalid="ignore", over="ignore"):
        return (vals * sc).reshape(R, C)


def dequantize(codes, scales, fmt, out="f32") -> np.ndarray:
    """Dequantize to FP32 (or to BF16 bits with ``out='bf16'``), one rounding of
    the exact value (overflow gives +-Inf, NaN scale gives NaN)."""
    from .formats import f64_to_bf16_bits
    exact = dequantize_exact(codes, scales, fmt)
    if out == "f32":
        with np.errstate(over="ignore"):
            return exact.astype(np.float32)
    if out == "bf16":
        return f64_to_bf16_bits(exact)
    raise ValueError(out)
