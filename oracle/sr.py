"""Stochastic-rounding MXFP4, row-wise (CPU oracle).

Test infrastructure only (see ``oracle/__init__``).

[FAF], the paragraph on the 37.2K tokens/s configuration: row gradients are
quantized to MXFP4 with stochastic rounding.  The page names the technique
without defining it.  The reading taken here is the textbook one, driven by
random bits the caller passes in:

* the block scale is the ordinary MX scale (same rule and clamp as the RNE
  path, ``oracle.mx.scale_exponent``); only the element cast changes;
* every element has its own uint32 random word r;
* the magnitude y = |V| / X is exact; if it is an E2M1 magnitude it is kept,
  at or above the largest magnitude (6) it saturates to 6, and strictly between
  adjacent magnitudes lo < hi it becomes hi iff
  r < floor(2^32 * (y - lo) / (hi - lo)), else lo -- up with probability
  (y - lo) / (hi - lo) to within 2^-32;
* the sign bit is copied (so -0 stays -0); a block holding NaN or Inf is
  encoded as on the RNE path (scale 0xFF, codes +-6).

Every quantity below is exact in float64: y has at most 24 significant bits,
lo <= y < hi <= 2 lo (or lo = 0), so y - lo is exact, (hi - lo) is a power of
two, and the threshold has at most 24 significant bits.
"""

import numpy as np

from .formats import E8M0_NAN, fmt_of
from .mx import BLOCK, pack_fp4, scale_exponent

# E2M1 magnitudes in code order 0..7
E2M1_MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def sr_threshold(y) -> tuple:
    """(lo_code, T) for magnitudes y >= 0 below 6: the element rounds up to
    lo_code + 1 iff r < T.  T = 0 for representable y."""
    y = np.asarray(y, dtype=np.float64)
    lo_code = np.searchsorted(E2M1_MAGS, y, side="right") - 1
    lo_code = np.clip(lo_code, 0, 6)
    lo = E2M1_MAGS[lo_code]
    span = E2M1_MAGS[lo_code + 1] - lo
    t = np.floor(np.ldexp((y - lo) / span, 32))
    return lo_code.astype(np.int64), t


def rounds_up(r, t) -> np.ndarray:
    """The stochastic decision: word r rounds up iff it falls below the threshold."""
    return r < t


def sr_cast_e2m1(y, r) -> np.ndarray:
    """E2M1 magnitude codes (0..7) of exact magnitudes y >= 0 with random words r."""
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(r, dtype=np.uint64).astype(np.float64)   # < 2^32: exact
    sat = y >= 6.0
    lo_code, t = sr_threshold(np.where(sat, 0.0, y))
    code = lo_code + rounds_up(r, t)
    return np.where(sat, 7, code).astype(np.int64)


def quantize_blocks_sr(blocks, rand, rule):
    """Stochastic-rounding MXFP4 of an array [..., 32] of FP32 values with one
    uint32 random word per element.  Returns (codes uint8 [..., 32], scales)."""
    f = fmt_of("e2m1")
    x = np.asarray(blocks, dtype=np.float32).astype(np.float64)
    r = np.asarray(rand, dtype=np.uint32)
    assert x.shape[-1] == BLOCK and r.shape == x.shape
    finite = np.all(np.isfinite(x), axis=-1)
    xf = np.where(np.isfinite(x), x, 0.0)
    amax = np.max(np.abs(xf), axis=-1)
    e = scale_exponent(amax, f, rule)
    scale = np.where(finite, (e + 127).astype(np.int64), E8M0_NAN)
    y = np.ldexp(np.abs(xf), (-e)[..., None].astype(np.int32))      # |V| / X, exact
    sign = np.where(np.signbit(x), f.sign_bit, 0)
    codes = sr_cast_e2m1(y, r) | sign
    codes = np.where(finite[..., None], codes, f.nan_code | sign)
    return codes.astype(np.uint8), scale.astype(np.uint8)


def quantize_rowwise_sr(x, rand, rule):
    """Row-wise stochastic-rounding MXFP4 of a 2-D FP32 array [R][C] with random
    words rand [R][C] (uint32).  Returns (packed codes [R][C/2], scales [R][C/32])."""
    x = np.asarray(x, dtype=np.float32)
    R, C = x.shape
    assert C % BLOCK == 0
    codes, scales = quantize_blocks_sr(x.reshape(R, C // BLOCK, BLOCK),
                                       np.asarray(rand, dtype=np.uint32).reshape(R, C // BLOCK, BLOCK), rule)
    return pack_fp4(codes.reshape(R, C)), scales
