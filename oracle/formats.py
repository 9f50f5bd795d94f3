"""Element and scale formats of OCP MX, as exact integer / float64 arithmetic.

Test infrastructure only (see ``oracle/__init__``).

Definitions followed ([UE8M0] glossary entries "FP8 (E4M3/E5M2)", "EU8M0",
"MXFP8" and the note on special values):

* E4M3 - 1 sign, 4 exponent (bias 7), 3 mantissa bits.  No infinities; the only
  NaN magnitude is S.1111.111.  Largest finite value 1.75 * 2^8 = 448, smallest
  subnormal 2^-9.
* E5M2 - 1 sign, 5 exponent (bias 15), 2 mantissa bits, IEEE-754 specials:
  exponent field 31 with mantissa 0 is +-Inf, with mantissa != 0 is NaN.
  Largest finite 1.75 * 2^15 = 57344, smallest subnormal 2^-16.
* E2M1 - 1 sign, 2 exponent (bias 1), 1 mantissa bit, no specials:
  magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
* E2M3 - 1 sign, 2 exponent (bias 1), 3 mantissa bits, no specials (FP6 of the
  MXFP8/6/4 family named on the page): largest 1.875 * 4 = 7.5, smallest
  subnormal 2^-3.
* E3M2 - 1 sign, 3 exponent (bias 3), 2 mantissa bits, no specials: largest
  1.75 * 16 = 28, smallest subnormal 2^-4.
* E8M0 - unsigned, 8 exponent bits, no mantissa: code c in [0, 254] is 2^(c-127),
  code 255 is NaN.

Element casts round to nearest, ties to even, and saturate: a finite magnitude
beyond the largest finite value becomes that value ([UE8M0] section 4, on the
scale algorithm clamping values above the upper limit).  Infinite inputs
saturate the same way; NaN inputs give the format's NaN (E2M1, E2M3 and E3M2
have none, so they give the largest magnitude with the input's sign).
"""

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class ElemFormat:
    name: str
    ebits: int
    mbits: int
    bias: int
    emax: int        # unbiased exponent of the largest finite value
    max_mant: int    # integer significand (with hidden bit) of the largest value, in units of 2^-mbits
    has_inf: bool
    nan_code: int    # canonical positive NaN code (E2M1: largest magnitude, no NaN exists)

    @property
    def bits(self) -> int:
        return 1 + self.ebits + self.mbits

    @property
    def emin(self) -> int:
        """Unbiased exponent of the smallest normal value."""
        return 1 - self.bias

    @property
    def max_value(self) -> float:
        return float(self.max_mant) * 2.0 ** (self.emax - self.mbits)

    @property
    def min_subnormal(self) -> float:
        return 2.0 ** (self.emin - self.mbits)

    @property
    def sign_bit(self) -> int:
        return 1 << (self.ebits + self.mbits)

    @property
    def max_code(self) -> int:
        """Positive code of the largest finite value."""
        return ((self.emax + self.bias) << self.mbits) | (self.max_mant - (1 << self.mbits))


# OCP E4M3 ("E4M3FN"): exponent field 15 is an ordinary binade except mantissa 111 (NaN).
E4M3 = ElemFormat("e4m3", ebits=4, mbits=3, bias=7, emax=8, max_mant=0b1110, has_inf=False, nan_code=0x7F)
# OCP E5M2: exponent field 31 is reserved for Inf/NaN.
E5M2 = ElemFormat("e5m2", ebits=5, mbits=2, bias=15, emax=15, max_mant=0b111, has_inf=True, nan_code=0x7F)
# OCP E2M1 (FP4): no Inf/NaN.
E2M1 = ElemFormat("e2m1", ebits=2, mbits=1, bias=1, emax=2, max_mant=0b11, has_inf=False, nan_code=0x7)

# OCP E2M3 / E3M2 (FP6): no Inf/NaN.
E2M3 = ElemFormat("e2m3", ebits=2, mbits=3, bias=1, emax=2, max_mant=0b1111, has_inf=False, nan_code=0x1F)
E3M2 = ElemFormat("e3m2", ebits=3, mbits=2, bias=3, emax=4, max_mant=0b111, has_inf=False, nan_code=0x1F)

FORMATS = {"e4m3": E4M3, "e5m2": E5M2, "e2m1": E2M1, "e2m3": E2M3, "e3m2": E3M2}


def fmt_of(f) -> ElemFormat:
    return FORMATS[f] if isinstance(f, str) else f


# ----------------------------------------------------------------------------
# decode
# ----------------------------------------------------------------------------

def decode(codes, fmt) -> np.ndarray:
    """Exact value of each element code as float64 (NaN / +-Inf for specials).

    Subnormal (exponent field 0): M * 2^(emin - mbits); normal:
    (2^mbits + M) * 2^(E - bias - mbits).
    """
    f = fmt_of(fmt)
    c = np.asarray(codes).astype(np.int64) & ((1 << f.bits) - 1)
    sign = (c >> (f.ebits + f.mbits)) & 1
    ef = (c >> f.mbits) & ((1 << f.ebits) - 1)
    mf = c & ((1 << f.mbits) - 1)
    sub = ef == 0
    sig = np.where(sub, mf, mf + (1 << f.mbits)).astype(np.float64)
    exp = np.where(sub, f.emin, ef - f.bias) - f.mbits
    mag = np.ldexp(sig, exp.astype(np.int32))
    top = (1 << f.ebits) - 1
    if f.name == "e4m3":
        mag = np.where((ef == top) & (mf == (1 << f.mbits) - 1), np.nan, mag)
    elif f.name == "e5m2":
        mag = np.where((ef == top) & (mf == 0), np.inf, mag)
        mag = np.where((ef == top) & (mf != 0), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


def is_nan_code(codes, fmt) -> np.ndarray:
    return np.isnan(decode(codes, fmt))


# ----------------------------------------------------------------------------
# encode: round to nearest even, then saturate
# ----------------------------------------------------------------------------

def _split_f64(v: np.ndarray):
    """Exact decomposition |v| = sig * 2^exp2 with sig a non-negative integer < 2^53."""
    m, e = np.frexp(np.abs(v))             # |v| = m * 2^e, m in [0.5, 1)
    sig = np.ldexp(m, 53).astype(np.int64)  # exact: m has at most 53 significant bits
    exp2 = e.astype(np.int64) - 53
    return sig, exp2


def encode(values, fmt) -> np.ndarray:
    """RNE + saturating cast of exact values (float64 array) to element codes (uint8).

    The value is taken exactly (float64 holds every FP32 value and every value
    an FP32 scaled by a power of two in the MX range can take).  Steps:
      1. NaN -> canonical NaN with the input's sign; +-Inf -> +-max.
      2. For finite v: the quantum of the binade that holds |v| (never below the
         subnormal quantum) is 2^qe; n = round-half-even(|v| / 2^qe) as an exact
         integer.
      3. n * 2^qe larger than the largest finite value -> the largest finite value.
      4. Assemble sign | exponent field | mantissa field.
    """
    f = fmt_of(fmt)
    v = np.asarray(values, dtype=np.float64)
    shape = v.shape
    v = v.reshape(-1)
    neg = np.signbit(v)
    nan = np.isnan(v)
    inf = np.isinf(v)
    fin = np.where(nan | inf, 0.0, v)

    sig, exp2 = _split_f64(fin)
    zero = sig == 0
    # true exponent E of |v| (|v| in [2^E, 2^(E+1)))
    msb = np.frexp(np.where(zero, 1.0, sig.astype(np.float64)))[1].astype(np.int64) - 1
    E = exp2 + msb
    qe = np.maximum(E, f.emin) - f.mbits           # exponent of one quantum
    shift = qe - exp2                               # |v| / 2^qe = sig * 2^-shift

    # exact round-half-even of sig * 2^-shift
    left = np.clip(-shift, 0, 62)
    right = np.clip(shift, 0, 62)
    q = (sig << left) >> right
    rem = sig - ((sig >> right) << right)
    half = np.where(right > 0, np.left_shift(np.int64(1), np.maximum(right - 1, 0)), 0)
    up = (right > 0) & ((rem > half) | ((rem == half) & ((q & 1) == 1)))
    n = q + up.astype(np.int64)

    # a carry out of the significand moves to the next binade
    carry = n >= (1 << (f.mbits + 1))
    n = np.where(carry, n >> 1, n)
    qe = np.where(carry, qe + 1, qe)

    # saturation: compare n * 2^qe with max_mant * 2^(emax - mbits)
    top_qe = f.emax - f.mbits
    over = (qe > top_qe) | ((qe == top_qe) & (n > f.max_mant))
    over |= inf

    subnormal = n < (1 << f.mbits)                  # only when qe == emin - mbits
    efield = np.where(subnormal | (n == 0), 0, qe + f.mbits + f.bias)
    mfield = np.where(subnormal | (n == 0), n, n - (1 << f.mbits))
    mag_code = (efield << f.mbits) | mfield
    mag_code = np.where(zero & ~inf, 0, mag_code)
    mag_code = np.where(over, f.max_code, mag_code)
    mag_code = np.where(nan, f.nan_code, mag_code)
    code = mag_code | np.where(neg, f.sign_bit, 0)
    return code.astype(np.uint8).reshape(shape)


# ----------------------------------------------------------------------------
# E8M0 scale
# ----------------------------------------------------------------------------

E8M0_NAN = 0xFF
E8M0_BIAS = 127


def e8m0_decode(codes) -> np.ndarray:
    """2^(c - 127) as float64 for c in [0, 254]; NaN for 255 ([UE8M0] glossary 'EU8M0')."""
    c = np.asarray(codes).astype(np.int64)
    val = np.ldexp(np.ones(c.shape), (c - E8M0_BIAS).astype(np.int32))
    return np.where(c == E8M0_NAN, np.nan, val)


# ----------------------------------------------------------------------------
# FP32 / BF16 helpers (plain IEEE definitions)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x) -> np.ndarray:
    """Round an FP32 array to BF16 (nearest, ties to even); NaN stays a quiet NaN."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    lsb = (b >> 16) & 1
    r = ((b + 0x7FFF + lsb) >> 16) & 0xFFFF
    r = np.where(nan, ((b >> 16) | 0x40) & 0xFFFF, r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round exact float64 values to BF16 (nearest, ties to even, with subnormals).

    Goes through the element-format machinery with an 8-exponent-bit, 7-mantissa
    -bit IEEE format, so that it is a single rounding of the exact value.
    """
    v = np.asarray(x, dtype=np.float64)
    sig, exp2 = _split_f64(np.where(np.isfinite(v), v, 0.0))
    zero = sig == 0
    msb = np.frexp(np.where(zero, 1.0, sig.astype(np.float64)))[1].astype(np.int64) - 1
    E = exp2 + msb
    qe = np.maximum(E, -126) - 7
    shift = qe - exp2
    left = np.clip(-shift, 0, 62)
    right = np.clip(shift, 0, 62)
    q = (sig << left) >> right
    rem = sig - ((sig >> right) << right)
    half = np.where(right > 0, np.left_shift(np.int64(1), np.maximum(right - 1, 0)), 0)
    up = (right > 0) & ((rem > half) | ((rem == half) & ((q & 1) == 1)))
    n = q + up.astype(np.int64)
    carry = n >= 256
    n = np.where(carry, n >> 1, n)
    qe = np.where(carry, qe + 1, qe)
    sub = n < 128
    ef = np.where(sub | (n == 0), 0, qe + 7 + 127)
    mf = np.where(sub | (n == 0), n, n - 128)
    over = ef >= 255
    mag = np.where(over, 0x7F80, (ef << 7) | mf)
    mag = np.where(zero, 0, mag)
    mag = np.where(np.isinf(v), 0x7F80, mag)
    mag = np.where(np.isnan(v), 0x7FC0, mag)
    return (mag | np.where(np.signbit(v), 0x8000, 0)).astype(np.uint16)
