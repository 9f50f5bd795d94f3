"""Independent second implementations used to pin the oracle.

Nothing here shares code with ``oracle/``: these are brute-force searches over
decoded value tables (taken from torch's FP8 dtypes where they exist),
``fractions.Fraction`` arithmetic, and scans over candidate exponents.  Each
``check_*`` function takes the implementation under test as an argument so that
the planted-mistake tests can feed it a broken variant.
"""

from fractions import Fraction

import numpy as np
import torch

# E2M1 magnitudes: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit, no specials.
E2M1_MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def table_from_torch(name: str) -> np.ndarray:
    """Decoded value of every code 0..255 using torch's own FP8 dtypes."""
    dt = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}[name]
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(dt).to(torch.float64).numpy()


# FP6 magnitudes in code order, written from the format definitions (OCP MX):
# subnormals M * 2^(1 - bias - mbits), normals (1 + M / 2^mbits) * 2^(E - bias).
E2M3_MAGNITUDES = [m / 8 for m in range(8)] + [(1 + m / 8) * 2.0 ** e for e in range(0, 3) for m in range(8)]
E3M2_MAGNITUDES = [m / 16 for m in range(4)] + [(1 + m / 4) * 2.0 ** e for e in range(-2, 5) for m in range(4)]
BITS = {"e4m3": 8, "e5m2": 8, "e2m1": 4, "e2m3": 6, "e3m2": 6}


def table(name: str) -> np.ndarray:
    small = {"e2m1": E2M1_MAGNITUDES, "e2m3": E2M3_MAGNITUDES, "e3m2": E3M2_MAGNITUDES}
    if name in small:
        mags = np.array(small[name])
        return np.concatenate([mags, -mags])
    return table_from_torch(name)


def nearest_even_codes(values: np.ndarray, name: str) -> np.ndarray:
    """Brute-force encoder: nearest finite code, ties to the code with an even
    last bit, beyond the largest finite value -> the largest finite value.

    Works on |v| over the sorted positive finite codes, then restores the sign.
    """
    tab = table(name)
    nbits = BITS[name]
    half = 1 << (nbits - 1)
    pos_codes = np.arange(half)
    pos_vals = tab[:half]
    ok = np.isfinite(pos_vals)
    pos_codes, pos_vals = pos_codes[ok], pos_vals[ok]
    order = np.argsort(pos_vals)
    pos_codes, pos_vals = pos_codes[order], pos_vals[order]
    v = np.asarray(values, dtype=np.float64)
    a = np.abs(v)
    hi = np.clip(np.searchsorted(pos_vals, a, side="left"), 0, pos_vals.size - 1)
    lo = np.clip(hi - 1, 0, pos_vals.size - 1)
    dlo = np.abs(a - pos_vals[lo])
    dhi = np.abs(pos_vals[hi] - a)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (pos_codes[hi] % 2 == 0))
    code = np.where(pick_hi, pos_codes[hi], pos_codes[lo])
    code = np.where(a >= pos_vals[-1], pos_codes[-1], code)
    return (code | np.where(np.signbit(v), half, 0)).astype(np.uint8)


# ----------------------------------------------------------------------------
# Fraction-based scalar MX quantizer (tiny inputs only)
# ----------------------------------------------------------------------------

def frac_max(name: str) -> Fraction:
    tab = table(name)
    return Fraction(float(np.nanmax(tab[np.isfinite(tab)])))


def frac_emax(name: str) -> int:
    """Exponent of the largest finite value: largest k with 2^k <= max."""
    m = frac_max(name)
    k = 0
    while Fraction(2) ** (k + 1) <= m:
        k += 1
    return k


def scan_floor_exponent(amax: Fraction, name: str) -> int:
    """floor(log2 amax) - emax by scanning powers of two."""
    k = -400
    while Fraction(2) ** (k + 1) <= amax:
        k += 1
    return k - frac_emax(name)


def scan_ceil_exponent(amax: Fraction, name: str) -> int:
    """Smallest integer e with amax <= max * 2^e, by scanning."""
    m = frac_max(name)
    e = -400
    while amax > m * Fraction(2) ** e:
        e += 1
    return e


def frac_nearest_code(v: Fraction, name: str) -> int:
    """Nearest-even finite code of an exact rational, saturating, by scanning all codes."""
    tab = table(name)
    nbits = BITS[name]
    half = 1 << (nbits - 1)
    best = None
    a = abs(v)
    for c in range(half):
        t = tab[c]
        if not np.isfinite(t):
            continue
        d = abs(a - Fraction(float(t)))
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    c = best[1]
    mx = frac_max(name)
    if a >= mx:
        c = int(np.where(tab[:half] == float(mx))[0][0])
    return c | (half if v < 0 else 0)


def frac_quantize_block(block, name: str, rule: str):
    """Scalar MX quantization of one finite block by exact rational arithmetic.
    Returns (codes list, scale code)."""
    xs = [Fraction(float(x)) for x in block]
    amax = max(abs(x) for x in xs)
    if amax == 0:
        e = -127
    else:
        e = scan_floor_exponent(amax, name) if rule == "floor" else scan_ceil_exponent(amax, name)
        e = max(-127, min(127, e))
    scale = e + 127
    codes = []
    for xv, xf in zip(block, xs):
        c = frac_nearest_code(xf / Fraction(2) ** e, name)
        if xf == 0 and np.signbit(xv):
            c |= 1 << (BITS[name] - 1)
        codes.append(c)
    return codes, scale


def frac_decode(code: int, name: str) -> Fraction:
    return Fraction(float(table(name)[code]))


def frac_dot(a_vals, b_vals) -> Fraction:
    return sum((Fraction(float(x)) * Fraction(float(y)) for x, y in zip(a_vals, b_vals)), Fraction(0))
