"""Planted mistakes: each test breaks the oracle in one plausible way (on the CPU,
in a local variant) and checks that the corresponding pin catches it.  This
shows that the pins constrain the oracle rather than restate it."""

import numpy as np

from oracle import formats as F
from oracle import hadamard, mx
from tests import test_oracle_formats as tf
from tests import test_oracle_hadamard_gemm as th
from tests import test_oracle_mx as tm


def _values():
    return tf._bf16_times_scales()[::7]


def test_truncating_encoder_is_caught():
    def trunc(values, fmt):
        v = np.asarray(values, np.float64)
        # round toward zero by shaving a little off before the RNE cast
        return F.encode(v * (1 - 2.0 ** -6), fmt)
    assert not tf.check_encoder_vs_bruteforce(trunc, "e4m3", _values())


def test_ties_away_encoder_is_caught():
    def away(values, fmt):
        v = np.asarray(values, np.float64)
        return F.encode(v * (1 + 2.0 ** -30), fmt)
    assert not tf.check_encoder_vs_bruteforce(away, "e2m1", np.array([0.25, 0.75, 1.25, 2.5, 5.0]))


def test_non_saturating_encoder_is_caught():
    def nosat(values, fmt):
        c = F.encode(values, fmt).astype(np.int64)
        f = F.fmt_of(fmt)
        over = np.abs(np.asarray(values)) > f.max_value * 1.0625
        return np.where(over, f.nan_code | (c & f.sign_bit), c).astype(np.uint8)
    assert not tf.check_encoder_vs_bruteforce(nosat, "e4m3", _values())


def test_scale_rule_off_by_one_is_caught():
    def floor_plus_one(amax, fmt, rule):
        return np.minimum(mx.scale_exponent(amax, fmt, rule) + 1, 127)
    assert not tm.check_scale_rule(floor_plus_one, "e4m3", "floor")


def test_ceil_rule_using_floor_is_caught():
    def ceil_as_floor(amax, fmt, rule):
        return mx.scale_exponent(amax, fmt, "floor")
    assert not tm.check_scale_rule(ceil_as_floor, "e5m2", "ceil")


def test_scale_rule_without_emax_is_caught():
    def no_emax(amax, fmt, rule):
        return np.clip(mx.scale_exponent(amax, fmt, rule) + F.fmt_of(fmt).emax - 7, -127, 127)
    assert not tm.check_scale_rule(no_emax, "e2m1", "ceil")


def test_block_quantizer_dropping_sign_is_caught():
    def unsigned(blocks, fmt, rule):
        c, s = mx.quantize_blocks(np.abs(blocks), fmt, rule)
        return c, s
    assert not tm.check_block_quantizer(unsigned, "e4m3", "ceil")


def test_block_quantizer_with_wrong_block_axis_is_caught():
    def transposed(blocks, fmt, rule):
        b = np.asarray(blocks)
        n = b.shape[0] // 32 * 32
        c, s = mx.quantize_blocks(b, fmt, rule)
        c2, s2 = mx.quantize_blocks(b[:n].reshape(-1, 32, 32).transpose(0, 2, 1).reshape(n, 32), fmt, rule)
        c[:n] = c2
        s[:n] = s2
        return c, s
    assert not tm.check_block_quantizer(transposed, "e5m2", "floor")


def test_hadamard_with_wrong_sign_or_order_is_caught():
    def wrong_sign(x, mask):
        return hadamard.hadamard32(x, mask ^ 1)

    def reversed_order(x, mask):
        return hadamard.hadamard32(np.asarray(x)[..., ::-1], mask)
    assert not th.check_hadamard_exact(wrong_sign)
    assert not th.check_hadamard_exact(reversed_order)


def test_gemm_with_transposed_scale_or_missing_alpha_is_caught():
    from oracle import gemm

    def no_alpha(*a, **k):
        k.pop("alpha", None)
        return gemm.gemm_ref(*a, **k)

    def scale_off(a, sa, fa, b, sb, fb, alpha=1.0):
        return gemm.gemm_ref(a, np.roll(sa, 1, axis=1), fa, b, sb, fb, alpha=alpha)
    assert not th.check_gemm_fraction(no_alpha, "e4m3", "e4m3")
    assert not th.check_gemm_fraction(scale_off, "e4m3", "e4m3")
