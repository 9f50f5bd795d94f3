"""Pins for the oracle's MX block quantizer, scale rules and dequantizer (CPU only)."""

from fractions import Fraction

import numpy as np
import pytest

import workloads
from oracle import formats as F
from oracle import mx
from tests import pins

FMTS = ["e4m3", "e5m2", "e2m1", "e2m3", "e3m2"]
RULES = ["floor", "ceil"]


# ---------------------------------------------------------------- scale rules

def _amax_samples(name):
    f = F.FORMATS[name]
    g = np.random.default_rng(5)
    rnd = (g.integers(1, 0x7F800000, size=3000, dtype=np.int64).astype(np.uint32)).view(np.float32)
    # destmax * 2^k and its FP32 neighbours: where the two rules differ
    k = np.arange(-140, 120, 3)
    edge = f.max_value * np.exp2(k)
    edge = edge[edge < 3.0e38].astype(np.float32)
    near = np.concatenate([edge, np.nextafter(edge, np.float32(0)), np.nextafter(edge, np.float32(np.inf))])
    pow2 = np.exp2(np.arange(-149, 128)).astype(np.float32)
    sub = (np.arange(1, 200, dtype=np.uint32)).view(np.float32)
    return np.concatenate([rnd, near, pow2, sub]).astype(np.float64)


def check_scale_rule(scale_exponent, name, rule) -> bool:
    a = _amax_samples(name)
    got = scale_exponent(a, F.FORMATS[name], rule)
    scan = pins.scan_floor_exponent if rule == "floor" else pins.scan_ceil_exponent
    want = np.array([max(-127, min(127, scan(Fraction(float(x)), name))) for x in a])
    return bool(np.array_equal(got, want))


@pytest.mark.parametrize("name", FMTS)
@pytest.mark.parametrize("rule", RULES)
def test_scale_rule_against_scan(name, rule):
    assert check_scale_rule(mx.scale_exponent, name, rule)


@pytest.mark.parametrize("name", FMTS)
def test_ceil_never_saturates_and_floor_puts_amax_in_top_binade(name):
    f = F.FORMATS[name]
    a = _amax_samples(name)
    a = a[(a > 2.0 ** -100) & (a < 2.0 ** 100)]
    ec = mx.scale_exponent(a, f, "ceil")
    assert np.all(a * np.exp2(-ec) <= f.max_value)
    assert np.all(a * np.exp2(-(ec - 1)) > f.max_value)
    ef = mx.scale_exponent(a, f, "floor")
    r = a * np.exp2(-ef)
    assert np.all((r >= 2.0 ** f.emax) & (r < 2.0 ** (f.emax + 1)))


def test_zero_block_and_clamps():
    for name in FMTS:
        for rule in RULES:
            e = mx.scale_exponent(np.array([0.0, 2.0 ** -149, float(np.finfo(np.float32).max)]), name, rule)
            assert e[0] == -127 and e[1] == -127 and -127 <= e[2] <= 127


# ---------------------------------------------------------------- block quantizer vs Fraction scalar

def _tiny_blocks():
    g = np.random.default_rng(9)
    blocks = [workloads.special_blocks()]
    for kind in ("normal", "wide", "rows"):
        blocks.append(workloads.random_tensor((6, 32), seed=len(blocks), kind=kind))
    ties = (g.integers(-12, 13, size=(4, 32)) * 0.25).astype(np.float32)   # many exact ties
    blocks.append(ties)
    return np.concatenate(blocks)


def check_block_quantizer(quantize_blocks, name, rule) -> bool:
    blocks = _tiny_blocks()
    finite = np.all(np.isfinite(blocks), axis=1)
    blocks = blocks[finite]
    codes, scales = quantize_blocks(blocks, F.FORMATS[name], rule)
    for i, blk in enumerate(blocks):
        want_codes, want_scale = pins.frac_quantize_block(blk, name, rule)
        if scales[i] != want_scale or list(codes[i]) != want_codes:
            return False
    return True


@pytest.mark.parametrize("name", FMTS)
@pytest.mark.parametrize("rule", RULES)
def test_block_quantizer_against_fraction_scalar(name, rule):
    assert check_block_quantizer(mx.quantize_blocks, name, rule)


@pytest.mark.parametrize("name", FMTS)
def test_nonfinite_blocks(name):
    f = F.FORMATS[name]
    blk = np.linspace(-3, 3, 32).astype(np.float32)
    blk[4] = np.nan
    blk[6] = -np.inf
    codes, scale = mx.quantize_blocks(blk[None], f, "ceil")
    assert scale[0] == F.E8M0_NAN
    assert np.all((codes[0].astype(int) & (f.sign_bit - 1)) == f.nan_code)
    assert np.array_equal(codes[0] >> (f.bits - 1), np.signbit(blk).astype(np.uint8))


# ---------------------------------------------------------------- invariants on larger inputs

def _inputs():
    return [workloads.wide_range_f32(64, 256), workloads.random_tensor((64, 256), 3, "wide"),
            workloads.bf16_to_f32(workloads.activation_bf16(64, 128))]


@pytest.mark.parametrize("name", FMTS)
@pytest.mark.parametrize("rule", RULES)
def test_power_of_two_equivariance_and_sign_symmetry(name, rule):
    f = F.FORMATS[name]
    for x in _inputs():
        q, s = mx.quantize_rowwise(x, f, rule)
        q = mx.unpack_codes(q, f)
        for j in (-3, 5):
            q2, s2 = mx.quantize_rowwise((x * np.float32(2.0 ** j)).astype(np.float32), f, rule)
            ok = (s > 20) & (s < 230) & (s2 > 0)       # away from the clamps
            assert np.array_equal(s2[ok].astype(int), s[ok].astype(int) + j)
            rows_ok = np.repeat(ok, 32, axis=1)
            assert np.array_equal(mx.unpack_codes(q2, f)[rows_ok], q[rows_ok])
        qn, sn = mx.quantize_rowwise(-x, f, rule)
        assert np.array_equal(sn, s)
        assert np.array_equal(mx.unpack_codes(qn, f), q ^ f.sign_bit)


@pytest.mark.parametrize("name", FMTS)
@pytest.mark.parametrize("rule", RULES)
def test_permutation_within_block(name, rule):
    f = F.FORMATS[name]
    x = workloads.random_tensor((16, 128), 4, "wide")
    perm = np.random.default_rng(1).permutation(32)
    xp = x.reshape(16, 4, 32)[:, :, perm].reshape(16, 128)
    q, s = mx.quantize_rowwise(x, f, rule)
    qp, sp = mx.quantize_rowwise(xp, f, rule)
    q, qp = mx.unpack_codes(q, f), mx.unpack_codes(qp, f)
    assert np.array_equal(s, sp)
    assert np.array_equal(q.reshape(16, 4, 32)[:, :, perm], qp.reshape(16, 4, 32))


@pytest.mark.parametrize("name", FMTS)
@pytest.mark.parametrize("rule", RULES)
def test_idempotence_and_error_bound(name, rule):
    f = F.FORMATS[name]
    for x in _inputs():
        q, s = mx.quantize_rowwise(x, f, rule)
        d1 = mx.dequantize(q, s, f)
        q2, s2 = mx.quantize_rowwise(d1, f, rule)
        d2 = mx.dequantize(q2, s2, f)
        assert np.array_equal(d1, d2)
        if rule == "floor":
            assert np.array_equal(q, q2) and np.array_equal(s, s2)
        # error <= half a quantum of the element's binade at the block scale, unless saturated
        X = np.repeat(F.e8m0_decode(s), 32, axis=1)
        v = np.abs(x.astype(np.float64)) / X
        E = np.floor(np.log2(np.where(v > 0, v, 1.0)))
        quantum = np.exp2(np.maximum(E, f.emin) - f.mbits) * X
        err = np.abs(d1.astype(np.float64) - x)
        sat = v > f.max_value
        assert np.all(err[~sat] <= quantum[~sat] / 2)
        if rule == "ceil":
            assert not sat.any()


def test_scale_bytes_per_element():
    x = workloads.wide_range_f32(32, 256)
    for name in FMTS:
        q, s = mx.quantize_rowwise(x, name, "ceil")
        assert s.size * 32 == x.size
        assert q.nbytes * 8 == x.size * F.FORMATS[name].bits


def test_colwise_is_rowwise_of_transpose():
    x = workloads.random_tensor((64, 96), 8, "rows")
    qr, sr, qc, sc = mx.quantize_dual(x, "e4m3", "ceil")
    q_t, s_t = mx.quantize_rowwise(np.ascontiguousarray(x.T), "e4m3", "ceil")
    assert np.array_equal(qc, q_t) and np.array_equal(sc, s_t)
    assert qc.shape == (96, 64) and sc.shape == (96, 2)


# ---------------------------------------------------------------- dequantize

@pytest.mark.parametrize("name", FMTS)
def test_dequantize_exact_against_fraction(name):
    g = np.random.default_rng(2)
    nb = 1 << F.FORMATS[name].bits
    codes = g.integers(0, nb, size=(8, 64)).astype(np.uint8)
    scales = g.integers(0, 255, size=(8, 2)).astype(np.uint8)
    scales[0, 0] = 0
    scales[1, 1] = 254
    packed = mx.pack_codes(codes, name)
    d = mx.dequantize_exact(packed, scales, name)
    for i in range(8):
        for j in range(64):
            t = pins.table(name)[codes[i, j]]
            if not np.isfinite(t):
                assert not np.isfinite(d[i, j])
                continue
            assert Fraction(float(d[i, j])) == Fraction(float(t)) * Fraction(2) ** (int(scales[i, j // 32]) - 127)
    f32 = mx.dequantize(packed, scales, name)
    fin = np.isfinite(d) & (np.abs(d) <= np.finfo(np.float32).max)
    assert np.array_equal(f32[fin].astype(np.float64), d[fin])   # FP32 holds every in-range value


def test_dequantize_nan_scale():
    q = np.zeros((1, 32), np.uint8)
    s = np.array([[255]], np.uint8)
    assert np.isnan(mx.dequantize(q, s, "e4m3")).all()


def test_tensor_amax_ignores_nan():
    x = np.array([[1.0, -7.0, np.nan, 3.0]], np.float32)
    assert mx.tensor_amax(x) == 7.0
    assert mx.tensor_amax(np.zeros((2, 2), np.float32)) == 0.0


def test_gemm_scale_layout_literal_positions():
    """The GEMM scale layout by hand: 3 lines x 32 K-blocks, value 100 * line + kb.
    Flat byte order: stage 0 (kb 0..15) of line 0, line 1, line 2, then stage 1."""
    lines, kblocks = 3, 32
    s = (100 * np.arange(lines)[:, None] + np.arange(kblocks)[None, :]).astype(np.uint8)
    g = mx.scales_to_gemm_layout(s).reshape(-1)
    assert g.size == lines * kblocks
    assert list(g[:4]) == [0, 1, 2, 3]              # line 0, kb 0..3
    assert g[15] == 15 and g[16] == 100 and g[31] == 115   # line 0 kb 15, line 1 kb 0 / 15
    assert g[32] == 200 and g[47] == 215            # line 2, kb 0 / 15
    assert g[48] == 16 and g[64] == 116 and g[95] == 231   # stage 1: line 0 kb 16, line 1 kb 16, line 2 kb 31
    # byte (line, kb) at ((kb // 16) * lines + line) * 16 + kb % 16, for every entry
    for line in range(lines):
        for kb in range(kblocks):
            assert g[((kb // 16) * lines + line) * 16 + kb % 16] == s[line, kb]
    assert np.array_equal(mx.scales_from_gemm_layout(g, lines, kblocks), s)


def test_planted_line_major_gemm_layout_is_caught(monkeypatch):
    """A plausible wrong layout (each line's stages contiguous, i.e. row-major
    regrouped) is a permutation too and round-trips; the literal pin must reject it."""
    def wrong(scales):
        s = np.asarray(scales, dtype=np.uint8)
        return s.reshape(s.shape[0], -1, 16).copy()
    monkeypatch.setattr(mx, "scales_to_gemm_layout", wrong)
    with pytest.raises(AssertionError):
        test_gemm_scale_layout_literal_positions()
