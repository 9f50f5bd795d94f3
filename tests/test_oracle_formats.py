"""Pins for the oracle's element and scale codecs (CPU only)."""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import formats as F
from tests import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")


def golden():
    with open(GOLDEN) as f:
        return {c["name"]: c for c in json.load(f)["constants"]}


# ---------------------------------------------------------------- page constants

def test_printed_e4m3_constants():
    g = golden()
    assert F.E4M3.max_value == g["e4m3_max"]["value"] == 1.75 * 2 ** 8
    assert F.E4M3.min_subnormal == g["e4m3_min_subnormal"]["value"] == 2.0 ** -9
    binades = math.log2(F.E4M3.max_value / F.E4M3.min_subnormal)
    assert abs(binades - g["e4m3_binades"]["value"]) < g["e4m3_binades"]["tolerance"]
    nan_codes = [c for c in range(128) if np.isnan(F.decode(c, F.E4M3))]
    assert len(nan_codes) == g["e4m3_nan_magnitude_patterns"]["value"]


def test_printed_e5m2_ieee_specials():
    assert golden()["e5m2_ieee_specials"]["value"]
    d = F.decode(np.arange(256), F.E5M2)
    assert np.isinf(d).sum() == 2 and d[0x7C] == np.inf and d[0xFC] == -np.inf
    # IEEE: exponent field all ones with non-zero mantissa is NaN
    assert np.isnan(d[[0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF]]).all()
    assert np.isfinite(d).sum() == 248


def test_printed_e8m0_range_and_nan():
    g = golden()
    v = F.e8m0_decode(np.arange(256))
    assert v[0] == 2.0 ** g["e8m0_exp_min"]["value"]
    assert v[254] == 2.0 ** g["e8m0_exp_max"]["value"]
    assert np.isnan(v[255]) and g["e8m0_has_nan"]["value"]
    assert (v[:255] > 0).all() and not g["e8m0_signed"]["value"]
    # every finite code is a power of two, strictly increasing
    assert np.all(np.diff(np.log2(v[:255])) == 1.0)


def test_printed_scale_budget():
    g = golden()
    k = g["block_size_k"]["value"]
    assert k * 8 + 8 == g["bits_per_block_e8m0"]["value"]
    assert k * 8 + 32 == g["bits_per_block_fp32_scale"]["value"]
    assert 1 - 8 / 32 == g["scale_traffic_reduction"]["value"]


# ---------------------------------------------------------------- decode

@pytest.mark.parametrize("name", ["e4m3", "e5m2"])
def test_decode_matches_torch_fp8_dtypes(name):
    ours = F.decode(np.arange(256), name)
    ref = pins.table_from_torch(name)
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()
    # sign of zero
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0])


def test_decode_e2m1_table():
    ours = F.decode(np.arange(16), "e2m1")
    assert list(ours[:8]) == pins.E2M1_MAGNITUDES
    assert list(-ours[8:]) == pins.E2M1_MAGNITUDES
    assert np.signbit(ours[8])


@pytest.mark.parametrize("name", ["e2m3", "e3m2"])
def test_decode_fp6_tables(name):
    ours = F.decode(np.arange(64), name)
    mags = pins.E2M3_MAGNITUDES if name == "e2m3" else pins.E3M2_MAGNITUDES
    assert list(ours[:32]) == mags and list(-ours[32:]) == mags
    assert np.signbit(ours[32])
    # the OCP extremes: E2M3 max 7.5, smallest subnormal 0.125; E3M2 max 28, 0.0625
    f = F.FORMATS[name]
    assert (f.max_value, f.min_subnormal) == ((7.5, 0.125) if name == "e2m3" else (28.0, 0.0625))


def test_fp4_packing_is_a_little_endian_nibble_stream():
    """E2M1 codes are packed two per byte, element 2j in the low nibble of byte j:
    the same little-endian bit-stream rule as FP6, at 4 bits (the pages are silent
    on the packing; this pins the reading, literal bytes written out by hand)."""
    from oracle import mx
    # codes 0x1, 0x2, 0xF, 0x0 -> bytes 0x21 (element 0 low, element 1 high), 0x0F
    assert list(mx.pack_fp4(np.array([0x1, 0x2, 0xF, 0x0]))) == [0x21, 0x0F]
    assert list(mx.pack_fp4(np.array([0x8, 0x7, 0x0, 0xC]))) == [0x78, 0xC0]
    assert list(mx.unpack_fp4(np.array([0x21, 0x0F], dtype=np.uint8))) == [0x1, 0x2, 0xF, 0x0]
    g = np.random.default_rng(8)
    c = g.integers(0, 16, size=(5, 64)).astype(np.uint8)
    p = mx.pack_fp4(c)
    assert p.shape == (5, 32) and np.array_equal(mx.unpack_fp4(p), c)
    # bit i of the stream is bit i % 4 of element i // 4
    stream = np.unpackbits(p[0], bitorder="little")
    assert np.array_equal(stream.reshape(64, 4), np.unpackbits(c[0][:, None], axis=1, bitorder="little")[:, :4])
    # through the block quantizer: a block 1, -2, 6, 0.5, 0, ... (amax 6, scale 2^0) gives
    # E2M1 codes 0x2, 0xC, 0x7, 0x1, 0, ... -> bytes 0xC2, 0x17, 0x00 ...
    x = np.zeros((1, 32), np.float32)
    x[0, :4] = [1.0, -2.0, 6.0, 0.5]
    q, s = mx.quantize_rowwise(x, "e2m1", "ceil")
    assert list(s[0]) == [127]
    assert list(q[0]) == [0xC2, 0x17] + [0] * 14


def test_planted_high_nibble_first_fp4_packing_is_caught(monkeypatch):
    """A consistent pack / unpack pair with element 2j in the HIGH nibble passes
    every round-trip check; the literal-byte pin must still reject it."""
    from oracle import mx

    def wrong_pack(codes):
        c = np.asarray(codes).astype(np.uint8)
        return (((c[..., 0::2] & 0xF) << 4) | (c[..., 1::2] & 0xF)).astype(np.uint8)

    def wrong_unpack(packed):
        p = np.asarray(packed).astype(np.uint8)
        out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
        out[..., 0::2] = p >> 4
        out[..., 1::2] = p & 0xF
        return out
    monkeypatch.setattr(mx, "pack_fp4", wrong_pack)
    monkeypatch.setattr(mx, "unpack_fp4", wrong_unpack)
    with pytest.raises(AssertionError):
        test_fp4_packing_is_a_little_endian_nibble_stream()


def test_fp6_packing_is_a_little_endian_bit_stream():
    from oracle import mx
    # codes 1, 2, 3, 4 -> 24-bit word 1 | 2 << 6 | 3 << 12 | 4 << 18 = 0x103081
    assert list(mx.pack_fp6(np.array([1, 2, 3, 4]))) == [0x81, 0x30, 0x10]
    assert list(mx.pack_fp6(np.array([0x3F, 0, 0, 0x3F]))) == [0x3F, 0x00, 0xFC]
    g = np.random.default_rng(9)
    c = g.integers(0, 64, size=(5, 64)).astype(np.uint8)
    p = mx.pack_fp6(c)
    assert p.shape == (5, 48) and np.array_equal(mx.unpack_fp6(p), c)
    # bit i of the stream is bit i % 6 of element i // 6
    stream = np.unpackbits(p[0], bitorder="little")
    assert np.array_equal(stream.reshape(64, 6), np.unpackbits(c[0][:, None], axis=1, bitorder="little")[:, :6])


def test_planted_big_endian_fp6_packing_is_caught(monkeypatch):
    from oracle import mx

    def wrong(codes):
        c = np.asarray(codes).astype(np.uint32) & 0x3F
        g = c.reshape(c.shape[:-1] + (c.shape[-1] // 4, 4))
        word = (g[..., 0] << 18) | (g[..., 1] << 12) | (g[..., 2] << 6) | g[..., 3]
        out = np.stack([(word >> 16) & 0xFF, (word >> 8) & 0xFF, word & 0xFF], axis=-1)
        return out.reshape(c.shape[:-1] + (c.shape[-1] * 3 // 4,)).astype(np.uint8)
    monkeypatch.setattr(mx, "pack_fp6", wrong)
    with pytest.raises(AssertionError):
        test_fp6_packing_is_a_little_endian_bit_stream()


@pytest.mark.parametrize("name", ["e4m3", "e5m2", "e2m1", "e2m3", "e3m2"])
def test_code_enumeration(name):
    f = F.FORMATS[name]
    n = 1 << f.bits
    d = F.decode(np.arange(n), f)
    fin = np.isfinite(d)
    expected_finite = {"e4m3": 254, "e5m2": 248, "e2m1": 16, "e2m3": 64, "e3m2": 64}[name]
    assert fin.sum() == expected_finite
    # decode -> encode is the identity on every non-NaN code (Inf saturates)
    e = F.encode(d[fin], f)
    assert np.array_equal(e, np.arange(n)[fin])
    # positive finite codes increase strictly with the code integer
    pos = d[: n // 2][fin[: n // 2]]
    assert np.all(np.diff(pos) > 0)
    assert F.decode(f.max_code, f) == f.max_value


# ---------------------------------------------------------------- encode

def _bf16_times_scales():
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    v = bits.view(np.float32).astype(np.float64)
    v = v[np.isfinite(v)]
    ks = np.arange(-140, 141, 7)
    return (v[None, :] * np.exp2(ks)[:, None]).reshape(-1)


def check_encoder_vs_bruteforce(encode, name, values) -> bool:
    a = encode(values, F.FORMATS[name]).astype(np.int64)
    b = pins.nearest_even_codes(values, name).astype(np.int64)
    return bool(np.array_equal(a, b))


@pytest.mark.parametrize("name", ["e4m3", "e5m2", "e2m1", "e2m3", "e3m2"])
def test_encode_all_bf16_patterns_at_many_scales(name):
    assert check_encoder_vs_bruteforce(F.encode, name, _bf16_times_scales())


@pytest.mark.parametrize("name", ["e4m3", "e5m2", "e2m1", "e2m3", "e3m2"])
def test_encode_midpoints_and_neighbours(name):
    f = F.FORMATS[name]
    d = F.decode(np.arange(1 << (f.bits - 1)), f)
    d = np.sort(d[np.isfinite(d)])
    mids = (d[:-1] + d[1:]) / 2
    mids = np.concatenate([mids, [f.max_value * 1.0625, f.max_value * 2, d[1] / 2]])
    m32 = mids.astype(np.float32)
    vals = np.concatenate([m32, np.nextafter(m32, np.float32(np.inf)), np.nextafter(m32, np.float32(0))])
    vals = np.concatenate([vals, -vals]).astype(np.float64)
    assert check_encoder_vs_bruteforce(F.encode, name, vals)


@pytest.mark.parametrize("name", ["e4m3", "e5m2", "e2m1", "e2m3", "e3m2"])
def test_encode_random_fp32_bits(name):
    g = np.random.default_rng(7)
    bits = g.integers(0, 1 << 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    # bring the exponents into the interesting window around the format
    scaled = np.ldexp(np.frexp(v.astype(np.float64))[0], g.integers(-30, 30, size=v.size).astype(np.int32))
    assert check_encoder_vs_bruteforce(F.encode, name, scaled)


@pytest.mark.parametrize("name,dt", [("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)])
def test_encode_matches_torch_cast_in_range(name, dt):
    f = F.FORMATS[name]
    v = _bf16_times_scales()
    v = v[np.abs(v) <= f.max_value].astype(np.float32)
    ref = torch.from_numpy(v).to(dt).view(torch.uint8).numpy()
    ours = F.encode(v.astype(np.float64), f)
    assert np.array_equal(ours, ref)


def test_encode_e2m1_ties():
    # exact halfway cases between E2M1 neighbours go to the even code
    vals = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, -0.25, -5.0])
    expect = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, -0.0, -4.0]
    got = F.decode(F.encode(vals, "e2m1"), "e2m1")
    assert list(got) == expect
    assert np.signbit(got[-2])


def test_encode_fp6_ties_and_specials():
    # halfway cases go to the even code; NaN -> largest magnitude with its sign; no Inf
    got = F.decode(F.encode(np.array([0.0625, 0.1875, 7.25, 7.75, 100.0, -np.inf, np.nan]), "e2m3"), "e2m3")
    assert list(got[:5]) == [0.0, 0.25, 7.0, 7.5, 7.5] and got[5] == -7.5 and got[6] == 7.5
    got = F.decode(F.encode(np.array([0.03125, 26.0, 30.0, -1e9]), "e3m2"), "e3m2")
    assert list(got) == [0.0, 24.0, 28.0, -28.0]


def test_encode_specials():
    for name in ("e4m3", "e5m2"):
        f = F.FORMATS[name]
        c = F.encode(np.array([np.nan, np.inf, -np.inf, -0.0, 1e300, -1e-300]), f)
        assert np.isnan(F.decode(c[0], f))
        assert c[1] == f.max_code and c[2] == f.max_code | 0x80     # saturate, never Inf
        assert c[3] == 0x80 and c[4] == f.max_code and c[5] == 0x80


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(3)
    bits = g.integers(0, 1 << 32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[~np.isnan(x)]
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.f32_to_bf16_bits(x), ref)
    assert np.array_equal(F.f64_to_bf16_bits(x.astype(np.float64)), ref)
