"""Pins of the stochastic-rounding MXFP4 oracle (oracle/sr.py).

Each pin is fixed by the reading of stochastic rounding, not by re-typing the
oracle: exact unbiasedness over a uniform grid of random words, the two extreme
words giving the grid ceiling / floor found by brute force, agreement with the
round-to-nearest encoder on representable values, the same block scales as the
RNE path, monotonicity in r, and planted mistakes that the pins must catch."""

import numpy as np
import pytest

from oracle import formats as ofmt
from oracle import mx as omx
from oracle import sr as osr

MAGS = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def grid_ceil(y):
    return min(m for m in MAGS if m >= y) if y <= 6 else 6.0


def grid_floor(y):
    return max(m for m in MAGS if m <= y) if y <= 6 else 6.0


def off_grid_values(rng, n):
    """Magnitudes strictly between neighbours, with the fraction a multiple of 1/256."""
    lo_i = rng.integers(0, 7, n)
    j = rng.integers(1, 256, n)
    lo = np.array(MAGS)[lo_i]
    span = np.array(MAGS)[lo_i + 1] - lo
    return lo + span * j / 256.0, lo, span, j


def test_unbiased_exactly_over_a_uniform_word_grid():
    """With r = k 2^24 (k = 0..255) every off-grid y rounds up exactly 256 * frac
    times, so the mean of the cast is y exactly."""
    rng = np.random.default_rng(1)
    y, lo, span, j = off_grid_values(rng, 300)
    ks = np.arange(256, dtype=np.uint64) << 24
    codes = osr.sr_cast_e2m1(np.repeat(y[:, None], 256, 1), np.broadcast_to(ks, (300, 256)))
    mags = np.array(MAGS)[codes]
    assert np.array_equal(mags.mean(axis=1), y)
    assert np.array_equal((mags > lo[:, None]).sum(axis=1), j)


def test_extreme_words_give_grid_ceiling_and_floor():
    rng = np.random.default_rng(2)
    y = np.concatenate([rng.uniform(0, 6, 2000), np.array(MAGS), rng.uniform(6, 50, 20),
                        np.ldexp(1.0, -np.arange(1, 60)).astype(np.float64)])
    up = np.array(MAGS)[osr.sr_cast_e2m1(y, np.zeros_like(y, dtype=np.uint64))]
    down = np.array(MAGS)[osr.sr_cast_e2m1(y, np.full(y.shape, 2**32 - 1, dtype=np.uint64))]
    # r = 0 takes the ceiling unless the fraction is below the word's resolution 2^-32
    lo, hi = np.array([grid_floor(v) for v in y]), np.array([grid_ceil(v) for v in y])
    frac = np.where(hi > lo, (np.minimum(y, 6.0) - lo) / np.where(hi > lo, hi - lo, 1.0), 0.0)
    assert np.array_equal(up, np.where(frac * 2.0**32 >= 1.0, hi, lo))
    assert np.array_equal(down, lo)


def test_always_a_neighbour_and_rne_on_representable_values():
    rng = np.random.default_rng(3)
    y = rng.uniform(0, 7, 5000)
    r = rng.integers(0, 2**32, 5000, dtype=np.uint64)
    got = np.array(MAGS)[osr.sr_cast_e2m1(y, r)]
    lo = np.array([grid_floor(v) for v in y])
    hi = np.array([grid_ceil(v) for v in y])
    assert np.all((got == lo) | (got == hi))
    rep = np.array(MAGS)
    codes_rep = osr.sr_cast_e2m1(np.repeat(rep, 50), rng.integers(0, 2**32, 400, dtype=np.uint64))
    assert np.array_equal(codes_rep, ofmt.encode(np.repeat(rep, 50), "e2m1").astype(np.int64))


def test_monotone_in_the_random_word():
    rng = np.random.default_rng(4)
    y = rng.uniform(0, 6, 50)
    rs = np.sort(rng.integers(0, 2**32, 400, dtype=np.uint64))
    codes = osr.sr_cast_e2m1(np.repeat(y[:, None], 400, 1), np.broadcast_to(rs, (50, 400)))
    assert np.all(np.diff(codes, axis=1) <= 0)          # rounding up is a prefix of the word range


@pytest.mark.parametrize("rule", ["floor", "ceil"])
def test_block_scales_and_specials_follow_the_rne_path(rule):
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((64, 32)) * np.exp2(rng.integers(-30, 30, (64, 1)))).astype(np.float32)
    x[3, :] = 0.0
    x[4, :] = -0.0
    x[5, 7] = np.nan
    x[6, 2] = -np.inf
    x[7, 5] = -0.0
    r = rng.integers(0, 2**32, x.shape, dtype=np.uint64).astype(np.uint32)
    codes, scales = osr.quantize_blocks_sr(x, r, rule)
    _, rne_scales = omx.quantize_blocks(x, "e2m1", rule)
    assert np.array_equal(scales, rne_scales)
    for row in (5, 6):                 # non-finite block: the E2M1 'NaN' code (+-6) with each input's sign
        assert np.array_equal(codes[row], 0x7 | (np.signbit(x[row]).astype(np.uint8) << 3))
    assert np.all(codes[3] == 0) and np.all(codes[4] == 0x8) and codes[7, 5] == 0x8
    # every finite code is one of the two grid neighbours of |x| / X
    e = scales[8:].astype(np.int64) - 127
    y = np.abs(x[8:].astype(np.float64)) * np.exp2(-e)[:, None]
    mags = np.array(MAGS)[codes[8:] & 7]
    assert np.all((mags == np.vectorize(grid_floor)(y)) | (mags == np.vectorize(grid_ceil)(y)))
    assert np.array_equal(codes[8:] >> 3, np.signbit(x[8:]).astype(np.uint8))


def test_mean_tracks_the_input_statistically():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((1, 32)).astype(np.float32)
    n = 4000
    r = rng.integers(0, 2**32, (n, 32), dtype=np.uint64).astype(np.uint32)
    codes, scales = osr.quantize_blocks_sr(np.repeat(x, n, 0), r, "ceil")
    deq = omx.dequantize_exact(omx.pack_fp4(codes), scales, "e2m1")
    # per element: |mean - x| within 6 sigma of a two-point variable of span <= 2 X
    X = np.exp2(float(scales[0]) - 127)
    assert np.all(np.abs(deq.mean(axis=0) - x[0]) <= 6 * (2 * X) / 2 / np.sqrt(n))


def test_rowwise_layout_matches_blocks():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((8, 128)).astype(np.float32)
    r = rng.integers(0, 2**32, x.shape, dtype=np.uint64).astype(np.uint32)
    q, s = osr.quantize_rowwise_sr(x, r, "ceil")
    c2, s2 = osr.quantize_blocks_sr(x.reshape(8, 4, 32), r.reshape(8, 4, 32), "ceil")
    assert np.array_equal(q, omx.pack_fp4(c2.reshape(8, 128))) and np.array_equal(s, s2)


# ---- planted mistakes: each wrong variant of the oracle must fail a pin above

def test_planted_off_by_one_comparison_is_caught(monkeypatch):
    orig = osr.sr_threshold

    def wrong(y):                      # "r <= T" instead of "r < T"
        lo, t = orig(y)
        return lo, np.where(t > 0, t + 1, 0)
    monkeypatch.setattr(osr, "sr_threshold", wrong)
    with pytest.raises(AssertionError):
        test_unbiased_exactly_over_a_uniform_word_grid()


def test_planted_complement_probability_is_caught(monkeypatch):
    orig = osr.sr_threshold

    def wrong(y):                      # up with probability 1 - frac
        lo, t = orig(y)
        return lo, np.where(t > 0, 2.0**32 - t, 0)
    monkeypatch.setattr(osr, "sr_threshold", wrong)
    with pytest.raises(AssertionError):
        test_unbiased_exactly_over_a_uniform_word_grid()


def test_planted_reversed_word_direction_is_caught(monkeypatch):
    # up iff r >= 2^32 - T: the right probability, the opposite end of the word range
    monkeypatch.setattr(osr, "rounds_up", lambda r, t: (t > 0) & (r >= 2.0**32 - t))
    with pytest.raises(AssertionError):
        test_extreme_words_give_grid_ceiling_and_floor()
