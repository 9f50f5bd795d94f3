"""Pins for the oracle's per-tensor delayed-scaling quantizer (CPU only).

The page states the behaviour, not a worked example: the history is a window of
the last n per-tensor amaxes, the next scale is max(window) / fp8_max / margin,
and the cast multiplies by the current multiplier.  These tests check that
behaviour from outside: window length, what the published scale does to the
next cast, the empty / non-finite history rule, and the margin.
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import delayed
from oracle import formats as F


def _tensor(amax, seed, shape=(32, 64)):
    x = workloads.random_tensor(shape, seed, "normal")
    x = x / np.abs(x).max() * np.float32(amax)
    x.reshape(-1)[np.argmax(np.abs(x))] = np.float32(amax)
    return x.astype(np.float32)


@pytest.mark.parametrize("fmt,fp8_max", [("e4m3", 448.0), ("e5m2", 57344.0)])
def test_next_scale_maps_history_max_onto_fp8_max(fmt, fp8_max):
    ring = delayed.Ring(16)
    x = _tensor(3.7, 0)
    delayed.quantize_delayed(x, fmt, ring, 0, fp8_max, 1.0)
    # the second cast of the same tensor puts its amax on (or next to) the top code
    q, _, _ = delayed.quantize_delayed(x, fmt, ring, 1, fp8_max, 1.0)
    top = F.decode(q, fmt)
    assert np.nanmax(np.abs(top)) == fp8_max
    # and the dequantized tensor is close to the input
    deq = top * np.float64(ring.s)
    f = F.FORMATS[fmt]
    # RNE: at most half a quantum, i.e. 2^-(mbits+1) relative, or half the smallest subnormal
    tol = np.maximum(np.abs(x) * 2.0 ** -(f.mbits + 1), float(ring.s) * f.min_subnormal / 2)
    assert np.all(np.abs(deq - x) <= tol * (1 + 1e-6))


def test_window_length_and_history_index():
    n = 16
    ring = delayed.Ring(n)
    spike = _tensor(1000.0, 1)
    small = [_tensor(1.0 + t / 64, 2 + t) for t in range(40)]
    delayed.quantize_delayed(spike, "e4m3", ring, 0, 448.0, 1.0)
    s_spike = ring.s
    for t in range(1, n):
        delayed.quantize_delayed(small[t], "e4m3", ring, t % n, 448.0, 1.0)
        assert ring.s == s_spike                        # the spike is still in the window
    delayed.quantize_delayed(small[n], "e4m3", ring, n % n, 448.0, 1.0)
    assert ring.s < s_spike                              # overwritten after n steps
    largest = max(float(np.abs(small[t]).max()) for t in range(1, n + 1))
    assert float(ring.s) == pytest.approx(largest / 448.0, rel=2 ** -23)


def test_scale_uses_float32_division_once_each():
    ring = delayed.Ring(4)
    a = np.float32(1234.5677)
    x = _tensor(a, 3)
    delayed.quantize_delayed(x, "e4m3", ring, 2, 448.0, 1.0)
    # compare with torch's float32 division (an independent IEEE implementation)
    s = torch.tensor(float(a), dtype=torch.float32) / torch.tensor(448.0, dtype=torch.float32)
    m = torch.tensor(1.0, dtype=torch.float32) / s
    assert ring.s == np.float32(s.item()) and ring.m == np.float32(m.item())


def test_empty_and_nonfinite_history_keep_scale():
    ring = delayed.Ring(8)
    delayed.quantize_delayed(np.zeros((32, 32), np.float32), "e4m3", ring, 0, 448.0, 1.0)
    assert ring.s == 1.0 and ring.m == 1.0
    x = _tensor(2.0, 4)
    delayed.quantize_delayed(x, "e4m3", ring, 1, 448.0, 1.0)
    s = ring.s
    y = x.copy()
    y[0, 0] = np.inf
    delayed.quantize_delayed(y, "e4m3", ring, 2, 448.0, 1.0)
    assert ring.s == s


def test_margin_divides_scale():
    r1, r2 = delayed.Ring(4), delayed.Ring(4)
    x = _tensor(100.0, 5)
    delayed.quantize_delayed(x, "e4m3", r1, 0, 448.0, 1.0)
    delayed.quantize_delayed(x, "e4m3", r2, 0, 448.0, 2.0)
    assert r2.s == r1.s / 2


def test_cast_is_multiply_then_one_rounding():
    # with m = 1 the cast is the plain saturating FP8 cast of x, which torch
    # implements independently for in-range values
    x = _tensor(400.0, 6)
    q = delayed.cast_per_tensor(x, 1.0, "e4m3")
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, ref)
    q = delayed.cast_per_tensor(x, 2.0, "e4m3")          # 800 saturates to 448
    assert F.decode(q, "e4m3").max() == 448.0


def test_transposed_output_and_amax():
    ring = delayed.Ring(16)
    x = _tensor(5.0, 7, shape=(64, 96))
    x[3, 3] = np.nan
    q, qT, a = delayed.quantize_delayed(x, "e5m2", ring, 0, 57344.0, 1.0)
    assert np.array_equal(qT, q.T) and a == np.float32(5.0)


def test_ring_layout_roundtrip():
    ring = delayed.Ring(16)
    delayed.quantize_delayed(_tensor(9.0, 8), "e4m3", ring, 5, 448.0, 1.0)
    arr = ring.as_array()
    assert arr.shape == (20,) and arr[5] == np.float32(9.0) and arr[18] == 0 and arr[19] == 0
    r2 = delayed.Ring.from_array(arr)
    assert r2.s == ring.s and r2.m == ring.m and np.array_equal(r2.hist, ring.hist)
