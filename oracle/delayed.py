"""Per-tensor FP8 quantization with delayed scaling (CPU oracle).

Test infrastructure only (see ``oracle/__init__``).

[FP8PY] (module docstring, ``quantize`` docstring and commit message): a tensor
is cast to FP8 with one multiplier for the whole tensor while its amax is taken
in the same pass; with a ring state, the amax is folded into the history slot
``hist[hist_idx]`` and the next scale is published as
max(hist) / fp8_max / pow2_margin.  Readings where the page is silent or
contradicts itself:

* the ring holds [hist[0..n-1] | s | m | amax | ticket]; s is the dequantization
  scale (x ~ q * s), m = fl32(1 / s) is the multiplier the cast uses (the page
  calls the passed scale a multiplier but publishes a dequantization scale; the
  slot it labels 'legacy' carries m here);
* the cast is y = fl32(x * m) followed by one RNE + saturating cast;
* s <- fl32(fl32(h / fp8_max) / margin) and m <- fl32(1 / s) when
  0 < h = max(hist) < inf; otherwise s and m keep their values;
* initially hist = 0, s = m = 1; the amax slot reads 0 after every call;
* the per-tensor amax ignores NaN entries.
"""

import numpy as np

from .formats import encode, fmt_of
from .mx import tensor_amax


def cast_per_tensor(x, multiplier, fmt) -> np.ndarray:
    """q = sat(RNE_fmt(fl32(x * m))) for an FP32 array x and FP32 scalar m."""
    y = np.asarray(x, dtype=np.float32) * np.float32(multiplier)   # one FP32 rounding
    return encode(y.astype(np.float64), fmt_of(fmt))


class Ring:
    """Host model of the device ring state of one tensor stream."""

    def __init__(self, hist_len: int):
        self.hist = np.zeros(hist_len, dtype=np.float32)
        self.s = np.float32(1.0)
        self.m = np.float32(1.0)

    def as_array(self, scratch_words: int = 0) -> np.ndarray:
        """The buffer layout between calls: [hist | s | m | amax(=0) | ticket(=0)],
        followed by `scratch_words` zero words when the buffer carries extra
        ticket scratch."""
        return np.concatenate([self.hist, np.array([self.s, self.m, 0.0, 0.0], dtype=np.float32),
                               np.zeros(scratch_words, dtype=np.float32)])

    @classmethod
    def from_array(cls, arr, scratch_words: int = 0):
        arr = np.asarray(arr, dtype=np.float32)
        n = arr.size - 4 - scratch_words
        r = cls(n)
        r.hist = arr[:n].copy()
        r.s = np.float32(arr[n])
        r.m = np.float32(arr[n + 1])
        return r

    def fold(self, amax, hist_idx: int, fp8_max: float, margin: float):
        """Write amax into the history window, then derive the next scale."""
        self.hist[hist_idx] = np.float32(amax)
        h = np.float32(np.max(self.hist))
        if h > 0 and np.isfinite(h):
            s = np.float32(np.float32(h / np.float32(fp8_max)) / np.float32(margin))
            self.s = s
            self.m = np.float32(np.float32(1.0) / s)


def quantize_delayed(x, fmt, ring: Ring, hist_idx: int, fp8_max: float, margin: float):
    """One call: cast with the ring's current multiplier, then fold.

    Returns (q [R][C], qT [C][R], amax).  Mutates ``ring``.
    """
    x = np.asarray(x, dtype=np.float32)
    q = cast_per_tensor(x, ring.m, fmt)
    a = tensor_amax(x)
    ring.fold(a, hist_idx, fp8_max, margin)
    return q, np.ascontiguousarray(q.T), a
