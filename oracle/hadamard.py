"""Fixed-sign 32-point Walsh-Hadamard preconditioning (CPU oracle).

Test infrastructure only (see ``oracle/__init__``).

[FAF] (the MXFP4 recipe paragraph) applies a 32-point Hadamard transform with a
fixed sign vector to each 32-element block of the weight-gradient GEMM's
reduction dimension before MXFP4 quantization.  The page gives no formula; the
reading taken here:

* the sign vector is a 32-bit mask drawn once from the seed: element j of every
  block is negated when bit j is set;
* the transform is the unnormalised Sylvester Hadamard matrix H32 (entries +-1),
  applied as the in-place fast transform with butterfly stages of span
  h = 1, 2, 4, 8, 16, each pair (i, i+h) with (i & h) == 0 becoming
  (v_i + v_{i+h}, v_i - v_{i+h});
* every addition is one FP32 operation rounded to nearest even, in exactly that
  order (so a GPU doing the same additions reproduces the bits);
* both GEMM operands get the same transform along the reduction axis; since
  H32 H32^T = 32 I, the GEMM multiplies its result by alpha = 1/32;
* a NaN produced by the additions (from a NaN input, or Inf - Inf) has no sign
  that IEEE 754 fixes, so every NaN leaving the transform has its sign bit
  cleared; Inf and finite results keep their signs.
"""

import numpy as np


def sign_flip(blocks, sign_mask: int) -> np.ndarray:
    x = np.asarray(blocks, dtype=np.float32)
    bits = (np.uint64(sign_mask) >> np.arange(32, dtype=np.uint64)) & np.uint64(1)
    return np.where(bits.astype(bool), -x, x).astype(np.float32)


def hadamard32(blocks, sign_mask: int) -> np.ndarray:
    """Sign flip then unnormalised FWHT over the last axis (length 32), in FP32."""
    v = sign_flip(blocks, sign_mask).copy()
    assert v.shape[-1] == 32
    h = 1
    while h < 32:
        for i in range(32):
            if i & h == 0:
                a = v[..., i].copy()
                b = v[..., i + h].copy()
                v[..., i] = a + b          # float32 + float32 -> float32, RNE
                v[..., i + h] = a - b
        h *= 2
    bits = v.view(np.uint32)
    return np.where(np.isnan(v), (bits & np.uint32(0x7FFFFFFF)).view(np.float32), v)
