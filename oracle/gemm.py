"""Block-scaled (MX) GEMM reference (CPU oracle).

Test infrastructure only (see ``oracle/__init__``).

[UE8M0] (MX definition paragraph): the matrix unit consumes the scale X and the
element codes Q_i of both operands and accumulates their products; the result is
requantized only if the next operator needs MX.  The MXFP8 study on the same
page emulates this by quantizing the GEMM inputs and running the product in
high precision.  The oracle does exactly that: dequantize both operands exactly
(float64 holds every value) and multiply them in float64.

Layout: A is [M][K] codes with scales [M][K/32]; B is given as [N][K] codes with
scales [N][K/32] (both K-contiguous, the "NT" layout); C = alpha * A B^T.
"""

import numpy as np

from .formats import f64_to_bf16_bits
from .mx import dequantize_exact


def gemm_ref(a, sa, fmt_a, b, sb, fmt_b, alpha=1.0, rows=None, cols=None) -> np.ndarray:
    """float64 C = alpha * deq(A) deq(B)^T, optionally only for the given row / column indices."""
    A = dequantize_exact(a if rows is None else np.asarray(a)[rows],
                         sa if rows is None else np.asarray(sa)[rows], fmt_a)
    B = dequantize_exact(b if cols is None else np.asarray(b)[cols],
                         sb if cols is None else np.asarray(sb)[cols], fmt_b)
    return float(alpha) * (A @ B.T)


def gemm_ref_bf16(*args, **kw) -> np.ndarray:
    """The reference rounded once to BF16 (bits)."""
    return f64_to_bf16_bits(gemm_ref(*args, **kw))


def rel_frobenius(c, ref) -> float:
    c = np.asarray(c, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(c - ref) / (den if den > 0 else 1.0))


def mm_fp8_ref(a, b, fmt, scale, trans_a=False, trans_b=False, bias=None) -> np.ndarray:
    """Per-tensor FP8 GEMM reference: float64 op(a) @ op(b) * scale (+ bias).

    [FP8PY] (``mm_fp8``): a and b are FP8 codes of one format, 2-D or 3-D, the
    batch dimension broadcast as in matmul; op(x) is x transposed in its last two
    dimensions when the matching flag is set (the flag and an inner-transposed
    view are the same request); ``scale`` is the combined dequantization scale
    of both operands; ``bias`` (BF16 bits, length n) is added in the epilogue.
    The codes decode exactly to float64; the product, the scale and the bias
    are applied in float64 in that order: (a @ b) * scale + bias."""
    from .formats import bf16_bits_to_f32, decode
    A = decode(np.asarray(a), fmt)
    B = decode(np.asarray(b), fmt)
    if trans_a:
        A = np.swapaxes(A, -1, -2)
    if trans_b:
        B = np.swapaxes(B, -1, -2)
    C = np.matmul(A, B) * float(np.float32(scale))
    if bias is not None:
        C = C + bf16_bits_to_f32(np.asarray(bias, dtype=np.uint16)).astype(np.float64)
    return C
