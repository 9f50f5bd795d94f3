"""Pins for the oracle's Hadamard preconditioning and GEMM reference (CPU only)."""

from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg
import torch

import workloads
from oracle import gemm, hadamard, mx
from tests import pins


def _signs(mask):
    return np.array([-1.0 if (mask >> j) & 1 else 1.0 for j in range(32)])


def check_hadamard_exact(h32) -> bool:
    """On small integers every FP32 addition is exact, so the transform must equal
    the Sylvester matrix product scipy builds, times the sign diagonal."""
    g = np.random.default_rng(0)
    x = g.integers(-1000, 1000, size=(64, 32)).astype(np.float32)
    mask = 0x9E3779B9
    got = h32(x, mask).astype(np.float64)
    H = scipy.linalg.hadamard(32).astype(np.float64)
    want = (x.astype(np.float64) * _signs(mask)) @ H.T
    return bool(np.array_equal(got, want))


def test_hadamard_equals_sylvester_product_on_integers():
    assert check_hadamard_exact(hadamard.hadamard32)


def test_hadamard_close_to_sylvester_on_reals():
    x = workloads.random_tensor((256, 32), 1, "normal")
    mask = 0x12345678
    got = hadamard.hadamard32(x, mask).astype(np.float64)
    H = scipy.linalg.hadamard(32).astype(np.float64)
    want = (x.astype(np.float64) * _signs(mask)) @ H.T
    # five rounded additions, each error <= 2^-24 of its magnitude (<= 32 max|x|)
    bound = 5 * 2.0 ** -24 * 32 * np.abs(x).max(axis=1, keepdims=True)
    assert np.all(np.abs(got - want) <= bound)


def test_hadamard_orthogonality_and_gemm_invariance():
    H = scipy.linalg.hadamard(32)
    assert np.array_equal(H @ H.T, 32 * np.eye(32, dtype=H.dtype))
    g = np.random.default_rng(4)
    A = g.integers(-8, 9, size=(8, 64)).astype(np.float32)
    B = g.integers(-8, 9, size=(6, 64)).astype(np.float32)
    mask = 0xDEADBEEF
    At = hadamard.hadamard32(A.reshape(8, 2, 32), mask).reshape(8, 64).astype(np.float64)
    Bt = hadamard.hadamard32(B.reshape(6, 2, 32), mask).reshape(6, 64).astype(np.float64)
    assert np.array_equal(At @ Bt.T / 32.0, A.astype(np.float64) @ B.T.astype(np.float64))


def test_hadamard_mask_zero_is_plain_fwht_and_identity_twice():
    x = np.random.default_rng(5).integers(-50, 50, size=(10, 32)).astype(np.float32)
    y = hadamard.hadamard32(hadamard.hadamard32(x, 0), 0)
    assert np.array_equal(y, 32 * x)


def test_hadamard_nonfinite_signs():
    """Non-finite inputs: an Inf propagates as +-Inf with the signs of its column
    of H32 (an IEEE-defined sign); a NaN, or Inf - Inf, makes NaNs, which leave
    the transform with a clear sign bit whatever the input NaN's sign."""
    H = scipy.linalg.hadamard(32)
    x = np.zeros((3, 32), np.float32)
    x[0, 5] = np.inf                             # column 5 of H32, times +Inf
    x[1, 9] = -np.float32(np.nan)                # a NaN with its sign bit set
    x[2, 3], x[2, 4] = np.inf, np.inf            # +Inf +- Inf: NaN where H32's signs differ
    y = hadamard.hadamard32(x, 0)
    assert np.array_equal(y[0], np.where(H[:, 5] > 0, np.inf, -np.inf).astype(np.float32))
    assert np.isnan(y[1]).all() and not np.signbit(y[1]).any()
    differ = H[:, 3] != H[:, 4]
    assert np.isnan(y[2][differ]).all() and not np.signbit(y[2][differ]).any()
    assert np.array_equal(y[2][~differ], np.where(H[~differ, 3] > 0, np.inf, -np.inf).astype(np.float32))
    # through the MX quantizer: a NaN block's codes are the positive NaN code (E2M1: +6)
    q, s = mx.quantize_rowwise(x[1:2], "e4m3", "ceil", hadamard_mask=0xFFFFFFFF)
    assert list(s[0]) == [0xFF] and (q == 0x7F).all()
    q, s = mx.quantize_rowwise(x[1:2], "e2m1", "ceil", hadamard_mask=0)
    assert list(s[0]) == [0xFF] and (mx.unpack_fp4(q) == 0x7).all()


def test_planted_nan_sign_passthrough_is_caught(monkeypatch):
    """An oracle that leaves the sign of the NaNs numpy's additions produce must
    fail the pin above (numpy keeps the input NaN's sign bit through a + b)."""
    def passthrough(blocks, sign_mask):
        v = hadamard.sign_flip(blocks, sign_mask).copy()
        h = 1
        while h < 32:
            for i in range(32):
                if i & h == 0:
                    a, b = v[..., i].copy(), v[..., i + h].copy()
                    v[..., i], v[..., i + h] = a + b, a - b
            h *= 2
        return v
    monkeypatch.setattr(hadamard, "hadamard32", passthrough)
    with pytest.raises(AssertionError):
        test_hadamard_nonfinite_signs()


# ---------------------------------------------------------------- GEMM

def _quantized_pair(M, N, K, fa, fb, rule="ceil", seed=0):
    A = workloads.random_tensor((M, K), seed, "normal")
    # give consecutive K-blocks different magnitudes so that every block scale matters
    A = (A * np.exp2(np.arange(K) // 32 * 5 % 17)[None, :]).astype(np.float32)
    B = workloads.random_tensor((N, K), seed + 1, "rows")
    qa, sa = mx.quantize_rowwise(A, fa, rule)
    qb, sb = mx.quantize_rowwise(B, fb, rule)
    return qa, sa, qb, sb


def check_gemm_fraction(gemm_ref, fa, fb) -> bool:
    M, N, K = 3, 4, 64
    qa, sa, qb, sb = _quantized_pair(M, N, K, fa, fb, seed=3)
    got = gemm_ref(qa, sa, fa, qb, sb, fb, alpha=0.5)
    ua = mx.unpack_fp4(qa) if fa == "e2m1" else qa
    ub = mx.unpack_fp4(qb) if fb == "e2m1" else qb
    for i in range(M):
        for j in range(N):
            av = [pins.frac_decode(int(ua[i, k]), fa) * Fraction(2) ** (int(sa[i, k // 32]) - 127) for k in range(K)]
            bv = [pins.frac_decode(int(ub[j, k]), fb) * Fraction(2) ** (int(sb[j, k // 32]) - 127) for k in range(K)]
            exact = Fraction(1, 2) * sum((x * y for x, y in zip(av, bv)), Fraction(0))
            if exact == 0:
                if got[i, j] != 0:
                    return False
            elif abs(Fraction(float(got[i, j])) - exact) > abs(exact) * Fraction(1, 2 ** 40):
                return False
    return True


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e2m1", "e2m1")])
def test_gemm_reference_against_fraction(fa, fb):
    assert check_gemm_fraction(gemm.gemm_ref, fa, fb)


def test_gemm_unit_scales_reduce_to_torch_fp8_matmul():
    g = np.random.default_rng(8)
    qa = g.integers(0, 256, size=(16, 64)).astype(np.uint8)
    qb = g.integers(0, 256, size=(8, 64)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x01
    qb[(qb & 0x7F) == 0x7F] = 0x02
    ones_a = np.full((16, 2), 127, np.uint8)
    ones_b = np.full((8, 2), 127, np.uint8)
    got = gemm.gemm_ref(qa, ones_a, "e4m3", qb, ones_b, "e4m3")
    ta = torch.from_numpy(qa).view(torch.float8_e4m3fn).to(torch.float64)
    tb = torch.from_numpy(qb).view(torch.float8_e4m3fn).to(torch.float64)
    assert np.allclose(got, (ta @ tb.T).numpy(), rtol=1e-14, atol=0)


def test_gemm_sampled_rows_cols_match_full():
    qa, sa, qb, sb = _quantized_pair(40, 24, 128, "e4m3", "e4m3")
    full = gemm.gemm_ref(qa, sa, "e4m3", qb, sb, "e4m3")
    rows = np.array([0, 7, 39])
    cols = np.array([3, 23])
    part = gemm.gemm_ref(qa, sa, "e4m3", qb, sb, "e4m3", rows=rows, cols=cols)
    assert np.array_equal(part, full[np.ix_(rows, cols)])


def test_bf16_output_rounding_error_of_exact_product():
    """The BF16 output alone puts about 1.6e-3 relative Frobenius error on a
    Gaussian-like product, which is why the GEMM parity bound is taken against
    the BF16-rounded reference."""
    qa, sa, qb, sb = _quantized_pair(64, 64, 256, "e4m3", "e4m3")
    ref = gemm.gemm_ref(qa, sa, "e4m3", qb, sb, "e4m3")
    bf = workloads.bf16_to_f32(gemm.gemm_ref_bf16(qa, sa, "e4m3", qb, sb, "e4m3"))
    err = gemm.rel_frobenius(bf, ref)
    assert 5e-4 < err < 3e-3
