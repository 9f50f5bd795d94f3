"""Pins of the per-tensor FP8 GEMM oracle (oracle.gemm.mm_fp8_ref).

Pinned to things other than itself: torch's own FP8 decode plus torch.matmul
(batch broadcasting included), a Fraction brute force written with explicit
indices over the stored layouts, the transposed-view identity, the bias and
scale laws, and planted mistakes that these pins must catch."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as ofmt
from oracle import gemm as og

TORCH_FP8 = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


def finite_codes(rng, shape, fmt):
    """Random finite FP8 codes (NaN / Inf codes redrawn)."""
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    bad = ~np.isfinite(ofmt.decode(c, fmt))
    while bad.any():
        c[bad] = rng.integers(0, 256, size=int(bad.sum())).astype(np.uint8)
        bad = ~np.isfinite(ofmt.decode(c, fmt))
    return c


def torch_ref(a, b, fmt, scale, ta, tb, bias):
    A = torch.from_numpy(a).view(TORCH_FP8[fmt]).double()
    B = torch.from_numpy(b).view(TORCH_FP8[fmt]).double()
    A = A.mT if ta else A
    B = B.mT if tb else B
    C = torch.matmul(A, B) * float(np.float32(scale))
    if bias is not None:
        C = C + torch.from_numpy(bias.view(np.int16)).view(torch.bfloat16).double()
    return C.numpy()


SHAPES = [  # (a stored shape builder, b stored shape builder) via (batch_a, batch_b)
    (None, None), (3, None), (None, 3), (3, 3), (1, 3), (3, 1)]


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("ta", [False, True])
@pytest.mark.parametrize("tb", [False, True])
@pytest.mark.parametrize("batches", SHAPES)
def test_against_torch_decode_and_matmul(fmt, ta, tb, batches):
    rng = np.random.default_rng(hash((fmt, ta, tb, batches)) % 2**32)
    M, N, K = 5, 7, 48
    ba, bb = batches
    sa = (K, M) if ta else (M, K)
    sb = (N, K) if tb else (K, N)
    a = finite_codes(rng, sa if ba is None else (ba,) + sa, fmt)
    b = finite_codes(rng, sb if bb is None else (bb,) + sb, fmt)
    bias = ofmt.f32_to_bf16_bits(rng.standard_normal(N).astype(np.float32))
    scale = np.float32(0.37)
    got = og.mm_fp8_ref(a, b, fmt, scale, ta, tb, bias)
    want = torch_ref(a, b, fmt, scale, ta, tb, bias)
    assert got.shape == want.shape
    # E4M3 sums are exact in float64 at this K; E5M2 products span more than 53 bits
    tol = 0.0 if fmt == "e4m3" else 1e-12
    assert np.allclose(got, want, rtol=tol, atol=tol * np.abs(want).max())


def fraction_brute_force(a, b, fmt, scale, ta, tb, bias):
    """C[p][m][n] = sum_k A(p, m, k) B(p, k, n) * scale + bias[n], indices spelled out
    over the stored arrays (no transposes, no matmul)."""
    va = ofmt.decode(a, fmt)
    vb = ofmt.decode(b, fmt)
    a3 = va if va.ndim == 3 else va[None]
    b3 = vb if vb.ndim == 3 else vb[None]
    P = max(a3.shape[0], b3.shape[0])
    M = a3.shape[2] if ta else a3.shape[1]
    K = a3.shape[1] if ta else a3.shape[2]
    N = b3.shape[1] if tb else b3.shape[2]
    bv = ofmt.bf16_bits_to_f32(bias).astype(np.float64) if bias is not None else np.zeros(N)
    out = np.zeros((P, M, N))
    for p in range(P):
        pa, pb = (p if a3.shape[0] > 1 else 0), (p if b3.shape[0] > 1 else 0)
        for m in range(M):
            for n in range(N):
                s = Fraction(0)
                for k in range(K):
                    x = a3[pa, k, m] if ta else a3[pa, m, k]
                    y = b3[pb, n, k] if tb else b3[pb, k, n]
                    s += Fraction(float(x)) * Fraction(float(y))
                out[p, m, n] = float(s * Fraction(float(np.float32(scale))) + Fraction(float(bv[n])))
    return out if (va.ndim == 3 or vb.ndim == 3) else out[0]


@pytest.mark.parametrize("ta,tb", [(False, False), (True, False), (False, True), (True, True)])
def test_against_fraction_brute_force(ta, tb):
    rng = np.random.default_rng(11)
    M, N, K = 3, 4, 6
    a = finite_codes(rng, (2,) + ((K, M) if ta else (M, K)), "e4m3")
    b = finite_codes(rng, (K, N) if not tb else (N, K), "e4m3")
    bias = ofmt.f32_to_bf16_bits(rng.standard_normal(N).astype(np.float32))
    got = og.mm_fp8_ref(a, b, "e4m3", np.float32(1.5), ta, tb, bias)
    want = fraction_brute_force(a, b, "e4m3", np.float32(1.5), ta, tb, bias)
    assert np.array_equal(got, want)


def test_transposed_storage_is_the_same_request():
    rng = np.random.default_rng(12)
    a = finite_codes(rng, (6, 64), "e4m3")
    b = finite_codes(rng, (64, 10), "e4m3")
    c0 = og.mm_fp8_ref(a, b, "e4m3", 1.0)
    c1 = og.mm_fp8_ref(np.ascontiguousarray(a.T), b, "e4m3", 1.0, trans_a=True)
    c2 = og.mm_fp8_ref(a, np.ascontiguousarray(b.T), "e4m3", 1.0, trans_b=True)
    assert np.array_equal(c0, c1) and np.array_equal(c0, c2)


def test_scale_and_bias_laws():
    rng = np.random.default_rng(13)
    a = finite_codes(rng, (4, 32), "e5m2")
    b = finite_codes(rng, (32, 6), "e5m2")
    base = og.mm_fp8_ref(a, b, "e5m2", 1.0)
    assert np.array_equal(og.mm_fp8_ref(a, b, "e5m2", 0.25), base * 0.25)      # power-of-two scale: exact
    bias = ofmt.f32_to_bf16_bits(np.arange(6, dtype=np.float32) - 2.5)
    with_bias = og.mm_fp8_ref(a, b, "e5m2", 0.25, bias=bias)
    assert np.array_equal(with_bias - base * 0.25, np.broadcast_to(np.arange(6) - 2.5, (4, 6)))
    zero = np.zeros((4, 32), np.uint8)                                        # code 0 = +0
    assert np.array_equal(og.mm_fp8_ref(zero, b, "e5m2", 3.0, bias=bias), np.broadcast_to(np.arange(6) - 2.5, (4, 6)))


def test_scale_is_taken_as_float32():
    a = np.array([[0x38]], np.uint8)        # E4M3 1.0
    b = np.array([[0x38]], np.uint8)
    assert og.mm_fp8_ref(a, b, "e4m3", 0.1)[0, 0] == float(np.float32(0.1))


# ---- planted mistakes: each wrong variant must fail a pin above

def _plant(monkeypatch, fn):
    monkeypatch.setattr(og, "mm_fp8_ref", fn)


def test_planted_ignored_transpose_is_caught(monkeypatch):
    orig = og.mm_fp8_ref

    def wrong(a, b, fmt, scale, trans_a=False, trans_b=False, bias=None):
        return orig(a, b, fmt, scale, trans_a, False, bias)      # the transpose of b dropped
    _plant(monkeypatch, wrong)
    b = finite_codes(np.random.default_rng(14), (8, 8), "e4m3")
    a = finite_codes(np.random.default_rng(15), (8, 8), "e4m3")
    with pytest.raises(AssertionError):
        assert np.array_equal(og.mm_fp8_ref(a, b, "e4m3", 1.0, trans_b=True),
                              fraction_brute_force(a, b, "e4m3", 1.0, False, True, None))


def test_planted_bias_before_scale_is_caught(monkeypatch):
    orig = og.mm_fp8_ref

    def wrong(a, b, fmt, scale, trans_a=False, trans_b=False, bias=None):
        c = orig(a, b, fmt, 1.0, trans_a, trans_b, bias)
        return c * float(np.float32(scale))
    _plant(monkeypatch, wrong)
    with pytest.raises(AssertionError):
        test_scale_and_bias_laws()


def test_planted_wrong_broadcast_is_caught(monkeypatch):
    orig = og.mm_fp8_ref

    def wrong(a, b, fmt, scale, trans_a=False, trans_b=False, bias=None):
        if np.ndim(b) == 3 and np.ndim(a) == 3 and a.shape[0] == 1:   # uses batch 0 of b everywhere
            b = np.repeat(np.asarray(b)[:1], b.shape[0], 0)
        return orig(a, b, fmt, scale, trans_a, trans_b, bias)
    _plant(monkeypatch, wrong)
    with pytest.raises(AssertionError):
        test_against_torch_decode_and_matmul("e4m3", False, False, (1, 3))
