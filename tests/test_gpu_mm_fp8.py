"""GPU parity of the per-tensor FP8 GEMM (mm_fp8) against the oracle's float64
op(a) @ op(b) * scale + bias.

Bounds (as for the block-scaled GEMM): the BF16 output is compared with the
reference rounded once to BF16 within 1e-3 relative Frobenius error, and every
element within one BF16 rounding (2^-8 relative) plus 2^-10 * scale *
sum_k |a_k b_k| of the float64 reference -- the matrix unit's fixed-point
accumulation window -- which any wrong pairing of rows, columns, batches or
layouts misses by orders of magnitude (the aggregate is graded from 256 outputs
up; below that a single 1-ulp BF16 flip exceeds it).  Integer-valued operands, whose FP32
sums are exact, are compared bit for bit."""

import numpy as np
import pytest
import torch

import workloads
from oracle import formats as ofmt
from oracle import gemm as og
from tests.gpu_util import assert_bytes_equal, host, import_library, tile_strata, upload_bf16_bits, upload_u8

pytestmark = pytest.mark.gpu

mxa = import_library()

BF16_TOL = 1e-3
ELEM_REL = 2.0 ** -10
TORCH_FP8 = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
LAYOUTS = [(False, False), (True, False), (False, True), (True, True)]


def codes(shape, seed, fmt, spread=4.0):
    """FP8 codes of N(0,1) * 2^U(-spread, spread) draws (oracle encoder, RNE)."""
    g = workloads.rng(3000 + seed)
    v = g.standard_normal(shape) * np.exp2(g.uniform(-spread, spread, size=shape))
    return ofmt.encode(v, fmt).astype(np.uint8)


def stored(shape_mk, trans, batch=None):
    """Stored shape of an operand whose op() is [rows][cols] = shape_mk."""
    r, c = shape_mk
    s = (c, r) if trans else (r, c)
    return s if batch is None else (batch,) + s


def as_fp8(x: np.ndarray, fmt: str) -> torch.Tensor:
    return upload_u8(x).view(TORCH_FP8[fmt])


def bf16_f64(bits):
    return workloads.bf16_to_f32(bits).astype(np.float64)


def scale_tensor(v):
    return torch.tensor([v], dtype=torch.float32, device="cuda")


def check(c_bits, a, b, fmt, scale, ta, tb, bias, what):
    ref = og.mm_fp8_ref(a, b, fmt, scale, ta, tb, bias)
    A = np.abs(ofmt.decode(a, fmt))
    B = np.abs(ofmt.decode(b, fmt))
    mag = np.matmul(np.swapaxes(A, -1, -2) if ta else A, np.swapaxes(B, -1, -2) if tb else B) * float(scale)
    got = bf16_f64(c_bits)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if got.size >= 256:
        # an aggregate: below a few hundred outputs one legitimate 1-ulp BF16 flip of
        # an exact value near a rounding boundary exceeds it on its own
        err = og.rel_frobenius(got, bf16_f64(og.f64_to_bf16_bits(ref)))
        assert err <= BF16_TOL, (what, err)
    bad = np.abs(got - ref) > 2.0 ** -8 * np.abs(ref) + ELEM_REL * mag + 1e-30
    assert not bad.any(), f"{what}: {bad.sum()} outputs outside the bound, first {np.argwhere(bad)[:4].tolist()}"


def run(a, b, fmt, scale, ta, tb, bias):
    bt = None if bias is None else upload_bf16_bits(bias)
    return host(mxa.mm_fp8(as_fp8(a, fmt), as_fp8(b, fmt), scale_tensor(scale), ta, tb, bt))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("shape", [(128, 128, 128), (200, 136, 96), (1, 7, 16), (64, 300, 512), (250, 260, 1040)])
def test_mm_fp8_small_parity(fmt, ta, tb, shape):
    M, N, K = shape
    a = codes(stored((M, K), ta), M + K, fmt)
    b = codes(stored((K, N), tb), N + K + 1, fmt)
    bias = ofmt.f32_to_bf16_bits(workloads.random_tensor((N,), 5, "normal") * 8)
    check(run(a, b, fmt, 0.3125, ta, tb, bias), a, b, fmt, 0.3125, ta, tb, bias, f"{shape}")
    check(run(a, b, fmt, 1.5, ta, tb, None), a, b, fmt, 1.5, ta, tb, None, f"{shape} no bias")


# 256 x 256-tile path shapes: one tile at the minimum K; 6 tiles; one wide tile row at K = 3 * 1024
TILED = [(256, 256, 1024), (512, 768, 2048), (256, 1024, 3072), (272, 400, 1024),   # ragged tiles
         (256, 256, 128), (512, 256, 640)]                                                # K past the last pair


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("shape", TILED)
def test_mm_fp8_tiled_parity(fmt, ta, tb, shape):
    M, N, K = shape
    a = codes(stored((M, K), ta), 7 + M, fmt)
    b = codes(stored((K, N), tb), 9 + N, fmt)
    bias = ofmt.f32_to_bf16_bits(workloads.random_tensor((N,), 6, "normal") * 64)
    check(run(a, b, fmt, 0.0078125, ta, tb, bias), a, b, fmt, 0.0078125, ta, tb, bias, f"{shape}")


@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("shape", [(96, 80, 64), (256, 512, 1024)])
@pytest.mark.parametrize("batches", [(3, None), (None, 3), (3, 3), (1, 3), (3, 1)])
def test_mm_fp8_batched(ta, tb, shape, batches):
    M, N, K = shape
    ba, bb = batches
    a = codes(stored((M, K), ta, ba), 11, "e4m3")
    b = codes(stored((K, N), tb, bb), 12, "e4m3")
    bias = ofmt.f32_to_bf16_bits(workloads.random_tensor((N,), 7, "normal"))
    check(run(a, b, "e4m3", 0.25, ta, tb, bias), a, b, "e4m3", 0.25, ta, tb, bias, f"{shape} {batches}")


@pytest.mark.parametrize("shape", [(96, 80, 64), (512, 256, 1024)])
def test_transposed_views_fold_into_the_layout(shape):
    M, N, K = shape
    a = codes((M, K), 13, "e4m3")
    b = codes((K, N), 14, "e4m3")
    sc = scale_tensor(0.5)
    A, B = as_fp8(a, "e4m3"), as_fp8(b, "e4m3")
    At = as_fp8(np.ascontiguousarray(a.T), "e4m3")        # stored [K][M]
    Bt = as_fp8(np.ascontiguousarray(b.T), "e4m3")        # stored [N][K]
    base = mxa.mm_fp8(A, B, sc)
    assert torch.equal(mxa.mm_fp8(At.t(), B, sc), base)               # view of the transpose, no flag
    assert torch.equal(mxa.mm_fp8(At, B, sc, trans_a=True), base)      # flag on the stored transpose
    assert torch.equal(mxa.mm_fp8(A, Bt.t(), sc), base)
    assert torch.equal(mxa.mm_fp8(A, Bt, sc, trans_b=True), base)
    assert torch.equal(mxa.mm_fp8(A.t(), B, sc, trans_a=True), base)   # view and flag cancel
    check(host(base), a, b, "e4m3", 0.5, False, False, None, "views")


@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("shape", [(96, 80, 64), (256, 256, 1024)])
def test_mm_fp8_integer_operands_bit_exact(ta, tb, shape):
    """Small integers: every FP32 partial sum is exact, so the only rounding is the
    final BF16 one of the exact value (scale a power of two, integer bias)."""
    M, N, K = shape
    g = workloads.rng(3100 + M)
    a = ofmt.encode(g.integers(-3, 4, size=stored((M, K), ta)).astype(np.float64), "e4m3").astype(np.uint8)
    b = ofmt.encode(g.integers(-3, 4, size=stored((K, N), tb)).astype(np.float64), "e4m3").astype(np.uint8)
    bias = ofmt.f32_to_bf16_bits(g.integers(-100, 100, size=N).astype(np.float32))
    got = run(a, b, "e4m3", 0.5, ta, tb, bias)
    want = og.f64_to_bf16_bits(og.mm_fp8_ref(a, b, "e4m3", 0.5, ta, tb, bias))
    assert_bytes_equal(got.view(np.uint16), want, f"{shape} {ta} {tb}")


def test_mm_fp8_k0_writes_the_bias():
    a = torch.empty((5, 0), dtype=torch.float8_e4m3fn, device="cuda")
    b = torch.empty((0, 7), dtype=torch.float8_e4m3fn, device="cuda")
    bias = ofmt.f32_to_bf16_bits(np.arange(7, dtype=np.float32) - 3)
    out = host(mxa.mm_fp8(a, b, scale_tensor(2.0), bias=upload_bf16_bits(bias)))
    assert np.array_equal(out.view(np.uint16), np.broadcast_to(bias, (5, 7)))
    out = host(mxa.mm_fp8(a, b, scale_tensor(2.0)))
    assert np.all(out.view(np.uint16) == 0)


def test_mm_fp8_binding_errors():
    a = torch.zeros((64, 64), dtype=torch.float8_e4m3fn, device="cuda")
    b = torch.zeros((48, 64), dtype=torch.float8_e4m3fn, device="cuda")
    with pytest.raises(ValueError):
        mxa.mm_fp8(a, b, scale_tensor(1.0))                  # inner dimensions differ
    with pytest.raises(ValueError):
        mxa.mm_fp8(a, a.view(torch.float8_e5m2), scale_tensor(1.0))   # mixed formats
    with pytest.raises(ValueError):
        mxa.mm_fp8(a[:, ::2], a[::2], scale_tensor(1.0))      # strided view
    with pytest.raises(ValueError):
        mxa.mm_fp8(a, a, 1.0)                                 # scale must be a device tensor


def field_codes(shape, seed, fmt):
    """Random finite FP8 codes drawn field by field: sign, an exponent field in a
    mid range (values ~2^-3 .. 2^4) and any mantissa."""
    g = workloads.rng(3200 + seed)
    sign = g.integers(0, 2, size=shape, dtype=np.uint8)
    mant = g.integers(0, 8 if fmt == "e4m3" else 4, size=shape, dtype=np.uint8)
    if fmt == "e4m3":
        return (sign << 7) | (g.integers(4, 11, size=shape, dtype=np.uint8) << 3) | mant
    return (sign << 7) | (g.integers(12, 19, size=shape, dtype=np.uint8) << 2) | mant


@pytest.mark.parametrize("tb", [True, False])
def test_mm_fp8_full_size(tb):
    """The linear-layer workload: x [8192][4096] times w [14336][4096] (x @ w.t(),
    K-contiguous) or w stored [4096][14336] (N-contiguous), with bias: one whole
    row from every 256-row output tile and one whole column from every
    256-column tile against the oracle, so every tile of the launch is checked."""
    M, N, K = 8192, 14336, 4096
    x = field_codes((M, K), 21, "e4m3")
    w = field_codes((N, K) if tb else (K, N), 22, "e4m3")
    bias = ofmt.f32_to_bf16_bits(workloads.random_tensor((N,), 8, "normal"))
    out = run(x, w, "e4m3", 0.015625, False, tb, bias)
    rows = tile_strata(M, 256, 23)
    cols = tile_strata(N, 256, 24)
    check(out[rows], x[rows], w, "e4m3", 0.015625, False, tb, bias, "full-size rows")
    ws = w[cols] if tb else w[:, cols]
    check(out[:, cols], x, ws, "e4m3", 0.015625, False, tb, bias[cols], "full-size columns")