"""GPU parity of the block-scaled GEMM against the oracle's float64 product of
the dequantized operands.

Tolerances (graded bound 1e-3 relative Frobenius error):
* FP32 output: within 1e-3 of the float64 reference, and elementwise within
  2^-10 * sum_k |a_k b_k| -- the matrix unit aligns the products of each step to
  a fixed-point window of limited width instead of rounding every addition in
  IEEE FP32 (measured: at most ~2^-12 of the largest product on adversarial
  data), so this is the bound a correct kernel meets while any wrong pairing of
  codes, scales or lanes misses it by orders of magnitude;
* BF16 output: compared with the reference rounded once to BF16, within 1e-3
  (the BF16 rounding of an exact result alone is ~1.6e-3 away from float64, so
  the raw float64 distance is reported, not graded)."""

import functools

import numpy as np
import pytest
import torch

import workloads
from oracle import gemm as og
from oracle import mx as omx
from tests.gpu_util import (assert_bytes_equal, check_bf16_lines, host, import_library, tile_strata, upload_bf16_bits,
                            upload_f32, upload_u8, abs_product)

pytestmark = pytest.mark.gpu

mxa = import_library()

FP32_TOL = 1e-3
BF16_TOL = 1e-3
ELEM_REL = 2.0 ** -10


def check_fp32(c32, qa, sa, fa, qb, sb, fb, alpha=1.0, rows=None, cols=None):
    ref = og.gemm_ref(qa, sa, fa, qb, sb, fb, alpha=alpha, rows=rows, cols=cols)
    mag = abs(alpha) * (np.abs(omx.dequantize_exact(qa, sa, fa)) @ np.abs(omx.dequantize_exact(qb, sb, fb)).T)
    err = og.rel_frobenius(c32, ref)
    assert err <= FP32_TOL, err
    bad = np.abs(c32.astype(np.float64) - ref) > ELEM_REL * mag
    assert not bad.any(), f"{bad.sum()} outputs outside the accumulation bound"
    return ref


def bf16_to_f64(bits):
    return workloads.bf16_to_f32(bits).astype(np.float64)


def quantized_operands(M, N, K, fa, fb, seed):
    A = workloads.random_tensor((M, K), seed, "normal")
    A = (A * np.exp2((np.arange(K) // 32) % 7 - 3)[None, :]).astype(np.float32)
    B = workloads.random_tensor((N, K), seed + 1, "rows")
    qa, sa = omx.quantize_rowwise(A, fa, "ceil")
    qb, sb = omx.quantize_rowwise(B, fb, "ceil")
    return qa, sa, qb, sb


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e5m2"),
                                   ("e2m1", "e2m1")])
@pytest.mark.parametrize("shape", [(128, 128, 128), (200, 136, 96), (64, 300, 512), (1, 7, 32)])
def test_gemm_small_parity(fa, fb, shape):
    M, N, K = shape
    qa, sa, qb, sb = quantized_operands(M, N, K, fa, fb, seed=M + N + K)
    args = (upload_u8(qa), upload_u8(sa), upload_u8(qb), upload_u8(sb), fa, fb, 0.75)
    c32 = host(mxa.mx_gemm(*args, out_dtype=torch.float32))
    ref = check_fp32(c32, qa, sa, fa, qb, sb, fb, alpha=0.75)
    c16 = host(mxa.mx_gemm(*args, out_dtype=torch.bfloat16))
    assert og.rel_frobenius(bf16_to_f64(c16), bf16_to_f64(og.f64_to_bf16_bits(ref))) <= BF16_TOL


@pytest.mark.parametrize("fa,fb", [("e2m3", "e2m3"), ("e3m2", "e2m3"), ("e2m3", "e3m2"), ("e3m2", "e3m2")])
@pytest.mark.parametrize("shape", [(128, 128, 128), (200, 136, 192), (64, 300, 512), (1, 7, 64), (256, 384, 1024),
                                   (96, 160, 320), (130, 258, 704)])   # whole K-steps of 256, then a partial one
def test_gemm_fp6_parity(fa, fb, shape):
    """MXFP6 operands (bit-stream packed as mx_quantize writes them).  K of 512
    and 1024 run on the 256 x 256 LDS-DMA path; the others on the 128 x 128
    path, whose FP6 K-steps are 256 long: K of 64, 128, 192, 320 and 704 end on
    a partial step, zero-filled past K."""
    M, N, K = shape
    qa, sa, qb, sb = quantized_operands(M, N, K, fa, fb, seed=M + N + K + 1)
    args = (upload_u8(qa), upload_u8(sa), upload_u8(qb), upload_u8(sb), fa, fb, 0.75)
    c32 = host(mxa.mx_gemm(*args, out_dtype=torch.float32))
    ref = check_fp32(c32, qa, sa, fa, qb, sb, fb, alpha=0.75)
    c16 = host(mxa.mx_gemm(*args, out_dtype=torch.bfloat16))
    assert og.rel_frobenius(bf16_to_f64(c16), bf16_to_f64(og.f64_to_bf16_bits(ref))) <= BF16_TOL


def test_gemm_fp6_integer_exact():
    """Operands whose products and sums are exact in FP32 (small integers on the
    E2M3 grid at scale 2^0) give the exact integer product."""
    g = np.random.default_rng(71)
    M, N, K = 64, 96, 256
    A = g.integers(-7, 8, size=(M, K)).astype(np.float32) / 1.0
    B = g.integers(-7, 8, size=(N, K)).astype(np.float32)
    A[:, ::32] = 7.0                                  # every block's amax is 7 -> scale 2^0 under CEIL (max 7.5)
    B[:, ::32] = -7.0
    qa, sa = omx.quantize_rowwise(A, "e2m3", "ceil")
    qb, sb = omx.quantize_rowwise(B, "e2m3", "ceil")
    assert (sa == 127).all() and (sb == 127).all()
    c = host(mxa.mx_gemm(upload_u8(qa), upload_u8(sa), upload_u8(qb), upload_u8(sb), "e2m3", "e2m3", 1.0,
                         out_dtype=torch.float32))
    assert np.array_equal(c, (A.astype(np.float64) @ B.astype(np.float64).T).astype(np.float32))


def test_gemm_fp6_bad_k_raises():
    q = torch.zeros((64, 72), dtype=torch.uint8, device="cuda")       # K = 96: not a multiple of 64
    s = torch.zeros((64, 3), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        mxa.mx_gemm(q, s, q, s, "e2m3", "e2m3")


# Shapes on the 256 x 256-tile LDS-DMA path (K a multiple of 512, N of 8):
# one tile at the minimum K; 6 tiles (no XCD regrouping); 8 tiles (regrouped
# across XCDs, one tile column); a wide tile row at K = 3 * 1024 (odd number of
# 16-K-block scale stages per unrolled pass).
TILED_SHAPES = [(256, 256, 1024), (512, 768, 2048), (2048, 256, 1024), (256, 1024, 3072),
                # ragged last tile row / column (rows past M, N read as zeros, stores masked)
                (300, 264, 1024), (520, 1000, 2048),
                # K of 512 / 1536: the last unrolled body has stages past K (they load zeros)
                (256, 512, 512), (264, 256, 1536)]


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e5m2"),
                                   ("e2m1", "e2m1"), ("e2m3", "e2m3"), ("e3m2", "e2m3"), ("e2m3", "e3m2")])
@pytest.mark.parametrize("shape", TILED_SHAPES)
def test_gemm_tiled_path_parity(fa, fb, shape):
    M, N, K = shape
    qa, sa, qb, sb = quantized_operands(M, N, K, fa, fb, seed=M + 2 * N + 3 * K)
    args = (upload_u8(qa), upload_u8(sa), upload_u8(qb), upload_u8(sb), fa, fb, -1.25)
    c32 = host(mxa.mx_gemm(*args, out_dtype=torch.float32))
    ref = check_fp32(c32, qa, sa, fa, qb, sb, fb, alpha=-1.25)
    c16 = host(mxa.mx_gemm(*args, out_dtype=torch.bfloat16))
    assert og.rel_frobenius(bf16_to_f64(c16), bf16_to_f64(og.f64_to_bf16_bits(ref))) <= BF16_TOL


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1", "e2m3"])
def test_gemm_tiled_path_exact_on_integer_valued_operands(fmt):
    """Integer-valued operands on the tiled path: exact whatever the summation
    order, so any misplaced code, scale byte or lane shows as an exact mismatch."""
    g = np.random.default_rng(19)
    M, N, K = 512, 256, 2048
    vals = np.array([0, 1, 2, 3, 4, -1, -2, -3, -4], np.float32) if fmt == "e2m1" else \
        np.arange(-7, 8).astype(np.float32) if fmt == "e2m3" else np.arange(-16, 17).astype(np.float32)
    A = g.choice(vals, size=(M, K)).astype(np.float32) * np.exp2((np.arange(K) // 32) % 5 - 2)[None, :]
    B = g.choice(vals, size=(N, K)).astype(np.float32)
    qa, sa = omx.quantize_rowwise(A.astype(np.float32), fmt, "ceil")
    qb, sb = omx.quantize_rowwise(B, fmt, "ceil")
    ref = og.gemm_ref(qa, sa, fmt, qb, sb, fmt)
    c = host(mxa.mx_gemm(upload_u8(qa), upload_u8(sa), upload_u8(qb), upload_u8(sb), fmt, fmt, 1.0,
                         out_dtype=torch.float32))
    assert np.array_equal(c.astype(np.float64), ref)


@pytest.mark.parametrize("ldc,dtype", [(576, torch.float32), (520, torch.bfloat16), (516, torch.bfloat16)])
def test_gemm_tiled_shape_with_ldc(ldc, dtype):
    """ldc > N: 16-byte-aligned rows stay on the tiled path, others (516 BF16)
    take the general kernel; columns past N are never written."""
    M, N, K = 256, 512, 1024
    qa, sa, qb, sb = quantized_operands(M, N, K, "e4m3", "e4m3", 23)
    out = torch.full((M, ldc), 7.0, dtype=dtype, device="cuda")
    mxa.mx_gemm(upload_u8(qa), upload_u8(sa), upload_u8(qb), upload_u8(sb), "e4m3", "e4m3", 1.0, out=out[:, :N])
    o = host(out.float())
    ref = og.gemm_ref(qa, sa, "e4m3", qb, sb, "e4m3")
    if dtype == torch.float32:
        check_fp32(o[:, :N], qa, sa, "e4m3", qb, sb, "e4m3")
    else:
        assert og.rel_frobenius(o[:, :N].astype(np.float64), bf16_to_f64(og.f64_to_bf16_bits(ref))) <= BF16_TOL
    assert (o[:, N:] == 7.0).all()


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_gemm_exact_on_integer_valued_operands(fmt):
    """Small integers times powers of two: every partial sum is exact in FP32, so
    the output equals the float64 product bit for bit whatever the order."""
    g = np.random.default_rng(9)
    M, N, K = 96, 160, 256
    vals = np.array([0, 1, 2, 3, 4, -1, -2, -3, -4], np.float32) if fmt == "e2m1" else \
        np.arange(-16, 17).astype(np.float32)
    A = g.choice(vals, size=(M, K)).astype(np.float32)
    B = g.choice(vals, size=(N, K)).astype(np.float32)
    qa, sa = omx.quantize_rowwise(A, fmt, "ceil")
    qb, sb = omx.quantize_rowwise(B, fmt, "ceil")
    ref = og.gemm_ref(qa, sa, fmt, qb, sb, fmt)
    c = host(mxa.mx_gemm(upload_u8(qa), upload_u8(sa), upload_u8(qb), upload_u8(sb), fmt, fmt, 1.0,
                         out_dtype=torch.float32))
    assert np.array_equal(c.astype(np.float64), ref)


def test_gemm_ldc_and_k_zero():
    qa, sa, qb, sb = quantized_operands(64, 40, 64, "e4m3", "e4m3", 3)
    out = torch.full((64, 56), 7.0, dtype=torch.float32, device="cuda")
    mxa.mx_gemm(upload_u8(qa), upload_u8(sa), upload_u8(qb), upload_u8(sb), "e4m3", "e4m3", 1.0, out=out[:, :40])
    o = host(out)
    check_fp32(o[:, :40], qa, sa, "e4m3", qb, sb, "e4m3")
    assert (o[:, 40:] == 7.0).all()                       # columns past N untouched
    z = torch.empty((0,), dtype=torch.uint8, device="cuda")
    c = torch.full((8, 8), 3.0, dtype=torch.float32, device="cuda")
    st = mxa.lib.mx_gemm(z.data_ptr(), z.data_ptr(), 0, z.data_ptr(), z.data_ptr(), 0, 0, 8, 8, 0, 1.0,
                         c.data_ptr(), 0, 8, torch.cuda.current_stream().cuda_stream)
    assert st == 0 and (host(c) == 0).all()               # empty sum


def test_mlp_mxfp8_gemm_full_size():
    """A 8192 x 4096 activations, W 14336 x 4096 weights, both MXFP8 E4M3 with the
    round-up rule along K, BF16 out, in the bench's launch configuration.  Both
    quantized operands are compared in full; the product on one row from every
    256-row output tile (whole rows) and one column from every 256-column tile
    (whole columns), so every 256 x 256 tile of the launch is checked, segment
    by segment."""
    a_bits, w_bits = workloads.mlp_operands()
    qa, sa = mxa.mx_quantize(upload_bf16_bits(a_bits), "e4m3", "ceil", "row")
    qw, sw = mxa.mx_quantize(upload_bf16_bits(w_bits), "e4m3", "ceil", "row")
    c = host(mxa.mx_gemm(qa, sa, qw, sw, "e4m3", "e4m3", 1.0, out_dtype=torch.bfloat16))
    oqa, osa = omx.quantize_rowwise(workloads.bf16_to_f32(a_bits), "e4m3", "ceil")
    oqw, osw = omx.quantize_rowwise(workloads.bf16_to_f32(w_bits), "e4m3", "ceil")
    assert_bytes_equal(host(sa), osa, "A scales")
    assert_bytes_equal(host(qa), oqa, "A codes")
    assert_bytes_equal(host(sw), osw, "W scales")
    assert_bytes_equal(host(qw), oqw, "W codes")
    rows = tile_strata(8192, 256, 44)
    cols = tile_strata(14336, 256, 45)
    op = (oqa, osa, "e4m3", oqw, osw, "e4m3")
    ref_r = og.gemm_ref(*op, rows=rows)
    check_bf16_lines(c[rows], ref_r, abs_product(*op, rows=rows), BF16_TOL, "rows")
    ref_c = og.gemm_ref(*op, cols=cols)
    check_bf16_lines(np.ascontiguousarray(c[:, cols].T), ref_c.T, abs_product(*op, cols=cols).T, BF16_TOL,
                     "columns")
    assert og.rel_frobenius(bf16_to_f64(c[rows]), ref_r) <= 4e-3        # BF16 output rounding only


@functools.lru_cache(maxsize=1)
def wgrad_oracle():
    """The oracle's Hadamard + column-wise MXFP4 quantization of both weight-gradient
    operands, whole (computed once per test session)."""
    g_bits, x_bits, mask = workloads.weight_grad_operands()
    ogq, ogs = omx.quantize_colwise_t(workloads.bf16_to_f32(g_bits), "e2m1", "ceil", hadamard_mask=mask)
    oxq, oxs = omx.quantize_colwise_t(workloads.bf16_to_f32(x_bits), "e2m1", "ceil", hadamard_mask=mask)
    return ogq, ogs, oxq, oxs


def wgrad_gpu():
    g_bits, x_bits, mask = workloads.weight_grad_operands()
    gq, gs = mxa.mx_quantize(upload_bf16_bits(g_bits), "e2m1", "ceil", "col", hadamard_mask=mask)
    xq, xs = mxa.mx_quantize(upload_bf16_bits(x_bits), "e2m1", "ceil", "col", hadamard_mask=mask)
    return gq, gs, xq, xs


def test_hadamard_mxfp4_quant_full_size():
    """G, X BF16 8192 tokens x 4096: fixed-sign Hadamard + column-wise MXFP4
    quantization along tokens, in the bench's launch configuration; every code
    and scale of both operands against the oracle."""
    got = wgrad_gpu()
    want = wgrad_oracle()
    for g, w, what in zip(got, want, ("G codes", "G scales", "X codes", "X scales")):
        assert_bytes_equal(host(g), w, what)


def test_hadamard_mxfp4_wgrad_gemm_full_size():
    """dW = (1/32) Gq^T Xq (4096 x 4096, K = 8192 tokens) with BF16 out: one row
    from every 256-row tile and one column from every 256-column tile, whole."""
    gq, gs, xq, xs = wgrad_gpu()
    dw = host(mxa.mx_gemm(gq, gs, xq, xs, "e2m1", "e2m1", 1.0 / 32, out_dtype=torch.bfloat16))
    ogq, ogs, oxq, oxs = wgrad_oracle()
    rows = tile_strata(4096, 256, 55)
    cols = tile_strata(4096, 256, 56)
    op = (ogq, ogs, "e2m1", oxq, oxs, "e2m1", 1.0 / 32)
    ref_r = og.gemm_ref(*op, rows=rows)
    check_bf16_lines(dw[rows], ref_r, abs_product(*op, rows=rows), BF16_TOL, "rows")
    ref_c = og.gemm_ref(*op, cols=cols)
    check_bf16_lines(np.ascontiguousarray(dw[:, cols].T), ref_c.T, abs_product(*op, cols=cols).T, BF16_TOL,
                     "columns")


