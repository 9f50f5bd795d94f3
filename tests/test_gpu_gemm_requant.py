"""GPU parity of the GEMM with MX re-quantization in the epilogue.

The kernel's FP32 result is the one ``mx_gemm`` writes with FP32 output (the same
MFMA sequence and the same alpha multiply), so its re-quantization is checked
bit for bit against the oracle's row-wise MX quantizer applied to that FP32
output -- the code decisions are taken in the same precision on both sides.  The
FP32 result itself is checked against the oracle's float64 product."""

import numpy as np
import pytest
import torch

import workloads
from oracle import gemm as og
from oracle import mx as omx
from tests.gpu_util import assert_bytes_equal, host, import_library, tile_strata, upload_u8

pytestmark = pytest.mark.gpu

mxa = import_library()


def operands(M, N, K, fa, fb, seed):
    A = workloads.random_tensor((M, K), seed, "normal")
    B = workloads.random_tensor((N, K), seed + 1, "rows")
    qa, sa = omx.quantize_rowwise(A, fa, "ceil")
    qb, sb = omx.quantize_rowwise(B, fb, "ceil")
    return qa, sa, qb, sb


def check(shape, fa, fb, fc, rc, alpha, seed):
    M, N, K = shape
    qa, sa, qb, sb = operands(M, N, K, fa, fb, seed)
    args = (upload_u8(qa), upload_u8(sa), upload_u8(qb), upload_u8(sb), fa, fb, alpha)
    c32 = host(mxa.mx_gemm(*args, out_dtype=torch.float32))
    q, s, a = mxa.mx_gemm_requant(*args, fmt_c=fc, rule_c=rc, amax=True)
    wq, ws = omx.quantize_rowwise(c32, fc, rc)
    assert_bytes_equal(host(s), ws, f"{shape} {fa}x{fb}->{fc} {rc} scales")
    assert_bytes_equal(host(q), wq, f"{shape} {fa}x{fb}->{fc} {rc} codes")
    assert host(a)[0] == omx.tensor_amax(c32)
    return qa, sa, qb, sb, c32


SHAPES = [(256, 256, 1024), (512, 768, 2048), (300, 288, 1024), (256, 256, 512), (200, 160, 96), (64, 96, 64),
          (1, 32, 32)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e2m1", "e2m1")])
@pytest.mark.parametrize("fc", ["e4m3", "e5m2", "e2m1"])
def test_requant_parity(shape, fa, fb, fc):
    for rc in ("floor", "ceil"):
        qa, sa, qb, sb, c32 = check(shape, fa, fb, fc, rc, 0.75, sum(shape))
    if shape[0] * shape[1] >= 4096:
        ref = og.gemm_ref(qa, sa, fa, qb, sb, fb, alpha=0.75)
        assert og.rel_frobenius(c32, ref) <= 1e-3


def test_requant_nonfinite_and_zero_blocks():
    """alpha large enough to overflow FP32 in some blocks (Inf -> scale 0xFF, NaN codes),
    and zero rows (scale code 0)."""
    M, N, K = 256, 256, 1024
    qa, sa, qb, sb = operands(M, N, K, "e4m3", "e4m3", 77)
    qa[5, :] = 0
    qb[17, :] = 0
    args = (upload_u8(qa), upload_u8(sa), upload_u8(qb), upload_u8(sb), "e4m3", "e4m3")
    for alpha in (3.0e37, 1.0):
        c32 = host(mxa.mx_gemm(*args, alpha, out_dtype=torch.float32))
        for fc in ("e4m3", "e2m1"):
            q, s = mxa.mx_gemm_requant(*args, alpha, fmt_c=fc, rule_c="ceil")
            wq, ws = omx.quantize_rowwise(c32, fc, "ceil")
            assert_bytes_equal(host(s), ws, f"alpha {alpha} {fc} scales")
            assert_bytes_equal(host(q), wq, f"alpha {alpha} {fc} codes")
        if alpha > 1:
            assert np.isinf(c32).any()


def test_requant_full_size():
    """The MLP up-projection (8192 x 4096 x (14336 x 4096)^T) re-quantized to MXFP8 E4M3:
    one whole row from every 256-row output tile (every tile of the launch)
    against the oracle quantizer of the FP32 result, which itself is held to the
    GEMM tolerance against the float64 product on those rows."""
    M, N, K = 8192, 14336, 4096
    a_bits, w_bits = workloads.mlp_operands()
    xa = torch.from_numpy(a_bits.view(np.int16)).view(torch.bfloat16).cuda()
    xw = torch.from_numpy(w_bits.view(np.int16)).view(torch.bfloat16).cuda()
    qa, sa = mxa.mx_quantize(xa, "e4m3", "ceil", "row")
    qw, sw = mxa.mx_quantize(xw, "e4m3", "ceil", "row")
    c32 = mxa.mx_gemm(qa, sa, qw, sw, "e4m3", "e4m3", 1.0, out_dtype=torch.float32)
    q, s, am = mxa.mx_gemm_requant(qa, sa, qw, sw, "e4m3", "e4m3", 1.0, fmt_c="e4m3", rule_c="ceil", amax=True)
    rows = tile_strata(M, 256, 5)
    c32h = host(c32)
    c = c32h[rows]
    wq, ws = omx.quantize_rowwise(c, "e4m3", "ceil")
    assert_bytes_equal(host(s)[rows], ws, "scales")
    assert_bytes_equal(host(q)[rows], wq, "codes")
    assert host(am)[0] == omx.tensor_amax(c32h)
    ref = og.gemm_ref(host(qa)[rows], host(sa)[rows], "e4m3", host(qw), host(sw), "e4m3")
    assert og.rel_frobenius(c, ref) <= 1e-3
