"""GPU parity of the GEMM scale layout ([K/512][lines][16], written by the
quantizers and read by the GEMMs and the dequantizer): the quantizers' scales
equal the oracle's row-major scales moved by the oracle's permutation, the
codes are unchanged, and a GEMM on GEMM-layout scales is bit-identical to the
same GEMM on row-major scales (the same products in the same order)."""

import numpy as np
import pytest
import torch

import workloads
from oracle import mx as omx
from tests.gpu_util import (assert_bytes_equal, f32_of_input, host, import_library, upload_bf16_bits, upload_f32,
                            upload_f16_from_f32)

pytestmark = pytest.mark.gpu

mxa = import_library()


def make_input(x32, dtype):
    if dtype == "f32":
        return upload_f32(x32)
    if dtype == "bf16":
        return upload_bf16_bits(workloads.to_bf16_bits(x32.astype(np.float64)))
    return upload_f16_from_f32(x32)


@pytest.mark.parametrize("dtype", ["bf16", "f32", "f16"])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2", "e2m1"])
@pytest.mark.parametrize("orient", ["row", "col"])
@pytest.mark.parametrize("had", [False, True])
def test_quantize_gemm_scales(dtype, fmt, orient, had):
    # 1024 x 1536 (row-wise: 48 K-blocks = 3 stages per row; column-wise: 32 K-blocks), ragged
    # against the 128 / 256-wide tiles; a second shape with a single stage
    mask = 0x13572468 if had else None
    for shape, seed in (((1024, 1536), 81), ((512, 544), 82)):
        if orient == "col" and shape[0] % 512:
            continue
        if orient == "row" and shape[1] % 512:
            continue
        x = make_input(workloads.random_tensor(shape, seed, "rows"), dtype)
        xs = f32_of_input(x)
        q, s = mxa.mx_quantize(x, fmt, "ceil", orient, hadamard_mask=mask, scale_layout="gemm")
        ref = omx.quantize_rowwise if orient == "row" else omx.quantize_colwise_t
        wq, ws = ref(xs, fmt, "ceil", hadamard_mask=mask)
        assert tuple(s.shape) == (ws.shape[1] // 16, ws.shape[0], 16)
        assert_bytes_equal(host(s), omx.scales_to_gemm_layout(ws), f"{shape} scales")
        assert_bytes_equal(host(q), wq, f"{shape} codes")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_dual_gemm_scales(dtype, fmt):
    x = make_input(workloads.random_tensor((1024, 1536), 83, "wide"), dtype)
    xs = f32_of_input(x)
    qr, sr, qc, sc = mxa.mx_quantize_dual(x, fmt, "ceil", scale_layout="gemm")
    wqr, wsr, wqc, wsc = omx.quantize_dual(xs, fmt, "ceil")
    assert_bytes_equal(host(sr), omx.scales_to_gemm_layout(wsr), "row scales")
    assert_bytes_equal(host(sc), omx.scales_to_gemm_layout(wsc), "col scales")
    assert_bytes_equal(host(qr), wqr, "row codes")
    assert_bytes_equal(host(qc), wqc, "col codes")


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
@pytest.mark.parametrize("orient", ["row", "col"])
def test_dequantize_gemm_scales(fmt, orient):
    x = upload_f32(workloads.random_tensor((512, 1024), 84, "rows"))
    q, s = mxa.mx_quantize(x, fmt, "ceil", orient)
    qg, sg = mxa.mx_quantize(x, fmt, "ceil", orient, scale_layout="gemm")
    d = mxa.mx_dequantize(q, s, 512, 1024, fmt, orient)
    dg = mxa.mx_dequantize(qg, sg, 512, 1024, fmt, orient, scale_layout="gemm")
    assert torch.equal(d.view(torch.int32), dg.view(torch.int32))


@pytest.mark.parametrize("fmt,shape", [("e4m3", (512, 768, 1024)),     # the 256 x 256 path, ragged N
                                       ("e4m3", (300, 224, 512)),      # partial tiles
                                       ("e5m2", (256, 256, 1536)),
                                       ("e2m1", (512, 512, 2048)),
                                       ("e2m1", (96, 160, 512)),
                                       ("e2m3", (256, 256, 1024))])     # FP6: the 128 x 128 path
def test_gemm_gemm_scales_bit_identical(fmt, shape):
    M, N, K = shape
    A = workloads.random_tensor((M, K), 85, "rows")
    B = workloads.random_tensor((N, K), 86, "wide")
    qa, sa = omx.quantize_rowwise(A, fmt, "ceil")
    qb, sb = omx.quantize_rowwise(B, fmt, "ceil")
    u8 = lambda t: torch.from_numpy(np.ascontiguousarray(t)).cuda()   # noqa: E731
    for out_dtype in (torch.float32, torch.bfloat16):
        c = mxa.mx_gemm(u8(qa), u8(sa), u8(qb), u8(sb), fmt, fmt, 0.5, out_dtype=out_dtype)
        cg = mxa.mx_gemm(u8(qa), u8(omx.scales_to_gemm_layout(sa)), u8(qb), u8(omx.scales_to_gemm_layout(sb)), fmt,
                         fmt, 0.5, out_dtype=out_dtype, scale_layout="gemm")
        assert torch.equal(c.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32),
                           cg.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32)), f"{shape} {out_dtype}"
    if fmt != "e2m3":
        r = mxa.mx_gemm_requant(u8(qa), u8(sa), u8(qb), u8(sb), fmt, fmt, 0.5, "e4m3", "ceil")
        rg = mxa.mx_gemm_requant(u8(qa), u8(omx.scales_to_gemm_layout(sa)), u8(qb), u8(omx.scales_to_gemm_layout(sb)),
                                 fmt, fmt, 0.5, "e4m3", "ceil", scale_layout="gemm")
        assert torch.equal(r[0], rg[0]) and torch.equal(r[1], rg[1])


def test_gemm_scales_full_size_workloads():
    """Both bench GEMMs at full size with the operands quantized straight into the
    GEMM layout: the scales are the row-major ones permuted, and the products are
    bit-identical to the row-major runs (whose parity the full-size GEMM tests check)."""
    a_bits, w_bits = workloads.mlp_operands()
    xa, xw = upload_bf16_bits(a_bits), upload_bf16_bits(w_bits)
    qa, sa = mxa.mx_quantize(xa, "e4m3", "ceil", "row")
    qw, sw = mxa.mx_quantize(xw, "e4m3", "ceil", "row")
    qag, sag = mxa.mx_quantize(xa, "e4m3", "ceil", "row", scale_layout="gemm")
    qwg, swg = mxa.mx_quantize(xw, "e4m3", "ceil", "row", scale_layout="gemm")
    assert torch.equal(qa, qag) and torch.equal(qw, qwg)
    assert_bytes_equal(host(sag), omx.scales_to_gemm_layout(host(sa)), "A scales")
    assert_bytes_equal(host(swg), omx.scales_to_gemm_layout(host(sw)), "W scales")
    c = mxa.mx_gemm(qa, sa, qw, sw, "e4m3", "e4m3", 1.0)
    cg = mxa.mx_gemm(qag, sag, qwg, swg, "e4m3", "e4m3", 1.0, scale_layout="gemm")
    assert torch.equal(c.view(torch.int16), cg.view(torch.int16))
    del xa, xw, qa, qw, qag, qwg, c, cg
    g_bits, x_bits, mask = workloads.weight_grad_operands()
    G, X = upload_bf16_bits(g_bits), upload_bf16_bits(x_bits)
    ops, opsg = [], []
    for t in (G, X):
        ops.append(mxa.mx_quantize(t, "e2m1", "ceil", "col", hadamard_mask=mask))
        opsg.append(mxa.mx_quantize(t, "e2m1", "ceil", "col", hadamard_mask=mask, scale_layout="gemm"))
    for (q, s), (qg, sg) in zip(ops, opsg):
        assert torch.equal(q, qg)
        assert_bytes_equal(host(sg), omx.scales_to_gemm_layout(host(s)), "wgrad scales")
    d = mxa.mx_gemm(ops[0][0], ops[0][1], ops[1][0], ops[1][1], "e2m1", "e2m1", 1.0 / 32)
    dg = mxa.mx_gemm(opsg[0][0], opsg[0][1], opsg[1][0], opsg[1][1], "e2m1", "e2m1", 1.0 / 32, scale_layout="gemm")
    assert torch.equal(d.view(torch.int16), dg.view(torch.int16))


def test_gemm_scale_layout_shape_errors():
    x = torch.zeros((512, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        mxa.mx_quantize(x, "e4m3", "ceil", "row", scale_layout="gemm")        # cols 256 is not a multiple of 512
    q = torch.zeros((64, 256), dtype=torch.uint8, device="cuda")
    s = torch.zeros((64, 8), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        mxa.mx_gemm(q, s, q, s, "e4m3", "e4m3", scale_layout="gemm")          # K 256
