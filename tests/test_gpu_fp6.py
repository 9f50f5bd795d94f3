"""GPU parity of MXFP6 (E2M3, E3M2): row-wise quantization and dequantization
against the oracle, bit-exact codes (packed bit stream), scales, amax and
dequantized values."""

import numpy as np
import pytest
import torch

import workloads
from oracle import formats as F
from oracle import gemm as og
from oracle import mx as omx
from tests.gpu_util import (assert_bytes_equal, assert_float_equal, check_bf16_lines, f32_of_input, host,
                            import_library, tile_strata, upload_bf16_bits, upload_f16_from_f32, upload_f32, upload_u8,
                            abs_product)

pytestmark = pytest.mark.gpu

mxa = import_library()

FP6 = ["e2m3", "e3m2"]
RULES = ["floor", "ceil"]


def make_input(x32, dtype):
    if dtype == "f32":
        return upload_f32(x32)
    if dtype == "bf16":
        return upload_bf16_bits(workloads.to_bf16_bits(x32.astype(np.float64)))
    return upload_f16_from_f32(x32)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("fmt", FP6)
@pytest.mark.parametrize("rule", RULES)
def test_fp6_rowwise_parity(dtype, fmt, rule):
    for shape, seed, kind in (((96, 256), 61, "rows"), ((64, 320), 62, "wide"), ((200, 96), 63, "normal")):
        x = make_input(workloads.random_tensor(shape, seed, kind), dtype)
        xs = f32_of_input(x)
        q, s, a = mxa.mx_quantize(x, fmt, rule, "row", amax=True)
        wq, ws = omx.quantize_rowwise(xs, fmt, rule)
        assert_bytes_equal(host(s), ws, f"{shape} scales")
        assert_bytes_equal(host(q), wq, f"{shape} codes")
        assert host(a)[0] == omx.tensor_amax(xs)


@pytest.mark.parametrize("fmt", FP6)
@pytest.mark.parametrize("rule", RULES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fp6_every_bf16_pattern_and_specials(fmt, rule, dtype):
    """Every finite BF16 value in blocks sweeping the exponent range, plus special
    blocks; BF16 input runs the hardware-convert kernel, FP32 the integer encoder."""
    blocks = np.concatenate([workloads.all_bf16_blocks(), workloads.special_blocks()])
    x = make_input(blocks.reshape(-1, 32), dtype)
    x32 = f32_of_input(x)
    q, s = mxa.mx_quantize(x, fmt, rule, "row")
    wq, ws = omx.quantize_rowwise(x32, fmt, rule)
    assert_bytes_equal(host(s), ws, "scales")
    assert_bytes_equal(host(q), wq, "codes")


@pytest.mark.parametrize("fmt", FP6)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_fp6_dequantize_parity(fmt, out_dtype):
    g = np.random.default_rng(64)
    rows, cols = 96, 160
    codes = g.integers(0, 64, size=(rows, cols)).astype(np.uint8)
    scales = g.integers(0, 256, size=(rows, cols // 32)).astype(np.uint8)
    scales[0, 0], scales[1, 0], scales[2, 0] = 0, 254, 255
    packed = omx.pack_fp6(codes)
    out = host(mxa.mx_dequantize(upload_u8(packed), upload_u8(scales), rows, cols, fmt, "row", out_dtype))
    kind = "f32" if out_dtype == torch.float32 else "bf16"
    want = omx.dequantize(packed, scales, fmt, out=kind)
    if kind == "f32":
        assert_float_equal(out, want, "f32")
    else:
        gotb, wantb = out.view(np.uint16), want.astype(np.uint16)
        nan = np.isnan(workloads.bf16_to_f32(wantb))
        assert_bytes_equal(np.where(nan, 0, gotb), np.where(nan, 0, wantb), "bf16")
        assert np.all(np.isnan(workloads.bf16_to_f32(gotb))[nan])


@pytest.mark.parametrize("fmt", FP6)
def test_fp6_roundtrip_error_bound(fmt):
    x32 = workloads.random_tensor((128, 256), 65, "rows")
    x = upload_f32(x32)
    q, s = mxa.mx_quantize(x, fmt, "ceil", "row")
    d = host(mxa.mx_dequantize(q, s, 128, 256, fmt, "row", torch.float32))
    assert_float_equal(d, omx.dequantize(host(q), host(s), fmt), "roundtrip")
    f = F.FORMATS[fmt]
    X = np.repeat(F.e8m0_decode(host(s)), 32, axis=1)
    v = np.abs(x32.astype(np.float64)) / X
    quantum = np.exp2(np.maximum(np.floor(np.log2(np.where(v > 0, v, 1.0))), f.emin) - f.mbits) * X
    assert np.all(np.abs(d - x32) <= quantum / 2)


def test_fp6_full_size():
    """BF16 8192 x 4096 activation to MXFP6 E3M2, row-wise: every code and scale
    against the oracle."""
    bits = workloads.activation_bf16(8192, 4096)
    q, s = mxa.mx_quantize(upload_bf16_bits(bits), "e3m2", "ceil", "row")
    wq, ws = omx.quantize_rowwise(workloads.bf16_to_f32(bits), "e3m2", "ceil")
    assert_bytes_equal(host(s), ws, "scales")
    assert_bytes_equal(host(q), wq, "codes")


def test_fp6_gemm_full_size():
    """The bench's MXFP6 GEMM: A 8192 x 4096 and W 14336 x 4096 quantized row-wise to
    E2M3 (round-up rule), BF16 out, on the 256 x 256 path.  Operands compared in
    full; the product on one whole row from every 128-row band and one whole
    column from every 128-column band (so every 256 x 256 output tile of the
    launch twice), segment by segment."""
    a_bits, w_bits = workloads.mlp_operands()
    qa, sa = mxa.mx_quantize(upload_bf16_bits(a_bits), "e2m3", "ceil", "row")
    qw, sw = mxa.mx_quantize(upload_bf16_bits(w_bits), "e2m3", "ceil", "row")
    c = host(mxa.mx_gemm(qa, sa, qw, sw, "e2m3", "e2m3", 1.0, out_dtype=torch.bfloat16))
    oqa, osa = omx.quantize_rowwise(workloads.bf16_to_f32(a_bits), "e2m3", "ceil")
    oqw, osw = omx.quantize_rowwise(workloads.bf16_to_f32(w_bits), "e2m3", "ceil")
    assert_bytes_equal(host(qa), oqa, "A codes")
    assert_bytes_equal(host(qw), oqw, "W codes")
    assert_bytes_equal(host(sa), osa, "A scales")
    assert_bytes_equal(host(sw), osw, "W scales")
    rows = tile_strata(8192, 128, 61)
    cols = tile_strata(14336, 128, 62)
    op = (oqa, osa, "e2m3", oqw, osw, "e2m3")
    ref_r = og.gemm_ref(*op, rows=rows)
    check_bf16_lines(c[rows], ref_r, abs_product(*op, rows=rows), 1e-3, "rows", seg=128)
    ref_c = og.gemm_ref(*op, cols=cols)
    check_bf16_lines(np.ascontiguousarray(c[:, cols].T), ref_c.T, abs_product(*op, cols=cols).T, 1e-3, "columns",
                     seg=128)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("fmt", FP6)
@pytest.mark.parametrize("rule", RULES)
def test_fp6_colwise_and_dual_parity(dtype, fmt, rule):
    # ragged tiles: 160 rows (one full and one partial 128-row tile), 200 / 224 / 96 columns;
    # a single 32 x 32 block
    for shape, seed, kind in (((160, 200), 67, "wide"), ((96, 96), 68, "rows"), ((288, 416), 69, "normal"),
                              ((160, 224), 70, "wide"), ((32, 32), 71, "normal")):
        x = make_input(workloads.random_tensor(shape, seed, kind), dtype)
        xs = f32_of_input(x)
        q, s, a = mxa.mx_quantize(x, fmt, rule, "col", amax=True)
        wq, ws = omx.quantize_colwise_t(xs, fmt, rule)
        assert_bytes_equal(host(s), ws, f"{shape} col scales")
        assert_bytes_equal(host(q), wq, f"{shape} col codes")
        assert host(a)[0] == omx.tensor_amax(xs)
        if shape[1] % 32 == 0:
            qr, sr, qc, sc, a = mxa.mx_quantize_dual(x, fmt, rule, amax=True)
            wqr, wsr, wqc, wsc = omx.quantize_dual(xs, fmt, rule)
            assert_bytes_equal(host(sr), wsr, f"{shape} dual row scales")
            assert_bytes_equal(host(qr), wqr, f"{shape} dual row codes")
            assert_bytes_equal(host(sc), wsc, f"{shape} dual col scales")
            assert_bytes_equal(host(qc), wqc, f"{shape} dual col codes")
            assert host(a)[0] == omx.tensor_amax(xs)


@pytest.mark.parametrize("fmt", FP6)
def test_fp6_dual_special_blocks(fmt):
    blocks = workloads.special_blocks()
    x32 = np.zeros((64, 64), np.float32)
    x32[:18, :32] = blocks
    x32[32:64, 32:50] = blocks.T
    x32[40, :] = np.nan
    x32[:, 60] = -np.inf
    for dtype in ("f32", "bf16"):
        x = make_input(x32, dtype)
        xs = f32_of_input(x)
        for rule in ("floor", "ceil"):
            qr, sr, qc, sc = mxa.mx_quantize_dual(x, fmt, rule)
            wqr, wsr, wqc, wsc = omx.quantize_dual(xs, fmt, rule)
            for got, want, what in ((sr, wsr, "row scales"), (qr, wqr, "row codes"), (sc, wsc, "col scales"),
                                    (qc, wqc, "col codes")):
                assert_bytes_equal(host(got), want, f"{dtype} {rule} {what}")


@pytest.mark.parametrize("fmt", FP6)
def test_fp6_colwise_dequantize(fmt):
    g = np.random.default_rng(70)
    rows, cols = 96, 136
    codes = g.integers(0, 64, size=(cols, rows)).astype(np.uint8)      # stored transposed
    scales = g.integers(0, 256, size=(cols, rows // 32)).astype(np.uint8)
    packed = omx.pack_fp6(codes)
    out = host(mxa.mx_dequantize(upload_u8(packed), upload_u8(scales), rows, cols, fmt, "col", torch.float32))
    assert_float_equal(out, omx.dequantize(packed, scales, fmt).T, "col dequant")


def test_fp6_unsupported_paths_raise():
    x = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        mxa.mx_quantize(x, "e2m3", "ceil", "row", hadamard_mask=1)
    with pytest.raises(ValueError):
        mxa.mx_quantize_dual(torch.zeros((64, 48), dtype=torch.bfloat16, device="cuda"), "e3m2")
    q, s = mxa.mx_quantize(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"), "e2m3", "ceil", "row")
    assert q.shape == (0, 48)
