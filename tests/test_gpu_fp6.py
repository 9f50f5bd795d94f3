"""GPU parity of MXFP6 (E2M3, E3M2): row-wise quantization and dequantization
against the oracle, bit-exact codes (packed bit stream), scales, amax and
dequantized values."""

import numpy as np
import pytest
import torch

import workloads
from oracle import formats as F
from oracle import mx as omx
from tests.gpu_util import (assert_bytes_equal, assert_float_equal, f32_of_input, host, upload_bf16_bits,
                            upload_f16_from_f32, upload_f32, upload_u8)

pytestmark = pytest.mark.gpu

mxa = pytest.importorskip("mx_block_scaled_quantize_amd")

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


def test_fp6_full_size_sampled_rows():
    """BF16 8192 x 4096 activation to MXFP6 E3M2: sampled rows against the oracle."""
    bits = workloads.cfg2(8192, 4096)
    q, s = mxa.mx_quantize(upload_bf16_bits(bits), "e3m2", "ceil", "row")
    qh, sh = host(q), host(s)
    rows = np.concatenate([[0, 8191], np.random.default_rng(66).choice(8192, 30, replace=False)])
    wq, ws = omx.quantize_rowwise(workloads.bf16_to_f32(bits[rows]), "e3m2", "ceil")
    assert_bytes_equal(sh[rows], ws, "scales")
    assert_bytes_equal(qh[rows], wq, "codes")


def test_fp6_unsupported_paths_raise():
    x = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    for call in (lambda: mxa.mx_quantize(x, "e2m3", "ceil", "col"),
                 lambda: mxa.mx_quantize(x, "e2m3", "ceil", "row", hadamard_mask=1),
                 lambda: mxa.mx_quantize_dual(x, "e3m2"),
                 lambda: mxa.mx_dequantize(torch.zeros((64, 48), dtype=torch.uint8, device="cuda"),
                                           torch.zeros((64, 2), dtype=torch.uint8, device="cuda"), 64, 64, "e2m3",
                                           "col")):
        with pytest.raises(ValueError):
            call()
    q, s = mxa.mx_quantize(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"), "e2m3", "ceil", "row")
    assert q.shape == (0, 48)
