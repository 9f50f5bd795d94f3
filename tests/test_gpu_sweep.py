"""Seeded random sweeps over shapes, formats, rules, input types and scale layouts,
each case compared with the oracle exactly as the targeted tests do: quantized
bytes and scales bit for bit, dequantized values bit for bit, GEMM results within
the FP32 bounds of test_gpu_gemm (1e-3 relative Frobenius and the per-element
accumulation bound).  The cases are drawn from one fixed seed, so a failure names a
reproducible case; every failing case is listed, not just the first."""

import numpy as np
import pytest
import torch

import workloads
from oracle import mx as omx
from tests.gpu_util import (assert_float_equal, f32_of_input, host, import_library, upload_bf16_bits,
                            upload_f16_from_f32, upload_f32, upload_u8)
from tests.test_gpu_gemm import check_fp32

pytestmark = pytest.mark.gpu

mxa = import_library()

FORMATS = ["e4m3", "e5m2", "e2m1", "e2m3", "e3m2"]
GEMM_PAIRS = [("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e5m2"), ("e2m1", "e2m1"),
              ("e2m3", "e2m3"), ("e3m2", "e2m3"), ("e2m3", "e3m2"), ("e3m2", "e3m2")]


def _input(rng, R, C, dtype, seed):
    """A device input and the exact FP32 values the oracle sees."""
    x32 = workloads.random_tensor((R, C), seed, ["normal", "wide", "rows"][seed % 3])
    if dtype == "f32":
        x = upload_f32(x32)
    elif dtype == "bf16":
        x = upload_bf16_bits(workloads.to_bf16_bits(x32.astype(np.float64)))
    else:
        x = upload_f16_from_f32(x32)
    return x, f32_of_input(x)


def _report(failures, n):
    assert not failures, f"{len(failures)} of {n} cases failed:\n" + "\n".join(failures[:40])


def test_quantize_random_cases():
    """Row-wise, column-wise and dual quantization: 300 random cases (rows and columns
    multiples of 32 up to 1248, every format, both rules, FP32/BF16/FP16 input, and
    the GEMM scale layout for the FP8 and FP4 formats in about a third of them)."""
    rng = np.random.default_rng(20261203)
    failures = []
    n = 300
    for i in range(n):
        fmt = FORMATS[rng.integers(len(FORMATS))]
        rule = ["floor", "ceil"][rng.integers(2)]
        kind = ["row", "col", "dual"][rng.integers(3)]
        dtype = ["f32", "bf16", "f16"][rng.integers(3)]
        R, C = 32 * int(rng.integers(1, 40)), 32 * int(rng.integers(1, 40))
        layout = "row"
        if fmt not in ("e2m3", "e3m2") and rng.random() < 0.3:   # no GEMM scale layout for FP6
            R, C = R - R % 512 or 512, C - C % 512 or 512
            layout = "gemm"
        seed = int(rng.integers(1 << 30))
        case = f"{kind} {fmt} {rule} {dtype} {R}x{C} layout={layout} seed={seed}"
        try:
            x, xs = _input(rng, R, C, dtype, seed)
            gl = omx.scales_to_gemm_layout if layout == "gemm" else (lambda s: s)
            if kind == "row":
                q, s = mxa.mx_quantize(x, fmt, rule, "row", scale_layout=layout)
                want = omx.quantize_rowwise(xs, fmt, rule)
                got = (host(q), host(s))
                want = (want[0], gl(want[1]))
            elif kind == "col":
                q, s = mxa.mx_quantize(x, fmt, rule, "col", scale_layout=layout)
                want = omx.quantize_colwise_t(xs, fmt, rule)
                got = (host(q), host(s))
                want = (want[0], gl(want[1]))
            else:
                outs = mxa.mx_quantize_dual(x, fmt, rule, scale_layout=layout)
                w = omx.quantize_dual(xs, fmt, rule)
                got = tuple(host(t) for t in outs)
                want = (w[0], gl(w[1]), w[2], gl(w[3]))
            if not all(a.shape == b.shape and np.array_equal(a, b) for a, b in zip(got, want)):
                failures.append(case)
        except Exception as e:   # noqa: BLE001 -- every case is reported
            failures.append(f"{case}: {type(e).__name__}: {str(e)[:160]}")
    _report(failures, n)


def test_dequantize_random_cases():
    """Dequantization to FP32 and BF16, both orientations, both scale layouts: 150
    random cases, half on oracle-quantized data and half on arbitrary codes and
    scale bytes (NaN codes and scale 255 included); FP32 compared bit for bit (any
    NaN matches any NaN), BF16 bit for bit outside NaN, NaN positions equal."""
    rng = np.random.default_rng(20261204)
    failures = []
    n = 150
    for i in range(n):
        fmt = FORMATS[rng.integers(len(FORMATS))]
        orient = ["row", "col"][rng.integers(2)]
        out = ["f32", "bf16"][rng.integers(2)]
        R, C = 32 * int(rng.integers(1, 40)), 32 * int(rng.integers(1, 40))
        layout = "row"
        if fmt not in ("e2m3", "e3m2") and rng.random() < 0.3:
            R, C = R - R % 512 or 512, C - C % 512 or 512
            layout = "gemm"
        arbitrary = bool(rng.integers(2))
        seed = int(rng.integers(1 << 30))
        case = f"{orient} {fmt} -> {out} {R}x{C} layout={layout} arbitrary={arbitrary} seed={seed}"
        try:
            lines, length = (R, C) if orient == "row" else (C, R)
            if arbitrary:
                g = np.random.default_rng(seed)
                codes = g.integers(0, 1 << omx.fmt_of(fmt).bits, size=(lines, length)).astype(np.uint8)
                q = omx.pack_codes(codes, fmt)
                s = g.integers(0, 256, size=(lines, length // 32)).astype(np.uint8)
            else:
                x32 = workloads.random_tensor((R, C), seed, ["normal", "wide", "rows"][seed % 3])
                q, s = (omx.quantize_rowwise if orient == "row" else omx.quantize_colwise_t)(x32, fmt, "ceil")
            want = omx.dequantize(q, s, fmt, out=out)
            if orient == "col":
                want = np.ascontiguousarray(want.T)
            sd = omx.scales_to_gemm_layout(s) if layout == "gemm" else s
            got = host(mxa.mx_dequantize(upload_u8(q), upload_u8(sd), R, C, fmt, orient,
                                         out_dtype=torch.float32 if out == "f32" else torch.bfloat16,
                                         scale_layout=layout))
            if out == "f32":
                assert_float_equal(got, want, case)
            else:
                gn, wn = (got & 0x7FFF) > 0x7F80, (want & 0x7FFF) > 0x7F80
                if not (np.array_equal(gn, wn) and np.array_equal(np.where(gn, 0, got), np.where(wn, 0, want))):
                    failures.append(case)
        except Exception as e:   # noqa: BLE001
            failures.append(f"{case}: {type(e).__name__}: {str(e)[:160]}")
    _report(failures, n)


def test_gemm_random_cases():
    """Block-scaled GEMM: 200 random cases over every format pair, M and N up to 560
    (N a multiple of 8), K on both kernels (multiples of 512 for the 256 x 256 one,
    any multiple of 32 -- 64 for FP6 -- for the other), both scale layouts, several
    alphas; FP32 out against the float64 product of the dequantized operands."""
    rng = np.random.default_rng(20261205)
    failures = []
    n = 200
    for i in range(n):
        fa, fb = GEMM_PAIRS[rng.integers(len(GEMM_PAIRS))]
        M = int(rng.integers(1, 560))
        N = max(8, int(rng.integers(1, 560)) // 8 * 8)
        g = 64 if fa in ("e2m3", "e3m2") else 32
        K = 512 * int(rng.integers(1, 4)) if rng.random() < 0.5 else g * int(rng.integers(1, 1600 // g))
        layout = "gemm" if (K % 512 == 0 and rng.random() < 0.5) else "row"
        alpha = float(rng.choice([1.0, 0.5, 1.0 / 32, 3.0]))
        seed = int(rng.integers(1 << 30))
        case = f"{fa}x{fb} M={M} N={N} K={K} layout={layout} alpha={alpha} seed={seed}"
        try:
            A = workloads.random_tensor((M, K), seed, "normal")
            A = (A * np.exp2(((np.arange(K) // 32) % 7) - 3)[None, :]).astype(np.float32)
            B = workloads.random_tensor((N, K), seed + 1, "rows")
            qa, sa = omx.quantize_rowwise(A, fa, "ceil")
            qb, sb = omx.quantize_rowwise(B, fb, "ceil")
            ga, gb = (omx.scales_to_gemm_layout(sa), omx.scales_to_gemm_layout(sb)) if layout == "gemm" else (sa, sb)
            c = host(mxa.mx_gemm(upload_u8(qa), upload_u8(ga), upload_u8(qb), upload_u8(gb), fa, fb, alpha,
                                 out_dtype=torch.float32, scale_layout=layout))
            check_fp32(c, qa, sa, fa, qb, sb, fb, alpha=alpha)
        except Exception as e:   # noqa: BLE001
            failures.append(f"{case}: {type(e).__name__}: {str(e)[:160]}")
    _report(failures, n)
