"""Seeded random sweeps over shapes, formats, rules, input types and scale layouts,
each case compared with the oracle exactly as the targeted tests do: quantized
bytes and scales bit for bit, dequantized values bit for bit, delayed-scaling
codes, amax and the whole ring bit for bit, GEMM results within the bounds of
test_gpu_gemm and test_gpu_mm_fp8 (1e-3 relative Frobenius and the per-element
accumulation bound), re-quantized GEMM outputs bit for bit.  The cases are drawn from one fixed seed, so a failure names a
reproducible case; every failing case is listed, not just the first."""

import numpy as np
import pytest
import torch

import workloads
from oracle import delayed as odl
from oracle import formats as ofmt
from oracle import mx as omx
from tests import test_gpu_mm_fp8 as tmm
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


def test_delayed_random_cases():
    """Per-tensor delayed scaling: 60 random cases of three successive steps (rows a
    multiple of 32 up to 1536, columns of 8 up to 1536, every layout, FP32 / BF16 /
    FP16 input, both formats, history length 1 to 40 with random slots, random
    fp8_max and margin, with and without ticket scratch): codes, amax and the whole
    ring after every step, the scratch left zero."""
    rng = np.random.default_rng(20261206)
    failures = []
    n = 60
    for i in range(n):
        layout = ["row", "transposed", "dual"][rng.integers(3)]
        dtype = ["f32", "bf16", "f16"][rng.integers(3)]
        fmt = ["e4m3", "e5m2"][rng.integers(2)]
        R, C = 32 * int(rng.integers(1, 49)), 8 * int(rng.integers(1, 193))
        hist_len = int(rng.integers(1, 41))
        fp8_max = float(rng.choice([448.0, 57344.0, 240.0, 1.0]))
        margin = float(rng.choice([1.0, 2.0, 0.75]))
        scratch = bool(rng.integers(2))
        seed = int(rng.integers(1 << 30))
        case = (f"{layout} {fmt} {dtype} {R}x{C} hist_len={hist_len} fp8_max={fp8_max} margin={margin} "
                f"scratch={scratch} seed={seed}")
        try:
            ring = mxa.new_ring(hist_len)
            tickets = mxa.new_tickets() if scratch else None
            oring = odl.Ring(hist_len)
            g = np.random.default_rng(seed)
            for t in range(3):
                idx = int(g.integers(hist_len))
                x32 = (g.standard_normal((R, C)) * np.exp2(g.uniform(-12, 12))).astype(np.float32)
                if dtype == "f32":
                    x = upload_f32(x32)
                elif dtype == "bf16":
                    x = upload_bf16_bits(workloads.to_bf16_bits(x32.astype(np.float64)))
                else:
                    x = upload_f16_from_f32(x32)
                xs = f32_of_input(x)
                q, qT, a = mxa.fp8_quantize_delayed(x, ring, idx, fmt, layout, fp8_max, margin, amax=True,
                                                    tickets=tickets)
                wq, wqT, wa = odl.quantize_delayed(xs, fmt, oring, idx, fp8_max, margin)
                ok = host(a)[0] == wa
                if q is not None:
                    ok = ok and np.array_equal(host(q), wq)
                if qT is not None:
                    ok = ok and np.array_equal(host(qT), wqT)
                gr, wr = host(ring), oring.as_array()
                ok = ok and np.array_equal(gr.view(np.uint32), np.asarray(wr, dtype=np.float32).view(np.uint32))
                if tickets is not None:
                    ok = ok and int(torch.count_nonzero(tickets)) == 0
                if not ok:
                    failures.append(f"{case} step {t}")
                    break
        except Exception as e:   # noqa: BLE001
            failures.append(f"{case}: {type(e).__name__}: {str(e)[:160]}")
    _report(failures, n)


def test_mm_fp8_random_cases():
    """Per-tensor FP8 GEMM: 80 random cases (M, N up to 600, K up to 2100, both formats,
    every transpose combination, random scale, with and without bias, sometimes a
    batch of 2 or 3 on either side)."""
    rng = np.random.default_rng(20261207)
    failures = []
    n = 80
    for i in range(n):
        fmt = ["e4m3", "e5m2"][rng.integers(2)]
        ta, tb = bool(rng.integers(2)), bool(rng.integers(2))
        M, N = int(rng.integers(1, 600)), int(rng.integers(1, 600))
        K = 16 * int(rng.integers(1, 132)) if rng.random() < 0.5 else 128 * int(rng.integers(1, 17))
        scale = float(np.exp2(rng.integers(-12, 3)) * rng.choice([1.0, 1.25, 0.75]))
        batch = [None, None, (2, None), (None, 3), (3, 3)][rng.integers(5)] if K <= 1024 else (None, None)
        use_bias = bool(rng.integers(2))
        seed = int(rng.integers(1 << 20))
        case = f"{fmt} ta={ta} tb={tb} M={M} N={N} K={K} scale={scale} batch={batch} bias={use_bias} seed={seed}"
        try:
            ba, bb = batch if batch else (None, None)
            a = tmm.codes(tmm.stored((M, K), ta, ba), seed, fmt)
            b = tmm.codes(tmm.stored((K, N), tb, bb), seed + 1, fmt)
            bias = (ofmt.f32_to_bf16_bits(workloads.random_tensor((N,), seed % 97, "normal") * 4)
                    if use_bias else None)
            tmm.check(tmm.run(a, b, fmt, scale, ta, tb, bias), a, b, fmt, scale, ta, tb, bias, case)
        except Exception as e:   # noqa: BLE001
            failures.append(f"{case}: {type(e).__name__}: {str(e)[:200]}")
    _report(failures, n)


def test_requant_random_cases():
    """GEMM with MX re-quantization in the epilogue: 60 random cases (FP8 and FP4
    operand pairs, M up to 600, N a multiple of 32 up to 608, K on both GEMM kernels,
    every output format and rule, random alpha): codes, scales and amax bit for bit
    against the oracle's row-wise quantizer applied to mx_gemm's FP32 output."""
    rng = np.random.default_rng(20261208)
    failures = []
    n = 60
    pairs = [("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e4m3", "e5m2"), ("e2m1", "e2m1")]
    for i in range(n):
        fa, fb = pairs[rng.integers(len(pairs))]
        fc = ["e4m3", "e5m2", "e2m1"][rng.integers(3)]
        rc = ["floor", "ceil"][rng.integers(2)]
        M, N = int(rng.integers(1, 600)), 32 * int(rng.integers(1, 20))
        K = 512 * int(rng.integers(1, 4)) if rng.random() < 0.5 else 32 * int(rng.integers(1, 50))
        alpha = float(rng.choice([1.0, 0.75, 1.0 / 32, 5.0]))
        seed = int(rng.integers(1 << 30))
        case = f"{fa}x{fb}->{fc} {rc} M={M} N={N} K={K} alpha={alpha} seed={seed}"
        try:
            A = workloads.random_tensor((M, K), seed, "normal")
            B = workloads.random_tensor((N, K), seed + 1, "rows")
            qa, sa = omx.quantize_rowwise(A, fa, "ceil")
            qb, sb = omx.quantize_rowwise(B, fb, "ceil")
            args = (upload_u8(qa), upload_u8(sa), upload_u8(qb), upload_u8(sb), fa, fb, alpha)
            c32 = host(mxa.mx_gemm(*args, out_dtype=torch.float32))
            q, s_, a = mxa.mx_gemm_requant(*args, fmt_c=fc, rule_c=rc, amax=True)
            wq, ws = omx.quantize_rowwise(c32, fc, rc)
            if not (np.array_equal(host(q), wq) and np.array_equal(host(s_), ws)
                    and host(a)[0] == omx.tensor_amax(c32)):
                failures.append(case)
        except Exception as e:   # noqa: BLE001
            failures.append(f"{case}: {type(e).__name__}: {str(e)[:160]}")
    _report(failures, n)
