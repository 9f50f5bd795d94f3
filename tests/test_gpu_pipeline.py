"""End-to-end parity of the per-tensor FP8 training flow of the AstrAI fp8.py page:
the delayed-scaling quantizer casts activations and weights with the scales their
rings hold, and mm_fp8 consumes the codes with scale = s_x * s_w taken from the
rings on the device (no host round trip), plus a bias.  Every step is compared
with the oracle's composition of the same steps."""

import numpy as np
import pytest
import torch

import workloads
from oracle import delayed as odl
from oracle import formats as ofmt
from oracle import gemm as og
from tests.gpu_util import host, upload_bf16_bits, import_library

pytestmark = pytest.mark.gpu

mxa = import_library()


@pytest.mark.parametrize("shape", [(256, 384, 512), (512, 512, 1024)])
def test_delayed_quantize_then_mm_fp8(shape):
    M, N, K = shape
    ring_x, ring_w = mxa.new_ring(16), mxa.new_ring(16)
    ox, ow = odl.Ring(16), odl.Ring(16)
    bias_bits = ofmt.f32_to_bf16_bits(workloads.random_tensor((N,), 9, "normal"))
    bias = upload_bf16_bits(bias_bits)
    for t in range(3):     # step 0 casts with s = 1; later steps with the folded scales
        xb = workloads.to_bf16_bits(workloads.random_tensor((M, K), 100 + t, "normal").astype(np.float64))
        wb = workloads.to_bf16_bits(workloads.random_tensor((N, K), 200 + t, "normal").astype(np.float64) * 0.02)
        xs, ws = workloads.bf16_to_f32(xb), workloads.bf16_to_f32(wb)
        # the scale the next GEMM uses is the one these casts used: read it before the fold
        sx_dev, sw_dev = ring_x[16:17].clone(), ring_w[16:17].clone()
        sx, sw = ox.s, ow.s
        xq, _ = mxa.fp8_quantize_delayed(upload_bf16_bits(xb), ring_x, t, "e4m3", "row")
        wq, _ = mxa.fp8_quantize_delayed(upload_bf16_bits(wb), ring_w, t, "e4m3", "row")
        wxq, _, _ = odl.quantize_delayed(xs, "e4m3", ox, t, 448.0, 1.0)
        wwq, _, _ = odl.quantize_delayed(ws, "e4m3", ow, t, 448.0, 1.0)
        assert np.array_equal(host(xq), wxq) and np.array_equal(host(wq), wwq)
        scale = sx_dev * sw_dev                        # s_x s_w in FP32 on the device
        out = host(mxa.mm_fp8(xq.view(torch.float8_e4m3fn), wq.view(torch.float8_e4m3fn).t(), scale, bias=bias))
        s_ref = np.float32(np.float32(sx) * np.float32(sw))
        ref = og.mm_fp8_ref(wxq, wwq, "e4m3", s_ref, trans_b=True, bias=bias_bits)
        got = workloads.bf16_to_f32(out.view(np.uint16)).astype(np.float64)
        assert og.rel_frobenius(got, workloads.bf16_to_f32(og.f64_to_bf16_bits(ref)).astype(np.float64)) <= 1e-3
        # the codes times the scales approximate the real product (the scale is a dequantization scale)
        if t > 0:
            exact = xs.astype(np.float64) @ ws.astype(np.float64).T + workloads.bf16_to_f32(bias_bits)
            assert og.rel_frobenius(got, exact) < 0.1
