"""Maximum sizes: tensors past 2^31 elements, where 32-bit index arithmetic would
wrap.  Inputs come from torch's seeded device generator (no quantization
arithmetic); sampled rows and columns on both sides of the 2^31-element boundary
are compared with the oracle."""

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import gemm as og
from oracle import mx as omx
from tests.gpu_util import assert_bytes_equal, host, import_library

pytestmark = pytest.mark.gpu

mxa = import_library()


def bf16_host_f32(t: torch.Tensor) -> np.ndarray:
    return (t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)


def test_quantize_past_2_31_elements():
    R, C = 65600, 32768                        # 2.15e9 elements; row 65536 starts at element 2^31
    g = torch.Generator(device="cuda").manual_seed(20261202)
    x = torch.randn((R, C), dtype=torch.bfloat16, device="cuda", generator=g)
    rows = np.array([0, 65535, 65536, 65537, R - 1, 12345, 50000])
    cols = np.array([0, 1, 16384, C - 1])
    qr, sr = mxa.mx_quantize(x, "e4m3", "ceil", "row")
    xr = bf16_host_f32(x[torch.from_numpy(rows).cuda()])
    wq, ws = omx.quantize_rowwise(xr, "e4m3", "ceil")
    assert_bytes_equal(host(sr[torch.from_numpy(rows).cuda()]), ws, "row scales")
    assert_bytes_equal(host(qr[torch.from_numpy(rows).cuda()]), wq, "row codes")
    del qr, sr
    q_r, s_r, q_c, s_c = mxa.mx_quantize_dual(x, "e4m3", "ceil")
    assert_bytes_equal(host(q_r[torch.from_numpy(rows).cuda()]), wq, "dual row codes")
    xc = bf16_host_f32(x[:, torch.from_numpy(cols).cuda()])          # [R][4]
    wqc, wsc = omx.quantize_colwise_t(xc, "e4m3", "ceil")
    assert_bytes_equal(host(s_c[torch.from_numpy(cols).cuda()]), wsc, "dual col scales")
    assert_bytes_equal(host(q_c[torch.from_numpy(cols).cuda()]), wqc, "dual col codes")


def test_gemm_output_past_2_31_elements():
    M = N = 49152                              # 2.4e9 outputs; row 43691 starts past element 2^31
    K = 512
    g = torch.Generator(device="cuda").manual_seed(7)
    # finite E4M3 codes: exponent field below 15 (so never the NaN pattern), any sign and mantissa
    def codes(shape):
        e = torch.randint(3, 12, shape, device="cuda", generator=g, dtype=torch.int32)
        m = torch.randint(0, 8, shape, device="cuda", generator=g, dtype=torch.int32)
        s = torch.randint(0, 2, shape, device="cuda", generator=g, dtype=torch.int32)
        return ((s << 7) | (e << 3) | m).to(torch.uint8)
    qa, qb = codes((M, K)), codes((N, K))
    sa = torch.randint(120, 134, (M, K // 32), device="cuda", generator=g, dtype=torch.int32).to(torch.uint8)
    sb = torch.randint(120, 134, (N, K // 32), device="cuda", generator=g, dtype=torch.int32).to(torch.uint8)
    c = mxa.mx_gemm(qa, sa, qb, sb, "e4m3", "e4m3", 0.5, out_dtype=torch.bfloat16)
    rows = np.array([0, 43690, 43691, 43692, M - 1])
    ri = torch.from_numpy(rows).cuda()
    got = (c[ri].contiguous().view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    ref = og.gemm_ref(host(qa[ri]), host(sa[ri]), "e4m3", host(qb), host(sb), "e4m3", alpha=0.5)
    want = (og.f64_to_bf16_bits(ref).astype(np.uint32) << 16).view(np.float32)
    assert og.rel_frobenius(got.astype(np.float64), want.astype(np.float64)) <= 1e-3
