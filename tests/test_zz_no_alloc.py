"""The allocation-free delayed-scaling entry point (fp8_quantize_delayed_static,
ticket scratch inside the library) against fp8_quantize_delayed with a caller
scratch buffer, through the C ABI: two calls in a row on the same ring state,
the second on a smaller input; codes, amax and the whole ring must be identical
after each call."""

import numpy as np
import pytest
import torch

import workloads
from tests.gpu_util import import_library, upload_bf16_bits

pytestmark = pytest.mark.gpu

mxa = import_library()

FMT = {"e4m3": 0, "e5m2": 1}
LAYOUT = {"row": 0, "transposed": 1, "dual": 2}


def call(static, x, fmt, layout, ring, hist_idx, tickets):
    R, C = x.shape
    q = torch.zeros((R, C), dtype=torch.uint8, device=x.device) if layout != "transposed" else None
    qT = torch.zeros((C, R), dtype=torch.uint8, device=x.device) if layout != "row" else None
    amax = torch.zeros(1, dtype=torch.float32, device=x.device)
    fp8_max = 448.0 if fmt == "e4m3" else 57344.0
    args = [x.data_ptr(), 1, R, C, FMT[fmt], LAYOUT[layout], None if q is None else q.data_ptr(),
            None if qT is None else qT.data_ptr(), ring.data_ptr(), ring.numel() - 4, hist_idx, fp8_max, 1.0,
            amax.data_ptr()]
    sp = torch.cuda.current_stream().cuda_stream
    if static:
        st = mxa.lib.fp8_quantize_delayed_static(*args, sp)
    else:
        st = mxa.lib.fp8_quantize_delayed(*args, tickets.data_ptr(), sp)
    assert st == 0, mxa.lib.mx_status_str(st).decode()
    torch.cuda.synchronize()
    return q, qT, amax


@pytest.mark.parametrize("layout,fmt", [("transposed", "e4m3"), ("dual", "e5m2"), ("row", "e4m3")])
def test_static_scratch_matches_caller_scratch(layout, fmt):
    tickets = mxa.new_tickets()
    ring_a, ring_b = mxa.new_ring(16), mxa.new_ring(16)
    stream = "act" if fmt == "e4m3" else "grad"
    # a large call (more workgroups than ticket groups), then a smaller one
    for t, (rows, cols) in enumerate(((2304, 4096), (256, 512))):
        x = upload_bf16_bits(workloads.delayed_step(stream, t, rows=rows, cols=cols))
        qa, qTa, aa = call(True, x, fmt, layout, ring_a, t, None)
        qb, qTb, ab = call(False, x, fmt, layout, ring_b, t, tickets)
        if qa is not None:
            assert torch.equal(qa, qb), f"call {t}: row codes differ"
        if qTa is not None:
            assert torch.equal(qTa, qTb), f"call {t}: transposed codes differ"
        assert torch.equal(aa, ab), f"call {t}: amax differs"
        assert torch.equal(ring_a, ring_b), f"call {t}: ring state differs"
        assert int(torch.count_nonzero(tickets)) == 0
        r = ring_a.cpu().numpy()
        assert r[16] > 0 and r[18] == 0 and r[19] == 0   # a scale was published; amax / ticket words cleared
