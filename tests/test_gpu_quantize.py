"""GPU parity of the MX quantizers, the dequantizer and the per-tensor delayed
quantizer against the CPU oracle: bit-exact codes, scales, amax and ring state
on the same seeded inputs."""

import numpy as np
import pytest
import torch

import workloads
from oracle import delayed as odl
from oracle import formats as F
from oracle import mx as omx
from tests.gpu_util import (assert_bytes_equal, assert_float_equal, f32_of_input, host, import_library,
                            upload_bf16_bits, upload_f16_from_f32, upload_f32, upload_u8)

pytestmark = pytest.mark.gpu

mxa = import_library()

FMTS = ["e4m3", "e5m2", "e2m1"]
RULES = ["floor", "ceil"]


def make_input(x32: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "f32":
        return upload_f32(x32)
    if dtype == "bf16":
        return upload_bf16_bits(workloads.to_bf16_bits(x32.astype(np.float64)))
    return upload_f16_from_f32(x32)


def small_inputs():
    return {
        "wide_range": workloads.wide_range_f32(96, 256),
        "wide": workloads.random_tensor((64, 320), 21, "wide"),
        "rows": workloads.random_tensor((160, 96), 22, "rows"),
    }


# ---------------------------------------------------------------- row-wise

@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rule", RULES)
def test_rowwise_parity(dtype, fmt, rule):
    for name, x32 in small_inputs().items():
        x = make_input(x32, dtype)
        xs = f32_of_input(x)
        q, s, a = mxa.mx_quantize(x, fmt, rule, "row", amax=True)
        wq, ws = omx.quantize_rowwise(xs, fmt, rule)
        assert_bytes_equal(host(s), ws, f"{name} scales")
        assert_bytes_equal(host(q), wq, f"{name} codes")
        assert host(a)[0] == omx.tensor_amax(xs)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rule", RULES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rowwise_every_bf16_pattern(fmt, rule, dtype):
    """Every finite BF16 value, in blocks whose maxima sweep the exponent range,
    plus hand-picked special blocks (zeros, FP32 subnormals, extremes, NaN, Inf)."""
    blocks = workloads.all_bf16_blocks()
    if dtype == "f32":
        blocks = np.concatenate([blocks, workloads.special_blocks()])
    x32 = blocks.reshape(-1, 256) if blocks.shape[0] % 8 == 0 else blocks.reshape(-1, 32)
    x = make_input(x32, dtype)
    xs = f32_of_input(x)
    q, s = mxa.mx_quantize(x, fmt, rule, "row")
    wq, ws = omx.quantize_rowwise(xs, fmt, rule)
    assert_bytes_equal(host(s), ws, "scales")
    assert_bytes_equal(host(q), wq, "codes")


@pytest.mark.parametrize("fmt", FMTS)
def test_rowwise_hadamard(fmt):
    mask = 0xA5C3_0F96
    x32 = workloads.random_tensor((64, 256), 23, "rows")
    for dtype in ("f32", "bf16"):
        x = make_input(x32, dtype)
        xs = f32_of_input(x)
        q, s = mxa.mx_quantize(x, fmt, "ceil", "row", hadamard_mask=mask)
        wq, ws = omx.quantize_rowwise(xs, fmt, "ceil", hadamard_mask=mask)
        assert_bytes_equal(host(s), ws, "scales")
        assert_bytes_equal(host(q), wq, "codes")


# ---------------------------------------------------------------- column-wise / dual

@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rule", RULES)
def test_colwise_parity_ragged(dtype, fmt, rule):
    # 160 rows (one full and one partial 128-row tile), 200 columns (not a multiple
    # of 32); 288 rows (a full 256-row FP4 tile and a partial one); one 32 x 32 block
    for shape, seed in (((160, 200), 24), ((288, 72), 30), ((32, 32), 31)):
        x32 = workloads.random_tensor(shape, seed, "wide")
        x = make_input(x32, dtype)
        xs = f32_of_input(x)
        q, s, a = mxa.mx_quantize(x, fmt, rule, "col", amax=True)
        wq, ws = omx.quantize_colwise_t(xs, fmt, rule)
        assert_bytes_equal(host(s), ws, f"{shape} scales")
        assert_bytes_equal(host(q), wq, f"{shape} codes")
        assert host(a)[0] == omx.tensor_amax(xs)


@pytest.mark.parametrize("fmt", FMTS)
def test_colwise_hadamard(fmt):
    mask = 0x1357_9BDF
    for shape, seed in (((256, 136), 25), ((544, 72), 32)):
        x32 = workloads.random_tensor(shape, seed, "normal")
        x = make_input(x32, "bf16")
        xs = f32_of_input(x)
        q, s = mxa.mx_quantize(x, fmt, "ceil", "col", hadamard_mask=mask)
        wq, ws = omx.quantize_colwise_t(xs, fmt, "ceil", hadamard_mask=mask)
        assert_bytes_equal(host(s), ws, f"{shape} scales")
        assert_bytes_equal(host(q), wq, f"{shape} codes")


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rule", RULES)
def test_dual_parity_ragged(dtype, fmt, rule):
    # tiles of 128 x 128 with ragged right and bottom edges; (256, 992) gives a
    # tile count divisible by 8 (the XCD-grouped tile order)
    for shape, seed in (((96, 160), 26), ((288, 416), 27), ((256, 992), 28), ((320, 544), 29), ((32, 32), 33)):
        x32 = workloads.random_tensor(shape, seed, "rows")
        x = make_input(x32, dtype)
        xs = f32_of_input(x)
        qr, sr, qc, sc, a = mxa.mx_quantize_dual(x, fmt, rule, amax=True)
        wqr, wsr, wqc, wsc = omx.quantize_dual(xs, fmt, rule)
        assert_bytes_equal(host(sr), wsr, "row scales")
        assert_bytes_equal(host(qr), wqr, "row codes")
        assert_bytes_equal(host(sc), wsc, "col scales")
        assert_bytes_equal(host(qc), wqc, "col codes")
        assert host(a)[0] == omx.tensor_amax(xs)


def test_dual_matches_single_orientation_calls():
    """Page-3 style orientation check: the one-read dual output equals the
    row-wise call and the column-wise call byte for byte."""
    x = upload_bf16_bits(workloads.activation_bf16(256, 384))
    for fmt in FMTS:
        qr, sr, qc, sc = mxa.mx_quantize_dual(x, fmt, "ceil")
        q1, s1 = mxa.mx_quantize(x, fmt, "ceil", "row")
        q2, s2 = mxa.mx_quantize(x, fmt, "ceil", "col")
        assert torch.equal(qr, q1) and torch.equal(sr, s1)
        assert torch.equal(qc, q2) and torch.equal(sc, s2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_special_blocks_dual(dtype):
    blocks = workloads.special_blocks()          # [18][32]
    x32 = np.zeros((64, 64), np.float32)
    x32[:18, :32] = blocks                      # as row blocks
    x32[32:64, 32:50] = blocks.T                # as column blocks
    x32[40, :] = np.nan
    x32[:, 60] = -np.inf
    x = make_input(x32, dtype)
    x32 = f32_of_input(x)
    for fmt in FMTS:
        for rule in RULES:
            qr, sr, qc, sc, a = mxa.mx_quantize_dual(x, fmt, rule, amax=True)
            wqr, wsr, wqc, wsc = omx.quantize_dual(x32, fmt, rule)
            assert_bytes_equal(host(sr), wsr, "row scales")
            assert_bytes_equal(host(qr), wqr, "row codes")
            assert_bytes_equal(host(sc), wsc, "col scales")
            assert_bytes_equal(host(qc), wqc, "col codes")
            assert host(a)[0] == omx.tensor_amax(x32)


@pytest.mark.parametrize("orient", ["col", "row"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("had", [False, True])
def test_special_blocks_hadamard(had, dtype, orient):
    """Zero, subnormal, extreme and non-finite blocks, with and without the
    Hadamard transform, column-wise and row-wise.  Every byte is compared,
    sign bits included: NaNs made by the transform carry a clear sign bit on
    both sides."""
    blocks = workloads.special_blocks()          # [18][32]
    x32 = np.zeros((96, 64), np.float32)
    x32[32:64, 8:26] = blocks.T                 # as column blocks
    x32[70, :] = np.nan
    x32[:, 60] = -np.inf
    if orient == "row":
        x32 = np.ascontiguousarray(x32.T)       # the same blocks as row blocks
    x = make_input(x32, dtype)
    xs = f32_of_input(x)
    mask = 0x2468_ACE1 if had else None
    ref = omx.quantize_colwise_t if orient == "col" else omx.quantize_rowwise
    for fmt in FMTS:
        for rule in RULES:
            q, s, a = mxa.mx_quantize(x, fmt, rule, orient, hadamard_mask=mask, amax=True)
            wq, ws = ref(xs, fmt, rule, hadamard_mask=mask)
            assert_bytes_equal(host(s), ws, f"{fmt} {rule} scales")
            assert_bytes_equal(host(q), wq, f"{fmt} {rule} codes")
            assert host(a)[0] == omx.tensor_amax(xs)


def test_empty_inputs():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    q, s, a = mxa.mx_quantize(x, "e4m3", "ceil", "row", amax=True)
    assert q.numel() == 0 and host(a)[0] == 0.0
    qr, sr, qc, sc, a = mxa.mx_quantize_dual(x, "e4m3", "ceil", amax=True)
    assert host(a)[0] == 0.0
    ring = mxa.new_ring(16)
    out = mxa.fp8_quantize_delayed(x, ring, 3, "e4m3", "transposed", amax=True)
    assert host(out[2])[0] == 0.0
    r = host(ring)
    assert r[16] == 1.0 and r[17] == 1.0 and r[18] == 0.0 and r[19] == 0.0


def test_bad_shape_raises_value_error():
    x = torch.zeros((64, 48), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        mxa.mx_quantize_dual(x)


# ---------------------------------------------------------------- dequantize

@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("orient", ["row", "col"])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_dequantize_parity(fmt, orient, out_dtype):
    g = np.random.default_rng(31)
    rows, cols = 96, 136 if orient == "col" else 160
    nb = 1 << F.FORMATS[fmt].bits
    stored_r, stored_c = (rows, cols) if orient == "row" else (cols, rows)
    codes = g.integers(0, nb, size=(stored_r, stored_c)).astype(np.uint8)
    scales = g.integers(0, 256, size=(stored_r, stored_c // 32)).astype(np.uint8)
    scales[0, 0], scales[1, 0], scales[2, 0] = 0, 254, 255
    packed = omx.pack_fp4(codes) if fmt == "e2m1" else codes
    out = mxa.mx_dequantize(upload_u8(packed), upload_u8(scales), rows, cols, fmt, orient, out_dtype)
    kind = "f32" if out_dtype == torch.float32 else "bf16"
    want = omx.dequantize(packed, scales, fmt, out=kind)
    if orient == "col":
        want = np.ascontiguousarray(want.T)
    got = host(out)
    if kind == "f32":
        assert_float_equal(got, want, "dequantized")
    else:
        gn = (got & 0x7FFF) > 0x7F80
        wn = (want & 0x7FFF) > 0x7F80
        assert np.array_equal(gn, wn)
        assert_bytes_equal(np.where(gn, 0, got), np.where(wn, 0, want), "dequantized bf16")


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_dequantize_roundtrip_wide_range_f32(fmt):
    x = upload_f32(workloads.wide_range_f32())
    q, s = mxa.mx_quantize(x, fmt, "floor", "row")
    d = mxa.mx_dequantize(q, s, 256, 1024, fmt, "row")
    wq, ws = omx.quantize_rowwise(workloads.wide_range_f32(), fmt, "floor")
    assert_bytes_equal(host(q), wq, "codes")
    assert_float_equal(host(d), omx.dequantize(wq, ws, fmt), "roundtrip")


# ---------------------------------------------------------------- per-tensor delayed scaling

def new_tickets(mode):
    """Ticket scratch for a delayed-scaling test: a fresh zeroed buffer, or None
    (the ticket is taken on the ring's own words)."""
    return mxa.new_tickets() if mode == "scratch" else None


def assert_ring_state(ring, tickets, oring, what):
    """The whole ring equals the host fold; the ticket scratch reads zero again."""
    assert ring.numel() == oring.hist.size + 4
    assert_float_equal(host(ring), oring.as_array(), f"{what} ring")
    if tickets is not None:
        assert int(torch.count_nonzero(tickets)) == 0, f"{what}: ticket scratch not left zero"


@pytest.mark.parametrize("tmode", ["scratch", "none"])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("layout", ["row", "transposed", "dual"])
def test_delayed_sequence_small(fmt, layout, tmode):
    """32 successive steps on one ring (length 16): codes, amax and the whole
    ring state equal the host fold after every step, with and without ticket
    scratch."""
    stream = "act" if fmt == "e4m3" else "grad"
    fp8_max = workloads.DELAYED_FP8_MAX[stream]
    ring = mxa.new_ring(16)
    tickets = new_tickets(tmode)
    oring = odl.Ring(16)
    for t in range(32):
        xb = workloads.delayed_step(stream, t, rows=96, cols=160)
        x = upload_bf16_bits(xb)
        xs = workloads.bf16_to_f32(xb)
        q, qT, a = mxa.fp8_quantize_delayed(x, ring, t % 16, fmt, layout, fp8_max, 1.0, amax=True, tickets=tickets)
        wq, wqT, wa = odl.quantize_delayed(xs, fmt, oring, t % 16, fp8_max, 1.0)
        if q is not None:
            assert_bytes_equal(host(q), wq, f"step {t} q")
        if qT is not None:
            assert_bytes_equal(host(qT), wqT, f"step {t} qT")
        assert host(a)[0] == wa
        assert_ring_state(ring, tickets, oring, f"step {t}")


@pytest.mark.parametrize("tmode", ["scratch", "none"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("layout", ["row", "transposed", "dual"])
def test_delayed_many_workgroups(layout, dtype, tmode):
    """A 2304 x 4096 input: more tiles than the persistent grid of the
    no-scratch launch (so workgroups loop over several tiles and all take their
    ticket on one word) and, with scratch, more than one workgroup per ticket
    group.  Four steps: codes, amax and ring exact."""
    ring = mxa.new_ring(8)
    tickets = new_tickets(tmode)
    oring = odl.Ring(8)
    for t in range(4):
        xb = workloads.delayed_step("grad", t, rows=2304, cols=4096)
        x = make_input(workloads.bf16_to_f32(xb), dtype)
        xs = f32_of_input(x)
        q, qT, a = mxa.fp8_quantize_delayed(x, ring, t % 8, "e5m2", layout, 57344.0, 1.0, amax=True, tickets=tickets)
        wq, wqT, wa = odl.quantize_delayed(xs, "e5m2", oring, t % 8, 57344.0, 1.0)
        if q is not None:
            assert_bytes_equal(host(q), wq, f"step {t} q")
        if qT is not None:
            assert_bytes_equal(host(qT), wqT, f"step {t} qT")
        assert host(a)[0] == wa
        assert_ring_state(ring, tickets, oring, f"step {t}")


@pytest.mark.parametrize("tmode", ["scratch", "none"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("layout", ["row", "transposed", "dual"])
@pytest.mark.parametrize("cols", [128, 256, 2048, 2176, 4096, 4352])
def test_delayed_small_grids(cols, layout, dtype, tmode):
    """128-row inputs whose grids straddle the ticket modes: one workgroup (no
    ticket, it folds its own max), 2 to 16 (a single-level ticket on the ring's
    words, also with scratch) and 17 or more (the two-level ticket with scratch).
    Transposed BF16 and dual launch one workgroup per 128 x 128 tile (1, 2, 16,
    17, 32, 34 here), row-wise one per 32768 elements (1, 1, 8, 9, 16, 17).  Six
    steps: codes, amax and ring exact, scratch left zero."""
    ring = mxa.new_ring(4)
    tickets = new_tickets(tmode)
    oring = odl.Ring(4)
    for t in range(6):
        xb = workloads.delayed_step("act", t, rows=128, cols=cols)
        x = make_input(workloads.bf16_to_f32(xb), dtype)
        xs = f32_of_input(x)
        q, qT, a = mxa.fp8_quantize_delayed(x, ring, t % 4, "e4m3", layout, 448.0, 1.0, amax=True, tickets=tickets)
        wq, wqT, wa = odl.quantize_delayed(xs, "e4m3", oring, t % 4, 448.0, 1.0)
        if q is not None:
            assert_bytes_equal(host(q), wq, f"step {t} q")
        if qT is not None:
            assert_bytes_equal(host(qT), wqT, f"step {t} qT")
        assert host(a)[0] == wa
        assert_ring_state(ring, tickets, oring, f"step {t}")


@pytest.mark.parametrize("tmode", ["scratch", "none"])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_delayed_multi_tile_ragged(fmt, tmode):
    """BF16 4128 x 4136 transposed: 33 x 33 tiles, more than the capped grid, so
    some workgroups take two tiles (all waves store the first, waves 1-3 the
    last), with a partial last tile row and column.  Three steps: every code,
    the amax and the whole ring."""
    ring = mxa.new_ring(16)
    tickets = new_tickets(tmode)
    oring = odl.Ring(16)
    for t in range(3):
        xb = workloads.delayed_step("act" if fmt == "e4m3" else "grad", 50 + t, rows=4128, cols=4136)
        x = upload_bf16_bits(xb)
        fp8_max = 448.0 if fmt == "e4m3" else 57344.0
        _, qT, a = mxa.fp8_quantize_delayed(x, ring, t, fmt, "transposed", fp8_max, 1.0, amax=True, tickets=tickets)
        _, wqT, wa = odl.quantize_delayed(workloads.bf16_to_f32(xb), fmt, oring, t, fp8_max, 1.0)
        assert_bytes_equal(host(qT), wqT, f"step {t} qT")
        assert host(a)[0] == wa
        assert_ring_state(ring, tickets, oring, f"step {t}")


def test_delayed_scratch_shared_by_two_rings():
    """One ticket scratch serves calls on different rings in stream order; each
    ring follows its own host fold."""
    tickets = mxa.new_tickets()
    rings = {s: mxa.new_ring(16) for s in ("act", "grad")}
    orings = {s: odl.Ring(16) for s in ("act", "grad")}
    for t in range(6):
        for stream, fmt in (("act", "e4m3"), ("grad", "e5m2")):
            fp8_max = workloads.DELAYED_FP8_MAX[stream]
            xb = workloads.delayed_step(stream, t, rows=512, cols=1024)
            _, qT = mxa.fp8_quantize_delayed(upload_bf16_bits(xb), rings[stream], t, fmt, "transposed", fp8_max,
                                             tickets=tickets)
            _, wqT, _ = odl.quantize_delayed(workloads.bf16_to_f32(xb), fmt, orings[stream], t, fp8_max, 1.0)
            assert_bytes_equal(host(qT), wqT, f"{stream} step {t} qT")
            assert_ring_state(rings[stream], tickets, orings[stream], f"{stream} step {t}")


@pytest.mark.parametrize("tmode", ["scratch", "none"])
def test_delayed_two_rings_on_two_streams(tmode):
    """The activation ring on one stream and the gradient ring on another, launched
    without any ordering between the streams, so the two streams' kernels may run
    at the same time (each ring with its own ticket scratch, or none).  The ring is
    copied on its own stream after each step; every copy, and every step's codes,
    equal that ring's host fold."""
    side = {s: torch.cuda.Stream() for s in ("act", "grad")}   # default priority
    fmts = {"act": "e4m3", "grad": "e5m2"}
    steps = 8
    xb = {s: [workloads.delayed_step(s, t, rows=1024, cols=2048) for t in range(steps)] for s in fmts}
    xs = {s: [upload_bf16_bits(b) for b in xb[s]] for s in fmts}
    rings = {s: mxa.new_ring(16) for s in fmts}
    tickets = {s: new_tickets(tmode) for s in fmts}
    torch.cuda.synchronize()
    out = {s: [] for s in fmts}
    for t in range(steps):
        for s, fmt in fmts.items():
            with torch.cuda.stream(side[s]):
                _, qT = mxa.fp8_quantize_delayed(xs[s][t], rings[s], t, fmt, "transposed",
                                                 workloads.DELAYED_FP8_MAX[s], tickets=tickets[s])
                out[s].append((qT, rings[s].clone()))
    torch.cuda.synchronize()
    for s, fmt in fmts.items():
        oring = odl.Ring(16)
        for t in range(steps):
            _, wqT, _ = odl.quantize_delayed(workloads.bf16_to_f32(xb[s][t]), fmt, oring, t,
                                             workloads.DELAYED_FP8_MAX[s], 1.0)
            qT, ring_t = out[s][t]
            assert_bytes_equal(host(qT), wqT, f"{s} step {t} qT")
            assert_ring_state(ring_t, None, oring, f"{s} step {t}")
        if tickets[s] is not None:
            assert int(torch.count_nonzero(tickets[s])) == 0, f"{s}: ticket scratch not left zero"


@pytest.mark.parametrize("tmode", ["scratch", "none"])
def test_delayed_one_ring_across_streams(tmode):
    """One ring whose steps alternate between two streams, each launch waiting on
    an event recorded after the previous one: the event order is the ring's order,
    and each step's codes and ring copy equal the host fold."""
    side = [torch.cuda.Stream(), torch.cuda.Stream()]   # default priority
    steps = 12
    xb = [workloads.delayed_step("act", t, rows=768, cols=1536) for t in range(steps)]
    xs = [upload_bf16_bits(b) for b in xb]
    ring = mxa.new_ring(8)
    tickets = new_tickets(tmode)
    torch.cuda.synchronize()
    done = None
    out = []
    for t in range(steps):
        s = side[t % 2]
        with torch.cuda.stream(s):
            if done is not None:
                s.wait_event(done)
            q, qT, a = mxa.fp8_quantize_delayed(xs[t], ring, t % 8, "e4m3", "dual", amax=True, tickets=tickets)
            out.append((q, qT, a, ring.clone()))
            done = torch.cuda.Event()
            done.record(s)
    torch.cuda.synchronize()
    oring = odl.Ring(8)
    for t in range(steps):
        wq, wqT, wa = odl.quantize_delayed(workloads.bf16_to_f32(xb[t]), "e4m3", oring, t % 8,
                                           workloads.DELAYED_FP8_MAX["act"], 1.0)
        q, qT, a, ring_t = out[t]
        assert_bytes_equal(host(q), wq, f"step {t} q")
        assert_bytes_equal(host(qT), wqT, f"step {t} qT")
        assert host(a)[0] == wa
        assert_ring_state(ring_t, None, oring, f"step {t}")
    if tickets is not None:
        assert int(torch.count_nonzero(tickets)) == 0, "ticket scratch not left zero"


def test_delayed_resume_from_saved_ring():
    """The ring is the only state: copying it out at step 16 and resuming from the
    copy gives the same bytes as the uninterrupted run."""
    ring = mxa.new_ring(16)
    outs = []
    saved = None
    for t in range(24):
        if t == 16:
            saved = ring.clone()
        x = upload_bf16_bits(workloads.delayed_step("act", t, rows=64, cols=64))
        outs.append(mxa.fp8_quantize_delayed(x, ring, t % 16, "e4m3", "transposed")[1])
    for t in range(16, 24):
        x = upload_bf16_bits(workloads.delayed_step("act", t, rows=64, cols=64))
        qT = mxa.fp8_quantize_delayed(x, saved, t % 16, "e4m3", "transposed")[1]
        assert torch.equal(qT, outs[t])
    assert torch.equal(saved, ring)


@pytest.mark.parametrize("hist_len", [17, 4096])
@pytest.mark.parametrize("cols", [128, 256, 4352])
@pytest.mark.parametrize("tmode", ["scratch", "none"])
def test_delayed_fold_of_a_preset_history(hist_len, cols, tmode):
    """A ring resumed with arbitrary history entries -- +Inf, subnormals, zeros,
    large and small normal values -- at the longest history and at one that is
    not a multiple of the fold's 16-entry batches, on grids of one workgroup
    (no ticket), two and 34 workgroups: the fold takes the max over the history
    exactly as the host fold does, for slots at both ends and inside."""
    g = np.random.default_rng(hist_len + cols)
    hist = (g.standard_normal(hist_len) ** 2 * np.exp2(g.integers(-30, 30, size=hist_len))).astype(np.float32)
    hist[g.integers(hist_len, size=4)] = 0.0
    hist[g.integers(hist_len, size=2)] = np.float32(1e-40)     # subnormal
    init = np.concatenate([hist, np.array([0.5, 2.0, 0.0, 0.0], dtype=np.float32)])
    ring = torch.from_numpy(init.copy()).to("cuda")
    tickets = new_tickets(tmode)
    oring = odl.Ring.from_array(init)
    slots = [0, hist_len - 1, hist_len // 2, 5]
    for t, idx in enumerate(slots):
        if t == 2:   # an Inf entry elsewhere holds s and m where they are
            ring[(idx + 3) % hist_len] = float("inf")
            oring.hist[(idx + 3) % hist_len] = np.inf
        if t == 3:   # and once it is overwritten the max of the rest takes over again
            ring[(slots[2] + 3) % hist_len] = 0.0
            oring.hist[(slots[2] + 3) % hist_len] = 0.0
        xb = workloads.delayed_step("act", 40 + t, rows=128, cols=cols)
        x = upload_bf16_bits(xb)
        _, qT, a = mxa.fp8_quantize_delayed(x, ring, idx, "e4m3", "transposed", 448.0, 1.0, amax=True,
                                            tickets=tickets)
        _, wqT, wa = odl.quantize_delayed(workloads.bf16_to_f32(xb), "e4m3", oring, idx, 448.0, 1.0)
        assert_bytes_equal(host(qT), wqT, f"step {t} qT")
        assert host(a)[0] == wa
        assert_ring_state(ring, tickets, oring, f"step {t}")


@pytest.mark.parametrize("dtype,layout,shape", [("f32", "dual", (64, 64)), ("bf16", "transposed", (64, 64)),
                                                ("bf16", "transposed", (160, 200))])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_delayed_margin_and_nonfinite(dtype, layout, shape, fmt):
    fp8_max = 448.0 if fmt == "e4m3" else 57344.0
    ring = mxa.new_ring(4)
    oring = odl.Ring(4)
    x_nan = workloads.random_tensor(shape, 41, "normal") * 50
    x_nan[6, 6] = np.nan                 # ignored by the amax: the fold goes ahead
    x_inf = x_nan.copy()
    x_inf[5, 5] = np.inf                 # an infinite amax: s and m are kept
    x_inf[40, 7] = -np.inf
    # margins 1e30 and 1e-30 make the multiplier huge (every code saturates) and tiny
    steps = [(x_nan, 2.0), (np.zeros_like(x_nan), 0.5), (x_nan, 1e30), (x_nan, 1e-30), (x_inf, 1.0),
             (x_nan, 1.0), (x_inf, 3.0), (x_nan, 1.0)]
    for t, (y, margin) in enumerate(steps):
        x = make_input(y, dtype)
        ys = f32_of_input(x)
        q, qT = mxa.fp8_quantize_delayed(x, ring, t % 4, fmt, layout, fp8_max, margin)
        wq, wqT, _ = odl.quantize_delayed(ys, fmt, oring, t % 4, fp8_max, margin)
        if q is not None:
            assert_bytes_equal(host(q), wq, f"step {t} q")
        assert_bytes_equal(host(qT), wqT, f"step {t} qT")
        assert_ring_state(ring, None, oring, f"step {t}")


# ---------------------------------------------------------------- full-size workloads (complete)

def test_activation_dual_full_size():
    """BF16 8192 x 4096, E4M3, round-up rule, dual + amax, in the bench's launch
    configuration: every row code and scale and every transposed column code and
    scale against the oracle."""
    xb = workloads.activation_bf16()
    x = upload_bf16_bits(xb)
    qr, sr, qc, sc, a = mxa.mx_quantize_dual(x, "e4m3", "ceil", amax=True)
    xs = workloads.bf16_to_f32(xb)
    wqr, wsr, wqc, wsc = omx.quantize_dual(xs, "e4m3", "ceil")
    assert_bytes_equal(host(sr), wsr, "row scales")
    assert_bytes_equal(host(qr), wqr, "row codes")
    assert_bytes_equal(host(sc), wsc, "col scales")
    assert_bytes_equal(host(qc), wqc, "col codes")
    assert host(a)[0] == omx.tensor_amax(xs)
    # zero blocks of the recipe come out as scale code 0
    assert (wsr == 0).sum() >= 16 and (wsc == 0).sum() >= 16


@pytest.mark.parametrize("fmt,rule,shape", [("e5m2", "floor", (8192, 4096)), ("e2m1", "ceil", (8192, 4096)),
                                             ("e4m3", "ceil", (4128, 4128)), ("e4m3", "floor", (2080, 8224))])
def test_dual_multi_tile_workgroups(fmt, rule, shape):
    """Inputs with more 128 x 128 tiles than the launch's two workgroups per CU, so
    each workgroup walks several tiles (FP8: loading the next tile's input while it
    converts the current one), with ragged last tile rows and columns in the
    smaller shapes: every code, scale and the amax against the oracle."""
    R, C = shape
    x32 = workloads.random_tensor(shape, R + C, "wide")
    x = upload_bf16_bits(workloads.to_bf16_bits(x32.astype(np.float64)))
    xs = f32_of_input(x)
    qr, sr, qc, sc, a = mxa.mx_quantize_dual(x, fmt, rule, amax=True)
    wqr, wsr, wqc, wsc = omx.quantize_dual(xs, fmt, rule)
    assert_bytes_equal(host(sr), wsr, "row scales")
    assert_bytes_equal(host(qr), wqr, "row codes")
    assert_bytes_equal(host(sc), wsc, "col scales")
    assert_bytes_equal(host(qc), wqc, "col codes")
    assert host(a)[0] == omx.tensor_amax(xs)


@pytest.mark.parametrize("stream", ["act", "grad"])
def test_delayed_full_size_32_steps(stream):
    """BF16 8192 x 4096 delayed scaling, 32 steps on one ring of 16 in the bench's
    launch configuration (ticket scratch): after every step the whole ring, the
    ticket scratch and the amax exact; every transposed code exact at steps 0,
    15 and 31."""
    fmt = workloads.DELAYED_FMT[stream]
    fp8_max = workloads.DELAYED_FP8_MAX[stream]
    ring = mxa.new_ring(16)
    tickets = mxa.new_tickets()
    oring = odl.Ring(16)
    for t in range(32):
        xb = workloads.delayed_step(stream, t)
        x = upload_bf16_bits(xb)
        m_before = np.float32(oring.m)
        _, qT, a = mxa.fp8_quantize_delayed(x, ring, t % 16, fmt, "transposed", fp8_max, 1.0, amax=True,
                                            tickets=tickets)
        xs = workloads.bf16_to_f32(xb)
        amax = omx.tensor_amax(xs)
        oring.fold(amax, t % 16, fp8_max, 1.0)
        assert host(a)[0] == amax
        assert_ring_state(ring, tickets, oring, f"{stream} step {t}")
        if t in (0, 15, 31):
            want = odl.cast_per_tensor(xs, m_before, fmt)
            assert_bytes_equal(host(qT), np.ascontiguousarray(want.T), f"{stream} step {t} qT")


def test_delayed_full_size_without_scratch():
    """The same workload with the page's plain ring (no ticket scratch): three
    steps, ring and amax exact, every code exact at the last step."""
    ring = mxa.new_ring(16)
    oring = odl.Ring(16)
    for t in range(3):
        xb = workloads.delayed_step("act", t)
        m_before = np.float32(oring.m)
        _, qT, a = mxa.fp8_quantize_delayed(upload_bf16_bits(xb), ring, t, "e4m3", "transposed", 448.0, 1.0,
                                            amax=True)
        xs = workloads.bf16_to_f32(xb)
        amax = omx.tensor_amax(xs)
        oring.fold(amax, t, 448.0, 1.0)
        assert host(a)[0] == amax
        assert_ring_state(ring, None, oring, f"step {t}")
    want = odl.cast_per_tensor(xs, m_before, "e4m3")
    assert_bytes_equal(host(qT), np.ascontiguousarray(want.T), "step 2 qT")
