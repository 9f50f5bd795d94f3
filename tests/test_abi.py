"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, and rejects bad arguments before touching the device."""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mx.h")

mxa = pytest.importorskip("mx_block_scaled_quantize_amd",
                          reason="libmx.so not built (run __graft_entry__.build())")

# These calls pass made-up device addresses that validation must reject before
# any launch; they are kept off machines with a GPU on principle.
import torch  # noqa: E402
if torch.cuda.is_available():
    pytest.skip("argument-validation tests use fake device addresses; CPU only", allow_module_level=True)
lib = mxa.lib

OK, NULL, SHAPE, ALIGN, UNSUP, LAUNCH, ARG = range(7)
FAKE = 0x10000   # an aligned, never-dereferenced address (validation fails first)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:mx_status_t|const char\*|int)\s+(\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(mxa.ENTRY_POINTS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", mxa.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_header_compiles_as_c():
    src = '#include "mx.h"\nint main(void){ return mx_abi_version() > 0 ? 0 : 1; }\n'
    r = subprocess.run(["gcc", "-std=c99", "-fsyntax-only", "-I", os.path.join(ROOT, "include"),
                        "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__", "-x", "c", "-"],
                       input=src, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_version_and_status_strings():
    assert lib.mx_abi_version() == 200
    for code in range(7):
        assert lib.mx_status_str(code).decode().startswith(mxa.STATUS[code])


def q(*a):
    return lib.mx_quantize(*a)


def test_mx_quantize_argument_errors():
    # (x, in, rows, cols, block, fmt, rule, orient, had, mask, q, s, layout, amax, stream)
    base = [FAKE, 1, 64, 64, 32, 0, 1, 0, 0, 0, FAKE, FAKE, 0, None, None]

    def call(**kw):
        args = list(base)
        names = ["x", "in_", "rows", "cols", "block", "fmt", "rule", "orient", "had", "mask", "q", "s", "layout", "amax",
                 "st"]
        for k, v in kw.items():
            args[names.index(k)] = v
        return lib.mx_quantize(*args)
    assert call(block=16) == UNSUP
    assert call(fmt=7) == UNSUP
    assert call(rule=5) == UNSUP
    assert call(in_=9) == UNSUP
    assert call(orient=3) == UNSUP
    assert call(rows=-1) == SHAPE
    assert call(cols=48) == SHAPE                    # row-wise needs cols % 32
    assert call(orient=1, rows=48) == SHAPE          # column-wise needs rows % 32
    assert call(orient=1, rows=64, cols=12) == SHAPE
    assert call(x=None) == NULL
    assert call(q=None) == NULL
    assert call(s=None) == NULL
    assert call(x=FAKE + 8) == ALIGN
    assert call(q=FAKE + 4) == ALIGN
    assert call(rows=0, x=None, q=None, s=None) == OK   # empty, nothing to do
    assert call(layout=2) == UNSUP                      # no such scale layout
    assert call(layout=1) == SHAPE                      # the GEMM layout groups 16 blocks: cols % 512
    assert call(layout=1, orient=1, rows=256, cols=512) == SHAPE   # column-wise: rows % 512
    assert call(layout=1, cols=512, fmt=3) == UNSUP     # not offered for FP6


def test_mx_quantize_dual_argument_errors():
    f = lib.mx_quantize_dual
    assert f(FAKE, 1, 64, 48, 32, 0, 1, FAKE, FAKE, FAKE, FAKE, 0, None, None) == SHAPE
    assert f(FAKE, 1, 48, 64, 32, 0, 1, FAKE, FAKE, FAKE, FAKE, 0, None, None) == SHAPE
    assert f(FAKE, 1, 64, 64, 32, 0, 1, FAKE, FAKE, None, FAKE, 0, None, None) == NULL
    assert f(FAKE, 1, 64, 64, 32, 0, 1, FAKE, FAKE, FAKE + 1, FAKE, 0, None, None) == ALIGN
    assert f(FAKE, 1, 64, 64, 64, 0, 1, FAKE, FAKE, FAKE, FAKE, 0, None, None) == UNSUP
    assert f(None, 1, 0, 64, 32, 0, 1, None, None, None, None, 0, None, None) == OK
    assert f(FAKE, 1, 512, 256, 32, 0, 1, FAKE, FAKE, FAKE, FAKE, 1, None, None) == SHAPE   # GEMM layout: both % 512
    assert f(FAKE, 1, 512, 512, 32, 3, 1, FAKE, FAKE, FAKE, FAKE, 1, None, None) == UNSUP   # not for FP6


def test_fp8_quantize_delayed_argument_errors():
    f = lib.fp8_quantize_delayed
    # (x, in, rows, cols, fmt, layout, q, qT, ring, hist_len, hist_idx, fp8_max, margin, amax, tickets, stream)
    good = [FAKE, 1, 64, 64, 0, 1, FAKE, FAKE, FAKE, 16, 0, 448.0, 1.0, None, FAKE, None]

    def call(i, v):
        a = list(good)
        a[i] = v
        return f(*a)
    assert call(4, 2) == UNSUP          # E2M1 has no per-tensor path
    assert call(4, 3) == UNSUP          # nor E2M3 / E3M2
    assert call(4, 4) == UNSUP
    assert call(5, 9) == UNSUP
    assert call(8, None) == NULL        # ring
    assert call(9, 0) == ARG            # hist_len
    assert call(10, 16) == ARG          # hist_idx out of range
    assert call(10, -1) == ARG
    assert call(11, 0.0) == ARG         # fp8_max
    assert call(12, float("nan")) == ARG
    assert call(12, float("inf")) == ARG
    assert call(2, 40) == SHAPE         # transposed output needs rows % 32
    assert call(3, 12) == SHAPE         # cols % 8
    assert call(7, None) == NULL        # qT for the transposed layout
    assert call(7, FAKE + 2) == ALIGN
    assert call(8, FAKE + 2) == ALIGN   # ring words are 4-byte aligned
    assert call(14, FAKE + 2) == ALIGN  # ticket scratch likewise


def test_fp8_quantize_delayed_static_argument_errors():
    """The allocation-free variant validates exactly as fp8_quantize_delayed does,
    before it looks up its scratch array (so no device is touched here)."""
    f = lib.fp8_quantize_delayed_static
    good = [FAKE, 1, 64, 64, 0, 1, FAKE, FAKE, FAKE, 16, 0, 448.0, 1.0, None, None]

    def call(i, v):
        a = list(good)
        a[i] = v
        return f(*a)
    assert call(4, 2) == UNSUP
    assert call(5, 9) == UNSUP
    assert call(8, None) == NULL
    assert call(8, FAKE + 2) == ALIGN
    assert call(9, 0) == ARG
    assert call(10, 16) == ARG
    assert call(11, 0.0) == ARG
    assert call(2, 40) == SHAPE
    assert call(7, None) == NULL
    assert call(0, FAKE + 8) == ALIGN


def test_ring_layout_is_the_pages():
    """The ring is [hist | scale | legacy | amax | done]: hist_len + 4 words, and the
    ticket scratch a separate optional buffer."""
    text = open(HEADER).read()
    assert re.search(r"#define MX_RING_WORDS\(hist_len\) \(\(hist_len\) \+ 4\)", text)
    assert re.search(r"#define MX_TICKET_WORDS 4096", text)
    assert mxa.ring_words(16) == 20 and mxa.TICKET_WORDS == 4096


def test_mx_dequantize_argument_errors():
    f = lib.mx_dequantize
    assert f(FAKE, FAKE, 64, 48, 32, 0, 0, 0, FAKE, 0, None) == SHAPE
    assert f(FAKE, FAKE, 48, 64, 32, 0, 1, 0, FAKE, 0, None) == SHAPE
    assert f(FAKE, FAKE, 64, 64, 32, 0, 0, 0, FAKE, 2, None) == UNSUP     # F16 output not offered
    assert f(FAKE, FAKE, 64, 64, 32, 0, 0, 0, None, 0, None) == NULL
    assert f(FAKE, FAKE, 64, 64, 32, 0, 0, 0, FAKE + 8, 0, None) == ALIGN
    assert f(None, None, 0, 0, 32, 0, 0, 0, None, 0, None) == OK
    assert f(FAKE, FAKE, 64, 64, 32, 0, 0, 1, FAKE, 0, None) == SHAPE    # GEMM layout needs cols % 512
    assert f(FAKE, FAKE, 64, 512, 32, 0, 0, 3, FAKE, 0, None) == UNSUP


def test_mx_gemm_argument_errors():
    f = lib.mx_gemm
    # (a, sa, fa, b, sb, fb, layout, M, N, K, alpha, c, c_dtype, ldc, stream)
    assert f(FAKE, FAKE, 0, FAKE, FAKE, 2, 0, 64, 64, 64, 1.0, FAKE, 1, 64, None) == UNSUP   # FP8 x FP4
    assert f(FAKE, FAKE, 3, FAKE, FAKE, 0, 0, 64, 64, 64, 1.0, FAKE, 1, 64, None) == UNSUP   # FP6 x FP8
    assert f(FAKE, FAKE, 3, FAKE, FAKE, 4, 0, 64, 64, 96, 1.0, FAKE, 1, 64, None) == SHAPE   # FP6: K % 64
    assert f(FAKE, FAKE, 0, FAKE, FAKE, 0, 0, 64, 64, 48, 1.0, FAKE, 1, 64, None) == SHAPE   # K % 32
    assert f(FAKE, FAKE, 0, FAKE, FAKE, 0, 0, 64, 64, 64, 1.0, FAKE, 1, 60, None) == SHAPE   # ldc < N
    assert f(FAKE, FAKE, 0, FAKE, FAKE, 0, 0, 64, 64, 64, 1.0, FAKE, 2, 64, None) == UNSUP   # F16 out
    assert f(None, FAKE, 0, FAKE, FAKE, 0, 0, 64, 64, 64, 1.0, FAKE, 1, 64, None) == NULL
    assert f(FAKE, FAKE, 0, FAKE, FAKE, 0, 0, 64, 64, 64, 1.0, FAKE + 1, 1, 64, None) == ALIGN   # odd BF16 address
    assert f(FAKE, FAKE, 0, FAKE, FAKE, 0, 0, 64, 64, 64, 1.0, FAKE + 2, 0, 64, None) == ALIGN   # FP32 needs 4 bytes
    assert f(FAKE + 8, FAKE, 0, FAKE, FAKE, 0, 0, 64, 64, 64, 1.0, FAKE, 1, 64, None) == ALIGN
    assert f(None, None, 0, None, None, 0, 0, 0, 64, 64, 1.0, None, 1, 64, None) == OK
    assert f(FAKE, FAKE, 0, FAKE, FAKE, 0, 1, 64, 64, 256, 1.0, FAKE, 1, 64, None) == SHAPE   # GEMM layout: K % 512
    assert f(FAKE, FAKE, 0, FAKE, FAKE, 0, 2, 64, 64, 512, 1.0, FAKE, 1, 64, None) == UNSUP   # no such layout


def test_mm_fp8_argument_errors():
    f = lib.mm_fp8
    # (a, b, fmt, batch, M, N, K, a_batched, b_batched, trans_a, trans_b, scale, bias, c, stream)
    assert f(FAKE, FAKE, 2, 1, 64, 64, 64, 0, 0, 0, 0, FAKE, None, FAKE, None) == UNSUP   # FP4 is not FP8
    assert f(FAKE, FAKE, 3, 1, 64, 64, 64, 0, 0, 0, 0, FAKE, None, FAKE, None) == UNSUP   # nor FP6
    assert f(FAKE, FAKE, 4, 1, 64, 64, 64, 0, 0, 0, 0, FAKE, None, FAKE, None) == UNSUP
    assert f(FAKE, FAKE, 0, 1, 64, 64, 40, 0, 0, 0, 0, FAKE, None, FAKE, None) == SHAPE   # K % 16
    assert f(FAKE, FAKE, 0, 70000, 64, 64, 64, 1, 1, 0, 0, FAKE, None, FAKE, None) == SHAPE   # batch limit
    assert f(FAKE, FAKE, 0, 1, -1, 64, 64, 0, 0, 0, 0, FAKE, None, FAKE, None) == SHAPE
    assert f(FAKE, FAKE, 0, 1, 64, 64, 64, 0, 0, 0, 0, None, None, FAKE, None) == NULL    # scale
    assert f(None, FAKE, 0, 1, 64, 64, 64, 0, 0, 0, 0, FAKE, None, FAKE, None) == NULL
    assert f(FAKE, FAKE, 0, 1, 64, 64, 64, 0, 0, 0, 0, FAKE, None, None, None) == NULL
    assert f(FAKE + 8, FAKE, 0, 1, 64, 64, 64, 0, 0, 0, 0, FAKE, None, FAKE, None) == ALIGN
    assert f(FAKE, FAKE, 1, 1, 64, 64, 64, 0, 0, 0, 0, FAKE, FAKE + 1, FAKE, None) == ALIGN   # odd bias
    assert f(FAKE, FAKE, 1, 1, 64, 64, 64, 0, 0, 0, 0, FAKE, None, FAKE + 1, None) == ALIGN   # odd c
    assert f(None, None, 0, 0, 64, 64, 64, 0, 0, 0, 0, None, None, None, None) == OK      # batch 0
    assert f(None, None, 0, 1, 0, 64, 64, 0, 0, 0, 0, None, None, None, None) == OK       # M 0


def test_mx_gemm_requant_argument_errors():
    f = lib.mx_gemm_requant
    # (a, sa, fa, b, sb, fb, layout, M, N, K, alpha, fc, rc, qc, sc, amax, stream)
    assert f(FAKE, FAKE, 0, FAKE, FAKE, 2, 0, 64, 64, 64, 1.0, 0, 1, FAKE, FAKE, None, None) == UNSUP   # FP8 x FP4
    assert f(FAKE, FAKE, 0, FAKE, FAKE, 0, 0, 64, 64, 64, 1.0, 3, 1, FAKE, FAKE, None, None) == UNSUP   # output format
    assert f(FAKE, FAKE, 0, FAKE, FAKE, 0, 0, 64, 64, 64, 1.0, 4, 1, FAKE, FAKE, None, None) == UNSUP   # E3M2 output
    assert f(FAKE, FAKE, 3, FAKE, FAKE, 3, 0, 64, 64, 64, 1.0, 0, 1, FAKE, FAKE, None, None) == UNSUP   # FP6 operands
    assert f(FAKE, FAKE, 3, FAKE, FAKE, 4, 0, 64, 64, 64, 1.0, 0, 1, FAKE, FAKE, None, None) == UNSUP
    assert f(FAKE, FAKE, 0, FAKE, FAKE, 0, 0, 64, 64, 64, 1.0, 0, 2, FAKE, FAKE, None, None) == UNSUP   # rule
    assert f(FAKE, FAKE, 0, FAKE, FAKE, 0, 0, 64, 48, 64, 1.0, 0, 1, FAKE, FAKE, None, None) == SHAPE   # N % 32
    assert f(FAKE, FAKE, 0, FAKE, FAKE, 0, 0, 64, 64, 48, 1.0, 0, 1, FAKE, FAKE, None, None) == SHAPE   # K % 32
    assert f(FAKE, FAKE, 0, FAKE, FAKE, 0, 0, 64, 64, 64, 1.0, 0, 1, None, FAKE, None, None) == NULL
    assert f(FAKE, FAKE, 0, FAKE, FAKE, 0, 0, 64, 64, 64, 1.0, 0, 1, FAKE, None, None, None) == NULL
    assert f(FAKE, FAKE, 0, FAKE, FAKE, 0, 0, 64, 64, 64, 1.0, 0, 1, FAKE + 8, FAKE, None, None) == ALIGN
    assert f(None, None, 0, None, None, 0, 0, 0, 64, 64, 1.0, 0, 1, None, None, None, None) == OK
    assert f(FAKE, FAKE, 0, FAKE, FAKE, 0, 1, 64, 64, 256, 1.0, 0, 1, FAKE, FAKE, None, None) == SHAPE


def test_mx_quantize_sr_argument_errors():
    f = lib.mx_quantize_sr
    # (x, in, rows, cols, block, fmt, rule, rand, q, scales, amax, stream)
    assert f(FAKE, 1, 64, 64, 32, 0, 1, FAKE, FAKE, FAKE, None, None) == UNSUP     # E4M3: SR is MXFP4 only
    assert f(FAKE, 1, 64, 64, 32, 3, 1, FAKE, FAKE, FAKE, None, None) == UNSUP     # E2M3
    assert f(FAKE, 1, 64, 64, 32, 4, 1, FAKE, FAKE, FAKE, None, None) == UNSUP     # E3M2
    assert f(FAKE, 1, 64, 48, 32, 2, 1, FAKE, FAKE, FAKE, None, None) == SHAPE
    assert f(FAKE, 1, 64, 64, 16, 2, 1, FAKE, FAKE, FAKE, None, None) == UNSUP     # block must be 32
    assert f(FAKE, 1, 64, 64, 32, 2, 1, None, FAKE, FAKE, None, None) == NULL      # no random words
    assert f(FAKE, 1, 64, 64, 32, 2, 1, FAKE + 4, FAKE, FAKE, None, None) == ALIGN
    assert f(None, 1, 0, 64, 32, 2, 1, None, None, None, None, None) == OK


def test_binding_rejects_host_tensors_and_bad_names():
    import torch
    x = torch.zeros(32, 32)
    with pytest.raises(ValueError):
        mxa.mx_quantize(x, "e4m3", "ceil", "row")
    with pytest.raises(ValueError):
        mxa.mx_quantize(x, "e3m4")
    err = mxa.MXValueError(SHAPE)
    assert isinstance(err, ValueError) and "MX_ERR_SHAPE" in str(err)
