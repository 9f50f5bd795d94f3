"""Python binding of libmx: OCP MX block quantization and block-scaled GEMM on
AMD Instinct MI355X (gfx950).

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of ``libmx.so`` (built from ``csrc/`` by ``_build.py``); PyTorch only
provides device memory and the current HIP stream.  There is no CPU fallback:
importing this module without the built library, or passing host tensors,
raises.

The functions carry the names of the C entry points declared in
``include/mx.h`` and return freshly allocated output tensors:

    mx_quantize(x, fmt, rule, orient, hadamard_mask=None, amax=False, scale_layout="row")
    mx_quantize_dual(x, fmt, rule, amax=False, scale_layout="row")
    fp8_quantize_delayed(x, ring, hist_idx, fmt, layout, fp8_max, margin, amax=False, tickets=None)
    mx_dequantize(q, scales, rows, cols, fmt, orient, out_dtype, scale_layout="row")
    mx_gemm(a, sa, b, sb, fmt_a, fmt_b, alpha, out_dtype, scale_layout="row")
    mx_quantize_sr(x, rand, rule, amax=False)
    mm_fp8(a, b, scale, trans_a, trans_b, bias, fmt)
    mx_gemm_requant(a, sa, b, sb, fmt_a, fmt_b, alpha, fmt_c, rule_c, amax=False, scale_layout="row")

scale_layout "row" stores E8M0 scales row-major [lines][K/32]; "gemm" stores them
in the GEMM layout [K/512][lines][16] (returned as a 3-D tensor of that shape).
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmx.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python -c 'import __graft_entry__ as g; g.build()' or python mx_block_scaled_quantize_amd/_build.py)")

# torch is imported first so that its HIP runtime is the one libmx binds to
lib = ctypes.CDLL(LIB_PATH)

# ---------------------------------------------------------------- enums (include/mx.h)
FMT = {"e4m3": 0, "e5m2": 1, "e2m1": 2, "e2m3": 3, "e3m2": 4}
DTYPE = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}
RULE = {"floor": 0, "ceil": 1}
ORIENT = {"row": 0, "col": 1}
SCALE_LAYOUT = {"row": 0, "gemm": 1}
LAYOUT = {"row": 0, "transposed": 1, "dual": 2}
STATUS = {0: "MX_OK", 1: "MX_ERR_NULL", 2: "MX_ERR_SHAPE", 3: "MX_ERR_ALIGN", 4: "MX_ERR_UNSUPPORTED",
          5: "MX_ERR_LAUNCH", 6: "MX_ERR_ARG"}
DEFAULT_FP8_MAX = {"e4m3": 448.0, "e5m2": 57344.0}
TICKET_WORDS = 4096             # MX_TICKET_WORDS


def ring_words(hist_len: int) -> int:
    """MX_RING_WORDS(hist_len): [hist | s | m | amax | ticket]."""
    return hist_len + 4

_p, _i64, _i32, _u32, _f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint32, ctypes.c_float
lib.mx_quantize.argtypes = [_p, _i32, _i64, _i64, _i32, _i32, _i32, _i32, _i32, _u32, _p, _p, _i32, _p, _p]
lib.mx_quantize_dual.argtypes = [_p, _i32, _i64, _i64, _i32, _i32, _i32, _p, _p, _p, _p, _i32, _p, _p]
lib.fp8_quantize_delayed.argtypes = [_p, _i32, _i64, _i64, _i32, _i32, _p, _p, _p, _i32, _i32, _f32, _f32, _p, _p, _p]
lib.mx_dequantize.argtypes = [_p, _p, _i64, _i64, _i32, _i32, _i32, _i32, _p, _i32, _p]
lib.mx_gemm.argtypes = [_p, _p, _i32, _p, _p, _i32, _i32, _i64, _i64, _i64, _f32, _p, _i32, _i64, _p]
lib.mx_quantize_sr.argtypes = [_p, _i32, _i64, _i64, _i32, _i32, _i32, _p, _p, _p, _p, _p]
lib.mm_fp8.argtypes = [_p, _p, _i32, _i64, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _p, _p, _p, _p]
lib.fp8_quantize_delayed_static.argtypes = [_p, _i32, _i64, _i64, _i32, _i32, _p, _p, _p, _i32, _i32, _f32, _f32, _p,
                                            _p]
lib.mx_gemm_requant.argtypes = [_p, _p, _i32, _p, _p, _i32, _i32, _i64, _i64, _i64, _f32, _i32, _i32, _p, _p, _p, _p]
for _f in (lib.mx_quantize, lib.mx_quantize_dual, lib.fp8_quantize_delayed, lib.mx_dequantize, lib.mx_gemm,
           lib.mx_quantize_sr, lib.mm_fp8, lib.mx_gemm_requant, lib.fp8_quantize_delayed_static):
    _f.restype = ctypes.c_int
lib.mx_status_str.argtypes = [ctypes.c_int]
lib.mx_status_str.restype = ctypes.c_char_p
lib.mx_abi_version.restype = ctypes.c_int

ENTRY_POINTS = ("mx_quantize", "mx_quantize_dual", "fp8_quantize_delayed", "mx_dequantize", "mx_gemm",
                "mx_quantize_sr", "mm_fp8", "mx_gemm_requant", "fp8_quantize_delayed_static", "mx_status_str",
                "mx_abi_version")


class MXError(RuntimeError):
    def __init__(self, status):
        self.status = status
        super().__init__(lib.mx_status_str(status).decode())


class MXValueError(MXError, ValueError):
    pass


def check(status: int):
    """Map a status code to an exception (argument errors -> ValueError)."""
    if status == 0:
        return
    if status in (2, 4, 6):
        raise MXValueError(status)
    raise MXError(status)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libmx works on device tensors only")
    return t.data_ptr()


def _stream(t):
    return torch.cuda.current_stream(t.device).cuda_stream


def _lookup(table, key, what):
    try:
        return table[key]
    except KeyError:
        raise ValueError(f"unsupported {what} {key!r} (expected one of {sorted(table, key=str)})") from None


def _amax_buf(amax, device):
    """amax=True -> a fresh zero accumulator; a float32 device tensor -> itself."""
    if isinstance(amax, torch.Tensor):
        if amax.dtype != torch.float32 or amax.numel() < 1:
            raise ValueError("amax accumulator must be a float32 tensor")
        return amax
    return torch.zeros(1, dtype=torch.float32, device=device) if amax else None


def _check_2d(x):
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("expected a contiguous 2-D tensor")


def scale_shape(lines: int, kblocks: int, layout: str):
    """Shape of a scale tensor: [lines][kblocks] row-major, [kblocks/16][lines][16] in the GEMM layout."""
    if _lookup(SCALE_LAYOUT, layout, "scale layout") == 0:
        return (lines, kblocks)
    if kblocks % 16:
        raise ValueError("the GEMM scale layout needs a blocked axis that is a multiple of 512")
    return (kblocks // 16, lines, 16)


def code_cols(n: int, fmt: str) -> int:
    """Bytes per row of n element codes (FP4 packs two per byte, FP6 four per three bytes)."""
    if fmt == "e2m1":
        return n // 2
    if fmt in ("e2m3", "e3m2"):
        return n * 3 // 4
    return n


def mx_quantize(x, fmt="e4m3", rule="ceil", orient="row", hadamard_mask=None, amax=False, scale_layout="row"):
    """MX quantization of a 2-D tensor.  Returns (q, scales) or (q, scales, amax).

    amax=True returns max |x| (NaN ignored) in a fresh 1-element tensor; pass a
    tensor instead to max-accumulate into it (running amax).

    orient='row': q [R][C] (FP4 [R][C/2], FP6 [R][3C/4]), scales [R][C/32].
    orient='col': q [C][R] (FP4 [C][R/2]), scales [C][R/32] (transposed storage).
    """
    _check_2d(x)
    R, C = x.shape
    f = _lookup(FMT, fmt, "format")
    o = _lookup(ORIENT, orient, "orientation")
    qr, qc = (R, C) if orient == "row" else (C, R)
    q = torch.empty((qr, code_cols(qc, fmt)), dtype=torch.uint8, device=x.device)
    s = torch.empty(scale_shape(qr, qc // 32, scale_layout), dtype=torch.uint8, device=x.device)
    a = _amax_buf(amax, x.device)
    check(lib.mx_quantize(_ptr(x), _lookup(DTYPE, x.dtype, "dtype"), R, C, 32, f, _lookup(RULE, rule, "rule"), o,
                          0 if hadamard_mask is None else 1, 0 if hadamard_mask is None else int(hadamard_mask),
                          _ptr(q), _ptr(s), SCALE_LAYOUT[scale_layout], _ptr(a), _stream(x)))
    return (q, s) if a is None else (q, s, a)


def mx_quantize_dual(x, fmt="e4m3", rule="ceil", amax=False, scale_layout="row"):
    """Row-wise and column-wise (transposed) MX copies from one read of x.
    Returns (q_row, s_row, q_colT, s_colT[, amax])."""
    _check_2d(x)
    R, C = x.shape
    f = _lookup(FMT, fmt, "format")
    qr = torch.empty((R, code_cols(C, fmt)), dtype=torch.uint8, device=x.device)
    sr = torch.empty(scale_shape(R, C // 32, scale_layout), dtype=torch.uint8, device=x.device)
    qc = torch.empty((C, code_cols(R, fmt)), dtype=torch.uint8, device=x.device)
    sc = torch.empty(scale_shape(C, R // 32, scale_layout), dtype=torch.uint8, device=x.device)
    a = _amax_buf(amax, x.device)
    check(lib.mx_quantize_dual(_ptr(x), _lookup(DTYPE, x.dtype, "dtype"), R, C, 32, f, _lookup(RULE, rule, "rule"),
                               _ptr(qr), _ptr(sr), _ptr(qc), _ptr(sc), SCALE_LAYOUT[scale_layout], _ptr(a),
                               _stream(x)))
    return (qr, sr, qc, sc) if a is None else (qr, sr, qc, sc, a)


def mx_quantize_sr(x, rand, rule="ceil", amax=False):
    """Row-wise MXFP4 with stochastic rounding driven by rand (uint32 words, one
    per element, same shape as x; any integer tensor of 4-byte elements).
    Returns (q [R][C/2], scales [R][C/32]) or (q, scales, amax)."""
    _check_2d(x)
    R, C = x.shape
    if rand.shape != x.shape or rand.element_size() != 4 or not rand.is_contiguous():
        raise ValueError("rand must be a contiguous tensor of 32-bit words shaped like x")
    q = torch.empty((R, C // 2), dtype=torch.uint8, device=x.device)
    s = torch.empty((R, C // 32), dtype=torch.uint8, device=x.device)
    a = _amax_buf(amax, x.device)
    check(lib.mx_quantize_sr(_ptr(x), _lookup(DTYPE, x.dtype, "dtype"), R, C, 32, FMT["e2m1"],
                             _lookup(RULE, rule, "rule"), _ptr(rand), _ptr(q), _ptr(s), _ptr(a), _stream(x)))
    return (q, s) if a is None else (q, s, a)


def _k_of(a, fmt):
    """Elements per row of a [rows][code bytes] operand: E2M1 packs 2 per byte, FP6 4 per 3 bytes."""
    if fmt == "e2m1":
        return a.shape[1] * 2
    if fmt in ("e2m3", "e3m2"):
        return a.shape[1] * 4 // 3
    return a.shape[1]


def mx_gemm_requant(a, sa, b, sb, fmt_a="e4m3", fmt_b="e4m3", alpha=1.0, fmt_c="e4m3", rule_c="ceil", amax=False,
                    scale_layout="row"):
    """C32 = fl32(alpha * deq(A) deq(B)^T), re-quantized row-wise to MX in the GEMM
    epilogue.  Returns (q [M][N] (E2M1: [M][N/2]), scales [M][N/32]) or (q, scales, amax)."""
    M = a.shape[0]
    N = b.shape[0]
    K = _k_of(a, fmt_a)
    fc = _lookup(FMT, fmt_c, "format")
    q = torch.empty((M, N // 2 if fmt_c == "e2m1" else N), dtype=torch.uint8, device=a.device)
    s = torch.empty((M, N // 32), dtype=torch.uint8, device=a.device)
    am = _amax_buf(amax, a.device)
    check(lib.mx_gemm_requant(_ptr(a), _ptr(sa), _lookup(FMT, fmt_a, "format"), _ptr(b), _ptr(sb),
                              _lookup(FMT, fmt_b, "format"), _lookup(SCALE_LAYOUT, scale_layout, "scale layout"),
                              M, N, K, float(alpha), fc, _lookup(RULE, rule_c, "rule"),
                              _ptr(q), _ptr(s), _ptr(am), _stream(a)))
    return (q, s) if am is None else (q, s, am)


def new_ring(hist_len: int, device="cuda") -> torch.Tensor:
    """A fresh delayed-scaling ring: [hist (zeros) | s = 1 | m = 1 | amax = 0 | ticket = 0]."""
    r = torch.zeros(ring_words(hist_len), dtype=torch.float32, device=device)
    r[hist_len] = 1.0
    r[hist_len + 1] = 1.0
    return r


def new_tickets(device="cuda") -> torch.Tensor:
    """Zeroed ticket scratch for fp8_quantize_delayed (MX_TICKET_WORDS uint32 words).
    Every call leaves it zero, so one buffer serves any number of ordered calls."""
    return torch.zeros(TICKET_WORDS, dtype=torch.int32, device=device)


def fp8_quantize_delayed(x, ring, hist_idx, fmt="e4m3", layout="transposed", fp8_max=None, margin=1.0, amax=False,
                         tickets=None):
    """Per-tensor FP8 cast with the ring's multiplier, then the on-device ring
    fold.  ``tickets`` (from new_tickets) spreads the workgroups' ticket over
    many cache lines; None takes it on the ring's own words (same result, slower
    on large tensors).  Returns (q or None, qT or None[, amax])."""
    _check_2d(x)
    R, C = x.shape
    if ring.dtype != torch.float32 or ring.dim() != 1 or not ring.is_contiguous() or ring.numel() < 5:
        raise ValueError("ring must be a contiguous 1-D float32 tensor of hist_len + 4 words")
    if tickets is not None and (tickets.element_size() != 4 or tickets.numel() < TICKET_WORDS
                                or not tickets.is_contiguous()):
        raise ValueError("tickets must be a contiguous tensor of MX_TICKET_WORDS 32-bit words")
    lay = _lookup(LAYOUT, layout, "layout")
    f = _lookup(FMT, fmt, "format")
    if fp8_max is None:
        fp8_max = _lookup(DEFAULT_FP8_MAX, fmt, "FP8 format")
    q = torch.empty((R, C), dtype=torch.uint8, device=x.device) if layout != "transposed" else None
    qT = torch.empty((C, R), dtype=torch.uint8, device=x.device) if layout != "row" else None
    a = torch.empty(1, dtype=torch.float32, device=x.device) if amax else None
    check(lib.fp8_quantize_delayed(_ptr(x), _lookup(DTYPE, x.dtype, "dtype"), R, C, f, lay, _ptr(q), _ptr(qT),
                                   _ptr(ring), ring.numel() - 4, int(hist_idx), float(fp8_max), float(margin),
                                   _ptr(a), _ptr(tickets), _stream(x)))
    return (q, qT, a) if amax else (q, qT)


def mx_dequantize(q, scales, rows, cols, fmt="e4m3", orient="row", out_dtype=torch.float32, scale_layout="row"):
    """Dequantize MX codes back to a [rows][cols] tensor of out_dtype (float32 or bfloat16)."""
    out = torch.empty((rows, cols), dtype=out_dtype, device=q.device)
    check(lib.mx_dequantize(_ptr(q), _ptr(scales), rows, cols, 32, _lookup(FMT, fmt, "format"),
                            _lookup(ORIENT, orient, "orientation"), _lookup(SCALE_LAYOUT, scale_layout, "scale layout"),
                            _ptr(out), _lookup(DTYPE, out_dtype, "dtype"),
                            _stream(q)))
    return out


def mx_gemm(a, sa, b, sb, fmt_a="e4m3", fmt_b="e4m3", alpha=1.0, out_dtype=torch.bfloat16, out=None,
            scale_layout="row"):
    """C = alpha * deq(A) deq(B)^T with A [M][K], B [N][K] codes (K-contiguous)."""
    M = a.shape[0]
    N = b.shape[0]
    K = _k_of(a, fmt_a)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    check(lib.mx_gemm(_ptr(a), _ptr(sa), _lookup(FMT, fmt_a, "format"), _ptr(b), _ptr(sb),
                      _lookup(FMT, fmt_b, "format"), _lookup(SCALE_LAYOUT, scale_layout, "scale layout"), M, N, K,
                      float(alpha), _ptr(out),
                      _lookup(DTYPE, out.dtype, "dtype"), out.stride(0), _stream(a)))
    return out


_FP8_DTYPES = {torch.float8_e4m3fn: "e4m3", torch.float8_e5m2: "e5m2"}


def _fp8_operand(x, name):
    """(tensor, batch, rows, cols, transposed_view) of a 2-D / 3-D FP8 operand: its
    last two dimensions must be dense row-major or the transpose of dense row-major."""
    if x.dim() not in (2, 3):
        raise ValueError(f"{name} must be 2-D or 3-D")
    if x.dtype not in _FP8_DTYPES and x.dtype != torch.uint8:
        raise ValueError(f"{name} must hold FP8 codes (float8_e4m3fn, float8_e5m2 or uint8)")
    r, c = x.shape[-2], x.shape[-1]
    sr, sc = x.stride(-2), x.stride(-1)
    if (sc == 1 and sr == c) or r <= 1 and sc == 1:
        tview = False
    elif sr == 1 and sc == r or c <= 1 and sr == 1:
        tview = True
    else:
        raise ValueError(f"{name}: the last two dimensions must be contiguous or a transposed contiguous view")
    batch = x.shape[0] if x.dim() == 3 else 1
    if batch > 1 and x.stride(0) != r * c:
        raise ValueError(f"{name}: batch stride must be rows * cols")
    return batch, r, c, tview


def mm_fp8(a, b, scale, trans_a=False, trans_b=False, bias=None, fmt=None):
    """Pre-quantized FP8 GEMM: op(a) @ op(b) * scale (+ bias), BF16 out.

    a, b: FP8 codes of one format (torch float8 tensors, or uint8 with ``fmt``),
    2-D or 3-D (batch broadcast as in matmul); a transposed view of a contiguous
    tensor is taken as stored, with the transpose folded into the layout.
    scale: a float32 device tensor with one element (the combined dequantization
    scale).  bias: BF16 [N] or None."""
    fa = _FP8_DTYPES.get(a.dtype)
    fb = _FP8_DTYPES.get(b.dtype)
    if fa and fb and fa != fb:
        raise ValueError("a and b must have the same FP8 format")
    f = fa or fb or fmt or "e4m3"
    if fmt is not None and fmt != f:
        raise ValueError("fmt does not match the operand dtype")
    ba, ra, ca, tva = _fp8_operand(a, "a")
    bb, rb, cb, tvb = _fp8_operand(b, "b")
    ka = bool(trans_a) != tva        # stored [K][M]
    kb = bool(trans_b) != tvb        # stored [N][K]
    M, K = (ca, ra) if trans_a else (ra, ca)
    K2, N = (cb, rb) if trans_b else (rb, cb)
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if ba != bb and ba != 1 and bb != 1:
        raise ValueError(f"batch dimensions {ba} and {bb} do not broadcast")
    batch = max(ba, bb)
    if not isinstance(scale, torch.Tensor):
        raise ValueError("scale must be a float32 device tensor with one element")
    if scale.dtype != torch.float32 or scale.numel() != 1:
        raise ValueError("scale must be a float32 device tensor with one element")
    if bias is not None and (bias.dtype != torch.bfloat16 or bias.dim() != 1 or bias.numel() != N
                             or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous BF16 vector of length N")
    shape = (batch, M, N) if (a.dim() == 3 or b.dim() == 3) else (M, N)
    out = torch.empty(shape, dtype=torch.bfloat16, device=a.device)
    check(lib.mm_fp8(_ptr(a), _ptr(b), FMT[f], batch, M, N, K, int(ba > 1), int(bb > 1), int(ka), int(kb),
                     _ptr(scale), _ptr(bias), _ptr(out), _stream(a)))
    return out
