"""Helpers for the GPU parity tests: uploads, downloads and mismatch reports."""

import numpy as np
import pytest
import torch


def dev():
    return torch.device("cuda", 0)


def upload_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev())


def upload_bf16_bits(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(dev())


def upload_f16_from_f32(x: np.ndarray) -> torch.Tensor:
    """FP32 values rounded to FP16 (torch RNE) on the host, then uploaded."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float16).to(dev())


def upload_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(dev())


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def f32_of_input(t: torch.Tensor) -> np.ndarray:
    """The exact FP32 values of a device input tensor (for the oracle)."""
    return t.float().cpu().numpy()


def assert_bytes_equal(got: np.ndarray, want: np.ndarray, what: str):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, f"{what}: shape {got.shape} != {want.shape}"
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        first = [(tuple(int(i) for i in b), int(got[tuple(b)]), int(want[tuple(b)])) for b in bad[:8]]
        raise AssertionError(f"{what}: {len(bad)} of {got.size} differ; first (index, gpu, oracle): {first}")


def assert_float_equal(got: np.ndarray, want: np.ndarray, what: str):
    """Bit-exact except that any NaN matches any NaN."""
    got = np.asarray(got, dtype=np.float32)
    want = np.asarray(want, dtype=np.float32)
    assert got.shape == want.shape, f"{what}: shape {got.shape} != {want.shape}"
    gn, wn = np.isnan(got), np.isnan(want)
    same = (got.view(np.uint32) == want.view(np.uint32)) | (gn & wn)
    if not same.all():
        bad = np.argwhere(~same)
        first = [(tuple(int(i) for i in b), float(got[tuple(b)]), float(want[tuple(b)])) for b in bad[:8]]
        raise AssertionError(f"{what}: {len(bad)} of {got.size} differ; first (index, gpu, oracle): {first}")


def import_library():
    """The package under test.  Where a GPU is present a missing or unloadable
    libmx.so is an error, so the GPU tests cannot pass by being skipped; without
    a GPU (where they are deselected anyway) the module is skipped."""
    if torch.cuda.is_available():
        import mx_block_scaled_quantize_amd as mxa
        return mxa
    return pytest.importorskip("mx_block_scaled_quantize_amd")


def tile_strata(n: int, tile: int, seed: int) -> np.ndarray:
    """One random index inside every `tile`-long block of range(n) (the last block
    may be ragged): a sample that touches every tile a launch of that tile size
    covers along this axis."""
    g = np.random.default_rng(seed)
    return np.array([s + int(g.integers(0, min(tile, n - s))) for s in range(0, n, tile)], dtype=np.int64)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def abs_product(qa, sa, fa, qb, sb, fb, alpha=1.0, rows=None, cols=None) -> np.ndarray:
    """|alpha| * |deq(A)| |deq(B)|^T on the selected rows / columns: the magnitude
    the matrix unit's accumulation error is measured against."""
    from oracle import mx as omx
    A = omx.dequantize_exact(qa if rows is None else np.asarray(qa)[rows],
                             sa if rows is None else np.asarray(sa)[rows], fa)
    B = omx.dequantize_exact(qb if cols is None else np.asarray(qb)[cols],
                             sb if cols is None else np.asarray(sb)[cols], fb)
    return abs(alpha) * (np.abs(A) @ np.abs(B).T)


def check_bf16_lines(got_bits: np.ndarray, ref: np.ndarray, mag: np.ndarray, tol: float, what: str, seg: int = 256):
    """BF16 GEMM output lines (rows of `got_bits`) against the float64 reference:
    * the relative Frobenius error of all of them against the reference rounded
      once to BF16 is within `tol` (the graded bound);
    * every element is within one BF16 rounding (2^-8 relative) plus
      2^-10 * sum_k |a_k b_k| (`mag`, the matrix unit's fixed-point accumulation
      window) of the reference -- a wrong code, scale, lane or tile pairing misses
      this by orders of magnitude.  A failure names the line and the `seg`-long
      segment (output tile) it falls in."""
    from oracle import gemm as og
    got = bf16_bits_to_f64(got_bits)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} != {ref.shape}"
    err = og.rel_frobenius(got, bf16_bits_to_f64(og.f64_to_bf16_bits(ref)))
    assert err <= tol, f"{what}: relative Frobenius error {err}"
    bad = np.abs(got - ref) > 2.0 ** -8 * np.abs(ref) + 2.0 ** -10 * mag + 1e-30
    if bad.any():
        i, j = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} outputs outside the bound; first at line {i}, element {j} "
                             f"(tile segment {j // seg}): got {got[i, j]}, reference {ref[i, j]}")
    return err
