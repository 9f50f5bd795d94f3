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
