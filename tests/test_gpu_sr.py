"""GPU parity of the stochastic-rounding MXFP4 quantizer (row-wise) against the
CPU oracle: bit-exact packed codes, scales and amax on the same seeded inputs
and the same seeded random words."""

import numpy as np
import pytest
import torch

import workloads
from oracle import mx as omx
from oracle import sr as osr
from tests.gpu_util import (assert_bytes_equal, f32_of_input, host, import_library, upload_bf16_bits,
                            upload_f16_from_f32, upload_f32)

pytestmark = pytest.mark.gpu

mxa = import_library()

RULES = ["floor", "ceil"]


def make_input(x32: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "f32":
        return upload_f32(x32)
    if dtype == "bf16":
        return upload_bf16_bits(workloads.to_bf16_bits(x32.astype(np.float64)))
    return upload_f16_from_f32(x32)


def upload_words(r: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(r, dtype=np.uint32).view(np.int32)).cuda()


def check_sr(x32, r, dtype, rule, what):
    x = make_input(x32, dtype)
    xs = f32_of_input(x)
    q, s, a = mxa.mx_quantize_sr(x, upload_words(r), rule, amax=True)
    wq, ws = osr.quantize_rowwise_sr(xs, r, rule)
    assert_bytes_equal(host(s), ws, f"{what} scales")
    assert_bytes_equal(host(q), wq, f"{what} codes")
    assert host(a)[0] == omx.tensor_amax(xs)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("rule", RULES)
def test_sr_parity(dtype, rule):
    # several 1024-chunk workgroups plus a ragged last one (rows * cols / 8 not a multiple of 1024)
    for shape, seed, kind in (((96, 256), 41, "rows"), ((64, 320), 42, "wide"), ((200, 96), 43, "normal")):
        x32 = workloads.random_tensor(shape, seed, kind)
        check_sr(x32, workloads.random_words(shape, seed), dtype, rule, f"{shape} {kind}")


@pytest.mark.parametrize("rule", RULES)
def test_sr_extreme_words(rule):
    """Words 0 and 2^32 - 1 take the grid ceiling and floor; 2^31 is the midpoint."""
    x32 = workloads.random_tensor((64, 256), 44, "normal")
    for w in (0, 1, 2**31, 2**32 - 1):
        check_sr(x32, np.full(x32.shape, w, np.uint32), "f32", rule, f"word {w:#x}")


@pytest.mark.parametrize("rule", RULES)
def test_sr_every_bf16_pattern_and_specials(rule):
    blocks = np.concatenate([workloads.all_bf16_blocks(), workloads.special_blocks()])
    x32 = blocks.reshape(-1, 32)
    r = workloads.random_words(x32.shape, 45)
    check_sr(x32, r, "f32", rule, "all bf16 + specials")
    x32 = np.zeros((64, 64), np.float32)
    x32[:18, :32] = workloads.special_blocks()
    x32[40, :] = np.nan
    x32[:, 60] = -np.inf
    check_sr(x32, workloads.random_words(x32.shape, 46), "f32", rule, "special rows")


def test_sr_threshold_boundaries():
    """Words at T - 1 and T for every off-grid value with a fraction of k/256:
    the decision flips exactly at the oracle's threshold."""
    k = np.arange(1, 256)
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    y = np.concatenate([mags[i] + (mags[i + 1] - mags[i]) * k / 256.0 for i in range(7)])
    x = np.concatenate([y, -y, [6.0] * 11]).astype(np.float32)      # every block holds 6: scale 2^0
    x = x[: (x.size // 32) * 32].reshape(-1, 32)
    x[:, 0] = 6.0
    _, t = osr.sr_threshold(np.abs(x.astype(np.float64)))
    t = t.astype(np.int64)
    for off in (-1, 0):
        r = np.clip(t + off, 0, 2**32 - 1).astype(np.uint32)
        check_sr(x, r, "f32", "ceil", f"threshold{off:+d}")


def test_sr_cfg_size_full():
    """The bench workload (BF16 8192 x 4096 gradient, one word per element): every
    code and scale against the oracle."""
    x_bits = workloads.activation_bf16(8192, 4096)
    r = workloads.random_words((8192, 4096), 47)
    q, s = mxa.mx_quantize_sr(upload_bf16_bits(x_bits), upload_words(r), "ceil")
    wq, ws = osr.quantize_rowwise_sr(workloads.bf16_to_f32(x_bits), r, "ceil")
    assert_bytes_equal(host(s), ws, "scales")
    assert_bytes_equal(host(q), wq, "codes")


def test_sr_empty_and_errors():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    q, s, a = mxa.mx_quantize_sr(x, torch.empty((0, 64), dtype=torch.int32, device="cuda"), amax=True)
    assert q.numel() == 0 and host(a)[0] == 0.0
    x = torch.zeros((64, 48), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        mxa.mx_quantize_sr(x, torch.zeros((64, 48), dtype=torch.int32, device="cuda"))
    x = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        mxa.mx_quantize_sr(x, torch.zeros((64, 32), dtype=torch.int32, device="cuda"))
