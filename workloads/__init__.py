"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests,
``__graft_entry__.smoke()`` and ``bench.py``.

This module holds no quantization arithmetic: it only draws random numbers and
rounds FP32 draws to BF16 storage (through torch's CPU cast, round to nearest
even).  Every generator is a pure function of its arguments.

Shapes follow the transformer layers the pages discuss ([UE8M0] MXFP8 study:
hidden 4096, sequence 8192; [FAF]: Llama-3 8B, MLP width 14336).  All inputs are
synthetic stand-ins; no dataset or checkpoint is involved.

BF16 tensors are returned as numpy uint16 bit patterns; ``bf16_to_f32`` widens
them (exactly) for consumers that want values.
"""

import numpy as np
import torch


def rng(config: int, stream: int = 0) -> np.random.Generator:
    """Generator for (config, stream): SeedSequence(config).spawn(stream + 1)[stream]."""
    return np.random.default_rng(np.random.SeedSequence(config).spawn(stream + 1)[stream])


def to_bf16_bits(x64: np.ndarray) -> np.ndarray:
    """float64 draws -> FP32 (numpy RNE) -> BF16 (torch RNE) bit patterns."""
    f32 = np.ascontiguousarray(np.asarray(x64, dtype=np.float64).astype(np.float32))
    return torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
# Workload recipes
# ----------------------------------------------------------------------------

def wide_range_f32(rows: int = 256, cols: int = 1024, seed: int = 1) -> np.ndarray:
    """FP32 [rows][cols]: N(0,1) * 2^u_row with u_row ~ U(-20, 20); 1% of the
    entries replaced by +-U(1e3, 1e4); then 4 random 32-element row blocks set to +0."""
    g = rng(seed)
    u = g.uniform(-20.0, 20.0, size=(rows, 1))
    x = g.standard_normal((rows, cols)) * np.exp2(u)
    n_out = int(round(0.01 * rows * cols))
    pos = g.choice(rows * cols, size=n_out, replace=False)
    sign = np.where(g.random(n_out) < 0.5, -1.0, 1.0)
    x.reshape(-1)[pos] = sign * g.uniform(1e3, 1e4, size=n_out)
    nblk = cols // 32
    for b in g.choice(rows * nblk, size=min(4, rows * nblk), replace=False):
        r, c = divmod(int(b), nblk)
        x[r, c * 32:(c + 1) * 32] = 0.0
    return x.astype(np.float32)


def activation_bf16(rows: int = 8192, cols: int = 4096, seed: int = 2) -> np.ndarray:
    """BF16 bits [rows][cols]: N(0,1) * 2^u_col with u_col ~ U(-8, 8) per column
    (channel); 0.1% of entries multiplied by 300; zero blocks: 16 aligned 32x32
    tiles, 16 row-only 1x32 and 16 column-only 32x1 blocks (fewer if small)."""
    g = rng(seed)
    u = g.uniform(-8.0, 8.0, size=(1, cols))
    x = g.standard_normal((rows, cols)) * np.exp2(u)
    n_out = int(round(0.001 * rows * cols))
    pos = g.choice(rows * cols, size=n_out, replace=False)
    x.reshape(-1)[pos] *= 300.0
    rb, cb = rows // 32, cols // 32
    k = min(16, rb * cb)
    for t in g.choice(rb * cb, size=k, replace=False):
        r, c = divmod(int(t), cb)
        x[r * 32:(r + 1) * 32, c * 32:(c + 1) * 32] = 0.0
    for t in g.choice(rows * cb, size=k, replace=False):
        r, c = divmod(int(t), cb)
        x[r, c * 32:(c + 1) * 32] = 0.0
    for t in g.choice(rb * cols, size=k, replace=False):
        r, c = divmod(int(t), cols)
        x[r * 32:(r + 1) * 32, c] = 0.0
    return to_bf16_bits(x)


DELAYED_FP8_MAX = {"act": 448.0, "grad": 57344.0}
DELAYED_FMT = {"act": "e4m3", "grad": "e5m2"}


def delayed_step(stream: str, t: int, rows: int = 8192, cols: int = 4096, seed: int = 3) -> np.ndarray:
    """BF16 bits for delayed-scaling step t of stream 'act' or 'grad':
    N(0,1) * 2^(sin(t/4) * 6), a fresh draw per (stream, step)."""
    sidx = {"act": 0, "grad": 1}[stream]
    g = rng(seed, stream=sidx * 64 + t)
    x = g.standard_normal((rows, cols)) * np.exp2(np.sin(t / 4.0) * 6.0)
    return to_bf16_bits(x)


def mlp_operands(M: int = 8192, N: int = 14336, K: int = 4096, seed: int = 4):
    """GEMM operands: activations A = BF16 N(0,1) [M][K], weights W = BF16
    N(0, 0.02) [N][K] (the K-contiguous B^T of an MLP up-projection)."""
    a = to_bf16_bits(rng(seed, 0).standard_normal((M, K)))
    w = to_bf16_bits(rng(seed, 1).standard_normal((N, K)) * 0.02)
    return a, w


def weight_grad_operands(tokens: int = 8192, width: int = 4096, seed: int = 5):
    """Weight-gradient operands: G = BF16 N(0, 1e-3) [tokens][width],
    X = BF16 N(0,1) [tokens][width], and a 32-bit sign mask."""
    g = to_bf16_bits(rng(seed, 0).standard_normal((tokens, width)) * 1e-3)
    x = to_bf16_bits(rng(seed, 1).standard_normal((tokens, width)))
    mask = int(rng(seed, 2).integers(0, 1 << 32, dtype=np.uint64))
    return g, x, mask


# ----------------------------------------------------------------------------
# Edge-case inputs for parity tests
# ----------------------------------------------------------------------------

def all_bf16_blocks(seed: int = 11) -> np.ndarray:
    """Every finite BF16 bit pattern exactly once, in blocks of 32 FP32 values.

    Patterns are shuffled and grouped so that each block's largest magnitude
    (which sets its scale) varies over the whole exponent range; returned as
    FP32 [n_blocks][32].
    """
    g = rng(seed)
    bits = np.arange(1 << 16, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    vals = vals[np.isfinite(vals)]
    # sort by magnitude, then cut into runs so that blocks hold neighbours in
    # exponent (small dynamic range, every exponent acts as a block maximum),
    # and also build blocks of random patterns (large dynamic range)
    order = np.argsort(np.abs(vals), kind="stable")
    near = vals[order]
    near = near[: near.size // 32 * 32].reshape(-1, 32)
    far = g.permutation(vals)
    far = far[: far.size // 32 * 32].reshape(-1, 32)
    return np.concatenate([near, far]).astype(np.float32)


def special_blocks() -> np.ndarray:
    """Hand-picked FP32 blocks: zeros of both signs, FP32 subnormals, the FP32
    extremes, NaN and Inf entries, a single non-zero entry, equal entries."""
    f = np.float32
    rows = []
    rows.append(np.zeros(32, f))
    z = np.zeros(32, f)
    z[1::2] = -0.0
    rows.append(z)
    rows.append((np.arange(1, 33, dtype=np.uint32)).view(np.float32))            # smallest subnormals
    rows.append(-(np.arange(1, 33, dtype=np.uint32) << 18).view(np.float32))    # larger subnormals
    rows.append(np.full(32, np.finfo(f).max, f))
    r = np.full(32, 1.0, f)
    r[3] = -np.finfo(f).max
    rows.append(r)
    r = np.linspace(-3, 3, 32).astype(f)
    r[7] = np.nan
    rows.append(r)
    r = np.linspace(-3, 3, 32).astype(f)
    r[9] = np.inf
    rows.append(r)
    r = np.linspace(-3, 3, 32).astype(f)
    r[0] = -np.inf
    rows.append(r)
    r = np.zeros(32, f)
    r[17] = f(2.0 ** -140)
    rows.append(r)
    r = np.zeros(32, f)
    r[5] = f(-1.0e30)
    rows.append(r)
    rows.append(np.full(32, f(448.0)))
    rows.append(np.full(32, f(449.0)))
    rows.append(np.full(32, f(-57344.0)))
    rows.append(np.full(32, f(6.0)))
    rows.append(np.full(32, f(5.0)))
    rows.append((2.0 ** np.arange(-15, 17)).astype(f))
    rows.append((-(2.0 ** np.arange(-40, -8))).astype(f))
    return np.stack(rows).astype(np.float32)


def random_tensor(shape, seed: int, kind: str = "normal") -> np.ndarray:
    """FP32 test tensor.  kinds: 'normal' N(0,1); 'wide' N(0,1) * 2^U(-30,30)
    per element; 'rows' N(0,1) * 2^U(-20,20) per row with 1% outliers."""
    g = rng(1000 + seed)
    if kind == "normal":
        x = g.standard_normal(shape)
    elif kind == "wide":
        x = g.standard_normal(shape) * np.exp2(g.uniform(-30, 30, size=shape))
    elif kind == "rows":
        x = g.standard_normal(shape) * np.exp2(g.uniform(-20, 20, size=(shape[0], 1)))
        flat = x.reshape(-1)
        n = max(1, flat.size // 100)
        pos = g.choice(flat.size, size=n, replace=False)
        flat[pos] = np.where(g.random(n) < 0.5, -1, 1) * g.uniform(1e3, 1e4, size=n)
    else:
        raise ValueError(kind)
    return x.astype(np.float32)


def random_words(shape, seed: int) -> np.ndarray:
    """uint32 random words (uniform over [0, 2^32)), the stochastic-rounding input."""
    return rng(2000 + seed).integers(0, 2**32, size=shape, dtype=np.uint64).astype(np.uint32)
