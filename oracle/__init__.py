"""CPU oracle for OCP microscaling (MX) block quantization and its consumers.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code, table or constant generator with
the HIP library under ``mx_block_scaled_quantize_amd/``; the only thing both
sides consume is the seeded synthetic inputs from ``workloads/``.

The oracle is plain, slow and exact:

* ``formats``  - element codecs (FP8 E4M3, FP8 E5M2, FP4 E2M1) and the E8M0
  scale, written from the format definitions as exact dyadic arithmetic on
  integers / float64 (every value involved is exactly representable there).
* ``mx``       - MX block quantization (block amax, shared power-of-two scale by
  the OCP round-down rule or the overflow-safe round-up rule, RNE + saturating
  element cast), row-wise / column-wise / dual, dequantization, per-tensor amax.
* ``delayed``  - per-tensor FP8 quantization with an amax-history ring folded
  into the next scale.
* ``hadamard`` - fixed-sign 32-point Walsh-Hadamard preconditioning.
* ``gemm``     - block-scaled GEMM reference: float64 product of the
  dequantized operands (the fake-quant emulation the MX studies use), and the
  per-tensor FP8 GEMM (op(a) @ op(b) * scale + bias, batch-broadcast).
* ``sr``       - stochastic-rounding MXFP4 with caller-supplied random words.

Sources (cited by page and section, see each function):
  [UE8M0]  "EU8M0 FP8 ... domestic compute chips" article (ag-981.com, news 240):
           the MX format definition, the E8M0 / E4M3 / E5M2 / E2M1 glossary,
           the scale-rounding discussion (OCP round-down vs. NVIDIA round-up),
           saturation, dual copies.
  [FP8PY]  AstrAI ``astrai/extension/ops/fp8.py`` page (commit 432dfec): the
           per-tensor quantize / quantize_dual / ring-state delayed scaling
           interface and its commit message.
  [FAF]    "Format-aware fusion" FP4 article (theaicronicle.com): MXFP4 with a
           fixed-sign 32-point Hadamard transform.

Parity status: every public function is pinned by the CPU tests in
``tests/test_oracle_*.py`` (closed forms, exhaustive enumeration, brute force,
independent library routines, invariants).  The pages print no worked numeric
example, so no function is pinned to printed input/output pairs; the printed
constants (E4M3 max 448, min 2^-9, E8M0 range, k = 32, 8 scale bits per block)
are pinned in ``tests/golden/``.  The packed storage of the sub-byte formats
(E2M1 two per byte, element 2j in the low nibble; FP6 as a little-endian bit
stream) is a reading, since the pages define no packing; it is pinned by
hand-written literal bytes, and a planted high-nibble-first (FP4) or
big-endian (FP6) packer must fail those pins.
"""

from . import formats, mx, delayed, hadamard, gemm, sr  # noqa: F401
