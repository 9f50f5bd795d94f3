"""The native library is built and loads.  Without it the library tests would
be skipped, not failed, so its absence fails here."""

import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_libmx_is_built_and_loads():
    path = os.path.join(ROOT, "mx_block_scaled_quantize_amd", "libmx.so")
    assert os.path.exists(path), "libmx.so is not built: run __graft_entry__.build()"
    import mx_block_scaled_quantize_amd as mxa
    assert mxa.lib.mx_abi_version() >= 100
