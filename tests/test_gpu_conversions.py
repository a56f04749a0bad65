"""The instruction-level conversions of the dispatch kernels (csrc/dc_convert.h) against what
they replace, over every binary32 input: the fp8 (E4M3, E5M2) and fp4 (E2M1) element codes of
gfx950's conversion instructions against the bit-level encoders of csrc/dc_device.h (every value
but the NaNs), the static int8 codes by magic-number addition against the rounding and clamping
of int8_code (every value), and the short division of the per-128-group scales against the correctly rounded
quotient (every b with the sign bit clear).  The parity tests compare the kernels with the oracle
on realistic inputs; this check covers the inputs they do not reach."""
import ctypes
import os

import pytest

from combine_quant_amd import build as B

NAMES = ("E4M3 codes", "E5M2 codes", "E2M1 codes", "448 / b", "57344 / b", "1 / b",
         "static int8 codes")


def _lib():
    if not os.path.exists(B.SELFCHECK_LIB):
        raise OSError(f"{B.SELFCHECK_LIB} is missing: build it with combine_quant_amd.build.build()")
    lib = ctypes.CDLL(B.SELFCHECK_LIB)
    lib.moe_dc_selfcheck_conversions.argtypes = [ctypes.POINTER(ctypes.c_ulonglong)]
    lib.moe_dc_selfcheck_conversions.restype = ctypes.c_int
    return lib


def test_selfcheck_library_exports_its_entry_point():
    assert hasattr(_lib(), "moe_dc_selfcheck_conversions")


@pytest.mark.gpu
def test_conversions_equal_the_bit_level_results_everywhere():
    import torch
    torch.cuda.init()
    counts = (ctypes.c_ulonglong * len(NAMES))()
    print("[conversions] exhaustive check of codes and divisions", flush=True)
    rc = _lib().moe_dc_selfcheck_conversions(counts)
    assert rc == 0, f"hipError {rc}"
    assert list(counts) == [0] * len(NAMES), dict(zip(NAMES, list(counts)))
