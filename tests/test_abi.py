"""The C-ABI library loads and exports every entry point that include/moe.h
declares (no compute: this runs without a GPU)."""

import ctypes
import os
import re

import pytest

from combine_top_route_moe_amd import _lib
from combine_top_route_moe_amd._build import LIB

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "moe.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_path():
    names = _declared()
    for fn in ("moe_route", "moe_permute", "moe_grouped_ffn", "moe_fake_quant_rows", "moe_combine"):
        assert fn in names


def test_library_exports_every_declared_symbol():
    if not os.path.exists(LIB):
        pytest.fail("libmoe.so is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB)
    for name in _declared():
        assert hasattr(lib, name), name
    assert set(_declared()) == set(_lib.SIGNATURES), "binding signatures out of sync with moe.h"


def test_host_only_entry_points():
    lib = _lib.load()
    assert lib.moe_status_string(0) == b"ok"
    assert b"gfx950" in lib.moe_status_string(-5)
    assert lib.moe_permute_capacity(512, 8, 64, 0) == 4096
    assert lib.moe_permute_capacity(16384, 8, 128, 1) == 2 * 16384 * 8
    assert lib.moe_permute_capacity(3, 1, 1, 1) == 4
    assert lib.moe_permute_workspace_bytes(512, 8, 64, 0) > 0
    assert lib.moe_grouped_ffn_workspace_bytes(4096, 64, 2048, 1024) >= 4096 * 1024 * 2
    # argument errors are reported synchronously, before any device work
    assert lib.moe_route(None, None, 4, 8, 9, 1, None, None, None) == -1        # K > E
    assert lib.moe_route(None, None, 4, 2048, 2, 1, None, None, None) == -2     # E > 1024
    assert lib.moe_grouped_ffn(None, None, None, 4, 100, 128, None, None, None, None, 16, 3,
                               None, 0, None, None) == -2                       # H % 128
    # FP8 weights: a selected stage needs its codes and its scales
    assert lib.moe_grouped_ffn_fp8(None, None, None, 4, 256, 128, None, None, None, None, None,
                                   None, 16, 3, None, 0, None, None) == -1
    assert lib.moe_grouped_ffn_fp8(None, None, None, 4, 256, 128, None, None, None, None, None,
                                   None, 16, 3 | 4, None, 0, None, None) == -1   # stage bits only
    assert lib.moe_pack_ffn_weights_fp8(None, None, 4, 256, 100, None, None, None, None, 0,
                                        None) == -2                              # I % 128
    assert lib.moe_pack_ffn_weights_fp8(None, None, 4, 256, 128, None, None, None, None, 2,
                                        None) == -1                              # unknown flag
    assert lib.moe_quant_rows_fp8(None, 0, 256, None, None, None, 0, None) == 0  # no rows
    assert lib.moe_quant_rows_fp8(None, 4, 256, None, None, None, 2, None) == -1  # stride < rows
    assert lib.moe_grouped_ffn_w8a8(None, None, 0, None, 1, None, None, 4, 256, 128, None, None,
                                    None, None, None, None, 16, 3, None, 0, None, None) == -1
    assert lib.moe_combine(None, 0, None, None, 0, 1, 128, None, None, None, None) == 0  # T = 0
    assert lib.moe_copy_bytes(None, None, 15, None) == -1
    assert lib.moe_read_bytes(None, 15, None, None) == -1        # not a multiple of 16
    assert lib.moe_read_bytes(None, 0, None, None) == 0          # nothing to read
    assert lib.moe_read_bytes(None, 16, None, None) == -1        # null pointers
