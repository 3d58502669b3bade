"""The bandwidth probe library on the CPU: it loads, exports what its header
declares, and rejects bad arguments with the documented status before any
HIP call (only rejected calls are made, so nothing is launched)."""
import ctypes
import os
import re

import pytest

from combine_moe_finalize_amd._paths import CSRC, PROBE_LIB_PATH

GRAIN = 16384
A, B = 0x10_0000_0000, 0x20_0000_0000      # fake device addresses, 256-byte aligned


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(PROBE_LIB_PATH):
        pytest.fail(f"{PROBE_LIB_PATH} is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(PROBE_LIB_PATH)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    L.moef_probe_read.argtypes = [vp, i64, vp, vp]
    L.moef_probe_copy.argtypes = [vp, vp, i64, vp]
    return L


def test_exports_the_header(lib):
    text = open(os.path.join(CSRC, "bandwidth_probes.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"^int\s+(\w+)\s*\(", text, flags=re.M))
    assert names == {"moef_probe_read", "moef_probe_copy", "moef_probe_empty", "moef_probe_mark"}
    for n in names:
        assert hasattr(lib, n)
    assert re.search(r"#define MOEF_PROBE_GRAIN 16384", text)


def test_rejections(lib):
    r, c = lib.moef_probe_read, lib.moef_probe_copy
    assert r(None, GRAIN, B, None) == 1 and r(A, GRAIN, None, None) == 1
    # one launch covers at most 2^32 - 1 work-items: 2^24 - 1 grains of 256 lanes
    for bad in (0, -GRAIN, GRAIN - 16, GRAIN + 16, GRAIN * (2 ** 24), GRAIN * (2 ** 31)):
        assert r(A, bad, B, None) == 2, bad
        assert c(A, B, bad, None) == 2, bad
    assert r(A + 8, GRAIN, B, None) == 4 and r(A, GRAIN, B + 2, None) == 4
    assert c(None, B, GRAIN, None) == 1 and c(A, None, GRAIN, None) == 1
    assert c(A + 4, B, GRAIN, None) == 4 and c(A, B + 8, GRAIN, None) == 4
    assert c(A, A + GRAIN - 16, GRAIN, None) == 6 and c(A + 16, A, GRAIN, None) == 6
