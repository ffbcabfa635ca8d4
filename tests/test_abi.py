"""C-ABI checks that need no GPU: the library loads, exports every symbol ``include/*.h``
declares, and rejects invalid arguments on the host before touching a device."""

import ctypes
import glob
import os
import re

import pytest

import mx_grouped_gemm_amd as bsg
from tests.conftest import ROOT

lib_missing = not os.path.exists(bsg.library_path())
pytestmark = pytest.mark.skipif(lib_missing, reason="libbsgemm.so not built")


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?\w+\s*\*?\s*(bsgemm_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return names


def test_header_declares_the_api():
    assert declared_functions() == set(bsg.EXPORTED)


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(bsg.library_path())
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for st in range(0, -7, -1):
        s = bsg.bsgemm_status_string(st)
        assert s and s != "unknown status"
    assert bsg.bsgemm_status_string(5) == "unknown status"


# Fake device addresses: validation must reject these calls before any pointer is used.
P16 = 0x10000
P4 = 0x10004
ODD = 0x10001


def grouped(A=P16, sa=P16, B=P16, sb=P16, eid=None, toff=None, T=0, C=P16, M=128, N=256, K=512,
            E=1, fmt=None):
    lib = bsg.load_library()
    fmt = bsg.make_fmt("e4m3", "e4m3", "blockwise", "bf16") if fmt is None else fmt
    return lib.bsgemm_grouped(A, sa, B, sb, eid, toff, T, C, M, N, K, E, fmt, None)


def test_grouped_validation():
    assert grouped(A=None) == -1
    assert grouped(C=None) == -1
    assert grouped(eid=P16, toff=None, T=1) == -1          # one of the two tile arrays missing
    assert grouped(N=100) == -2
    assert grouped(K=200) == -2
    assert grouped(M=-1) == -2
    assert grouped(N=0) == -2
    assert grouped(E=0) == -2
    assert grouped(A=ODD) == -3
    assert grouped(B=P4) == -3
    assert grouped(sa=ODD) == -3
    assert grouped(fmt=0) == -4
    assert grouped(fmt=bsg.make_fmt("e2m1", "e4m3", "blockwise", "bf16")) == -4
    assert grouped(fmt=bsg.make_fmt("e4m3", "e4m3", "blockwise", "bf16") | (9 << 12)) == -4
    assert grouped(fmt=1 << 20) == -4


def test_grouped_empty_is_noop():
    # M = 0, or a tile map with zero tiles: valid, nothing to enqueue, no device touched
    assert grouped(M=0) == 0
    assert grouped(eid=P16, toff=P16, T=0) == 0


def test_build_tiles_validation():
    lib = bsg.load_library()
    assert lib.bsgemm_build_tiles(P16, 0, 4, 1, P16, P16, P16, None) == -2
    assert lib.bsgemm_build_tiles(P16, 5000, 4, 1, P16, P16, P16, None) == -2
    assert lib.bsgemm_build_tiles(P16, 4, -1, 1, P16, P16, P16, None) == -2
    assert lib.bsgemm_build_tiles(None, 4, 4, 1, P16, P16, P16, None) == -1
    assert lib.bsgemm_build_tiles(P16, 4, 4, 1, P16, P16, None, None) == -1
    assert lib.bsgemm_build_tiles(ODD, 4, 4, 1, P16, P16, P16, None) == -3


def test_schedule_hint_validation():
    """The small-M schedule hint is accepted for blockwise only; other hint bits are rejected."""
    mx = bsg.make_fmt("e4m3", "e4m3", "mx", "f16")
    assert grouped(fmt=mx | bsg.SCHED_SMALL_M) == -4
    assert grouped(fmt=bsg.make_fmt("e4m3", "e4m3", "blockwise", "bf16") | (2 << 16)) == -4



def test_nvfp4_validation():
    """nvfp4 takes e2m1 x e2m1 only, K a multiple of 256 and 16-byte aligned scale bases."""
    nv = bsg.make_fmt("e2m1", "e2m1", "nv", "f16")
    assert grouped(fmt=bsg.make_fmt("e4m3", "e2m1", "nv", "f16")) == -4
    assert grouped(fmt=bsg.make_fmt("e2m1", "e4m3", "nv", "f16")) == -4
    assert grouped(fmt=nv | bsg.SCHED_SMALL_M) == -4
    assert grouped(fmt=nv, K=384) == -2
    assert grouped(fmt=nv, sa=P4) == -3
    assert grouped(fmt=nv, sb=P4) == -3
    assert grouped(fmt=nv, M=0) == 0


def test_grouped_ws_validation():
    """Workspace checks that come before any device use (M = 0 is a no-op otherwise)."""
    lib = bsg.load_library()
    fmt = bsg.make_fmt("e4m3", "e4m3", "blockwise", "bf16")
    args = (P16, P16, P16, P16, None, None, 0, P16, 0, 256, 512, 1, fmt)
    assert lib.bsgemm_grouped_ws(*args, None, 1 << 30, None) == -1      # workspace NULL
    assert lib.bsgemm_grouped_ws(*args, P16 + 16, 1 << 30, None) == -3  # not 256-byte aligned
    assert lib.bsgemm_grouped_ws(*args, P16, 1 << 30, None) == 0        # M = 0: nothing to do
    assert lib.bsgemm_grouped_workspace_size(None) == -1
