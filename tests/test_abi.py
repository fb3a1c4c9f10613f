"""The C-ABI library: it loads, exports every function its header declares,
and rejects bad arguments on the host before any GPU work."""
import ctypes
import os
import re

import pytest

import sparse_moe_transformer_softmax_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mi355x.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert "moe_layer_forward" in names and len(names) >= 10
    L = ctypes.CDLL(moe.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(moe._SIGS), set(names) ^ set(moe._SIGS)


def test_version_and_status_strings():
    assert moe.moe_version() == 10000
    assert moe.moe_status_string(0) == "ok"
    for st in range(-8, 0):
        assert moe.moe_status_string(st) != "unknown status"


def test_workspace_bytes():
    n = moe.moe_workspace_bytes(32, 2880, 2880, 32, 4)
    # at least the MX6x3 rows of x and h and the fp32 expert outputs
    assert n >= 32 * 90 * 80 + 128 * 90 * 80 + 128 * 2880 * 4
    assert n % 256 == 0
    assert moe.moe_workspace_bytes(32, 2880, 2880, 32, 0) == 0
    assert moe.moe_workspace_bytes(32, 2880, 2880, 3, 4) == 0
    assert moe.moe_workspace_bytes(32, 2881, 2880, 32, 4) == 0
    assert moe.moe_workspace_bytes(32, 2880, 2880, 300, 4) == 0


def _call(T=16, d=128, I=128, E=8, k=4, clamp=7.0, ptr=0x10000, out=0x900000):
    p = ctypes.c_void_p(ptr)
    return moe.lib().moe_layer_forward(*([p] * 9), T, d, I, E, k, clamp, ctypes.c_void_p(out), None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=100), -2), (dict(I=48), -2), (dict(E=0), -2), (dict(E=257), -2), (dict(k=0), -2),
    (dict(k=9, E=16), -2), (dict(k=5, E=4), -2), (dict(T=-1), -2), (dict(clamp=0.0), -2),
    (dict(clamp=float("nan")), -2), (dict(ptr=0), -1), (dict(ptr=0x10004), -4), (dict(out=0x10000), -7),
    (dict(out=0), -1),
])
def test_argument_errors_are_reported_on_the_host(kw, status):
    assert _call(**kw) == status


def test_zero_tokens_is_a_no_op():
    assert _call(T=0) == 0
    assert _call(T=0, ptr=0, out=0) == 0
    assert _call(T=0, d=100) == -2
