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


def _resid(x=0x10000, yb=None, yf=0x20000, xo=0x30000, no=0x40000, T=4, d=64, eps=1e-5):
    P = ctypes.c_void_p
    return moe.lib().moe_rmsnorm_residual(P(x), P(yb), P(yf), P(xo), P(no), T, d, eps, None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=48), -2), (dict(T=-1), -2), (dict(eps=-1.0), -2), (dict(yb=0x50000), -1), (dict(yf=None), -1),
    (dict(x=None), -1), (dict(xo=None), -1), (dict(xo=0x30004), -4), (dict(no=0x10040), -7),
    (dict(xo=0x10040), -7), (dict(no=0x30000), -7), (dict(xo=0x20000), -7),
])
def test_rmsnorm_residual_argument_errors(kw, status):
    assert _resid(**kw) == status


def test_rmsnorm_residual_zero_rows_is_a_no_op():
    assert _resid(T=0) == 0


def _attn(q=0x100000, k=0x200000, v=0x300000, sinks=0x400000, out=0x500000, B=2, Tq=8, S=16, q_pos0=4, Hq=16,
          Hkv=2, D=64, window=0):
    P = ctypes.c_void_p
    return moe.lib().moe_attn_forward(P(q), P(k), P(v), P(sinks), P(out), B, Tq, S, q_pos0, Hq, Hkv, D, window,
                                      None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=128), -3), (dict(Hkv=3), -3), (dict(Hq=96, Hkv=3), -3), (dict(Hq=64, Hkv=2), -3),
    (dict(S=0), -2), (dict(q_pos0=-1), -2), (dict(q_pos0=9), -2), (dict(Tq=-1), -2), (dict(window=-1), -2),
    (dict(B=-1), -2), (dict(Hkv=0), -2), (dict(q=None), -1), (dict(sinks=None), -1), (dict(out=None), -1),
    (dict(q=0x100008), -4), (dict(v=0x300008), -4), (dict(sinks=0x400002), -4), (dict(out=0x100000), -7),
    (dict(out=0x200100), -7), (dict(out=0x400000), -7),
])
def test_attention_argument_errors(kw, status):
    assert _attn(**kw) == status


def test_attention_empty_batch_is_a_no_op():
    assert _attn(B=0) == 0
    assert _attn(Tq=0, q=None, out=None) == 0


def _rope(x=0x100000, out=0x200000, n=8, H=4, D=64, pos0=0, theta=10000.0):
    P = ctypes.c_void_p
    return moe.lib().moe_attn_rope(P(x), P(out), n, H, D, pos0, theta, None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=63), -2), (dict(D=0), -2), (dict(D=258), -2), (dict(n=-1), -2), (dict(pos0=-3), -2),
    (dict(theta=1.0), -2), (dict(theta=float("nan")), -2), (dict(x=None), -1), (dict(out=None), -1),
    (dict(x=0x100004), -4), (dict(out=0x100040), -7),
])
def test_rope_argument_errors(kw, status):
    assert _rope(**kw) == status


def test_rope_empty_is_a_no_op():
    assert _rope(n=0, x=None, out=None) == 0


def _pack(codes=0x100000, scales=0x200000, E=2, N=64, K=128, co=0x300000, so=0x400000):
    P = ctypes.c_void_p
    return moe.lib().moe_pack_weights(P(codes), P(scales), E, N, K, P(co), P(so), None)


@pytest.mark.parametrize("kw,status", [
    (dict(N=63), -2), (dict(N=0), -2), (dict(K=96), -2), (dict(K=32), -2), (dict(E=0), -2),
    (dict(codes=None), -1), (dict(so=None), -1), (dict(codes=0x100008), -4), (dict(co=0x300004), -4),
    (dict(so=0x400002), -4), (dict(co=0x100000), -7), (dict(so=0x200000), -7), (dict(so=0x300010), -7),
])
def test_pack_weights_argument_errors(kw, status):
    assert _pack(**kw) == status


def test_packed_scale_bytes():
    # one 4-byte word per row and chunk of four 32-element blocks
    assert moe.moe_packed_scale_bytes(128, 5760, 2880) == 128 * 5760 * 4 * 23
    assert moe.moe_packed_scale_bytes(2, 64, 128) == 2 * 64 * 4
    assert moe.moe_packed_scale_bytes(2, 63, 128) == 0
    assert moe.moe_packed_scale_bytes(2, 64, 96) == 0


def test_packed_flag_needs_even_block_counts():
    P = ctypes.c_void_p
    # d or I not a multiple of 64 (an odd number of 32-element blocks) is
    # refused before any GPU work
    f = moe.lib().moe_layer_forward_ex
    args = [P(0x10000)] * 9
    assert f(*args, 32, 2880, 2848, 32, 4, 7.0, moe.MOE_LAYER_PACKED, P(0x900000), None, None, None, None,
             None) == -3
    assert f(*args, 4096, 2848, 2880, 32, 4, 7.0, moe.MOE_LAYER_PACKED, P(0x900000), None, None, None, None,
             None) == -3
    assert f(*args, 4096, 2880, 2880, 32, 4, 7.0, 16, P(0x900000), None, None, None, None, None) == -2


def test_one_and_two_term_flags_exclude_each_other():
    P = ctypes.c_void_p
    f = moe.lib().moe_layer_forward_ex
    args = [P(0x10000)] * 9
    both = moe.MOE_LAYER_MXFP6 | moe.MOE_LAYER_MX6X2
    assert f(*args, 32, 2880, 2880, 32, 4, 7.0, both, P(0x900000), None, None, None, None, None) == -2
