"""Python binding of libmoe_mi355x.so, the MI355X (gfx950) gpt-oss MoE MLP layer.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Tensors are torch CUDA tensors (torch supplies device memory and the
current stream); bf16 tensors are passed as raw 16-bit patterns.  If the
library has not been built the functions raise -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "MoeError", "lib", "moe_layer_forward", "moe_layer_forward_dbg", "moe_route",
    "moe_workspace_bytes", "moe_workspace_init", "moe_layer_forward_ws", "moe_rmsnorm",
    "moe_stack_forward", "moe_release", "moe_status_string", "moe_version", "LIB_PATH",
    "moe_timing_enable", "moe_timing_read", "KERNELS", "moe_layer_forward_mx6", "moe_layer_forward_mx6_dbg",
    "moe_layer_forward_ex", "MOE_LAYER_MXFP6", "MOE_LAYER_ALT_ACT", "moe_rmsnorm_residual",
    "moe_layer_forward_noalloc", "MOE_NOALLOC_SCRATCH_BYTES", "moe_attn_rope", "moe_attn_forward",
    "moe_pack_weights", "moe_packed_scale_bytes", "MOE_LAYER_PACKED", "packed_shapes", "MOE_LAYER_MX6X2",
]

MOE_LAYER_MXFP6 = 1
MOE_LAYER_ALT_ACT = 2
MOE_LAYER_PACKED = 4
MOE_LAYER_MX6X2 = 8
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_SIGS = {
    "moe_layer_forward": (_I, [_P] * 9 + [_I] * 5 + [_F, _P, _P]),
    "moe_layer_forward_dbg": (_I, [_P] * 9 + [_I] * 5 + [_F] + [_P] * 6),
    "moe_layer_forward_mx6": (_I, [_P] * 9 + [_I] * 5 + [_F, _P, _P]),
    "moe_layer_forward_noalloc": (_I, [_P] * 9 + [_I] * 5 + [_F, _P, _P]),
    "moe_layer_forward_mx6_dbg": (_I, [_P] * 9 + [_I] * 5 + [_F] + [_P] * 6),
    "moe_layer_forward_ex": (_I, [_P] * 9 + [_I] * 5 + [_F, _I] + [_P] * 6),
    "moe_route": (_I, [_P] * 3 + [_I] * 4 + [_P] * 4),
    "moe_workspace_bytes": (ctypes.c_size_t, [_I] * 5),
    "moe_workspace_init": (_I, [_P, ctypes.c_size_t, _P]),
    "moe_layer_forward_ws": (_I, [_P] * 9 + [_I] * 5 + [_F, _P, _P, ctypes.c_size_t, _P]),
    "moe_rmsnorm": (_I, [_P, _P, _I, _I, _F, _P]),
    "moe_rmsnorm_residual": (_I, [_P] * 5 + [_I, _I, _F, _P]),
    "moe_attn_rope": (_I, [_P, _P] + [_I] * 4 + [_F, _P]),
    "moe_attn_forward": (_I, [_P] * 5 + [_I] * 8 + [_P]),
    "moe_pack_weights": (_I, [_P, _P, _I, _I, _I, _P, _P, _P]),
    "moe_packed_scale_bytes": (ctypes.c_size_t, [_I, _I, _I]),
    "moe_stack_forward_ex": (_I, [_P, _I] + [_P] * 8 + [_I] * 5 + [_F, _F, _I, _P, _P]),
    "moe_stack_forward": (_I, [_P, _I] + [_P] * 8 + [_I] * 5 + [_F, _F, _P, _P]),
    "moe_release": (None, []),
    "moe_timing_enable": (_I, [_I]),
    "moe_timing_read": (_I, [_P, _P, _I]),
    "moe_status_string": (ctypes.c_char_p, [_I]),
    "moe_version": (_I, []),
}


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status} ({moe_status_string(status)})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Loads the HIP library (raises if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run python -m sparse_moe_transformer_softmax_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def moe_status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def moe_version() -> int:
    return lib().moe_version()


def moe_release() -> None:
    lib().moe_release()


KERNELS = ("route", "gateup_gemm", "down_gemm", "combine", "split_x")


def moe_timing_enable(on=True) -> None:
    """on: True (every kernel), False (off), or an iterable of names from KERNELS."""
    if on is True:
        mask = (1 << len(KERNELS)) - 1
    elif not on:
        mask = 0
    else:
        mask = 0
        for k in on:
            mask |= 1 << KERNELS.index(k)
    _ok("moe_timing_enable", lib().moe_timing_enable(mask))


def moe_timing_read(reset: bool = True) -> dict:
    """{kernel: (total_ms, launches)} since the last reset."""
    ms = (ctypes.c_double * 5)()
    n = (ctypes.c_int * 5)()
    _ok("moe_timing_read", lib().moe_timing_read(ctypes.cast(ms, _P), ctypes.cast(n, _P), 1 if reset else 0))
    return {k: (ms[i], n[i]) for i, k in enumerate(KERNELS)}


def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(t, name, dtype, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _ok(fn, st):
    if st != 0:
        raise MoeError(fn, st)


def packed_shapes(E: int, N: int, K: int):
    """Shapes of moe_pack_weights' outputs: codes [E, N/2, K], scales
    [E, ceil(K/128), N, 4]."""
    return (E, N // 2, K), (E, (K // 32 + 3) // 4, N, 4)


def _layer_ptrs(x, router_w, router_b, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2, packed=False):
    torch = _torch()
    T, d = x.shape
    E = router_w.shape[0]
    I = b13.shape[1] // 2
    if packed:
        c13, s13 = packed_shapes(E, 2 * I, d)
        c2, s2 = packed_shapes(E, d, I)
    else:
        c13, s13, c2, s2 = (E, 2 * I, d // 2), (E, 2 * I, d // 32), (E, d, I // 2), (E, d, I // 32)
    ptrs = [
        _check(x, "x", torch.bfloat16, (T, d)),
        _check(router_w, "router_w", torch.bfloat16, (E, d)),
        _check(router_b, "router_b", torch.float32, (E,)),
        _check(w13_codes, "w13_codes", torch.uint8, c13),
        _check(w13_scales, "w13_scales", torch.uint8, s13),
        _check(b13, "b13", torch.float32, (E, 2 * I)),
        _check(w2_codes, "w2_codes", torch.uint8, c2),
        _check(w2_scales, "w2_scales", torch.uint8, s2),
        _check(b2, "b2", torch.float32, (E, d)),
    ]
    return ptrs, T, d, I, E


def moe_layer_forward(x, router_w, router_b, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2,
                      k: int = 4, clamp: float = 7.0, out=None, stream=None, _fn="moe_layer_forward"):
    """out = MoE(x) in bf16 [T, d]; see include/moe_mi355x.h."""
    torch = _torch()
    ptrs, T, d, I, E = _layer_ptrs(x, router_w, router_b, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2)
    if out is None:
        out = torch.empty((T, d), dtype=torch.bfloat16, device=x.device)
    po = _check(out, "out", torch.bfloat16, (T, d))
    _ok(_fn, getattr(lib(), _fn)(*ptrs, T, d, I, E, k, clamp, po, _stream(stream)))
    return out


def moe_layer_forward_mx6(x, router_w, router_b, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2,
                          k: int = 4, clamp: float = 7.0, out=None, stream=None):
    """Activation-quantised fast mode (MXFP6 activations into the expert
    GEMMs); see include/moe_mi355x.h."""
    return moe_layer_forward(x, router_w, router_b, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2,
                             k=k, clamp=clamp, out=out, stream=stream, _fn="moe_layer_forward_mx6")


def moe_layer_forward_mx6_dbg(x, router_w, router_b, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2,
                              k: int = 4, clamp: float = 7.0, stream=None):
    """moe_layer_forward_dbg for the fast mode."""
    return moe_layer_forward_dbg(x, router_w, router_b, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2,
                                 k=k, clamp=clamp, stream=stream, _fn="moe_layer_forward_mx6_dbg")


def moe_layer_forward_noalloc(x, router_w, router_b, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2,
                              k: int = 4, clamp: float = 7.0, out=None, stream=None):
    """moe_layer_forward with its scratch in the library's static device
    array (no allocation inside the call; pass `out` to allocate nothing
    here either); see include/moe_mi355x.h."""
    return moe_layer_forward(x, router_w, router_b, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2,
                             k=k, clamp=clamp, out=out, stream=stream, _fn="moe_layer_forward_noalloc")


def moe_layer_forward_dbg(x, router_w, router_b, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2,
                          k: int = 4, clamp: float = 7.0, stream=None, _fn="moe_layer_forward_dbg"):
    """Returns (out bf16, out_f32, topk_id int32 [T,k], topk_w fp32 [T,k], counts int32 [E])."""
    torch = _torch()
    ptrs, T, d, I, E = _layer_ptrs(x, router_w, router_b, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2)
    dev = x.device
    out = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
    out_f32 = torch.empty((T, d), dtype=torch.float32, device=dev)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    counts = torch.empty((E,), dtype=torch.int32, device=dev)
    _ok(_fn, getattr(lib(), _fn)(
        *ptrs, T, d, I, E, k, clamp, _check(out, "out", torch.bfloat16), _check(out_f32, "out_f32", torch.float32),
        _check(ids, "ids", torch.int32), _check(w, "w", torch.float32), _check(counts, "counts", torch.int32),
        _stream(stream)))
    return out, out_f32, ids, w, counts


def moe_layer_forward_ex(x, router_w, router_b, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2,
                         k: int = 4, clamp: float = 7.0, flags: int = 0, debug: bool = False, out=None,
                         stream=None):
    """moe_layer_forward with flags (MOE_LAYER_MXFP6, MOE_LAYER_ALT_ACT, MOE_LAYER_PACKED,
    MOE_LAYER_MX6X2).
    debug=False: returns out; debug=True: (out, out_f32, topk_id, topk_w, counts)."""
    torch = _torch()
    ptrs, T, d, I, E = _layer_ptrs(x, router_w, router_b, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2,
                                   packed=bool(flags & MOE_LAYER_PACKED))
    dev = x.device
    if out is None:
        out = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
    po = _check(out, "out", torch.bfloat16, (T, d))
    if debug:
        out_f32 = torch.empty((T, d), dtype=torch.float32, device=dev)
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
        counts = torch.empty((E,), dtype=torch.int32, device=dev)
        extra = [_check(out_f32, "out_f32", torch.float32), _check(ids, "ids", torch.int32),
                 _check(w, "w", torch.float32), _check(counts, "counts", torch.int32)]
    else:
        extra = [None, None, None, None]
    _ok("moe_layer_forward_ex", lib().moe_layer_forward_ex(*ptrs, T, d, I, E, k, clamp, flags, po, *extra,
                                                           _stream(stream)))
    return (out, out_f32, ids, w, counts) if debug else out


def moe_route(x, router_w, router_b, k: int = 4, stream=None):
    """Returns (topk_id int32 [T,k], topk_w fp32 [T,k], counts int32 [E])."""
    torch = _torch()
    T, d = x.shape
    E = router_w.shape[0]
    px = _check(x, "x", torch.bfloat16, (T, d))
    pw = _check(router_w, "router_w", torch.bfloat16, (E, d))
    pb = _check(router_b, "router_b", torch.float32, (E,))
    ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    counts = torch.empty((E,), dtype=torch.int32, device=x.device)
    _ok("moe_route", lib().moe_route(px, pw, pb, T, d, E, k, _check(ids, "ids", torch.int32),
                                     _check(w, "w", torch.float32), _check(counts, "counts", torch.int32),
                                     _stream(stream)))
    return ids, w, counts


def moe_workspace_bytes(T: int, d: int, I: int, E: int, k: int) -> int:
    return int(lib().moe_workspace_bytes(T, d, I, E, k))


def moe_workspace_init(ws, stream=None) -> None:
    torch = _torch()
    _ok("moe_workspace_init", lib().moe_workspace_init(_check(ws, "ws", torch.uint8), ws.numel(), _stream(stream)))


def moe_layer_forward_ws(x, router_w, router_b, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2, ws,
                         k: int = 4, clamp: float = 7.0, out=None, stream=None):
    torch = _torch()
    ptrs, T, d, I, E = _layer_ptrs(x, router_w, router_b, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2)
    if out is None:
        out = torch.empty((T, d), dtype=torch.bfloat16, device=x.device)
    po = _check(out, "out", torch.bfloat16, (T, d))
    pws = _check(ws, "ws", torch.uint8)
    _ok("moe_layer_forward_ws", lib().moe_layer_forward_ws(*ptrs, T, d, I, E, k, clamp, po, pws, ws.numel(),
                                                           _stream(stream)))
    return out


def moe_rmsnorm(x, eps: float = 1e-5, out=None, stream=None):
    torch = _torch()
    T, d = x.shape
    if out is None:
        out = torch.empty_like(x)
    _ok("moe_rmsnorm", lib().moe_rmsnorm(_check(x, "x", torch.bfloat16, (T, d)),
                                         _check(out, "out", torch.bfloat16, (T, d)), T, d, eps, _stream(stream)))
    return out


def moe_rmsnorm_residual(x, y, eps: float = 1e-5, x_out=None, n_out=None, normalize: bool = True, stream=None):
    """x_out = bf16(x + y), n_out = bf16(RMSNorm(x_out)); y bf16 or fp32 [T, d].
    Returns (x_out, n_out) (n_out None when normalize is False)."""
    torch = _torch()
    T, d = x.shape
    px = _check(x, "x", torch.bfloat16, (T, d))
    if y.dtype == torch.float32:
        yb, yf = None, _check(y, "y", torch.float32, (T, d))
    else:
        yb, yf = _check(y, "y", torch.bfloat16, (T, d)), None
    if x_out is None:
        x_out = torch.empty_like(x)
    if n_out is None and normalize:
        n_out = torch.empty_like(x)
    pxo = _check(x_out, "x_out", torch.bfloat16, (T, d))
    pno = _check(n_out, "n_out", torch.bfloat16, (T, d)) if normalize else None
    _ok("moe_rmsnorm_residual", lib().moe_rmsnorm_residual(px, yb, yf, pxo, pno, T, d, eps, _stream(stream)))
    return x_out, (n_out if normalize else None)


def moe_attn_rope(x, pos0: int = 0, theta: float = 10000.0, out=None, stream=None):
    """Rotary encoding of x bf16 [n, H, D] at positions pos0 .. pos0 + n - 1
    (out may be x itself)."""
    torch = _torch()
    n, H, D = x.shape
    if out is None:
        out = torch.empty_like(x)
    _ok("moe_attn_rope", lib().moe_attn_rope(_check(x, "x", torch.bfloat16, (n, H, D)),
                                             _check(out, "out", torch.bfloat16, (n, H, D)), n, H, D, pos0,
                                             theta, _stream(stream)))
    return out


def moe_attn_forward(q, k, v, sinks, q_pos0: int = 0, window: int = 0, out=None, stream=None):
    """Grouped-query attention with per-head sink logits: q bf16 [B, Tq, Hq, D],
    k and v bf16 [B, S, Hkv, D], sinks fp32 [Hq]; window 0 is dense causal
    attention, otherwise the band of the last `window` positions."""
    torch = _torch()
    B, Tq, Hq, D = q.shape
    S, Hkv = k.shape[1], k.shape[2]
    if out is None:
        out = torch.empty_like(q)
    _ok("moe_attn_forward", lib().moe_attn_forward(
        _check(q, "q", torch.bfloat16, (B, Tq, Hq, D)), _check(k, "k", torch.bfloat16, (B, S, Hkv, D)),
        _check(v, "v", torch.bfloat16, (B, S, Hkv, D)), _check(sinks, "sinks", torch.float32, (Hq,)),
        _check(out, "out", torch.bfloat16, (B, Tq, Hq, D)), B, Tq, S, q_pos0, Hq, Hkv, D, window, _stream(stream)))
    return out


def moe_stack_forward(x0, layers, k: int = 4, clamp: float = 7.0, eps: float = 1e-5, out=None, stream=None,
                      flags: int = 0):
    """layers: list of dicts with router_w, router_b, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2
    (flags: MOE_LAYER_ALT_ACT, MOE_LAYER_PACKED; any set flag calls moe_stack_forward_ex)."""
    torch = _torch()
    T, d = x0.shape
    n = len(layers)
    keys = ["router_w", "router_b", "w13_codes", "w13_scales", "b13", "w2_codes", "w2_scales", "b2"]
    arrays = {kk: (ctypes.c_void_p * n)() for kk in keys}
    I = E = None
    for l, L in enumerate(layers):
        ptrs, _, _, I, E = _layer_ptrs(x0, *[L[kk] for kk in keys], packed=bool(flags & MOE_LAYER_PACKED))
        for kk, p in zip(keys, ptrs[1:]):
            arrays[kk][l] = p.value
    if out is None:
        out = torch.empty_like(x0)
    args = [_check(x0, "x0", torch.bfloat16, (T, d)), n] + [ctypes.cast(arrays[kk], ctypes.c_void_p) for kk in keys]
    if flags:
        _ok("moe_stack_forward_ex", lib().moe_stack_forward_ex(
            *args, T, d, I, E, k, clamp, eps, flags, _check(out, "out", torch.bfloat16, (T, d)), _stream(stream)))
    else:
        _ok("moe_stack_forward", lib().moe_stack_forward(
            *args, T, d, I, E, k, clamp, eps, _check(out, "out", torch.bfloat16, (T, d)), _stream(stream)))
    return out


def moe_pack_weights(codes, scales, stream=None):
    """Packed copies of one MXFP4 weight stack (codes uint8 [E, N, K/2],
    scales uint8 [E, N, K/32]) for MOE_LAYER_PACKED: returns (codes [E, N/2, K],
    scales [E, ceil(K/128), N, 4])."""
    torch = _torch()
    E, N, half = codes.shape
    K = 2 * half
    cs, ss = packed_shapes(E, N, K)
    co = torch.empty(cs, dtype=torch.uint8, device=codes.device)
    so = torch.empty(ss, dtype=torch.uint8, device=codes.device)
    _ok("moe_pack_weights", lib().moe_pack_weights(
        _check(codes, "codes", torch.uint8, (E, N, K // 2)), _check(scales, "scales", torch.uint8, (E, N, K // 32)),
        E, N, K, _check(co, "codes_out", torch.uint8, cs), _check(so, "scales_out", torch.uint8, ss),
        _stream(stream)))
    return co, so


def moe_packed_scale_bytes(E: int, N: int, K: int) -> int:
    return int(lib().moe_packed_scale_bytes(E, N, K))
