"""Plants plausible mistakes in the oracle (on the CPU, via monkeypatch) and
checks that at least one pin catches each of them."""
import numpy as np
import pytest

from oracle import moe_oracle as O
from tests import test_oracle_pins as P


def _swapped_nibbles(codes, scales):
    c = np.asarray(codes, dtype=np.uint8)
    return ORIG["mxfp4_dequant"](((c & 15) << 4) | (c >> 4), scales)


def _e8m0_bias_128(byte):
    s = np.asarray(byte, dtype=np.int64)
    return np.where(s == 255, np.nan, np.ldexp(1.0, s - 128))


def _softmax_wrong_sign(sel):
    e = np.exp(-(sel - sel.max(axis=1, keepdims=True)))
    return e / e.sum(axis=1, keepdims=True)


def _topk_ascending(logits, k):
    return np.argsort(logits, axis=1, kind="stable")[:, :k]


def _no_plus_one(g, u, c):
    gc = np.clip(g, -c, c)
    return gc * O.sigmoid(gc) * np.clip(u, -c, c)


def _unclamped_up(g, u, c):
    gc = np.clip(g, -c, c)
    return gc * O.sigmoid(gc) * (u + 1.0)


def _gate_up_swapped(xs, w13, b13, w2, b2, c):
    I = w13.shape[0] // 2
    a = xs @ w13.T + b13[None, :]
    return O.clamped_swiglu(a[:, I:], a[:, :I], c) @ w2.T + b2[None, :]


def _w2_transposed(xs, w13, b13, w2, b2, c):
    I = w13.shape[0] // 2
    a = xs @ w13.T + b13[None, :]
    return O.clamped_swiglu(a[:, :I], a[:, I:], c) @ w2 + b2[None, :]


def _b2_outside(xs, w13, b13, w2, b2, c):
    return ORIG["expert_ffn"](xs, w13, b13, w2, b2, c) - b2[None, :] + (b2[None, :] * 0.5)


def _gap_inner_slots(logits, k):
    srt = -np.sort(-logits, axis=1)
    return srt[:, k - 2] - srt[:, k - 1]


def _gap_wrong_end(logits, k):
    srt = np.sort(logits, axis=1)
    return srt[:, k] - srt[:, k - 1]


def _router_no_bias(x, wr, b):
    return x @ wr.T


def _rmsnorm_no_eps_mean(v, eps=1e-5):
    return v / np.sqrt(np.sum(v * v, axis=-1, keepdims=True) + eps)


ORIG = {n: getattr(O, n) for n in ("mxfp4_dequant", "expert_ffn")}

MUTATIONS = [
    ("mxfp4_dequant", _swapped_nibbles),
    ("e8m0_value", _e8m0_bias_128),
    ("selected_softmax", _softmax_wrong_sign),
    ("topk_experts", _topk_ascending),
    ("clamped_swiglu", _no_plus_one),
    ("clamped_swiglu", _unclamped_up),
    ("expert_ffn", _gate_up_swapped),
    ("expert_ffn", _w2_transposed),
    ("expert_ffn", _b2_outside),
    ("router_logits", _router_no_bias),
    ("topk_gap", _gap_inner_slots),
    ("topk_gap", _gap_wrong_end),
    ("rmsnorm", _rmsnorm_no_eps_mean),
]

PINS = [getattr(P, n) for n in dir(P) if n.startswith("test_") and n != "test_dense_masked_equals_sparse_tiny"
        and n != "test_format_sizes_match_pages"]


@pytest.mark.parametrize("name,fn", MUTATIONS, ids=[f.__name__ for _, f in MUTATIONS])
def test_some_pin_catches(monkeypatch, name, fn):
    monkeypatch.setattr(O, name, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutation {fn.__name__}"
