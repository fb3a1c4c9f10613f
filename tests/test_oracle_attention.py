"""Pins of the attention oracle (oracle/attention_oracle.py) against what the
mathematics fixes: closed forms on tiny inputs, invariants of causal and
banded attention and of rotary encoding, and special cases that reduce to a
library softmax.  Each pin is written so that a plausible mistake in the
oracle (a dropped scale or sink, an off-by-one band, a wrong head mapping,
the other rotary pairing) fails at least one of them; the mutation harness
at the end plants such mistakes and checks that."""
import math

import numpy as np
import pytest
from scipy.special import softmax as lib_softmax

from oracle import attention_oracle as A


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------------------
# rotary encoding
# ---------------------------------------------------------------------------

def test_rope_identity_at_position_zero():
    x = _rand((3, 2, 8), 1)
    assert np.array_equal(A.rope(x, np.zeros(3)), x)


def test_rope_closed_form_pairs_adjacent_elements():
    # D = 4: pair (0, 1) turns by pos * 1, pair (2, 3) by pos * 10000^(-1/2)
    e1 = np.array([[[0.0, 1.0, 0.0, 0.0]]])
    e2 = np.array([[[0.0, 0.0, 1.0, 0.0]]])
    r1 = A.rope(e1, np.array([1]))[0, 0]
    r2 = A.rope(e2, np.array([1]))[0, 0]
    assert np.allclose(r1, [-math.sin(1.0), math.cos(1.0), 0.0, 0.0], atol=1e-15)
    assert np.allclose(r2, [0.0, 0.0, math.cos(0.01), math.sin(0.01)], atol=1e-15)
    x = np.array([[[0.3, -0.7, 1.1, 0.2]]])
    r = A.rope(x, np.array([5]))[0, 0]
    c0, s0, c1, s1 = math.cos(5.0), math.sin(5.0), math.cos(0.05), math.sin(0.05)
    assert np.allclose(r, [0.3 * c0 + 0.7 * s0, 0.3 * s0 - 0.7 * c0, 1.1 * c1 - 0.2 * s1, 1.1 * s1 + 0.2 * c1],
                       atol=1e-14)


def test_rope_dot_products_depend_on_relative_position_only():
    q, k = _rand((1, 1, 64), 2), _rand((1, 1, 64), 3)
    for p, pk, delta in [(7, 3, 11), (100, 100, 900), (4095, 0, 37)]:
        a = float(np.sum(A.rope(q, np.array([p])) * A.rope(k, np.array([pk]))))
        b = float(np.sum(A.rope(q, np.array([p + delta])) * A.rope(k, np.array([pk + delta]))))
        assert abs(a - b) < 1e-9 * max(1.0, abs(a))


def test_rope_composes_and_keeps_pair_norms():
    x = _rand((4, 3, 16), 4)
    a, b = np.array([1, 5, 17, 300]), np.array([2, 9, 40, 1000])
    assert np.allclose(A.rope(A.rope(x, a), b), A.rope(x, a + b), atol=1e-12)
    y = A.rope(x, b)
    assert np.allclose(x[..., 0::2] ** 2 + x[..., 1::2] ** 2, y[..., 0::2] ** 2 + y[..., 1::2] ** 2, atol=1e-12)


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def _case(B=2, Tq=9, S=12, Hq=4, Hkv=2, D=8, seed=5):
    return _rand((B, Tq, Hq, D), seed), _rand((B, S, Hkv, D), seed + 1), _rand((B, S, Hkv, D), seed + 2), \
        _rand(Hq, seed + 3)


def test_zero_queries_average_the_visible_values():
    # every visible score is 0, so out = (sum of visible v) / (n + e^sink)
    _, k, v, sinks = _case()
    q = np.zeros((2, 9, 4, 8))
    for window, q_pos0 in [(0, 3), (4, 3), (1, 0), (20, 0)]:
        out = A.attention(q, k, v, sinks, q_pos0, window)
        for b in range(2):
            for i in range(9):
                p = q_pos0 + i
                lo = 0 if window == 0 else max(0, p - window + 1)
                for h in range(4):
                    g = h // 2
                    n = p - lo + 1
                    want = v[b, lo:p + 1, g].sum(axis=0) / (n + math.exp(sinks[h]))
                    assert np.allclose(out[b, i, h], want, atol=1e-13)


def test_band_of_one_without_sink_returns_own_value():
    q, k, v, _ = _case()
    out = A.attention(q, k, v, np.full(4, -np.inf), 3, 1)
    for i in range(9):
        for h in range(4):
            assert np.array_equal(out[:, i, h], v[:, 3 + i, h // 2])


def test_first_position_closed_form():
    # query 0 sees key 0 only: out = v0 * e^s / (e^s + e^sink), s = q.k0 / sqrt(D)
    D = 64
    q, k, v = _rand((1, 1, 1, D), 10), _rand((1, 1, 1, D), 11), _rand((1, 1, 1, D), 12)
    for sink in (-3.0, 0.0, 2.5):
        s = float(np.dot(q[0, 0, 0], k[0, 0, 0])) / 8.0
        want = v[0, 0, 0] * math.exp(s) / (math.exp(s) + math.exp(sink))
        out = A.attention(q, k, v, np.array([sink]), 0, 0)[0, 0, 0]
        assert np.allclose(out, want, atol=1e-14)


def test_two_keys_closed_form():
    D = 4
    q = np.array([[[[1.0, 2.0, 0.0, -1.0]]]])
    k = np.array([[[[0.5, 0.5, 1.0, 0.0]], [[-1.0, 1.0, 0.0, 2.0]]]])
    v = np.array([[[[1.0, 0.0, 0.0, 0.0]], [[0.0, 1.0, 0.0, 0.0]]]])
    s0, s1 = 1.5 / 2.0, (-1.0 + 2.0 - 2.0) / 2.0
    sink = 0.25
    den = math.exp(s0) + math.exp(s1) + math.exp(sink)
    out = A.attention(q, k, v, np.array([sink]), 1, 0)[0, 0, 0]
    assert np.allclose(out, [math.exp(s0) / den, math.exp(s1) / den, 0.0, 0.0], atol=1e-15)


def test_query_heads_share_their_group_kv_head():
    # 8 query heads over 2 kv heads: heads 0..3 read kv head 0, heads 4..7 kv head 1
    B, Tq, S, D = 1, 3, 5, 8
    q = np.zeros((B, Tq, 8, D))
    k = _rand((B, S, 2, D), 20)
    v = np.zeros((B, S, 2, D))
    v[:, :, 0, :] = 1.0
    v[:, :, 1, :] = 2.0
    out = A.attention(q, k, v, np.full(8, -np.inf), 2, 0)
    assert np.allclose(out[0, :, :, 0], np.array([[1, 1, 1, 1, 2, 2, 2, 2]] * Tq), atol=1e-14)


def test_band_equals_dense_inside_the_window():
    q, k, v, sinks = _case(Tq=12, S=12)
    dense = A.attention(q, k, v, sinks, 0, 0)
    band = A.attention(q, k, v, sinks, 0, 5)
    assert np.array_equal(dense[:, :5], band[:, :5])
    assert not np.allclose(dense[:, 5:], band[:, 5:])
    assert np.array_equal(A.attention(q, k, v, sinks, 0, 12), dense)


def test_future_and_out_of_band_keys_do_not_matter():
    q, k, v, sinks = _case(Tq=6, S=12)
    q_pos0, window = 4, 3          # positions 4..9 see keys p-2..p
    base = A.attention(q, k, v, sinks, q_pos0, window)
    k2, v2 = k.copy(), v.copy()
    k2[:, 10:] += 5.0
    v2[:, 10:] -= 3.0               # keys past every query
    k2[:, :2] += 5.0
    v2[:, :2] -= 3.0                # keys before every query's band (p - 2 >= 2)
    assert np.array_equal(A.attention(q, k2, v2, sinks, q_pos0, window), base)
    v3 = v.copy()
    v3[:, 4] += 1.0                 # inside the band of position 4 (and 5, 6)
    assert not np.allclose(A.attention(q, k, v3, sinks, q_pos0, window)[:, :3], base[:, :3])


def test_without_sink_equals_the_library_softmax():
    q, k, v, _ = _case()
    out = A.attention(q, k, v, np.full(4, -np.inf), 3, 0)
    for b in range(2):
        for h in range(4):
            s = q[b, :, h] @ k[b, :, h // 2].T / math.sqrt(8)
            mask = np.arange(12)[None, :] <= (3 + np.arange(9))[:, None]
            w = lib_softmax(np.where(mask, s, -np.inf), axis=1)
            assert np.allclose(out[b, :, h], w @ v[b, :, h // 2], atol=1e-13)


def test_sink_is_one_more_softmax_column_without_a_value():
    q, k, v, sinks = _case()
    out = A.attention(q, k, v, sinks, 3, 4)
    for b in range(2):
        for h in range(4):
            s = q[b, :, h] @ k[b, :, h // 2].T / math.sqrt(8)
            p = (3 + np.arange(9))[:, None]
            j = np.arange(12)[None, :]
            s = np.where((j <= p) & (j > p - 4), s, -np.inf)
            w = lib_softmax(np.concatenate([s, np.full((9, 1), sinks[h])], axis=1), axis=1)[:, :12]
            assert np.allclose(out[b, :, h], w @ v[b, :, h // 2], atol=1e-13)


def test_sampled_rows_equal_the_full_output():
    q, k, v, sinks = _case()
    full = A.attention(q, k, v, sinks, 3, 4)
    rows = [(0, 0, 0), (1, 8, 3), (0, 4, 2), (1, 2, 1)]
    got = A.attention_rows(q, k, v, sinks, 3, 4, rows)
    for n, (b, i, h) in enumerate(rows):
        assert np.allclose(got[n], full[b, i, h], atol=1e-14)


# ---------------------------------------------------------------------------
# planted mistakes: each must fail at least one pin above
# ---------------------------------------------------------------------------

def _no_scale(qh, kh):
    return qh @ kh.T


def _scale_by_d(qh, kh):
    return qh @ kh.T / qh.shape[-1]


def _band_off_by_one(pos, S, window):
    p = np.asarray(pos, dtype=np.int64)[:, None]
    j = np.arange(S, dtype=np.int64)[None, :]
    ok = j <= p
    if window > 0:
        ok = ok & (j >= p - window)
    return ok


def _not_causal(pos, S, window):
    p = np.asarray(pos, dtype=np.int64)[:, None]
    j = np.arange(S, dtype=np.int64)[None, :]
    return (j > p - window) if window > 0 else np.ones((p.shape[0], S), dtype=bool)


def _heads_round_robin(h, Hq, Hkv):
    return h % Hkv


def _sink_ignored(s, sink):
    return ORIG["sink_softmax"](s, -np.inf)


def _sink_counted_twice(s, sink):
    m = np.maximum(s.max(axis=1), float(sink))
    e = np.exp(s - m[:, None])
    return e / (e.sum(axis=1) + 2.0 * np.exp(float(sink) - m))[:, None]


def _rope_half_split(x, pos, theta=A.ROPE_THETA):
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    ang = A.rope_angles(pos, D, theta)[:, None, :]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :D // 2], x[..., D // 2:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def _rope_wrong_frequency(pos, D, theta=A.ROPE_THETA):
    i = np.arange(D // 2, dtype=np.float64)
    return np.asarray(pos, dtype=np.float64)[:, None] * (theta ** (-i / D))[None, :]


def _rope_backwards(x, pos, theta=A.ROPE_THETA):
    return ORIG["rope"](x, -np.asarray(pos), theta)


ORIG = {n: getattr(A, n) for n in ("sink_softmax", "rope")}

MUTATIONS = [
    ("scores", _no_scale),
    ("scores", _scale_by_d),
    ("key_mask", _band_off_by_one),
    ("key_mask", _not_causal),
    ("head_group", _heads_round_robin),
    ("sink_softmax", _sink_ignored),
    ("sink_softmax", _sink_counted_twice),
    ("rope", _rope_half_split),
    ("rope_angles", _rope_wrong_frequency),
    ("rope", _rope_backwards),
]

PINS = [f for n, f in sorted(globals().items()) if n.startswith("test_") and n != "test_some_pin_catches"]


@pytest.mark.parametrize("name,fn", MUTATIONS, ids=[f.__name__ for _, f in MUTATIONS])
def test_some_pin_catches(monkeypatch, name, fn):
    monkeypatch.setattr(A, name, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutation {fn.__name__}"
