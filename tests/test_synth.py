"""The seeded generator: determinism, stream independence and the value
distributions of the workloads."""
import numpy as np

from oracle import moe_oracle as O
from moe_inputs import synth
from moe_inputs.workloads import WORKLOADS


def test_deterministic_and_seed_sensitive():
    a = synth.gen_x(1, 8, 64)
    assert np.array_equal(a, synth.gen_x(1, 8, 64))
    assert not np.array_equal(a, synth.gen_x(2, 8, 64))
    e1 = synth.gen_experts(3, 2, 64, 32)
    e2 = synth.gen_experts(3, 2, 64, 32)
    for key in e1:
        assert np.array_equal(e1[key], e2[key])


def test_redraw_touches_only_named_rows():
    a = synth.gen_x(1, 16, 64)
    b = synth.gen_x(1, 16, 64, {3: 1, 9: 2})
    changed = np.nonzero(np.any(a != b, axis=1))[0].tolist()
    assert changed == [3, 9]
    c = synth.gen_x(1, 16, 64, {3: 2, 9: 2})
    assert not np.array_equal(b[3], c[3]) and np.array_equal(b[9], c[9])


def test_distributions():
    x = O.bf16_bits_to_f64(synth.gen_x(4, 256, 2880))
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    wr, br = synth.gen_router(4, 128, 2880)
    w = O.bf16_bits_to_f64(wr)
    assert abs(w.var() * 2880 - 1) < 0.02
    assert abs(br.var() - 0.1) < 0.04
    ex = synth.gen_experts(4, 2, 2880, 256)
    assert set(np.unique(ex["w13_scales"]).tolist()) == {121, 122, 123, 124}
    nib = np.concatenate([ex["w13_codes"] & 15, ex["w13_codes"] >> 4]).reshape(-1)
    cnt = np.bincount(nib, minlength=16) / nib.size
    assert np.all(np.abs(cnt - 1 / 16) < 0.002)
    assert abs(ex["b13"].std() - 0.1) < 0.005 and abs(ex["b2"].std() - 0.1) < 0.005


def test_zipf_bias_is_a_permuted_log_rank():
    wl = WORKLOADS["120b_prefill_zipf"]
    b = synth.zipf_router_bias(wl.seed, wl.E, 0.5)
    rank = np.rint(np.exp(-b.astype(np.float64) / 0.5)).astype(int)
    assert sorted(rank.tolist()) == list(range(1, wl.E + 1))
