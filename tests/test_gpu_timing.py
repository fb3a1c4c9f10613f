"""The library's per-kernel timing (moe_timing_enable / moe_timing_read),
which bench.py's roofline figures come from: every enabled kernel of a
layer call is counted once per launch with a positive duration (the expert
GEMMs by events their launch records itself, the other kernels by events
around their launch), disabled kernels are not counted, and timing leaves
the results bit for bit unchanged."""
import sys

import pytest

from moe_inputs.workloads import WORKLOADS, Workload
from oracle.workload_inputs import make_inputs
import sparse_moe_transformer_softmax_amd as moe
from tests.parity_util import KEYS, to_gpu

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "no GPU"
    moe.lib()
    return _t


@pytest.mark.parametrize("name,wl", [
    ("decode", WORKLOADS["20b_decode"]),                                              # folded combine
    ("prefill", Workload("prefill", T=1500, d=256, I=192, E=8, k=3, seed=0x5EED4200)),  # 128-row tiles + combine
])
def test_timing_counts_each_launch_and_changes_nothing(torch, name, wl):
    say(f"timing {name}")
    g = to_gpu(make_inputs(wl, condition=False))
    args = [g[k] for k in KEYS]
    ref = moe.moe_layer_forward(*args, k=wl.k, clamp=wl.clamp)
    torch.cuda.synchronize()
    moe.moe_timing_read(reset=True)
    moe.moe_timing_enable(True)
    n = 3
    for _ in range(n):
        out = moe.moe_layer_forward(*args, k=wl.k, clamp=wl.clamp)
    torch.cuda.synchronize()
    moe.moe_timing_enable(False)
    t = moe.moe_timing_read(reset=True)
    say(f"  {t}")
    assert torch.equal(out, ref)
    for kname in ("route", "gateup_gemm", "down_gemm"):
        ms, cnt = t[kname]
        assert cnt == n and ms > 0, (kname, t[kname])
    if name == "prefill":
        assert t["combine"][1] == n and t["combine"][0] > 0
    # only the enabled kernels are timed
    moe.moe_timing_enable(["gateup_gemm"])
    moe.moe_layer_forward(*args, k=wl.k, clamp=wl.clamp)
    torch.cuda.synchronize()
    moe.moe_timing_enable(False)
    t = moe.moe_timing_read(reset=True)
    assert t["gateup_gemm"][1] == 1 and t["route"][1] == 0 and t["down_gemm"][1] == 0
    # nothing is timed while timing is off
    moe.moe_layer_forward(*args, k=wl.k, clamp=wl.clamp)
    torch.cuda.synchronize()
    assert all(c == 0 for _, c in moe.moe_timing_read(reset=True).values())
