"""The allocation-free entry point (moe_layer_forward_noalloc), called
through the C ABI, against moe_layer_forward on the same inputs: two calls
in a row with the second on fewer tokens (the static scratch keeps the first
call's contents), at a decode size and at a prefill size, with the device's
free memory unchanged across the calls; and the size limit.  The runtime
places the library's static scratch array in device memory when the entry
point first takes its address on a GPU (its set-up), so free memory is
compared only after one call has been made."""
import numpy as np
import pytest

from oracle.workload_inputs import make_inputs
from moe_inputs.workloads import WORKLOADS, Workload
import sparse_moe_transformer_softmax_amd as moe
from tests.parity_util import KEYS, to_gpu


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "no GPU"
    moe.lib()
    return _t


def _pair(torch, g, T, k, clamp):
    args = [g["x"][:T].contiguous()] + [g[kk] for kk in KEYS[1:]]
    ref = torch.empty((T, g["x"].shape[1]), dtype=torch.bfloat16, device="cuda")
    got = torch.full_like(ref, 5.0)
    moe.moe_layer_forward(*args, k=k, clamp=clamp, out=ref)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    moe.moe_layer_forward_noalloc(*args, k=k, clamp=clamp, out=got)
    torch.cuda.synchronize()
    return ref, got, free0, torch.cuda.mem_get_info()[0]


@pytest.mark.gpu
@pytest.mark.parametrize("name,T1,T2", [("20b_decode", 32, 7), ("prefill_small", 600, 257)])
def test_noalloc_matches_layer_forward_on_two_calls(torch, name, T1, T2):
    wl = WORKLOADS[name] if name in WORKLOADS else Workload(name, T=600, d=256, I=192, E=8, k=4, seed=0x5EED9000)
    inp = make_inputs(wl)
    g = to_gpu(inp)
    print(f"[gpu-case] noalloc {name}: T={T1} then T={T2}", flush=True)
    # set-up: the first call on this GPU takes the scratch array's address
    setup = torch.empty((T2, g["x"].shape[1]), dtype=torch.bfloat16, device="cuda")
    moe.moe_layer_forward_noalloc(*([g["x"][:T2].contiguous()] + [g[kk] for kk in KEYS[1:]]), k=wl.k,
                                  clamp=wl.clamp, out=setup)
    torch.cuda.synchronize()
    for T in (T1, T2):
        ref, got, free0, free1 = _pair(torch, g, T, wl.k, wl.clamp)
        assert torch.equal(got, ref), f"T={T}: the allocation-free call differs"
        assert free1 == free0, f"T={T}: device free memory changed by {free0 - free1} bytes"


def test_noalloc_rejects_sizes_beyond_its_scratch():
    import ctypes
    P = ctypes.c_void_p(0x10000)
    # 4096 tokens at d = I = 2880, E = 32, k = 4 need about 340 MB of scratch
    st = moe.lib().moe_layer_forward_noalloc(*([P] * 9), 4096, 2880, 2880, 32, 4, 7.0,
                                             ctypes.c_void_p(0x90000000), None)
    assert st == -8
    assert moe.moe_workspace_bytes(4096, 2880, 2880, 32, 4) > moe.MOE_NOALLOC_SCRATCH_BYTES
    assert moe.moe_workspace_bytes(32, 2880, 2880, 32, 4) <= moe.MOE_NOALLOC_SCRATCH_BYTES
