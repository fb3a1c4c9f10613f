"""The packed weight layout (moe_pack_weights, MOE_LAYER_PACKED) on the GPU:
the packing is a byte permutation, checked bit for bit against the layout
written out in numpy here; and a layer (or the stack) on packed weights must
give bitwise the results of the same call on the row-major weights (the
kernels copy the same bytes into the same LDS places and do the same
arithmetic in the same order) -- at decode sizes (16- and 32-row tiles, the
combine folded into the down projection, more than 8 phases of K) and at
prefill sizes (64- and 128-row tiles)."""
import sys

import numpy as np
import pytest

from moe_inputs import synth
from moe_inputs.workloads import WORKLOADS, Workload
from oracle.workload_inputs import make_inputs
import sparse_moe_transformer_softmax_amd as moe
from tests.parity_util import KEYS, to_gpu

pytestmark = pytest.mark.gpu

WKEYS = ["w13_codes", "w13_scales", "w2_codes", "w2_scales"]


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "no GPU"
    moe.lib()
    return _t


def pack_reference(codes, scales):
    """The packed layout, written out: for each pair of rows and each chunk
    of four 32-element blocks, the even row's chunk bytes then the odd
    row's; scales chunk-major, four per row, 127 past the last block."""
    E, N, half = codes.shape
    K = 2 * half
    nblk = K // 32
    nchk = (nblk + 3) // 4
    out = np.empty((E, N // 2, K), dtype=np.uint8)
    for c in range(nchk):
        w = 16 * min(4, nblk - 4 * c)
        out[:, :, 128 * c:128 * c + w] = codes[:, 0::2, 64 * c:64 * c + w]
        out[:, :, 128 * c + w:128 * c + 2 * w] = codes[:, 1::2, 64 * c:64 * c + w]
    sc = np.full((E, nchk, N, 4), 127, dtype=np.uint8)
    for c in range(nchk):
        for q in range(4):
            if 4 * c + q < nblk:
                sc[:, c, :, q] = scales[:, :, 4 * c + q]
    return out, sc


@pytest.mark.parametrize("E,N,K", [(2, 64, 128), (3, 10, 192), (1, 2, 64), (4, 96, 2880), (2, 5760, 2880)])
def test_pack_is_the_written_out_permutation(torch, E, N, K):
    say(f"pack E={E} N={N} K={K}")
    codes, scales = synth.gen_mxfp4(77 + N, 20, 21, E, N, K)
    c_ref, s_ref = pack_reference(codes, scales)
    co, so = moe.moe_pack_weights(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(co.cpu().numpy(), c_ref)
    assert np.array_equal(so.cpu().numpy(), s_ref)


def _packed(torch, g):
    p = dict(g)
    p["w13_codes"], p["w13_scales"] = moe.moe_pack_weights(g["w13_codes"], g["w13_scales"])
    p["w2_codes"], p["w2_scales"] = moe.moe_pack_weights(g["w2_codes"], g["w2_scales"])
    return p


CASES = [
    ("tiny", None),
    ("20b_decode", None),
    ("qwen3_decode", None),
    ("20b_batch256", None),
    ("decode_k4160", Workload("decode_k4160", T=8, d=4160, I=64, E=8, k=4, seed=0x5EED3003)),
    ("20b_prefill", None),
    ("120b_prefill_zipf", None),
    ("stack_layer", Workload("stack_layer", T=2048, d=2880, I=2880, E=128, k=4, seed=0x5EED1007)),
    ("ragged", Workload("ragged", T=333, d=256, I=192, E=8, k=4, seed=0x5EED3001)),
    ("ragged_k8", Workload("ragged_k8", T=1000, d=384, I=320, E=16, k=8, seed=0x5EED3002)),
    ("wide64_ragged", Workload("wide64_ragged", T=600, d=320, I=384, E=64, k=4, seed=0x5EED3004)),
]


# every case with the stored activation reading, and the variant one (interleaved gate/up rows)
# on the shapes that exercise each kernel once
ALT_ON = ("tiny", "20b_decode", "qwen3_decode", "20b_prefill", "ragged", "ragged_k8", "wide64_ragged")
RUNS = [(n, w, 0) for n, w in CASES] + [(n, w, moe.MOE_LAYER_ALT_ACT) for n, w in CASES if n in ALT_ON]


@pytest.mark.parametrize("name,wl,alt", RUNS, ids=[f"{n}-alt{a}" for n, _, a in RUNS])
def test_packed_layer_equals_row_major_bitwise(torch, name, wl, alt):
    wl = wl or WORKLOADS[name]
    say(f"packed vs row-major {name} alt={alt}")
    inp = make_inputs(wl, condition=False)
    g = to_gpu(inp)
    p = _packed(torch, g)
    a = moe.moe_layer_forward_ex(*[g[k] for k in KEYS], k=wl.k, clamp=wl.clamp, flags=alt, debug=True)
    b = moe.moe_layer_forward_ex(*[p[k] for k in KEYS], k=wl.k, clamp=wl.clamp, flags=alt | moe.MOE_LAYER_PACKED,
                                 debug=True)
    torch.cuda.synchronize()
    for x, y, what in zip(a, b, ["out", "out_f32", "ids", "w", "counts"]):
        assert torch.equal(x, y), what


def test_packed_stack_equals_row_major_bitwise(torch):
    wl = WORKLOADS["120b_stack36"]
    n = 3
    say(f"packed stack vs row-major, {n} layers of the 120b stack")
    layers, packed, x0 = [], [], None
    for l in range(n):
        g = to_gpu(make_inputs(wl, layer=l, condition=False))
        if l == 0:
            x0 = g["x"]
        lk = {k: g[k] for k in KEYS[1:]}
        layers.append(lk)
        packed.append(_packed(torch, lk))
    a = moe.moe_stack_forward(x0, layers, k=wl.k, clamp=wl.clamp, eps=1e-5)
    b = moe.moe_stack_forward(x0, packed, k=wl.k, clamp=wl.clamp, eps=1e-5, flags=moe.MOE_LAYER_PACKED)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
