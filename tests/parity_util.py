"""Helpers of the GPU parity tests: upload of generated inputs, the bf16
output tolerance, and routing comparisons."""
from __future__ import annotations

import numpy as np

from oracle import moe_oracle as O

KEYS = ["x", "router_w", "router_b", "w13_codes", "w13_scales", "b13", "w2_codes", "w2_scales", "b2"]


def to_gpu(inp: dict, device="cuda:0") -> dict:
    import torch
    out = {}
    for kk in KEYS:
        a = np.ascontiguousarray(inp[kk])
        if a.dtype == np.uint16:
            t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(a)
        out[kk] = t.to(device)
    return out


def bf16_half_ulp(ref: np.ndarray) -> np.ndarray:
    """Half a bf16 unit in the last place at each reference value."""
    a = np.abs(ref)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126)
    return np.where(a > 0, 0.5 * np.exp2(e - 7), 0.5 * 2.0 ** -133)


def bf16_excess(out_bf16: np.ndarray, ref: np.ndarray) -> float:
    """max(|out - ref| - half ulp(ref)) / rms(ref): the error beyond the final
    bf16 rounding of the exact result, relative to the output rms."""
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return float(np.max(np.abs(out_bf16 - ref) - bf16_half_ulp(ref)) / rms)


def rel_max_err(out: np.ndarray, ref: np.ndarray) -> float:
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return float(np.max(np.abs(out - ref)) / rms)


TOL = 1e-2  # max |err| <= 1e-2 * rms(ref)
# gate weights, relative.  The pages fix no precision for the router; the
# kernel sums each logit's d = 2880 exact bf16 products in fp32, about d/32
# + 24 roundings of partial sums of order 1-3, i.e. a logit error of order
# sqrt(114) * 2^-24 * 2 ~ 2e-6 in the far tail, and a selected-softmax weight
# moves by at most twice the largest logit error in relative terms.  The
# largest error measured over every case (E 8 .. 256, d up to 4160) is
# 1.1e-6.
W_TOL = 4e-6


def bf16_tensor_to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def check_routing(ids_gpu: np.ndarray, w_gpu: np.ndarray, counts_gpu: np.ndarray, ref: dict, E: int):
    """Expert sets bit-exact per token, counts bit-exact, weights matched by
    expert id within W_TOL relative."""
    ids_ref, w_ref = ref["ids"], ref["w"]
    T, k = ids_ref.shape
    order_g = np.argsort(ids_gpu, axis=1, kind="stable")
    order_r = np.argsort(ids_ref, axis=1, kind="stable")
    sg = np.take_along_axis(ids_gpu, order_g, 1)
    sr = np.take_along_axis(ids_ref, order_r, 1)
    bad = np.nonzero(np.any(sg != sr, axis=1))[0]
    assert bad.size == 0, f"{bad.size} tokens with different expert sets, first {bad[:8]}"
    wg = np.take_along_axis(w_gpu, order_g, 1)
    wr = np.take_along_axis(w_ref, order_r, 1)
    werr = float(np.max(np.abs(wg - wr) / np.abs(wr)))
    print(f"[gpu-case]   gate weight max rel err {werr:.2e}", flush=True)
    assert werr <= W_TOL
    assert np.array_equal(counts_gpu, np.bincount(ids_ref.reshape(-1), minlength=E))
    # slots in descending logit order
    lg = np.take_along_axis(ref["logits"], ids_gpu.astype(np.int64), 1)
    assert np.all(np.diff(lg, axis=1) <= 1e-5)
