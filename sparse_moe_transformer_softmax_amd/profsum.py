"""Short text summaries of rocprofv3 CSV output, for the committed profiles.

    python -m sparse_moe_transformer_softmax_amd.profsum stats KERNEL_STATS_CSV [--cmd CMD]
    python -m sparse_moe_transformer_softmax_amd.profsum traffic --fetch CSV --write CSV \
        --kernel SUBSTR --copy-kernel SUBSTR --copy-bytes BYTES [--cmd CMD]
    python -m sparse_moe_transformer_softmax_amd.profsum busy COUNTER_CSV --kernel SUBSTR [--cmd CMD]

`stats` prints the per-kernel call count and mean/min/max duration from a
`--kernel-trace --stats --output-format csv` run.  `traffic` reads two
`--pmc FETCH_SIZE` / `--pmc WRITE_SIZE` counter-collection files (KiB per
dispatch), scales each counter by what it reads for a reference copy kernel
that moves a known number of bytes each way, and prints the HBM bytes per
launch of the kernel whose name contains SUBSTR, as `key: value` lines that
bench.py reads back (with the hash of the kernel sources they belong to).
`busy` prints the MFMA-busy share of a kernel from a `--pmc
SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE` run.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


# sources no MoE-layer kernel is built from (the attention steps beside the
# layer): a change there leaves the layer's counter summaries valid
NOT_LAYER_SOURCES = ("attention.hip",)


def src_sha() -> str:
    """Hash of the MoE layer's HIP sources (kernels, the launch code that
    picks them, the weight packing); a counter summary is valid only for
    these."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_moe_transformer_softmax_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if not f.endswith((".hip", ".h")) or f in NOT_LAYER_SOURCES:
            continue
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def short_name(n: str) -> str:
    n = n.strip('"')
    if n.startswith("void "):
        n = n[5:]
    return n if len(n) <= 90 else n[:87] + "..."


def cmd_stats(args) -> None:
    rows = list(csv.DictReader(open(args.csv)))
    print(f"# rocprofv3 kernel statistics")
    if args.cmd:
        print(f"# command: {args.cmd}")
    print(f"{'kernel':90s} {'calls':>6s} {'mean_us':>9s} {'min_us':>9s} {'max_us':>9s} {'pct':>6s}")
    for r in rows:
        print(f"{short_name(r['Name']):90s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} "
              f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} {float(r['Percentage']):6.2f}")


def per_dispatch(path: str, counter: str, substr: str):
    vals = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter or substr not in r["Kernel_Name"]:
            continue
        did = r["Dispatch_Id"]
        vals[did] = vals.get(did, 0.0) + float(r["Counter_Value"])
    return list(vals.values())


def cmd_traffic(args) -> None:
    f_k = per_dispatch(args.fetch, "FETCH_SIZE", args.kernel)
    w_k = per_dispatch(args.write, "WRITE_SIZE", args.kernel)
    f_c = per_dispatch(args.fetch, "FETCH_SIZE", args.copy_kernel)
    w_c = per_dispatch(args.write, "WRITE_SIZE", args.copy_kernel)
    if not (f_k and w_k and f_c and w_c):
        sys.exit(f"missing dispatches: kernel fetch {len(f_k)} write {len(w_k)}, copy fetch {len(f_c)} write {len(w_c)}")
    kib = 1024.0
    # the copy reads and writes copy_bytes: counter KiB -> true bytes
    f_scale = args.copy_bytes / (max(f_c) * kib)
    w_scale = args.copy_bytes / (max(w_c) * kib)
    fetch = statistics.mean(f_k) * kib * f_scale
    write = statistics.mean(w_k) * kib * w_scale
    print("# HBM traffic per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE counters")
    if args.cmd:
        for c in args.cmd:
            print(f"# command: {c}")
    print(f"kernel: {args.kernel}")
    print(f"dispatches: {len(f_k)} fetch, {len(w_k)} write")
    print(f"copy_reference: {args.copy_kernel} moving {args.copy_bytes} bytes each way")
    print(f"copy_fetch_KiB: {max(f_c):.1f}")
    print(f"copy_write_KiB: {max(w_c):.1f}")
    print(f"fetch_scale: {f_scale:.4f}")
    print(f"write_scale: {w_scale:.4f}")
    print(f"fetch_KiB_per_launch_raw: {statistics.mean(f_k):.1f}")
    print(f"write_KiB_per_launch_raw: {statistics.mean(w_k):.1f}")
    print(f"fetch_bytes_per_launch: {fetch:.0f}")
    print(f"write_bytes_per_launch: {write:.0f}")
    print(f"traffic_bytes_per_launch: {fetch + write:.0f}")
    print(f"src_sha: {src_sha()}")


def cmd_busy(args) -> None:
    """MFMA-busy share of one kernel from SQ_VALU_MFMA_BUSY_CYCLES (summed over
    every SIMD) and GRBM_GUI_ACTIVE (summed over the XCDs): busy /
    (simds * active / xcds)."""
    busy = per_dispatch(args.csv, "SQ_VALU_MFMA_BUSY_CYCLES", args.kernel)
    active = per_dispatch(args.csv, "GRBM_GUI_ACTIVE", args.kernel)
    sq = per_dispatch(args.csv, "SQ_BUSY_CYCLES", args.kernel)
    if not (busy and active):
        sys.exit(f"missing dispatches: busy {len(busy)} active {len(active)}")
    simds, xcds = args.cus * 4, args.xcds
    frac = statistics.mean(busy) / simds / (statistics.mean(active) / xcds)
    print("# MFMA-busy share of a kernel from rocprofv3 counters")
    if args.cmd:
        for c in args.cmd:
            print(f"# command: {c}")
    print(f"kernel: {args.kernel}")
    print(f"dispatches: {len(busy)}")
    print(f"SQ_VALU_MFMA_BUSY_CYCLES_per_dispatch: {statistics.mean(busy):.0f}")
    print(f"GRBM_GUI_ACTIVE_per_dispatch: {statistics.mean(active):.0f}")
    if sq:
        print(f"SQ_BUSY_CYCLES_per_dispatch: {statistics.mean(sq):.0f}")
    print(f"simds: {simds}")
    print(f"xcds: {xcds}")
    print(f"mfma_busy_frac: {frac:.4f}")
    print(f"src_sha: {src_sha()}")


def main(argv=None) -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--cmd", default="")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--copy-kernel", required=True)
    t.add_argument("--copy-bytes", type=float, required=True)
    t.add_argument("--cmd", action="append", default=[])
    b = sub.add_parser("busy")
    b.add_argument("csv")
    b.add_argument("--kernel", required=True)
    b.add_argument("--cus", type=int, default=256)
    b.add_argument("--xcds", type=int, default=8)
    b.add_argument("--cmd", action="append", default=[])
    args = ap.parse_args(argv)
    if args.cmd_name == "stats":
        cmd_stats(args)
    elif args.cmd_name == "busy":
        cmd_busy(args)
    else:
        cmd_traffic(args)


if __name__ == "__main__":
    main()
