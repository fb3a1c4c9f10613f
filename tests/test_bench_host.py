"""Host-side logic of the benchmark and of the profile summaries (no GPU)."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_traffic_is_scaled_by_the_copy_kernel(tmp_path, capsys):
    from sparse_moe_transformer_softmax_amd import profsum
    # the copy moves 1 MiB each way; its fetch counter reads half of that
    # (two dispatches of the kernel, counters split over two rows each)
    fetch = [dict(Dispatch_Id=1, Kernel_Name="bitwise_not_kernel", Counter_Name="FETCH_SIZE", Counter_Value=512.0)]
    write = [dict(Dispatch_Id=1, Kernel_Name="bitwise_not_kernel", Counter_Name="WRITE_SIZE", Counter_Value=1024.0)]
    for d, (fv, wv) in enumerate([(100.0, 10.0), (300.0, 30.0)], start=2):
        fetch += [dict(Dispatch_Id=d, Kernel_Name="my_gemm<1>", Counter_Name="FETCH_SIZE", Counter_Value=fv / 2)] * 2
        write += [dict(Dispatch_Id=d, Kernel_Name="my_gemm<1>", Counter_Name="WRITE_SIZE", Counter_Value=wv)]
    fp, wp = tmp_path / "f.csv", tmp_path / "w.csv"
    _counter_csv(fp, fetch)
    _counter_csv(wp, write)
    profsum.main(["traffic", "--fetch", str(fp), "--write", str(wp), "--kernel", "my_gemm<1>",
                  "--copy-kernel", "bitwise_not", "--copy-bytes", str(1 << 20)])
    out = dict(l.split(": ", 1) for l in capsys.readouterr().out.splitlines() if ": " in l and not l.startswith("#"))
    # mean raw fetch 200 KiB x 2 (scale) = 400 KiB; write 20 KiB x 1
    assert float(out["fetch_scale"]) == pytest.approx(2.0)
    assert float(out["write_scale"]) == pytest.approx(1.0)
    assert float(out["traffic_bytes_per_launch"]) == pytest.approx((400 + 20) * 1024)
    assert out["src_sha"].strip() == profsum.src_sha()


def test_traffic_summary_is_ignored_once_sources_change(tmp_path, monkeypatch):
    import bench
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic_gateup_gemm_wl.txt").write_text("traffic_bytes_per_launch: 1234\nsrc_sha: 0000000000000000\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.read_traffic("gateup_gemm", "wl") is None
    from sparse_moe_transformer_softmax_amd.profsum import src_sha
    (prof / "traffic_gateup_gemm_wl.txt").write_text(f"traffic_bytes_per_launch: 1234\nsrc_sha: {src_sha()}\n")
    assert bench.read_traffic("gateup_gemm", "wl") == 1234.0
    assert bench.read_traffic("down_gemm", "wl") is None
