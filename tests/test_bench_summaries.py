"""The benchmark's rocprofv3 summarizers on small synthetic CSV files shaped like
rocprofv3's: counters scaled by the copy probe, clusters of dispatches of one kernel
instance, the per-call traffic of the decode kernels, and the kernel-trace table."""

import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

GATE = "void sfn::(anonymous namespace)::decode_gate_local_kernel<1, 1, 1, 512, 2, 2>(sfn::DecodeArgs)"
RED = "void sfn::(anonymous namespace)::decode_reduce_kernel(sfn::DecodeArgs, int)"
NEG = ("void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(at::TensorIteratorBase&)"
       "::{lambda()#1}, std::array<char*, 2ul> >(int, ...)")
FILL = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float> >(int, ...)"
PROBE = 1 << 30


def _write_counters(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "x_counter_collection.csv"), "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Grid_Size", "Kernel_Name", "Workgroup_Size", "Counter_Name", "Counter_Value"])
        for i, (name, grid, wg, kib) in enumerate(rows):
            w.writerow([i + 1, grid, name, wg, counter, kib])


def _counter_dirs(tmp_path):
    # FETCH reports half the bytes (as on the hardware), WRITE all of them; the gate kernel
    # runs at two densities (two clusters), the reduce at one
    mb = lambda x: x * 1e6 / 1024.0  # bytes -> KiB as the counters report them
    fetch = [(NEG, 1 << 28, 256, PROBE / 2 / 1024.0)] * 3 + [(FILL, 1 << 20, 256, 1.0)]
    fetch += [(GATE, 256 * 512, 512, mb(180.0) / 2)] * 5 + [(GATE, 256 * 512, 512, mb(108.0) / 2)] * 4
    fetch += [(RED, 128 * 512, 512, mb(4.2) / 2)] * 9
    write = [(NEG, 1 << 28, 256, PROBE / 1024.0)] * 3 + [(FILL, 1 << 20, 256, 1.0)]
    write += [(GATE, 256 * 512, 512, mb(4.2))] * 9 + [(RED, 128 * 512, 512, mb(0.02))] * 9
    fd, wd = tmp_path / "fetch", tmp_path / "write"
    _write_counters(str(fd), "FETCH_SIZE", fetch)
    _write_counters(str(wd), "WRITE_SIZE", write)
    return str(fd), str(wd)


def test_kernel_traffic_scales_by_the_probe_and_splits_clusters(tmp_path, capsys):
    fd, wd = _counter_dirs(tmp_path)
    assert bench.summarize_kernel_traffic(fd, wd, PROBE, "cmd") == 0
    out = capsys.readouterr().out
    assert "FETCH x 2.0000, WRITE x 1.0000" in out
    rows = [ln for ln in out.splitlines() if ln.startswith("| `")]
    gate = [ln for ln in rows if "decode_gate_local_kernel<1,1,1,512,2,2>" in ln]
    assert len(gate) == 2, rows  # the two densities stay apart
    assert "| 256 x 512 | 5 | 180.00 |" in gate[0] and "| 4.20 |" in gate[0]
    assert "| 256 x 512 | 4 | 108.00 |" in gate[1]
    red = [ln for ln in rows if "decode_reduce_kernel" in ln]
    assert len(red) == 1 and "| 128 x 512 | 9 | 4.20 |" in red[0] and red[0].endswith("| 0.02 |")
    assert not any("elementwise" in ln for ln in rows)  # torch's kernels are left out


def test_traffic_per_call_sums_the_call_kernels(tmp_path, monkeypatch, capsys):
    fd, wd = _counter_dirs(tmp_path)
    target = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(target))
    assert bench.write_traffic((fd, wd), PROBE, "cmd") == 0
    res = json.load(open(target))
    # medians: gate read 180 MB (5 of 9 dispatches), written 4.2; reduce read 4.2, written 0.02
    assert res["bytes_per_call"] == pytest.approx((180.0 + 4.2 + 4.2 + 0.02) * 1e6, rel=1e-9)
    assert res["counters"]["FETCH_SIZE"]["scale"] == pytest.approx(2.0)
    assert res["kernel_hash"] == bench.kernel_hash()
    capsys.readouterr()


def test_missing_probe_is_an_error(tmp_path):
    d = tmp_path / "nop"
    _write_counters(str(d), "FETCH_SIZE", [(GATE, 256 * 512, 512, 1.0)])
    with pytest.raises(SystemExit):
        bench.summarize_kernel_traffic(str(d), str(d), PROBE, "cmd")


def test_kernel_trace_groups_by_instance_and_grid(tmp_path, capsys):
    d = tmp_path / "trace"
    os.makedirs(d)
    with open(d / "x_kernel_trace.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z", "Workgroup_Size_X",
                    "Workgroup_Size_Y", "Workgroup_Size_Z", "Start_Timestamp", "End_Timestamp"])
        for i, us in enumerate((30.0, 32.0, 34.0)):
            w.writerow([GATE, 256 * 512, 1, 1, 512, 1, 1, 1000 * i * 100, 1000 * i * 100 + int(us * 1000)])
        w.writerow([RED, 128 * 512, 1, 1, 512, 1, 1, 0, 4000])
        w.writerow([RED, 512 * 512, 1, 1, 512, 1, 1, 0, 8000])
        w.writerow([FILL, 1024, 1, 1, 256, 1, 1, 0, 1000])
    bench.summarize_trace(str(d), "cmd")
    out = capsys.readouterr().out
    assert "| `decode_gate_local_kernel<1,1,1,512,2,2>` | 256 x 512 | 3 | 32.00 | 32.00 | 30.00 | 34.00 |" in out
    assert "| `decode_reduce_kernel` | 128 x 512 | 1 | 4.00 |" in out
    assert "| `decode_reduce_kernel` | 512 x 512 | 1 | 8.00 |" in out
    assert "| (torch kernels: input generation, copies) | | 1 | 1.00 |" in out


def test_bench_refuses_more_than_one_gpu():
    """The benchmark measures one GPU: --gpus above 1 exits with status 2 and says so,
    before anything touches a device."""
    import subprocess
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU only" in res.stderr and res.stdout == ""
