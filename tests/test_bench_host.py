"""Host-side logic of bench.py (no GPU): the algorithmic byte count, the counter
calibration that turns rocprofv3 FETCH_SIZE / WRITE_SIZE readings into HBM bytes, and the
refusal of a multi-GPU run."""
import csv
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_of_the_metric_layer():
    # 2 planes of 4096 x 11008 bits + fp16 g (2 x 4096) + fp16 x (11008) + fp16 y (4096)
    assert bench.algorithmic_bytes(4096, 11008, 2) == 11_272_192 + 16_384 + 22_016 + 8_192
    assert bench.algorithmic_bytes(4096, 11008, 2) == 11_318_784
    assert bench.algorithmic_bytes(28672, 8192, 1, M=4) == 28672 * 8192 // 8 + 2 * 28672 + 2 * 4 * 8192 + 2 * 4 * 28672


def _write_counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Counter_Name", "Kernel_Name", "Dispatch_Id", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_counter_calibration(tmp_path):
    # FETCH_SIZE read at half scale on this part: the stream-read kernel's known bytes fix
    # the factor; WRITE_SIZE is calibrated on the weight copy. Two dispatches of the
    # product, each reported as two partial rows (summed per dispatch), median taken.
    nbytes = bench.algorithmic_bytes(bench.N_ROWS, bench.K_COLS, bench.K_PLANES)
    stream_kib = (nbytes // 256 * 256) / 1024.0 / 2.0          # half of the true bytes
    Kw = (bench.K_COLS + 31) // 32
    copy_bytes = bench.K_PLANES * bench.N_ROWS * ((Kw + 31) // 32 * 32) * 4
    prod = "void rb::(anonymous namespace)::gemv_nib1_kernel<2, 5, true, 1, 1, false>(unsigned int const*)"
    other = "void rb::(anonymous namespace)::gemv_nib_kernel<__half, __half, __half, 2, 3, 1, 16, 12>(unsigned int const*)"
    d = tmp_path / "run"
    d.mkdir()
    _write_counters(d / "f_counter_collection.csv", [
        {"Counter_Name": "FETCH_SIZE", "Kernel_Name": prod, "Dispatch_Id": 1, "Counter_Value": 2000.0},
        {"Counter_Name": "FETCH_SIZE", "Kernel_Name": prod, "Dispatch_Id": 1, "Counter_Value": 1000.0},
        {"Counter_Name": "FETCH_SIZE", "Kernel_Name": prod, "Dispatch_Id": 2, "Counter_Value": 3000.0},
        # the general-h kernel is another kernel: not counted
        {"Counter_Name": "FETCH_SIZE", "Kernel_Name": other, "Dispatch_Id": 6, "Counter_Value": 9000.0},
        {"Counter_Name": "FETCH_SIZE", "Kernel_Name": other, "Dispatch_Id": 7, "Counter_Value": 9000.0},
        {"Counter_Name": "FETCH_SIZE", "Kernel_Name": "stream_read_kernel", "Dispatch_Id": 3, "Counter_Value": stream_kib},
    ])
    _write_counters(d / "w_counter_collection.csv", [
        {"Counter_Name": "WRITE_SIZE", "Kernel_Name": prod, "Dispatch_Id": 4, "Counter_Value": 8.0},
        {"Counter_Name": "WRITE_SIZE", "Kernel_Name": "__amd_rocclr_copyBuffer", "Dispatch_Id": 5,
         "Counter_Value": copy_bytes / 1024.0},
    ])
    out = tmp_path / "rec.json"
    assert bench.summarize_counters(str(tmp_path), str(out)) == 0
    rec = json.loads(out.read_text())
    assert abs(rec["fetch_scale"] - 2.0) < 1e-9 and abs(rec["write_scale"] - 1.0) < 1e-12
    assert rec["fetch_kib_per_dispatch"] == 3000.0                 # both dispatches read 3000 KiB
    assert rec["hbm_bytes_per_launch"] == round(3000.0 * 1024 * 2.0 + 8.0 * 1024)
    assert rec["kernel_source_hash"] == bench.kernel_source_hash()


def test_multi_gpu_request_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_kernel_hash_ignores_comments_not_code(tmp_path, monkeypatch):
    src = "// header\nint f(int a) {  // add one\n  return a + 1; /* block\n comment */\n}\n"
    p = tmp_path / "k.hip"
    p.write_text(src)
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(p)])
    h0 = bench.kernel_source_hash()
    p.write_text(src.replace("// add one", "// adds one to a").replace("block\n comment", "other"))
    assert bench.kernel_source_hash() == h0
    p.write_text(src.replace("a + 1", "a + 2"))
    assert bench.kernel_source_hash() != h0
