"""Host-side logic of bench.py (CPU only): the GPU-count guard and the
conversion of rocprofv3 counter CSVs into HBM bytes per launch."""
import csv
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=_FIELDS)
        w.writeheader()
        for i, (name, kib) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": kib})


def test_traffic_from_counters_scales_by_calibration(tmp_path):
    calib = 256 << 20
    kern = "void pa::decode_partial_mfma_kernel<128, true>(pa::DecodeParams)"
    other = "void pa::decode_partial_kernel<float, 128, 1, 2, 4, 1>(pa::DecodeParams)"
    copy = "void at::native::vectorized_elementwise_kernel<4, AUnaryFunctor<float, float, float, MulFunctor<float>>>"
    # the counters read 10% high on the copy: the kernel's reading is scaled down by 1/1.1
    _csv(tmp_path / "f.csv", "FETCH_SIZE",
         [(copy, calib * 1.1 / 1024), (kern, 1100.0), (kern, 1100.0), (other, 5e6), (copy, calib * 1.1 / 1024)])
    _csv(tmp_path / "w.csv", "WRITE_SIZE", [(copy, calib / 1024), (kern, 10.0), (kern, 30.0)])
    out = tmp_path / "t.json"
    r = bench.traffic_from_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                                    "llama3_8b_bf16", "bf16", calib, str(out))
    assert r["fetch_size"]["dispatches"] == 2
    assert r["fetch_size"]["bytes_per_launch"] == 1000 * 1024
    assert r["write_size"]["bytes_per_launch"] == 20 * 1024
    assert r["bytes_per_launch"] == 1020 * 1024
    assert json.loads(out.read_text()) == r
    assert r["source_sha256_16"] == bench._src_hash("bf16")


def test_traffic_file_ignored_when_stale(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    p = tmp_path / "traffic_decode_partial_mfma_kernel_llama3_8b_bf16.json"
    p.write_text(json.dumps({"workload": "llama3_8b_bf16", "source_sha256_16": "0" * 16,
                             "bytes_per_launch": 5}))
    assert bench._traffic("llama3_8b_bf16", "bf16") is None
    p.write_text(json.dumps({"workload": "llama3_8b_bf16", "source_sha256_16": bench._src_hash("bf16"),
                             "bytes_per_launch": 5}))
    assert bench._traffic("llama3_8b_bf16", "bf16") == 5
    assert bench._traffic("big_batch_bf16", "bf16") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_of_the_write_kernel(tmp_path):
    """The write kernel's rows are picked by name (not the vLLM-layout write's),
    hashed against its own source and written to its own summary."""
    calib = 256 << 20
    copy = "void at::native::vectorized_elementwise_kernel<4, AUnaryFunctor<float, float, float, MulFunctor<float>>>"
    kern = "pa::write_kv_kernel(unsigned int __vector(4)*, unsigned int __vector(4)*, long const*)"
    vllm = "void pa::write_kv_vllm_kernel<unsigned short>(unsigned int __vector(4)*, unsigned short*)"
    _csv(tmp_path / "f.csv", "FETCH_SIZE", [(copy, calib / 2048), (kern, 300.0), (vllm, 9e6)])
    _csv(tmp_path / "w.csv", "WRITE_SIZE", [(copy, calib / 1024), (kern, 200.0), (vllm, 9e6)])
    r = bench.traffic_from_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                                    "write_65536_bf16", "write", calib, str(tmp_path / "t.json"))
    assert r["kernel"] == "write_kv_kernel" and r["fetch_size"]["dispatches"] == 1
    assert r["fetch_size"]["bytes_per_launch"] == 600 * 1024          # FETCH read half: scale 2
    assert r["bytes_per_launch"] == 800 * 1024
    assert r["source_sha256_16"] == bench._src_hash("write") != bench._src_hash("bf16")
    assert bench._traffic_file("write", "w").endswith("traffic_write_kv_kernel_w.json")


def test_traffic_in_vllm_layout(tmp_path, monkeypatch):
    """In vLLM's cache layout the write's counters come from the vLLM-layout
    kernel and go to a summary of their own, which a P09-layout line never
    reads (and the other way round)."""
    calib = 256 << 20
    copy = "void at::native::vectorized_elementwise_kernel<4, AUnaryFunctor<float, float, float, MulFunctor<float>>>"
    kern = "pa::write_kv_kernel(unsigned int __vector(4)*, unsigned int __vector(4)*, long const*)"
    vllm = "void pa::write_kv_vllm_kernel<unsigned short>(unsigned int __vector(4)*, unsigned short*)"
    _csv(tmp_path / "f.csv", "FETCH_SIZE", [(copy, calib / 2048), (kern, 9e6), (vllm, 300.0)])
    _csv(tmp_path / "w.csv", "WRITE_SIZE", [(copy, calib / 1024), (kern, 9e6), (vllm, 200.0)])
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    out = bench._traffic_file("write", "w", "vllm")
    assert out.endswith("traffic_write_kv_vllm_kernel_w_vllm.json")
    r = bench.traffic_from_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "w", "write", calib, out,
                                    "vllm")
    assert r["kernel"] == "write_kv_vllm_kernel" and r["layout"] == "vllm"
    assert r["bytes_per_launch"] == 800 * 1024
    assert bench._traffic("w", "write", "vllm") == 800 * 1024
    assert bench._traffic("w", "write") is None
    # the bf16 decode runs one template in both layouts: the layouts still keep separate files
    assert bench._traffic_file("bf16", "c", "vllm").endswith("traffic_decode_partial_mfma_kernel_c_vllm.json")
    assert bench._src_hash("f32", "vllm") == bench._src_hash("bf16") != bench._src_hash("f32")
