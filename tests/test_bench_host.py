"""Host-side logic of bench.py (no GPU): the stored counter figures are used only for the
kernel sources they were measured on, and the one-GPU limit is reported, not ignored."""
import json
import os
import shutil
import subprocess
import sys

import bench

CSRC = os.path.join(bench.ROOT, "bit_quantized_linear_vq_amd", "csrc")
WORKLOAD = "c2_qkv_w8a8_per_token"


def copy_tree(tmp_path):
    root = tmp_path / "repo"
    shutil.copytree(CSRC, root / "bit_quantized_linear_vq_amd" / "csrc")
    (root / "profiles").mkdir()
    return root


def write_traffic(root, gemm_sha, quant_sha):
    entry = {"kernel_sha": gemm_sha, "bytes_per_launch": 123, "quant_kernel_sha": quant_sha,
             "quant_fetch_bytes": 10, "quant_write_bytes": 5}
    (root / "profiles" / "qgemm_traffic.json").write_text(json.dumps({WORKLOAD: entry}))


def test_traffic_follows_the_kernel_sources(tmp_path, monkeypatch):
    root = copy_tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(root))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(root / "profiles" / "qgemm_traffic.json"))
    g0, q0 = bench.kernel_hash("k_qgemm.hip"), bench.kernel_hash("k_quant.hip")
    write_traffic(root, g0, q0)
    assert bench.load_traffic(WORKLOAD) == (123, 15)
    assert bench.load_traffic("no_such_workload") == (None, None)

    # A header the GEMM includes changes: its figure is dropped, the quantizer's kept.
    hdr = root / "bit_quantized_linear_vq_amd" / "csrc" / "gemm_common.h"
    hdr.write_text(hdr.read_text() + "\n// edited\n")
    assert bench.kernel_hash("k_qgemm.hip") != g0
    assert bench.kernel_hash("k_quant.hip") == q0
    assert bench.load_traffic(WORKLOAD) == (None, 15)

    # A header both include changes: both figures are dropped.
    common = root / "bit_quantized_linear_vq_amd" / "csrc" / "dev_common.h"
    common.write_text(common.read_text() + "\n// edited\n")
    assert bench.kernel_hash("k_quant.hip") != q0
    assert bench.load_traffic(WORKLOAD) == (None, None)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "GPU" in (r.stdout + r.stderr)
