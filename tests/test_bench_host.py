"""Host logic of bench.py (CPU): the one-GPU contract and the traffic field.

The roofline's `traffic` comes from a committed rocprofv3 summary and must
read null once the kernel's sources differ from those the counters were taken
on; a run asked for more than one GPU must exit with a message saying so.
"""
import json
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_kernel_sources_exist():
    for names in bench.KERNEL_SOURCES.values():
        for n in names:
            assert os.path.exists(os.path.join(ROOT, "combine_ep_route_topk_amd", "csrc", n)), n


@pytest.mark.parametrize("kernel", sorted(bench.KERNEL_SOURCES))
def test_traffic_reads_null_when_the_sources_changed(kernel, tmp_path, monkeypatch):
    src = os.path.join(ROOT, "profiles", f"traffic_{kernel}_dsv3.txt")
    if not os.path.exists(src):
        pytest.skip("no summary for this kernel")
    os.makedirs(tmp_path / "profiles")
    shutil.copytree(os.path.join(ROOT, "combine_ep_route_topk_amd", "csrc"),
                    tmp_path / "combine_ep_route_topk_amd" / "csrc")
    shutil.copy(src, tmp_path / "profiles")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    rec = json.loads([ln for ln in open(src) if ln.startswith("json:")][-1][5:])
    got = bench.traffic_for(kernel, "dsv3")
    # the committed summary matches the committed sources
    assert got == rec["hbm_bytes_per_launch"]
    # a change to any of the kernel's sources voids it
    first = bench.KERNEL_SOURCES[kernel][0]
    with open(tmp_path / "combine_ep_route_topk_amd" / "csrc" / first, "a") as f:
        f.write("\n// changed\n")
    assert bench.traffic_for(kernel, "dsv3") is None
    # and a workload without a summary has none
    assert bench.traffic_for(kernel, "decode") is None
