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
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    lines = open(src).read().splitlines()
    rec = json.loads([ln for ln in lines if ln.startswith("json:")][-1][5:])
    # a summary taken on these very sources is read ...
    rec["source_sha256_16"] = bench.src_digest(bench.KERNEL_SOURCES[kernel])
    body = [ln for ln in lines if not ln.startswith("json:")] + ["json:" + json.dumps(rec)]
    (tmp_path / "profiles" / f"traffic_{kernel}_dsv3.txt").write_text("\n".join(body) + "\n")
    assert bench.traffic_for(kernel, "dsv3") == rec["hbm_bytes_per_launch"]
    # ... and a change to any of the kernel's sources voids it
    for n in bench.KERNEL_SOURCES[kernel]:
        path = tmp_path / "combine_ep_route_topk_amd" / "csrc" / n
        keep = path.read_bytes()
        path.write_bytes(keep + b"\n// changed\n")
        assert bench.traffic_for(kernel, "dsv3") is None, n
        path.write_bytes(keep)
    assert bench.traffic_for(kernel, "dsv3") == rec["hbm_bytes_per_launch"]
    # a workload without a summary has none
    assert bench.traffic_for(kernel, "decode") is None


def test_committed_traffic_matches_its_digest_or_reads_null():
    """The committed summaries are read only where their digest is current."""
    for kernel, names in bench.KERNEL_SOURCES.items():
        src = os.path.join(ROOT, "profiles", f"traffic_{kernel}_dsv3.txt")
        if not os.path.exists(src):
            continue
        rec = json.loads([ln for ln in open(src) if ln.startswith("json:")][-1][5:])
        current = rec["source_sha256_16"] == bench.src_digest(names)
        assert bench.traffic_for(kernel, "dsv3") == (rec["hbm_bytes_per_launch"] if current else None)
