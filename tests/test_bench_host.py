"""Host-side tests of bench.py's own logic (no GPU): the one-GPU guard, the
option defaults it records, the algorithmic bytes the roofline divides by,
and the rule that a committed traffic figure is used only while the kernel
source it was measured on is unchanged."""

from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("argv,want", [
    ([], "auto"),
    (["--workload", "decode"], "auto"),
    (["--workload", "training"], "streaming"),
    (["--workload", "training", "--combine-stores", "cached"], "cached"),
    (["--workload", "prefill", "--combine-stores", "streaming"], "streaming"),
])
def test_combine_store_default_per_workload(monkeypatch, argv, want):
    monkeypatch.setattr(sys, "argv", ["bench.py", *argv])
    assert bench.parse().combine_stores == want


def test_prefill_algorithmic_bytes_from_the_definitions():
    # T = 4096 tokens of H = 7168 bf16 channels, top-8: x read once, each of
    # the T*k receive rows written once by dispatch and read once by combine,
    # y written once, plus the int32 / fp32 routing metadata
    c = workloads.get_config("prefill", 8.0)
    T, H, k = 4096, 7168, 8
    assert (c.T, c.H, c.k) == (T, H, k)
    ab = bench.algorithmic_bytes(c)
    assert ab["dispatch"] == 58_720_256 + 469_762_048 + 131_072          # x, rows, dst
    assert ab["combine"] == 469_762_048 + 2 * 131_072 + 58_720_256       # rows, dst + w, y
    assert ab["plan"] == 2 * 131_072                                       # ids read, dst written
    assert ab["plan"] + ab["dispatch"] + ab["combine"] == 1_057_619_968


def test_fp8_dispatch_bytes_count_codes_and_scales():
    c = workloads.get_config("prefill", 8.0)
    n = c.T * c.k
    ab = bench.algorithmic_bytes(c, fp8=True)
    assert ab["dispatch"] == c.T * c.H * 2 + n * (c.H + c.H // 128 * 4) + n * 4


def test_training_backward_bytes():
    c = workloads.get_config("training", 8.0)
    n, row = c.T * c.k, c.H * 2
    ab = bench.algorithmic_bytes(c)
    # gy once, the k expert rows read, the k gradient rows written, dst / w /
    # grad_w metadata
    assert ab["combine_bwd"] == c.T * row + 2 * n * row + 16 * n
    assert ab["dispatch_bwd"] == n * row + 4 * n + c.T * row


def _fake_tree(tmp_path, text):
    csrc = tmp_path / "combine_ep_plan_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "combine.hip").write_text(text)
    (csrc / "device.h").write_text("// helpers\n")
    (tmp_path / "profiles").mkdir()
    return csrc


def test_traffic_is_used_only_on_the_source_it_was_measured_on(tmp_path, monkeypatch):
    csrc = _fake_tree(tmp_path, "// combine v1\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h = bench.source_hash(bench.KERNEL_SOURCES["combine"])
    rec = {"workload": "prefill", "kernels": {
        "combine": {"source_hash": h, "bytes_per_launch": 529_560_080}}}
    (tmp_path / "profiles" / "traffic_prefill.json").write_text(json.dumps(rec))
    assert bench.traffic_for("prefill", "combine") == 529_560_080
    assert bench.traffic_for("prefill", "dispatch") is None          # not measured
    assert bench.traffic_for("training", "combine") is None          # no such file
    (csrc / "combine.hip").write_text("// combine v2\n")
    assert bench.traffic_for("prefill", "combine") is None          # kernel changed since


def test_committed_traffic_records_name_known_kernels():
    for wl in ("prefill", "training"):
        path = os.path.join(ROOT, "profiles", f"traffic_{wl}.json")
        with open(path) as fh:
            d = json.load(fh)
        assert d["workload"] == wl
        for op, rec in d["kernels"].items():
            assert op in bench.KERNEL_SOURCES
            # fabric bytes are the algorithmic bytes or a little more
            assert rec["algorithmic_bytes"] <= rec["bytes_per_launch"] <= 1.05 * rec["algorithmic_bytes"]
