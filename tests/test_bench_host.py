"""Host logic of bench.py that the reported roofline depends on (no GPU):
the source hash that keys the committed counter summaries, and the
arithmetic of those summaries."""
import json
import os
import shutil

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_101_amd", "csrc")
COUNTER_WORKLOADS = ["gqa40", "gqa40_tp8", "qwen", "prefix_shared", "fp8", "fp8_p512",
                     "prefill", "prefill_small"]


def _tree_copy(tmp_path):
    dst = tmp_path / "paged_kv_cache_101_amd" / "csrc"
    shutil.copytree(CSRC, dst)
    return tmp_path, dst


@pytest.mark.parametrize("workload", [None, "gqa40", "prefix_shared", "prefill"])
def test_kernel_hash_ignores_comments_and_spacing(tmp_path, workload):
    root, dst = _tree_copy(tmp_path)
    assert bench.kernel_hash(workload, root=str(root)) == bench.kernel_hash(workload)
    for f in ("decode_wave.h", "paged_prefill.hip"):
        p = dst / f
        text = p.read_text()
        p.write_text("// a new comment\n/* and a block\n   comment */\n" + text.replace("\n", "\n\n", 3))
    assert bench.kernel_hash(workload, root=str(root)) == bench.kernel_hash(workload)


@pytest.mark.parametrize("workload,f", [("gqa40", "decode_wave.h"), ("prefix_shared", "paged_prefill.hip"),
                                        ("prefill", "paged_prefill.hip"), ("prefill_small", "pkv_internal.h")])
def test_kernel_hash_follows_code(tmp_path, workload, f):
    root, dst = _tree_copy(tmp_path)
    p = dst / f
    p.write_text(p.read_text() + "\nnamespace pkv { constexpr int kHashProbe = 1; }\n")
    assert bench.kernel_hash(workload, root=str(root)) != bench.kernel_hash(workload)


def test_decode_hash_ignores_prefill_sources(tmp_path):
    # the plain decode launches nothing from paged_prefill.hip
    root, dst = _tree_copy(tmp_path)
    p = dst / "paged_prefill.hip"
    p.write_text(p.read_text() + "\nnamespace pkv { constexpr int kHashProbe = 1; }\n")
    assert bench.kernel_hash("gqa40", root=str(root)) == bench.kernel_hash("gqa40")


def _record(workload):
    path = os.path.join(ROOT, "profiles", bench.counter_file(workload))
    assert os.path.exists(path), path
    rec = None
    with open(path) as fh:
        for line in fh:
            if line.startswith("{"):
                rec = json.loads(line)
    assert rec is not None
    return rec


@pytest.mark.parametrize("workload", COUNTER_WORKLOADS)
def test_counter_summary_arithmetic(workload):
    """Bytes = KiB per dispatch x 1024 x the plain-copy scale, summed over the
    kernels of one call; the scale is the copy's bytes over what the counter
    read for it."""
    rec = _record(workload)
    cal = rec["copy_calibration"]
    assert cal["fetch_scale"] == pytest.approx(cal["bytes"] / (cal["fetch_kib"] * 1024), rel=1e-4)
    assert cal["write_scale"] == pytest.approx(cal["bytes"] / (cal["write_kib"] * 1024), rel=1e-4)
    rd = sum(k["fetch_kib_per_launch"] * 1024 * cal["fetch_scale"] for k in rec["kernels"].values())
    wr = sum(k["write_kib_per_launch"] * 1024 * cal["write_scale"] for k in rec["kernels"].values())
    t = rec["traffic_bytes_per_launch"]
    assert t["read"] == pytest.approx(rd, rel=1e-3)
    assert t["write"] == pytest.approx(wr, rel=1e-3)
    assert abs(t["total"] - (t["read"] + t["write"])) <= 1  # each rounded to whole bytes
    assert rec["read_over_algorithmic"] == pytest.approx(t["read"] / rec["algorithmic_read_bytes_per_launch"],
                                                         rel=1e-3)
    # every kernel of the call was seen on several dispatches
    assert all(k["dispatches"] >= 2 for k in rec["kernels"].values())


def test_counter_files_are_distinct():
    names = [bench.counter_file(w) for w in COUNTER_WORKLOADS]
    assert len(set(names)) == len(names)
