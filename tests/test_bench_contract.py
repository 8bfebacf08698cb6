"""Host-side checks of bench.py's contract: one GPU only, and the HBM traffic
figure it reports is taken from a committed counter summary only while the
profiled kernel source is unchanged."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def _fake_tree(tmp_path):
    for rel in [bench.KERNEL_SOURCES["main_bwd_dkdv"]] + bench.KERNEL_HEADERS:
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, rel), dst)
    (tmp_path / "profiles").mkdir()
    return tmp_path


def _write_profile(root, sha, nbytes):
    p = root / "profiles" / f"{bench.KERNEL_NAMES['main_bwd_dkdv']}_eagle3_256k.md"
    p.write_text("# summary\n\n- kernel: main_bwd_dkdv_kernel\n"
                 f"- source_sha: {sha}\n- hbm_bytes_per_launch: {nbytes}\n")


def test_traffic_is_read_while_the_source_matches(tmp_path, monkeypatch):
    root = _fake_tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(root))
    sha = bench.source_sha(bench.KERNEL_SOURCES["main_bwd_dkdv"])
    _write_profile(root, sha, "1.25e+12")
    assert bench.traffic_for("main_bwd_dkdv", "eagle3_256k") == pytest.approx(1.25e12)


def test_traffic_is_null_once_the_kernel_source_changed(tmp_path, monkeypatch):
    root = _fake_tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(root))
    sha = bench.source_sha(bench.KERNEL_SOURCES["main_bwd_dkdv"])
    _write_profile(root, sha, "1.25e+12")
    with open(root / bench.KERNEL_SOURCES["main_bwd_dkdv"], "a") as f:
        f.write("\n// edited\n")
    assert bench.traffic_for("main_bwd_dkdv", "eagle3_256k") is None
    # a shared header counts as part of the kernel too
    _write_profile(root, bench.source_sha(bench.KERNEL_SOURCES["main_bwd_dkdv"]), "1.25e+12")
    with open(root / bench.KERNEL_HEADERS[0], "a") as f:
        f.write("\n// edited\n")
    assert bench.traffic_for("main_bwd_dkdv", "eagle3_256k") is None


def test_traffic_is_null_without_a_summary(tmp_path, monkeypatch):
    root = _fake_tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(root))
    assert bench.traffic_for("main_bwd_dkdv", "eagle3_256k") is None
