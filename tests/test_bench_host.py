"""Host logic of bench.py, on the CPU: the one-GPU refusal, the rule that a
committed HBM-traffic figure is used only while its kernel's sources are
unchanged, and the roofline arithmetic."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_read_kv_skips_comments_and_blank_lines(tmp_path):
    f = tmp_path / "kv.txt"
    f.write_text("# a comment = not a key\n\nkernel = gemm_f6f4\nbytes_per_launch = 123\nsources = a b\n")
    assert bench.read_kv(str(f)) == {"kernel": "gemm_f6f4", "bytes_per_launch": "123", "sources": "a b"}


def _fake_tree(tmp_path, kernel_text):
    (tmp_path / "profiles").mkdir()
    (tmp_path / "k.hip").write_text(kernel_text)
    return tmp_path


def test_committed_traffic_only_while_sources_are_unchanged(tmp_path, monkeypatch):
    root = _fake_tree(tmp_path, "kernel v1")
    monkeypatch.setattr(bench, "ROOT", str(root))
    h = bench.source_hash(["k.hip"])
    (root / "profiles" / "traffic_kx_wl.txt").write_text(
        "kernel = kx\nlayer = wl\nbytes_per_launch = 4096\nsources = k.hip\nsource_hash = %s\n" % h)
    assert bench.committed_traffic("kx", "wl") == 4096
    (root / "k.hip").write_text("kernel v2")   # the kernel changed since the counters were taken
    assert bench.committed_traffic("kx", "wl") is None
    assert bench.committed_traffic("ky", "wl") is None   # no file at all


def test_committed_traffic_files_name_existing_sources():
    prof = os.path.join(ROOT, "profiles")
    files = [f for f in os.listdir(prof) if f.startswith("traffic_")]
    assert files
    for f in files:
        kv = bench.read_kv(os.path.join(prof, f))
        assert int(kv["bytes_per_launch"]) > 0
        srcs = kv["sources"].split()
        assert srcs and all(os.path.exists(os.path.join(ROOT, s)) for s in srcs), f


def test_roofline_arithmetic(monkeypatch):
    monkeypatch.setattr(bench, "_PEAKS", {"mfma_f6f4_TFLOPS": 8000.0, "hbm_read_8MiB_GBps": 2500.0})
    # 1.1e12 ops in 275 us: 4000 TFLOP/s, 0.396 of 10.1 PFLOP/s, 0.5 of the measured 8000
    r = bench.roofline("k", "mfma", 1_100_000_000_000, 275.0, "TFLOP/s", 10100.0, "mfma_f6f4_TFLOPS", 7, "d")
    assert r["achieved"] == pytest.approx(4000.0)
    assert r["frac"] == pytest.approx(4000.0 / 10100.0, abs=1e-4)
    assert r["frac_measured"] == pytest.approx(0.5)
    assert r["traffic"] == 7 and r["work_per_launch"] == 1_100_000_000_000 and r["us_per_launch"] == 275.0
    # bytes: 8 MB in 4 us = 2000 GB/s, 0.25 of 8 TB/s
    r = bench.roofline("k", "hbm", 8_000_000, 4.0, "GB/s", 8000.0, "hbm_read_8MiB_GBps")
    assert r["achieved"] == pytest.approx(2000.0)
    assert r["frac"] == pytest.approx(0.25)
    assert r["frac_measured"] == pytest.approx(0.8)
