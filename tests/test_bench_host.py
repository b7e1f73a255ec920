"""Host-side logic of bench.py (CPU only): the visible-pair counts behind
every TFLOP/s figure, the single-GPU contract of the command line, and the
rule that stored counter figures (clock bounds, HBM bytes) are used only for
the kernel source they were taken on."""

import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _brute(mask, n, window, offs=None):
    win = window if mask in ("sliding", "band", "prefix_lm") else None
    return int(oracle.visible(mask, n, n, win, doc_offsets=offs).sum())


@pytest.mark.parametrize("n", [1, 2, 3, 17, 64, 130])
def test_visible_pairs_equal_the_oracle_mask(n):
    for mask in ("none", "causal"):
        assert bench.visible_pairs(mask, n, 0) == _brute(mask, n, 0), (mask, n)
    for w in sorted({1, 2, 5, n - 1, n, n + 3} - {0}):
        if w >= 1:
            assert bench.visible_pairs("sliding", n, w) == _brute("sliding", n, w), ("sliding", n, w)
    for w in sorted({0, 1, 3, n - 1, n, n + 5}):
        if w >= 0:
            assert bench.visible_pairs("band", n, w) == _brute("band", n, w), ("band", n, w)
            assert bench.visible_pairs("prefix_lm", n, w) == _brute("prefix_lm", n, w), ("prefix_lm", n, w)
    rng = np.random.default_rng(n)
    for _ in range(4):
        cuts = sorted(rng.integers(0, n + 1, size=int(rng.integers(0, 5))).tolist())
        offs = np.array([0] + cuts + [n])
        for mask in ("document", "document_causal"):
            assert bench.visible_pairs(mask, n, 0, offs) == _brute(mask, n, 0, offs), (mask, n, offs)


def test_headline_flop_count():
    # 4 d flop per visible pair of the causal [4, 16, 2048, 64] workload
    assert 4 * 64 * bench.visible_pairs("causal", 2048, 0) * 4 * 16 == 34_376_515_584


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr


def test_stored_figures_need_the_current_kernel_source(tmp_path, monkeypatch):
    clock = tmp_path / "clock.json"
    traffic = tmp_path / "traffic.json"
    clock.write_text(json.dumps({"kernel_source_digest": "abc", "clock_ghz": 1.9, "clock_ghz_upper": 2.4}))
    traffic.write_text(json.dumps({"kernel_source_digest": "abc", "bytes_per_launch": 123}))
    monkeypatch.setattr(bench, "CLOCK_FILE", str(clock))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(traffic))
    assert bench.clock_for("abc") == (1.9, 2.4)
    assert bench.traffic_for("abc") == 123
    assert bench.clock_for("def") is None
    assert bench.traffic_for("def") is None
    monkeypatch.setattr(bench, "CLOCK_FILE", str(tmp_path / "missing.json"))
    assert bench.clock_for("abc") is None


def test_kernel_source_digest_follows_the_sources(tmp_path, monkeypatch):
    d0 = bench.kernel_source_digest()
    assert len(d0) == 16 and d0 == bench.kernel_source_digest()
    copy = tmp_path / "k.hip"
    copy.write_bytes(open(os.path.join(ROOT, bench.KERNEL_SOURCES[0]), "rb").read() + b"\n")
    rest = [os.path.join(ROOT, rel) for rel in bench.KERNEL_SOURCES[1:]]
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [os.path.join(ROOT, bench.KERNEL_SOURCES[0])] + rest)
    assert bench.kernel_source_digest() == d0          # absolute paths: the same bytes, the same digest
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(copy)] + rest)
    assert bench.kernel_source_digest() != d0
