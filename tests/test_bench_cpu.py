"""Host-side logic of bench.py that runs without a GPU: the one-GPU guard and
the reading of the committed HBM-traffic counter summary."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "exactly one GPU" in p.stdout + p.stderr


def _fake_root(tmp_path, sha, value="123456"):
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "k_traffic.md").write_text(
        "# title\n\n| a | b |\n  indented: 1\n"
        f"sources_sha256: {sha}\ntraffic_bytes_per_launch: {value}\n")
    for rel in bench.TRAFFIC_SOURCES:
        f = tmp_path / rel
        f.parent.mkdir(parents=True, exist_ok=True)
        f.write_text(rel)
    return str(tmp_path)


def test_traffic_read_only_while_sources_match(tmp_path, monkeypatch):
    root = _fake_root(tmp_path, "0" * 64)
    monkeypatch.setattr(bench, "ROOT", root)
    assert bench.measured_traffic("k") is None            # sources changed since
    assert bench.measured_traffic("missing") is None      # no summary at all
    sha = bench.sources_sha256()
    (tmp_path / "profiles" / "k_traffic.md").write_text(
        f"sources_sha256: {sha}\ntraffic_bytes_per_launch: 236041041\n")
    assert bench.measured_traffic("k") == 236041041.0
    (tmp_path / "profiles" / "k_traffic.md").write_text(
        f"sources_sha256: {sha}\ntraffic_bytes_per_launch: n/a\n")
    assert bench.measured_traffic("k") is None            # unparsable value


def test_sources_hash_covers_every_listed_file(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", _fake_root(tmp_path, ""))
    before = bench.sources_sha256()
    f = tmp_path / bench.TRAFFIC_SOURCES[-1]
    f.write_text(f.read_text() + " ")
    assert bench.sources_sha256() != before


@pytest.mark.parametrize("rel", bench.TRAFFIC_SOURCES)
def test_traffic_sources_exist(rel):
    assert os.path.isfile(os.path.join(ROOT, rel))
