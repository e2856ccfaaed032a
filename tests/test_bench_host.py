"""Host-side checks of bench.py (no GPU): the measured-traffic figure is tied to the backward kernel's own
sources, and more than one GPU is refused with a message."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

CSRC = ("selective_state_space_chunked_amd", "csrc")


def _copy_sources(tmp_path):
    dst = tmp_path.joinpath(*CSRC)
    dst.mkdir(parents=True)
    for f in ("selective.hpp", "real_selective.hip", "common.hpp", "kernels.hpp"):
        shutil.copy(os.path.join(ROOT, *CSRC, f), dst / f)
    return dst


def _hash_at(root, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(root))
    return bench.kernel_sources_sha256()


def test_traffic_hash_follows_the_backward_only(tmp_path, monkeypatch):
    dst = _copy_sources(tmp_path)
    h0 = _hash_at(tmp_path, monkeypatch)
    assert h0 == _hash_at(ROOT, monkeypatch)
    hdr = dst / "selective.hpp"
    text = hdr.read_text()
    # an edit inside the forward kernel leaves the figure valid
    fwd = text.index("// forward (SUMMARY")
    hdr.write_text(text[:fwd] + "// forward (SUMMARY" + text[fwd + len("// forward (SUMMARY"):].replace(
        "constexpr int kFwdStates = 8;", "constexpr int kFwdStates = 8;  // edited", 1))
    assert _hash_at(tmp_path, monkeypatch) == h0
    # an edit inside the backward kernel invalidates it
    hdr.write_text(text.replace("constexpr int kPresum = 4;", "constexpr int kPresum = 4;  // edited", 1))
    assert _hash_at(tmp_path, monkeypatch) != h0
    bwd = text.index("// backward.  Reverse over the tiles")
    hdr.write_text(text[:bwd] + text[bwd:].replace("if (SUMMARY) {", "if (SUMMARY) {  // edited", 1))
    assert _hash_at(tmp_path, monkeypatch) != h0


def test_stored_traffic_matches_the_current_sources():
    meas = bench.MEASURED_TRAFFIC["selective backward"]
    assert meas["sources_sha256"] == bench.kernel_sources_sha256()


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
