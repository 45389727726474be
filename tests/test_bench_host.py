"""bench.py's host-side logic, without a GPU: argument refusals, the
counter summaries behind the `traffic` field, the source hash."""
import os
import re
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr


@pytest.mark.parametrize("rows", ["0", "65"])
def test_decode_rows_range(rows):
    r = _run("--gemm", "--decode", "--rows", rows)
    assert r.returncode == 2
    assert "--rows must be in 1..64" in r.stderr


@pytest.mark.parametrize("rows", ["64", "8193"])
def test_prefill_rows_range(rows):
    r = _run("--gemm", "--rows", rows)
    assert r.returncode == 2
    assert "--rows must be in 65..8192" in r.stderr


def test_source_hash_is_stable():
    h = bench.kernel_source_hash()
    assert re.fullmatch(r"[0-9a-f]{16}", h)
    assert h == bench.kernel_source_hash(bench.KERNEL_SOURCES)
    assert h != bench.kernel_source_hash(bench.GEMM_SOURCES)


# Every committed HBM counter summary was taken on the current kernel
# sources: read_counters hands back its per-launch bytes (a kernel edit
# without new counters makes the bench report traffic null, and fails here).
SUMMARIES = [(bench.COUNTERS[w], bench.KERNEL_SOURCES) for w in (2, 3, 4, 5)] + [
             (bench.GEMM_COUNTERS, bench.GEMM_SOURCES),
             (bench.DECODE_COUNTERS[16], bench.GEMM_SOURCES), (bench.NORM_COUNTERS, bench.NORM_SOURCES)]


@pytest.mark.parametrize("rel,sources", SUMMARIES)
def test_counter_summaries_match_sources(rel, sources):
    text = open(os.path.join(ROOT, rel)).read()
    stated = float(re.search(r"^hbm_bytes_per_launch:\s*(\S+)", text, re.M).group(1))
    got = bench.read_counters(0, rel, sources)
    assert got == stated and got > 0


def test_counter_summary_of_other_sources_is_ignored(tmp_path):
    rel = bench.COUNTERS[3]
    text = open(os.path.join(ROOT, rel)).read()
    stale = re.sub(r"^kernel_source_hash:.*$", "kernel_source_hash: 0000000000000000", text, flags=re.M)
    p = tmp_path / "stale.txt"
    p.write_text(stale)
    assert bench.read_counters(0, str(p), bench.KERNEL_SOURCES) is None
    assert bench.read_counters(0, "profiles/no_such_file.txt") is None
    assert bench.read_counters(99) is None


def test_host_cpu_model_named():
    assert bench.host_cpu_model().strip()
