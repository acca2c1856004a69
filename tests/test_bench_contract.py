"""bench.py's host-side pieces, without a GPU: the committed counter
summaries parse, and each was taken on the kernel sources as they are now
(otherwise bench.py reports traffic as null, as it should, and the summary
needs a new counter run)."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

SUMMARIES = [
    (bench.TRAFFIC_FILE, bench.DECODE_SOURCES),
    (bench.PREFILL_TRAFFIC_FILE, bench.PREFILL_SOURCES),
    (bench.BACKWARD_TRAFFIC_FILE, bench.BACKWARD_SOURCES),
    (bench.PROJECTION_TRAFFIC_FILE, bench.PROJECTION_SOURCES),
]


@pytest.mark.parametrize("path,sources", SUMMARIES, ids=[os.path.basename(s[0]) for s in SUMMARIES])
def test_traffic_summary_matches_current_sources(path, sources):
    assert os.path.exists(path), path
    traffic = bench.read_traffic(bench.source_digest(sources), path)
    assert traffic is not None, f"{os.path.basename(path)} was taken on other kernel sources"
    assert traffic > 0


def test_read_traffic_rejects_other_sources(tmp_path):
    p = tmp_path / "t.md"
    p.write_text("kernel_source_digest: 0123456789abcdef\nfetch_bytes_per_launch: 1.5e9\nwrite_bytes_per_launch: 2e8\n")
    assert bench.read_traffic("0123456789abcdef", str(p)) == pytest.approx(1.7e9)
    assert bench.read_traffic("fedcba9876543210", str(p)) is None
    assert bench.read_traffic("0123456789abcdef", str(tmp_path / "missing.md")) is None


def test_more_than_one_gpu_is_refused():
    import subprocess
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2 and "one GPU" in res.stderr


def test_profile_commands_run_with_the_flags_bench_accepts():
    """Every bench.py command recorded in profiles/ uses only flags the
    benchmark accepts, and leaves out the context-only legs (--no-context), so
    that it reproduces the dispatch sequence its summary describes."""
    import re
    import subprocess
    helptext = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True,
                              text=True, timeout=120).stdout
    prof = os.path.join(ROOT, "profiles")
    n = 0
    for name in sorted(os.listdir(prof)):
        for line in open(os.path.join(prof, name)):
            if "python3 bench.py" not in line:
                continue
            n += 1
            args = line.split("python3 bench.py", 1)[1].split()
            for flag in (a for a in args if a.startswith("--")):
                assert re.search(rf"(^|\s){re.escape(flag)}(\s|$|,)", helptext), f"{name}: unknown flag {flag}"
            assert "--no-context" in args, f"{name}: command runs the context legs"
    assert n >= 6
