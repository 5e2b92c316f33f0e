"""Host logic of bench.py (CPU): the traffic figure is taken from a committed
counter summary only when that summary was measured on the current kernel
sources, the source hash follows the kernel's includes, the rocprofv3 csv
summary reports what the files hold, and the one-GPU limit is enforced."""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.fixture
def tree(tmp_path, monkeypatch):
    """A copy of the kernel sources and the header under a scratch root."""
    shutil.copytree(os.path.join(ROOT, "mxfp4_expert_weight_amd", "csrc"),
                    tmp_path / "mxfp4_expert_weight_amd" / "csrc",
                    ignore=shutil.ignore_patterns("*.o", "*.so"))
    shutil.copytree(os.path.join(ROOT, "include"), tmp_path / "include")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return tmp_path


def _write_profile(tree, kernel, workload, sha, traffic="1234567"):
    (tree / "profiles" / f"{kernel}_{workload}.txt").write_text(
        "# header: with a colon\n"
        "  indented: 1\n"
        f"traffic_bytes_per_launch: {traffic}\n"
        f"kernel_sources_sha256: {sha}\n")


def test_traffic_only_from_matching_sources(tree):
    sha = bench.kernel_source_hash("gateup_kernel")
    assert bench.recorded_traffic("w") is None                       # no summary
    _write_profile(tree, "gateup_kernel", "w", sha)
    assert bench.recorded_traffic("w") == 1234567.0
    _write_profile(tree, "gateup_kernel", "w", "0" * 64)              # other sources
    assert bench.recorded_traffic("w") is None
    _write_profile(tree, "gateup_kernel", "w", sha, traffic="n/a")   # unreadable figure
    assert bench.recorded_traffic("w") is None


def test_hash_follows_the_kernels_includes(tree):
    csrc = tree / "mxfp4_expert_weight_amd" / "csrc"
    gu, lm, every = (bench.kernel_source_hash("gateup_kernel"), bench.kernel_source_hash("lmhead_fp8_kernel"),
                     bench.kernel_source_hash())
    # the prefetch kernel's source is in no other translation unit
    with open(csrc / "prefetch.hip", "a") as f:
        f.write("\n// edit\n")
    assert bench.kernel_source_hash("gateup_kernel") == gu
    assert bench.kernel_source_hash("lmhead_fp8_kernel") == lm
    assert bench.kernel_source_hash() != every
    # a header that forward.hip reaches only through other headers
    with open(csrc / "common.h", "a") as f:
        f.write("\n// edit\n")
    assert bench.kernel_source_hash("gateup_kernel") != gu
    assert bench.kernel_source_hash("lmhead_fp8_kernel") != lm
    # a recorded summary taken before the edit no longer counts
    _write_profile(tree, "gateup_kernel", "w", gu)
    assert bench.recorded_traffic("w") is None


def test_committed_summaries_parse():
    """Every committed gate/up summary carries a hash and a traffic figure in
    the form recorded_traffic reads."""
    import glob
    files = glob.glob(os.path.join(ROOT, "profiles", "gateup_kernel_ling_m*.txt"))
    assert files
    for p in files:
        keys = [ln.split(":", 1)[0] for ln in open(p) if not ln.startswith((" ", "#", "|")) and ":" in ln]
        assert "kernel_sources_sha256" in keys, p
        if not p.endswith("_hint.txt"):
            assert "traffic_bytes_per_launch" in keys, p


def test_profile_summary(tmp_path, capsys):
    d = tmp_path / "run"
    d.mkdir()
    (d / "run_kernel_stats.csv").write_text(
        '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
        '"void moe::gateup_kernel<true, 8, false, false>(moe::ForwardArgs)",4,48000,12000.0,60.0,9000,15000,1.0\n'
        '"void moe::down_kernel<true, false>(moe::ForwardArgs)",4,20000,5000.0,25.0,4000,6000,1.0\n')
    (d / "run_counter_collection.csv").write_text(
        '"Kernel_Name","Counter_Name","Counter_Value"\n'
        '"gateup_kernel","FETCH_SIZE",100\n'
        '"gateup_kernel","FETCH_SIZE",300\n'
        '"down_kernel","FETCH_SIZE",7\n')
    bench.profile_summary([str(d)], "gateup_kernel")
    out = capsys.readouterr().out.splitlines()
    gu = [ln for ln in out if "gateup_kernel<" in ln][0].split()
    assert gu[-5:] == ["4", "12.00", "9.00", "15.00", "60.0"]
    assert any("down_kernel<" in ln and "5.00" in ln for ln in out)
    cnt = [ln for ln in out if "FETCH_SIZE" in ln]          # down_kernel is filtered out
    assert len(cnt) == 1 and "gateup_kernel" in cnt[0]
    m = re.search(r"n=\s*(\d+)\s+mean=\s*([0-9.]+)\s+median=\s*([0-9.]+)", cnt[0])
    assert m and (int(m.group(1)), float(m.group(2)), float(m.group(3))) == (2, 200.0, 200.0)


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                       env=e, timeout=120)
    assert r.returncode != 0
    assert "--gpus must be 1" in r.stderr
    assert r.stdout == ""
