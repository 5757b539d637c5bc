"""Host-side checks of bench.py's bookkeeping (no GPU).

* every HBM-counter summary under profiles/ names a kernel whose sources
  bench.py knows, carries a 16-hex source hash and a byte count;
* bench.py reports a summary's traffic only while the hash of the kernel's
  sources matches the one recorded with the counters (a changed kernel gets
  null, not stale numbers);
* more than one GPU is refused with a message;
* the all-pairs ablation counts each pair of key tiles once.
"""

import glob
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

SUMMARIES = sorted(glob.glob(os.path.join(ROOT, "profiles", "hbm_*.txt")))


def _fields(path):
    out = {}
    for line in open(path):
        m = re.match(r"^(\w+):\s*(\S+)", line)
        if m:
            out.setdefault(m.group(1), m.group(2))
    return out


def test_there_are_counter_summaries():
    assert SUMMARIES, "no profiles/hbm_*.txt"


@pytest.mark.parametrize("path", SUMMARIES, ids=[os.path.basename(p) for p in SUMMARIES])
def test_summary_fields(path):
    f = _fields(path)
    assert f.get("kernel") in bench.KERNEL_SOURCES, f.get("kernel")
    assert re.fullmatch(r"[0-9a-f]{16}", f.get("source_sha256_16", ""))
    assert int(f["traffic_bytes_per_launch"]) > 0
    name = os.path.basename(path)[len("hbm_"):-len(".txt")]
    assert name.startswith(f["kernel"] + "_")


@pytest.mark.parametrize("path", SUMMARIES, ids=[os.path.basename(p) for p in SUMMARIES])
def test_traffic_follows_the_source_hash(path, monkeypatch):
    f = _fields(path)
    kernel = f["kernel"]
    workload = os.path.basename(path)[len("hbm_") + len(kernel) + 1:-len(".txt")]
    current = bench.traffic_from_profile(kernel, workload)
    # either the sources are those the counters were taken on, or null
    assert current in (None, int(f["traffic_bytes_per_launch"]))
    # any other source list (a changed kernel) hashes differently: null
    monkeypatch.setitem(bench.KERNEL_SOURCES, kernel, ["zp_host.h"])
    assert bench.traffic_from_profile(kernel, workload) is None


def test_unknown_kernel_or_workload_has_no_traffic():
    assert bench.traffic_from_profile("compress", "no_such_workload") is None
    assert bench.traffic_from_profile("no_such_kernel", "8b_32L_8kv_32q_N4096") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_all_pairs_work_counts_each_tile_pair_once():
    # nt tiles give nt (nt + 1) / 2 tile pairs (the diagonal included), each
    # 2 b^2 d flops; for full tiles that is (n^2 + n b) d, about half the
    # 2 n^2 d of the whole Gram matrix
    assert bench.all_pairs_flops(1, 16, 128) == 2 * 16 * 16 * 128
    assert bench.all_pairs_flops(1, 32, 64) == 3 * 2 * 16 * 16 * 64
    assert bench.all_pairs_flops(1, 33, 64) == 6 * 2 * 16 * 16 * 64   # ragged: 3 tiles
    n, d = 4096, 128
    assert bench.all_pairs_flops(5, n, d) == 5 * (n * n + n * 16) * d
