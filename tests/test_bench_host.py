"""Host-side accounting of bench.py (CPU): the rows counted as algorithmic bytes, and the
committed traffic summary's source-hash check."""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def test_needed_rows_by_hand():
    K = 4
    T = np.array([1.0, 1.0, 0.0, 0.0, 0.7, 1.0], dtype=np.float32)
    n = np.array([0, 4, 2, 4, 1, 3], dtype=np.int32)
    status = np.array([0, 0, 0, 16, 0, 1], dtype=np.int32)   # 16: a note, 1: a data error
    # sampled n=0: 2; sampled all accepted: 2K+1 = 9; greedy n=2: 3; greedy all: K+1 = 5
    # (the note bit is no error); sampled n=1: 4; sampled with an error: every row, 9
    assert bench.needed_rows(T, n, status, K) == 2 + 9 + 3 + 5 + 4 + 9


def test_needed_rows_never_exceed_the_full_read():
    rng = np.random.default_rng(5)
    for K in (0, 1, 8):
        B = 200
        T = np.where(rng.random(B) < 0.25, 0.0, rng.random(B) + 0.1)
        n = rng.integers(0, K + 1, B)
        st = np.where(rng.random(B) < 0.05, 1, 0)
        full = int(sum(K + 1 + (K if t != 0 else 0) for t in T))
        got = bench.needed_rows(T, n, st, K)
        assert 0 < got <= full
        # with every draft accepted the rule needs every row
        assert bench.needed_rows(T, np.full(B, K), np.zeros(B, int), K) == full


def test_drawn_rows_by_hand():
    K = 3
    T = np.array([1.0, 1.0, 0.0, 1.0], dtype=np.float32)
    n = np.array([1, 3, 0, 2], dtype=np.int32)
    status = np.array([16, 0, 0, 1], dtype=np.int32)
    # residual draw (2 rows, the note bit is no error), bonus draw (1), greedy (0), error (0)
    assert bench.drawn_rows(T, n, status, K) == 3


def test_traffic_file_is_read_only_for_the_current_sources(tmp_path, monkeypatch):
    f = tmp_path / "traffic.md"
    f.write_text(f"kernel_source_sha256_16: {bench.kernel_source_hash()}\n"
                 "hbm_bytes_per_launch: 1.25e+09\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic(4) == 1.25e9
    assert bench.measured_traffic(3) is None      # counted on the B=256 K=8 workload only
    f.write_text("kernel_source_sha256_16: 0000000000000000\nhbm_bytes_per_launch: 1.25e+09\n")
    assert bench.measured_traffic(4) is None


def test_committed_traffic_summary_matches_the_sources():
    """The committed counter summary was taken on the kernel sources in the tree."""
    assert bench.measured_traffic(4) is not None
