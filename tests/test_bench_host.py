"""Host logic of bench.py (CPU only): the credited-work formula and the
reader of the committed HBM-traffic record.

The visible-pair counts are checked against a brute-force count of the mask
predicate (key j visible to query i: j <= i under the causal mask, and
|i - j| < window for a window), written here independently of bench.py's
closed forms.
"""
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def brute_pairs(N, causal, window):
    n = 0
    for i in range(N):
        for j in range(N):
            if causal and j > i:
                continue
            if window > 0 and not (i - j < window and j - i < window):
                continue
            n += 1
    return n


@pytest.mark.parametrize("N", [1, 2, 7, 32, 33, 100])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("window", [0, 1, 2, 5, 31, 99, 100, 1000])
def test_visible_pairs_match_the_mask(N, causal, window):
    assert bench.visible_pairs(N, causal, window) == brute_pairs(N, causal, window)


def test_credited_flops_convention():
    # 4 d flops per pair (S and P V); the full square, halved under the
    # causal mask (the metric's convention, not the N (N + 1) / 2 pairs);
    # the exact visible pairs under a window shorter than N.
    BH, N, d = 3, 64, 128
    assert bench.credited_fwd_flops(BH, N, d, False, 0) == 4.0 * BH * N * N * d
    assert bench.credited_fwd_flops(BH, N, d, True, 0) == 2.0 * BH * N * N * d
    assert bench.credited_fwd_flops(BH, N, d, True, 16) == 4.0 * d * BH * brute_pairs(N, True, 16)
    assert bench.credited_fwd_flops(BH, N, d, False, 16) == 4.0 * d * BH * brute_pairs(N, False, 16)
    assert bench.credited_fwd_flops(BH, N, d, True, N) == 2.0 * BH * N * N * d


def _record(tmp_path, kernel, sha, nbytes):
    rec = {"kernel": kernel, "workload": "test", "sources_sha256": sha,
           "hbm_bytes_per_launch": nbytes}
    p = tmp_path / "traffic.md"
    p.write_text("# traffic\n\n```json\n" + json.dumps(rec) + "\n```\n")
    return str(p)


def test_recorded_traffic_needs_matching_kernel_and_sources(tmp_path, monkeypatch):
    sha = bench.kernel_sources_sha256()
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", _record(tmp_path, "attn::k<1>", sha, 1234))
    assert bench.recorded_traffic("attn::k<1>") == 1234
    assert bench.recorded_traffic("attn::other<1>") is None
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", _record(tmp_path, "attn::k<1>", "0" * 64, 1234))
    assert bench.recorded_traffic("attn::k<1>") is None
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(tmp_path / "missing.md"))
    assert bench.recorded_traffic("attn::k<1>") is None


def test_sources_hash_covers_every_kernel_source(tmp_path, monkeypatch):
    # The hash changes when any .hip or .hpp file under csrc changes and
    # ignores other files.
    d = tmp_path / "csrc"
    d.mkdir()
    (d / "a.hip").write_text("x")
    (d / "b.hpp").write_text("y")
    (d / "notes.txt").write_text("z")
    monkeypatch.setattr(bench, "CSRC", str(d))
    h0 = bench.kernel_sources_sha256()
    (d / "notes.txt").write_text("changed")
    assert bench.kernel_sources_sha256() == h0
    (d / "b.hpp").write_text("y2")
    assert bench.kernel_sources_sha256() != h0
