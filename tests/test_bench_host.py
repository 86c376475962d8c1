"""Host logic of bench.py (CPU only): the visible-pair count behind the
counted FLOPs of masked workloads, and the rule that HBM traffic is reported
only while the kernel sources are the ones the counters were taken on.

The pair count is checked against the oracle's frame-window predicate by
brute force on small analogues (every anchor and see-all combination), and
against the long-video frame-pair count of 641 of 42 x 42 frames.
"""

import itertools
import json
import os

import numpy as np
import pytest

import bench
from oracle import FrameWindow


def _brute_pairs(F, T, C, R, first, last, see_all):
    w = FrameWindow(frames=F, tokens_per_frame=T, chunk_frames=C, radius_chunks=R,
                    anchor_first=bool(first), anchor_last=bool(last),
                    anchor_queries_see_all=bool(see_all))
    idx = np.arange(F * T)
    return int(w(idx, idx).sum())


def test_dense_pairs():
    for N in (1, 7, 4096):
        assert bench.visible_pairs(N, None) == N * N


@pytest.mark.parametrize("F,T,C,R", [(7, 3, 2, 1), (9, 2, 3, 1), (10, 1, 2, 2), (5, 4, 5, 1)])
def test_frame_window_pairs_match_oracle(F, T, C, R):
    for first, last, see_all in itertools.product((0, 1), repeat=3):
        mask = dict(frames=F, tokens_per_frame=T, chunk_frames=C, radius_chunks=R,
                    anchor_first=first, anchor_last=last, anchor_queries_see_all=see_all)
        assert bench.visible_pairs(F * T, mask) == _brute_pairs(F, T, C, R, first, last, see_all)


def test_long_video_pair_count():
    mask = dict(frames=42, tokens_per_frame=1560, chunk_frames=5, radius_chunks=1)
    assert bench.visible_pairs(42 * 1560, mask) == 641 * 1560 * 1560


def test_traffic_only_for_the_measured_sources(monkeypatch):
    path = os.path.join(bench.ROOT, "profiles", "traffic_image_dit_4096.json")
    rec = json.load(open(path))
    monkeypatch.setattr(bench, "kernel_sha", lambda: rec["kernel_sha256"])
    assert bench.traffic_record("image_dit_4096") == rec["hbm_bytes_per_launch"]
    monkeypatch.setattr(bench, "kernel_sha", lambda: "0" * 64)
    assert bench.traffic_record("image_dit_4096") is None
    assert bench.traffic_record("no_such_workload") is None
