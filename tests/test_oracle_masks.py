"""Pins for the oracle's chunked frame-window mask.

The page's printed figure is that a frame sees about 15 frames (its 5-frame
chunk and one chunk on each side); the rest is brute force with Python sets
over frames, written independently of the oracle's vectorised predicate.
"""

import json
import os

import numpy as np
import pytest

from oracle import FrameWindow

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "frame_window.json")


def _frames_seen_bruteforce(F, C, R, first, last, see_all, qf):
    """Set of key frames visible from query frame qf."""
    chunks = {}
    for f in range(F):
        chunks.setdefault(f // C, []).append(f)
    qc = qf // C
    seen = set()
    for c in range(qc - R, qc + R + 1):
        seen.update(chunks.get(c, []))
    if first:
        seen.add(0)
    if last:
        seen.add(F - 1)
    if see_all and ((first and qf == 0) or (last and qf == F - 1)):
        seen = set(range(F))
    return seen


def test_interior_frame_sees_fifteen_frames():
    g = json.load(open(GOLDEN))
    C, R = g["chunk_frames"], g["radius_chunks"]
    w = FrameWindow(frames=42, tokens_per_frame=1, chunk_frames=C, radius_chunks=R,
                    anchor_first=False, anchor_last=False)
    vis = w(np.arange(42), np.arange(42))
    # a frame in an interior chunk (chunk 3 = frames 15..19)
    assert vis[17].sum() == g["frames_seen_by_interior_frame_printed"]


@pytest.mark.parametrize("see_all,expected", [(False, 641), (True, 706)])
def test_long_video_frame_pair_count(see_all, expected):
    F = 42
    w = FrameWindow(frames=F, tokens_per_frame=1, chunk_frames=5, radius_chunks=1,
                    anchor_first=True, anchor_last=True, anchor_queries_see_all=see_all)
    vis = w(np.arange(F), np.arange(F))
    brute = sum(len(_frames_seen_bruteforce(F, 5, 1, True, True, see_all, qf)) for qf in range(F))
    assert vis.sum() == brute == expected


@pytest.mark.parametrize("F,T,C,R,first,last,see_all", [
    (7, 3, 2, 1, True, True, False),
    (7, 3, 2, 0, True, False, False),
    (9, 2, 3, 1, False, True, True),
    (5, 4, 5, 0, False, False, False),
    (11, 1, 2, 2, True, True, True),
])
def test_token_mask_matches_bruteforce(F, T, C, R, first, last, see_all):
    w = FrameWindow(frames=F, tokens_per_frame=T, chunk_frames=C, radius_chunks=R,
                    anchor_first=first, anchor_last=last, anchor_queries_see_all=see_all)
    n = F * T
    vis = w(np.arange(n), np.arange(n))
    for i in range(n):
        seen = _frames_seen_bruteforce(F, C, R, first, last, see_all, i // T)
        for j in range(n):
            assert vis[i, j] == ((j // T) in seen), (i, j)


def test_every_query_sees_its_own_frame():
    w = FrameWindow(frames=42, tokens_per_frame=1560, chunk_frames=5, radius_chunks=1)
    rows = np.arange(0, w.n_tokens, 997)
    vis = w(rows, np.arange(w.n_tokens))
    for a, i in enumerate(rows):
        f = i // 1560
        assert vis[a, f * 1560:(f + 1) * 1560].all()
