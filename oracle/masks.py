"""Chunked frame-window visibility with anchor frames, as a dense predicate.

TEST INFRASTRUCTURE (the oracle): never imported by the library.

Page "VDN-Minimax-H3 ... Stage A1" (yfxerp.com), the description of the local
window softmax branch and its configuration keys: the window is ``chunk: 5,
radius: 1`` -- a frame's own 5-frame chunk plus one chunk on either side, so a
frame sees about 15 frames -- and the first and last frames are anchors
(``anchor_frames: both``) that are exactly visible in the softmax mask.

Readings taken where the page is silent:

* tokens are flattened frame-major: token i belongs to frame i // T;
* chunks are consecutive runs of C frames starting at frame 0 (the last chunk
  may be shorter);
* key j is visible to query i iff |chunk(frame(i)) - chunk(frame(j))| <= R, or
  frame(j) is an enabled anchor frame;
* optionally (off by default) queries in an anchor frame see every key -- the
  other reading of the page's "visible in both directions".
"""

from dataclasses import dataclass

import numpy as np

__all__ = ["FrameWindow", "frame_window_visible"]


@dataclass(frozen=True)
class FrameWindow:
    frames: int
    tokens_per_frame: int
    chunk_frames: int
    radius_chunks: int
    anchor_first: bool = True
    anchor_last: bool = True
    anchor_queries_see_all: bool = False

    @property
    def n_tokens(self):
        return self.frames * self.tokens_per_frame

    def __call__(self, qi, ki):
        return frame_window_visible(qi, ki, self)


def frame_window_visible(qi, ki, w):
    """Bool matrix [len(qi), len(ki)]: may query qi[a] attend to key ki[b]."""
    qi = np.asarray(qi, dtype=np.int64)
    ki = np.asarray(ki, dtype=np.int64)
    qf = qi // w.tokens_per_frame
    kf = ki // w.tokens_per_frame
    qc = qf // w.chunk_frames
    kc = kf // w.chunk_frames
    vis = np.abs(qc[:, None] - kc[None, :]) <= w.radius_chunks
    key_anchor = np.zeros(kf.shape, dtype=bool)
    query_anchor = np.zeros(qf.shape, dtype=bool)
    if w.anchor_first:
        key_anchor |= kf == 0
        query_anchor |= qf == 0
    if w.anchor_last:
        key_anchor |= kf == w.frames - 1
        query_anchor |= qf == w.frames - 1
    vis |= key_anchor[None, :]
    if w.anchor_queries_see_all:
        vis |= query_anchor[:, None]
    return vis
