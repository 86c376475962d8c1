"""Workload shapes and seeded input recipes.

Shapes stand in for the pages' workloads (no dataset is used):

* ``tiny_fp32``            1 x 2 x 128 x 64, float32 -- the small case.
* ``image_dit_4096``       2 x 24 x 4096 x 128, bf16 -- a 64 x 64 latent-token
  image DiT.  Q, K RMS-normalised per head; tangents are TrigFlow-path
  velocities projected through random 128 x 128 maps.
* ``t2i_prefix_4352``      4 x 16 x (4096 + 256) x 64, bf16 -- image tokens
  plus a text prefix, tangents x 1e-2.
* ``video_dit_32760``      1 x 40 x 32760 x 128, bf16 -- 21 latent frames of
  30 x 52 tokens (480p 16:9 = 832 x 480 over a 16x spatial reduction); Q, K
  RMS-normalised; tangents x 0.1.
* ``long_video_65520``     1 x 24 x 65520 x 128, bf16 -- 42 such frames with a
  chunked window (5-frame chunks, radius 1, first and last frame anchors).

Every tensor is drawn in float64 from numpy's PCG64, one independent stream
per (tensor, batch, head) derived from ``SeedSequence([seed, tensor_id, b,
h])`` so that heads can be drawn in parallel, then rounded once to the
workload dtype with torch's round-to-nearest-even conversion.  Both the GPU
path and the oracle read those same rounded values.
"""

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "sample_rows", "to_float64"]

_TORCH_DTYPE = {"bf16": torch.bfloat16, "fp32": torch.float32}

# tensor ids of the per-slab random streams
_ID = {"q": 0, "k": 1, "v": 2, "dq": 3, "dk": 4, "dv": 5,
       "x0": 10, "eps": 11, "wq": 20, "wk": 21, "wv": 22, "t": 30}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str                    # "bf16" or "fp32"
    seed: int
    rms_qk: bool = False          # RMS-normalise Q and K per row
    tangents: str = "gaussian"    # "gaussian" or "trigflow"
    tangent_scale: float = 1.0
    mask: dict = field(default=None, hash=False, compare=False)
    n_kv: int = None              # key/value rows (None: N, self-attention)
    d_v: int = None               # value head dim (None: d)

    @property
    def Nkv(self):
        return self.N if self.n_kv is None else self.n_kv

    @property
    def dv(self):
        return self.d if self.d_v is None else self.d_v

    @property
    def flops(self):
        """Counted FLOPs of the dense definition per (batch, head): three
        products over d_qk (Q K^T, dQ K^T, Q dK^T) and three over d_v (P V,
        P dV, (P . dS) V), 2 Lq Lkv d each; 12 N^2 d when square."""
        return 6.0 * self.B * self.H * self.N * self.Nkv * (self.d + self.dv)


FRAME_WINDOW_65520 = {
    "frames": 42, "tokens_per_frame": 1560, "chunk_frames": 5,
    "radius_chunks": 1, "anchor_first": 1, "anchor_last": 1,
    "anchor_queries_see_all": 0,
}

WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_fp32", 1, 2, 128, 64, "fp32", 1001, tangent_scale=0.1),
        Workload("image_dit_4096", 2, 24, 4096, 128, "bf16", 1002,
                 rms_qk=True, tangents="trigflow"),
        Workload("t2i_prefix_4352", 4, 16, 4352, 64, "bf16", 1003,
                 tangent_scale=1e-2),
        Workload("video_dit_32760", 1, 40, 32760, 128, "bf16", 1004,
                 rms_qk=True, tangent_scale=0.1),
        Workload("long_video_65520", 1, 24, 65520, 128, "bf16", 1005,
                 tangent_scale=0.1, mask=FRAME_WINDOW_65520),
    ]
}


def _rng(seed, tid, b=0, h=0):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, b, h])))


def _rms_normalise(x, eps=1e-6):
    # RMSNorm with unit weight, per row over the head dimension (page "Обслуживание
    # Ideogram v4 менее чем за секунду", dev48.org, the RMSNorm epilogue section)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def _threads():
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:
        return 4


def make_inputs(w, seed=None):
    """Return a dict of CPU torch tensors q, dq [B, H, N, d], k, dk [B, H,
    Nkv, d], v, dv [B, H, Nkv, dv] (contiguous, in the workload dtype) plus
    ``scale`` (None = 1/sqrt(d)) and ``mask`` (a frame-window dict or None)."""
    seed = w.seed if seed is None else seed
    tdt = _TORCH_DTYPE[w.dtype]
    B, H, N, d = w.B, w.H, w.N, w.d
    rows = {"q": N, "k": w.Nkv, "v": w.Nkv}
    cols = {"q": d, "k": d, "v": w.dv}
    out = {n: torch.empty((B, H, rows[n[-1]], cols[n[-1]]), dtype=tdt)
           for n in ("q", "k", "v", "dq", "dk", "dv")}

    if w.tangents == "trigflow":
        if w.Nkv != N or w.dv != d:
            raise ValueError("the TrigFlow tangent recipe is for self-attention shapes")
        t = float(_rng(seed, _ID["t"]).uniform(0.0, math.pi / 2))
        wmat = {n: _rng(seed, _ID["w" + n]).standard_normal((d, d)) / math.sqrt(d)
                for n in ("q", "k", "v")}
    else:
        t, wmat = None, None

    def slab(bh):
        b, h = divmod(bh, H)
        for n in ("q", "k", "v"):
            x = _rng(seed, _ID[n], b, h).standard_normal((rows[n], cols[n]))
            if w.rms_qk and n in ("q", "k"):
                x = _rms_normalise(x)
            out[n][b, h] = torch.from_numpy(x).to(tdt)
        if w.tangents == "trigflow":
            x0 = _rng(seed, _ID["x0"], b, h).standard_normal((N, d))
            eps = _rng(seed, _ID["eps"], b, h).standard_normal((N, d))
            dx = -math.sin(t) * x0 + math.cos(t) * eps     # TrigFlow-path velocity
            for n in ("q", "k", "v"):
                out["d" + n][b, h] = torch.from_numpy(dx @ wmat[n]).to(tdt)
        else:
            for n in ("dq", "dk", "dv"):
                x = _rng(seed, _ID[n], b, h).standard_normal((rows[n[1]], cols[n[1]])) * w.tangent_scale
                out[n][b, h] = torch.from_numpy(x).to(tdt)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(slab, range(B * H)))
    out["scale"] = None
    out["mask"] = None if w.mask is None else dict(w.mask)
    out["trigflow_t"] = t
    return out


def to_float64(x):
    """Exact float64 numpy copy of a (CPU or GPU) torch tensor."""
    return x.detach().to("cpu", torch.float64).numpy()


def sample_rows(N, every=64, block=128, tokens_per_frame=None, edge_blocks=4):
    """Deterministic query-row sample for checks at full size.

    Every ``every``-th row, the rows on both sides of the first and last
    ``edge_blocks`` query-block boundaries, every row of the last (ragged)
    query block, and when ``tokens_per_frame`` is given the two rows around
    every frame boundary.
    """
    rows = set(range(0, N, every))
    nb = (N + block - 1) // block
    for b in list(range(min(edge_blocks, nb))) + list(range(max(0, nb - edge_blocks), nb)):
        for r in (b * block - 1, b * block, b * block + block - 1):
            if 0 <= r < N:
                rows.add(r)
    rows.update(range((nb - 1) * block, N))
    if tokens_per_frame:
        for f in range(0, N + 1, tokens_per_frame):
            for r in (f - 1, f):
                if 0 <= r < N:
                    rows.add(r)
    return np.array(sorted(rows), dtype=np.int64)
