"""Host-only checks of the C-ABI library: it loads, exports every function the
header declares, validates arguments without launching, and its tile
scheduler visits exactly the key tiles the oracle's mask makes visible.
No test here touches a GPU."""

import os
import re

import numpy as np
import pytest

import attention_jvp_amd as aj
from oracle import FrameWindow

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_jvp.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_jvp_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    declared = _declared_functions()
    assert "attn_jvp_fwd" in declared and "attn_jvp_fwd_strided" in declared
    lib = aj.load()
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(aj.exported_symbols()) == declared


def _layout(B, H, N, d):
    s = (H * N * d, N * d, d)
    lay = aj.Layout()
    for n in ("q", "k", "v", "dq", "dk", "dv", "o", "dout"):
        getattr(lay, n)[:] = s
    return lay


def _ptrs(B, H, N, d, esize, gap=1 << 20):
    """Fake, well-separated, 256-byte aligned device addresses (never used)."""
    size = B * H * N * d * esize + gap
    base = 1 << 40
    return [base + i * size for i in range(10)]


def _check(B=1, H=2, N=100, d=128, dtype=0, lay=None, mask=None, ptrs=None):
    esize = 2 if dtype == 0 else 4
    p = _ptrs(B, H, N, d, esize) if ptrs is None else ptrs
    lay = _layout(B, H, N, d) if lay is None else lay
    return aj.attn_jvp_check(*p, B, H, N, d, dtype, lay, mask)


def test_valid_arguments():
    assert _check() == 0
    for d in (16, 32, 64, 256):
        assert _check(d=d) == 0, d
    for d in (16, 32, 64):
        assert _check(d=d, dtype=1) == 0, d
    assert _check(N=65520, H=1, mask=dict(frames=42, tokens_per_frame=1560, chunk_frames=5,
                                          radius_chunks=1)) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), -1), (dict(H=-1), -1), (dict(N=0), -1), (dict(dtype=7), -1),
    (dict(d=96), -2), (dict(d=512), -2), (dict(d=8), -2), (dict(d=128, dtype=1), -2),
    (dict(d=256, dtype=1), -2),
])
def test_rejected_sizes(kw, status):
    assert _check(**kw) == status


def test_null_pointers_and_layout():
    p = _ptrs(1, 2, 100, 128, 2)
    for i in range(10):
        q = list(p)
        q[i] = None
        assert aj.attn_jvp_check(*q, 1, 2, 100, 128, 0, _layout(1, 2, 100, 128), None) == -1
    assert aj.attn_jvp_check(*p, 1, 2, 100, 128, 0, None, None) == -1


def test_tangent_strides_must_match_primal():
    for name in ("dq", "dk", "dv", "dout"):
        lay = _layout(1, 2, 100, 128)
        getattr(lay, name)[0] += 8
        assert _check(lay=lay) == -3, name


def test_alignment_and_overlap():
    lay = _layout(1, 2, 100, 128)
    lay.k[2] = 132            # row stride not a multiple of 8 bf16
    lay.dk[2] = 132
    assert _check(lay=lay) == -3
    p = _ptrs(1, 2, 100, 128, 2)
    p[1] += 2                  # K not 16-byte aligned
    assert _check(ptrs=p) == -3
    p = _ptrs(1, 2, 100, 128, 2)
    p[6] = p[0] + 256          # O overlaps Q
    assert _check(ptrs=p) == -3
    p = _ptrs(1, 2, 100, 128, 2)
    p[9] = p[8] + 4            # dLSE overlaps LSE
    assert _check(ptrs=p) == -3
    # a [B, N, H, d] buffer viewed as [B, H, N, d] is a valid layout
    B, H, N, d = 2, 3, 50, 64
    lay = aj.Layout()
    for n in ("q", "k", "v", "dq", "dk", "dv", "o", "dout"):
        getattr(lay, n)[:] = (N * H * d, d, H * d)
    assert _check(B=B, H=H, N=N, d=d, lay=lay) == 0


@pytest.mark.parametrize("mask", [
    dict(frames=41, tokens_per_frame=1560, chunk_frames=5, radius_chunks=1),
    dict(frames=42, tokens_per_frame=1560, chunk_frames=0, radius_chunks=1),
    dict(frames=42, tokens_per_frame=1560, chunk_frames=5, radius_chunks=-1),
])
def test_bad_mask(mask):
    assert _check(N=65520, H=1, mask=mask) == -4


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5, -6):
        assert aj.attn_jvp_status_string(s)
    assert aj.attn_jvp_status_string(-99) == "unknown status"


def test_tile_shape():
    assert aj.attn_jvp_tile_shape(0, 128) == (128, 64)    # bf16 d = 128: eight waves
    assert aj.attn_jvp_tile_shape(0, 64) == (192, 64)     # bf16 d = 64: twelve waves
    assert aj.attn_jvp_tile_shape(1, 64) == (64, 64)     # float32: four waves
    with pytest.raises(aj.AttnJvpError):
        aj.attn_jvp_tile_shape(1, 128)


def test_fwd_geometry_by_grid():
    # bf16 d = 64 without a mask: 64-row blocks and 32-key tiles where the
    # 192-row grid would end in a mostly idle round of the 256 CUs
    g = aj.attn_jvp_fwd_geometry
    assert g(2, 24, 4096, 4096, 64, 64, 0) == (64, 32)     # 4.1 rounds of 192 rows
    assert g(8, 24, 1024, 1024, 64, 64, 0) == (64, 32)
    assert g(8, 6, 1000, 1000, 64, 64, 0) == (64, 32)      # 2 rounds against 1
    assert g(4, 16, 4352, 4352, 64, 64, 0) == (192, 64)    # 5.75 rounds
    assert g(1, 16, 8192, 8192, 64, 64, 0) == (192, 64)
    assert g(1, 24, 16384, 16384, 64, 64, 0) == (64, 32)    # 8.1 rounds against 8
    assert g(1, 2, 300, 300, 64, 64, 0) == (192, 64)       # below one round either way
    # the default geometry everywhere else: masks, other head dims, float32
    mask = dict(frames=32, tokens_per_frame=128, chunk_frames=2, radius_chunks=1)
    assert g(2, 24, 4096, 4096, 64, 64, 0, mask) == aj.attn_jvp_tile_shape(0, 64)
    assert g(2, 24, 4096, 4096, 128, 128, 0) == aj.attn_jvp_tile_shape(0, 128)
    assert g(2, 24, 4096, 4096, 64, 128, 0) == aj.attn_jvp_tile_shape_ex(0, 64, 128)
    assert g(2, 24, 4096, 4096, 64, 64, 1) == aj.attn_jvp_tile_shape(1, 64)
    assert g(2, 24, 4096, 4096, 32, 32, 0) == aj.attn_jvp_tile_shape(0, 32)
    for args in ((0, 24, 4096, 4096, 64, 64, 0), (2, 24, 4096, 0, 64, 64, 0),
                 (2, 24, 4096, 4096, 48, 48, 0), (2, 24, 4096, 4096, 64, 64, 3)):
        with pytest.raises(aj.AttnJvpError):
            g(*args)


def test_tile_shape_unequal_head_dims():
    # eight waves x 16 rows while the resident registers fit two waves per
    # SIMD, else four; 64-key tiles while two LDS stages fit in 128 KiB
    assert aj.attn_jvp_tile_shape_ex(0, 128, 128) == (128, 64)
    assert aj.attn_jvp_tile_shape_ex(0, 128, 64) == (128, 64)
    assert aj.attn_jvp_tile_shape_ex(0, 256, 256) == (64, 32)
    assert aj.attn_jvp_tile_shape_ex(0, 256, 64) == (128, 32)
    assert aj.attn_jvp_tile_shape_ex(0, 64, 256) == (64, 32)
    assert aj.attn_jvp_tile_shape_ex(0, 16, 128) == (128, 64)
    assert aj.attn_jvp_tile_shape_ex(1, 16, 64) == (128, 64)
    assert aj.attn_jvp_tile_shape(0, 128) == aj.attn_jvp_tile_shape_ex(0, 128, 128)
    for args in ((0, 96, 64), (0, 64, 512), (1, 64, 128), (2, 64, 64)):
        with pytest.raises(aj.AttnJvpError):
            aj.attn_jvp_tile_shape_ex(*args)


def _check_ex(B=1, H=2, Nq=100, Nkv=300, dqk=64, dv=128, dtype=0, lay=None, mask=None,
              ptrs=None):
    esize = 2 if dtype == 0 else 4
    p = _ptrs(B, H, max(Nq, Nkv), max(dqk, dv), esize) if ptrs is None else ptrs
    return aj.attn_jvp_check_ex(*p, aj.Shape(B, H, Nq, Nkv, dqk, dv), dtype, lay, mask)


def test_check_ex_unequal_shapes():
    assert _check_ex() == 0
    assert _check_ex(Nq=300, Nkv=77, dqk=256, dv=16) == 0
    assert _check_ex(dqk=32, dv=64, dtype=1) == 0
    assert _check_ex(Nkv=0) == -1
    assert _check_ex(dqk=48) == -2
    assert _check_ex(dv=128, dtype=1) == -2
    # the frame window is a self-attention mask with one head dim
    fw = dict(frames=3, tokens_per_frame=100, chunk_frames=1, radius_chunks=0)
    assert _check_ex(Nq=300, Nkv=300, dqk=64, dv=64, mask=fw) == 0
    assert _check_ex(Nq=300, Nkv=300, dqk=64, dv=128, mask=fw) == -2
    assert _check_ex(Nq=100, Nkv=300, dqk=64, dv=64, mask=fw) == -4


def test_check_ex_extents_use_each_tensors_shape():
    # contiguous layouts of the general shape; O directly after V must pass,
    # O one row earlier overlaps V's last row
    B, H, Nq, Nkv, dqk, dv = 1, 2, 40, 96, 32, 128
    sizes = [B * H * n * d * 2 for n, d in ((Nq, dqk), (Nkv, dqk), (Nkv, dv),
                                             (Nq, dqk), (Nkv, dqk), (Nkv, dv),
                                             (Nq, dv), (Nq, dv))]
    base, p = 1 << 40, []
    for sz in sizes:
        p.append(base)
        base += sz
    p += [base, base + B * H * Nq * 4]
    shape = aj.Shape(B, H, Nq, Nkv, dqk, dv)
    assert aj.attn_jvp_check_ex(*p, shape, 0, None, None) == 0
    p2 = list(p)
    p2[6] -= dv * 2
    assert aj.attn_jvp_check_ex(*p2, shape, 0, None, None) == -3


def _tiles_with_visible_pairs(w, N, bm, bn):
    """Brute force with the oracle's mask: key tiles holding at least one
    visible (query, key) pair, per query block."""
    out = []
    kidx = np.arange(N)
    for q0 in range(0, N, bm):
        rows = np.arange(q0, min(q0 + bm, N))
        # visibility depends on the query's frame only: one row per frame
        _, first = np.unique(rows // w.tokens_per_frame, return_index=True)
        vis = w(rows[first], kidx).any(axis=0)
        tiles = {j // bn for j in np.nonzero(vis)[0]}
        out.append(len(tiles))
    return out


@pytest.mark.parametrize("F,T,C,R,first,last,see_all", [
    (42, 1560, 5, 1, 1, 1, 0),
    (42, 1560, 5, 1, 1, 1, 1),
    (21, 100, 3, 1, 1, 0, 0),
    (17, 37, 2, 0, 0, 1, 0),
    (9, 300, 4, 2, 0, 0, 0),
    (50, 7, 1, 0, 1, 1, 1),
])
def test_scheduler_visits_exactly_the_visible_tiles(F, T, C, R, first, last, see_all):
    N = F * T
    mask = dict(frames=F, tokens_per_frame=T, chunk_frames=C, radius_chunks=R,
                anchor_first=first, anchor_last=last, anchor_queries_see_all=see_all)
    got = aj.attn_jvp_visible_tiles(N, 0, 128, mask)
    w = FrameWindow(F, T, C, R, bool(first), bool(last), bool(see_all))
    bm, bn = aj.attn_jvp_tile_shape(0, 128)
    assert got == _tiles_with_visible_pairs(w, N, bm, bn)


def _bwd_tiles_with_visible_pairs(w, N, block, tile, keys):
    # brute force: per owned block, the streamed tiles holding a pair the
    # oracle's window shows (owned rows are keys when `keys`)
    idx = np.arange(N)
    out = []
    for r0 in range(0, N, block):
        rows = np.arange(r0, min(r0 + block, N))
        vis = (w(idx, rows) if keys else w(rows, idx)).any(axis=1 if keys else 0)
        out.append(len({j // tile for j in np.nonzero(vis)[0]}))
    return out


@pytest.mark.parametrize("F,T,C,R,first,last,see_all", [
    (21, 100, 3, 1, 1, 0, 0),
    (17, 37, 2, 0, 0, 1, 0),
    (9, 300, 4, 2, 0, 0, 0),
    (50, 7, 1, 0, 1, 1, 1),
    (12, 64, 2, 0, 1, 1, 1),
    (14, 90, 3, 1, 0, 0, 1),
])
@pytest.mark.parametrize("block,tile", [(64, 64), (128, 64), (256, 32)])
def test_backward_scheduler_visits_exactly_the_visible_tiles(F, T, C, R, first, last, see_all,
                                                             block, tile):
    N = F * T
    mask = dict(frames=F, tokens_per_frame=T, chunk_frames=C, radius_chunks=R,
                anchor_first=first, anchor_last=last, anchor_queries_see_all=see_all)
    w = FrameWindow(F, T, C, R, bool(first), bool(last), bool(see_all))
    for keys in (0, 1):
        got = aj.attn_jvp_bwd_visible_tiles(N, block, tile, keys, mask)
        assert got == _bwd_tiles_with_visible_pairs(w, N, block, tile, keys), (keys, got)
    dense = aj.attn_jvp_bwd_visible_tiles(N, block, tile, 1)
    assert dense == [(N + tile - 1) // tile] * ((N + block - 1) // block)


def test_dense_scheduler_visits_every_tile():
    got = aj.attn_jvp_visible_tiles(4352, 0, 64)
    assert got == [68] * 23          # 192-row query blocks at bf16 d = 64


def test_long_video_visited_fraction():
    mask = dict(frames=42, tokens_per_frame=1560, chunk_frames=5, radius_chunks=1)
    got = aj.attn_jvp_visible_tiles(65520, 0, 128, mask)
    _, bn = aj.attn_jvp_tile_shape(0, 128)
    total = len(got) * ((65520 + bn - 1) // bn)
    assert 0.36 < sum(got) / total < 0.38


def _bwd_ptrs(B, H, Nq, Nkv, d, esize):
    sizes = [B * H * n * d * esize for n in (Nq, Nkv, Nkv, Nq, Nq)] + [B * H * Nq * 4] + \
        [B * H * n * d * esize for n in (Nq, Nkv, Nkv)] + [B * H * Nq * 4]
    base, p = 1 << 40, []
    for sz in sizes:
        p.append(base)
        base += (sz + 255) // 256 * 256
    return p


def test_bwd_check():
    shape = aj.Shape(2, 3, 100, 260, 128, 128)
    p = _bwd_ptrs(2, 3, 100, 260, 128, 2)
    assert aj.attn_jvp_bwd_check(*p, shape, 0) == 0
    for d in (16, 32, 64, 256):
        sh = aj.Shape(1, 2, 50, 70, d, d)
        assert aj.attn_jvp_bwd_check(*_bwd_ptrs(1, 2, 50, 70, d, 2), sh, 0) == 0, d
    assert aj.attn_jvp_bwd_check(*_bwd_ptrs(1, 2, 50, 70, 64, 4), aj.Shape(1, 2, 50, 70, 64, 64), 1) == 0
    assert aj.attn_jvp_bwd_check(*p, aj.Shape(2, 3, 100, 260, 128, 64), 0) == -2   # d_qk != d_v
    assert aj.attn_jvp_bwd_check(*p, aj.Shape(2, 3, 100, 260, 96, 96), 0) == -2
    assert aj.attn_jvp_bwd_check(*_bwd_ptrs(1, 2, 50, 70, 128, 4), aj.Shape(1, 2, 50, 70, 128, 128), 1) == -2
    assert aj.attn_jvp_bwd_check(*p, aj.Shape(2, 3, 0, 260, 128, 128), 0) == -1
    q = list(p)
    q[5] = None                                     # LSE
    assert aj.attn_jvp_bwd_check(*q, shape, 0) == -1
    q = list(p)
    q[6] = p[0] + 512                               # dQ overlaps Q
    assert aj.attn_jvp_bwd_check(*q, shape, 0) == -3
    q = list(p)
    q[9] = p[5]                                     # delta overlaps LSE
    assert aj.attn_jvp_bwd_check(*q, shape, 0) == -3
    # frame-window mask: the forward's rules (square, frames x tokens = N)
    win = aj.Mask.frame_window(frames=5, tokens_per_frame=40, chunk_frames=2, radius_chunks=1)
    ps = _bwd_ptrs(1, 2, 200, 200, 64, 2)
    sq = aj.Shape(1, 2, 200, 200, 64, 64)
    assert aj.attn_jvp_bwd_check(*ps, sq, 0, None, win) == 0
    assert aj.attn_jvp_bwd_check(*_bwd_ptrs(1, 2, 200, 240, 64, 2), aj.Shape(1, 2, 200, 240, 64, 64),
                                 0, None, win) == -4                          # Lq != Lkv
    bad = aj.Mask.frame_window(frames=6, tokens_per_frame=40, chunk_frames=2, radius_chunks=1)
    assert aj.attn_jvp_bwd_check(*ps, sq, 0, None, bad) == -4                 # 240 tokens != 200


def test_library_matches_its_sources(monkeypatch):
    # the loaded library carries the digest of the sources it was built from
    import attention_jvp_amd.build as build
    lib = aj.load()
    assert lib.attn_jvp_build_id().decode() == build.source_digest()
    # a library older than the sources beside it is refused
    monkeypatch.setattr(build, "source_digest", lambda: "0" * 64)
    monkeypatch.setattr(aj, "_lib", None)
    with pytest.raises(ImportError, match="other sources"):
        aj.load()
    monkeypatch.undo()
    assert aj.load() is lib or aj.load() is not None
