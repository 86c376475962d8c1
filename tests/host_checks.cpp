// Host-side checks of the attn_jvp validation and planning code, built with
// the host compiler under AddressSanitizer and UndefinedBehaviorSanitizer
// (tests/test_host_sanitized.py builds and runs it; no GPU involved).
//
//  1. Work lists: for many frame-window masks (the long-video window, the
//     masks of the GPU tests, and edge shapes: one frame, one token per frame,
//     chunks larger than the sequence, radius 0 and beyond every chunk,
//     anchors on and off, anchor queries seeing everything) and every built
//     launch geometry, every tile index a block walks (visible_tiles for the
//     forward and the dQ launch, visible_query_tiles for the dK/dV launch) is
//     inside the sequence, the ranges are ascending and disjoint, and the set
//     of tiles equals the tiles holding a visible pair under a brute-force
//     predicate written here from the definition.
//  2. Argument validation on fabricated pointers (never dereferenced) and
//     sizes up to the limits of the types: every call returns a status, the
//     launch-size limits hold, and a set of known-bad calls is rejected.
//  3. Split planning: choose_splits and split_workspace over many shapes.
//  4. The tile walk: for random sets of up to three ascending disjoint
//     ranges (empty ones included), tile_walk / walk_at give, for every
//     index below tile_count, the tiles of the ranges in ascending order.
//
// Prints "host checks: ok" and exits 0, or prints the first failure and
// exits 1.

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "attn_jvp.h"
#include "host.h"

using namespace attn_jvp;

static int failures = 0;

#define CHECK(cond, ...)                                   \
  do {                                                     \
    if (!(cond)) {                                         \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);                        \
      fprintf(stderr, "\n");                               \
      if (++failures > 20) exit(1);                        \
    }                                                      \
  } while (0)

// The frame-window predicate from its definition: query frame qf sees key
// frame kf when their chunks are at most R apart, or kf is an anchor frame,
// or (see_all) qf is an anchor frame.
struct Window {
  int frames, tpf, chunk, radius, first, last, see_all;
  bool anchor(int f) const { return (first && f == 0) || (last && f == frames - 1); }
  bool visible(int q, int k) const {
    const int qf = q / tpf, kf = k / tpf;
    const int dc = qf / chunk - kf / chunk;
    if (dc <= radius && -dc <= radius) return true;
    if (anchor(kf)) return true;
    return see_all && anchor(qf);
  }
  attn_jvp_mask desc() const {
    attn_jvp_mask m;
    m.kind = ATTN_JVP_MASK_FRAME_WINDOW;
    m.frames = frames;
    m.tokens_per_frame = tpf;
    m.chunk_frames = chunk;
    m.radius_chunks = radius;
    m.anchor_first = first;
    m.anchor_last = last;
    m.anchor_queries_see_all = see_all;
    return m;
  }
};

// One block's work list against brute force.  keys: the block owns keys
// and walks query tiles (the transpose).
static void check_block(const Window &w, const MaskDev &m, int r0, int r1, int BN, bool keys,
                        const char *what) {
  const int N = w.frames * w.tpf;
  const int ntiles = (N + BN - 1) / BN;
  const TileRanges tr = keys ? visible_query_tiles(m, r0, r1, N, BN)
                             : visible_tiles(m, r0, r1, N, BN);
  CHECK(tr.n >= 1 && tr.n <= 3, "%s: %d ranges", what, tr.n);
  for (int i = 0; i < tr.n; ++i) {
    CHECK(0 <= tr.lo[i] && tr.lo[i] < tr.hi[i] && tr.hi[i] <= ntiles,
          "%s: range %d [%d, %d) of %d tiles (rows %d..%d)", what, i, tr.lo[i], tr.hi[i],
          ntiles, r0, r1);
    if (i > 0) CHECK(tr.hi[i - 1] < tr.lo[i], "%s: ranges %d, %d touch or overlap", what, i - 1, i);
  }
  for (int i = tr.n; i < 3; ++i)
    CHECK(tr.lo[i] == 0 && tr.hi[i] == 0, "%s: unused range %d not empty", what, i);
  std::vector<char> walked(ntiles, 0);
  const int n = tile_count(tr);
  for (int it = 0; it < n; ++it) {
    const int t = tile_at(tr, it);
    CHECK(t >= 0 && t < ntiles, "%s: tile %d out of [0, %d)", what, t, ntiles);
    if (t < 0 || t >= ntiles) return;
    CHECK(!walked[t], "%s: tile %d walked twice", what, t);
    walked[t] = 1;
    if (it > 0) CHECK(t > tile_at(tr, it - 1), "%s: tiles not ascending", what);
  }
  // visibility depends on frames only, and every frame between the first
  // and the last row of a contiguous row range holds one of its rows: a tile
  // holds a visible pair iff some (block frame, tile frame) pair is visible
  const int f0 = r0 / w.tpf, f1 = (r1 - 1) / w.tpf;
  for (int t = 0; t < ntiles; ++t) {
    bool any = false;
    const int g0 = t * BN / w.tpf, g1 = ((t + 1) * BN < N ? (t + 1) * BN - 1 : N - 1) / w.tpf;
    for (int a = f0; a <= f1 && !any; ++a)
      for (int b = g0; b <= g1 && !any; ++b)
        any = keys ? w.visible(b * w.tpf, a * w.tpf) : w.visible(a * w.tpf, b * w.tpf);
    CHECK(walked[t] == (any ? 1 : 0), "%s: rows %d..%d tile %d walked %d, visible pair %d",
          what, r0, r1, t, walked[t], any);
  }
}

static void check_window(const Window &w) {
  const attn_jvp_mask desc = w.desc();
  const int N = w.frames * w.tpf;
  CHECK(check_mask(&desc, N, N) == ATTN_JVP_OK, "mask rejected");
  const MaskDev m = to_dev(&desc);
  char what[160];
  // forward geometries and the backward launches' rows / tiles
  const int rows[] = {16, 64, 128, 192, 256};
  const int tiles[] = {32, 64};
  for (int br : rows)
    for (int bn : tiles) {
      for (int keys = 0; keys < 2; ++keys) {
        snprintf(what, sizeof what, "F%d T%d C%d R%d a%d%d%d rows%d tile%d %s", w.frames, w.tpf,
                 w.chunk, w.radius, w.first, w.last, w.see_all, br, bn, keys ? "keys" : "queries");
        for (int r0 = 0; r0 < N; r0 += br) check_block(w, m, r0, r0 + br < N ? r0 + br : N, bn,
                                                       keys != 0, what);
      }
    }
}

static void check_work_lists() {
  // small analogues and edge shapes, exhaustively
  const int F[] = {1, 2, 3, 5, 7, 11};
  const int T[] = {1, 3, 17, 40, 64};
  const int C[] = {1, 2, 3, 5, 13};
  const int R[] = {0, 1, 2, 9};
  for (int f : F)
    for (int t : T)
      for (int c : C)
        for (int r : R)
          for (int a = 0; a < 8; ++a) {
            if (f * t > 2000) continue;
            check_window(Window{f, t, c, r, a & 1, (a >> 1) & 1, (a >> 2) & 1});
          }
  // the masks of the GPU tests
  const Window gpu[] = {{7, 37, 2, 1, 1, 1, 0},  {9, 64, 3, 0, 1, 0, 0}, {6, 50, 2, 0, 0, 1, 1},
                        {11, 40, 1, 1, 1, 1, 0}, {5, 100, 5, 0, 0, 0, 0}, {12, 30, 2, 0, 1, 1, 1},
                        {8, 33, 3, 1, 0, 0, 1},  {10, 60, 2, 0, 1, 1, 0}, {10, 30, 2, 1, 1, 1, 0}};
  for (const Window &w : gpu) check_window(w);
  // the long-video window at full size: bounds and brute force on the
  // frame grid (a tile is visible when some pair of its frames is)
  const Window lv{42, 1560, 5, 1, 1, 1, 0};
  const attn_jvp_mask desc = lv.desc();
  const MaskDev m = to_dev(&desc);
  const int N = lv.frames * lv.tpf;
  const FwdGeom g = fwd_geom(2, 128, 128);
  int64_t walked = 0;
  for (int keys = 0; keys < 2; ++keys)
    for (int r0 = 0; r0 < N; r0 += g.block_m) {
      const int r1 = r0 + g.block_m < N ? r0 + g.block_m : N;
      const TileRanges tr = keys ? visible_query_tiles(m, r0, r1, N, g.block_n)
                                 : visible_tiles(m, r0, r1, N, g.block_n);
      const int n = tile_count(tr);
      if (!keys) walked += n;
      for (int it = 0; it < n; ++it) {
        const int t = tile_at(tr, it);
        CHECK(t >= 0 && t * g.block_n < N, "long video: tile %d", t);
        bool any = false;
        const int f0 = r0 / lv.tpf, f1 = (r1 - 1) / lv.tpf;
        const int kf0 = t * g.block_n / lv.tpf;
        const int kf1 = ((t + 1) * g.block_n < N ? (t + 1) * g.block_n - 1 : N - 1) / lv.tpf;
        for (int a = f0; a <= f1 && !any; ++a)
          for (int b = kf0; b <= kf1 && !any; ++b)
            any = keys ? lv.visible(b * lv.tpf, a * lv.tpf) : lv.visible(a * lv.tpf, b * lv.tpf);
        CHECK(any, "long video: tile %d of rows %d..%d holds no visible frame pair", t, r0, r1);
      }
    }
  printf("long-video forward work list: %lld of %lld tiles\n", (long long)walked,
         (long long)((N + g.block_m - 1) / g.block_m) * ((N + g.block_n - 1) / g.block_n));
}

// Fabricated, 256-byte aligned, non-overlapping device addresses.
struct Fake {
  uintptr_t next = (uintptr_t)1 << 40;
  void *get(size_t bytes) {
    void *p = (void *)next;
    next += (bytes + 4095) & ~(size_t)4095;
    next += 4096;
    return p;
  }
};

static void check_validation() {
  Fake f;
  const attn_jvp_shape s = {2, 24, 4096, 4096, 128, 128};
  const attn_jvp_layout L = contiguous(s);
  const size_t t = (size_t)2 * 24 * 4096 * 128 * 2;
  void *p[8];
  for (int i = 0; i < 8; ++i) p[i] = f.get(t);
  float *lse = (float *)f.get(2 * 24 * 4096 * 4), *dlse = (float *)f.get(2 * 24 * 4096 * 4);
  CHECK(check_args(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], lse, dlse, &s, ATTN_JVP_BF16,
                   &L, nullptr) == ATTN_JVP_OK, "image-DiT call rejected");
  // outputs overlapping an input
  CHECK(check_args(p[0], p[1], p[2], p[3], p[4], p[5], p[1], p[7], lse, dlse, &s, ATTN_JVP_BF16,
                   &L, nullptr) == ATTN_JVP_ESTRIDE, "overlap accepted");
  // misaligned pointer
  CHECK(check_args((char *)p[0] + 2, p[1], p[2], p[3], p[4], p[5], p[6], p[7], lse, dlse, &s,
                   ATTN_JVP_BF16, &L, nullptr) == ATTN_JVP_ESTRIDE, "misaligned accepted");
  // unbuilt head dim
  attn_jvp_shape s2 = s;
  s2.head_dim_qk = 96;
  CHECK(check_args(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], lse, dlse, &s2, ATTN_JVP_BF16,
                   &L, nullptr) == ATTN_JVP_EUNSUPPORTED, "d=96 accepted");
  // float32 d = 128 is not built
  CHECK(check_args(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], lse, dlse, &s, ATTN_JVP_FP32,
                   &L, nullptr) == ATTN_JVP_EUNSUPPORTED, "fp32 d=128 accepted");
  // a tangent stride that differs from its primal's
  attn_jvp_layout L2 = L;
  L2.dk[2] = 136;
  CHECK(check_args(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], lse, dlse, &s, ATTN_JVP_BF16,
                   &L2, nullptr) == ATTN_JVP_ESTRIDE, "tangent stride accepted");
  // launches whose work-item count exceeds 32 bits (sizes are not checked
  // against memory here: the pointers are fabricated)
  attn_jvp_shape big = {1, 1 << 20, 1 << 14, 128, 128, 128};
  const attn_jvp_layout LB = contiguous(big);
  const int st = check_args(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], lse, dlse, &big,
                            ATTN_JVP_BF16, &LB, nullptr);
  CHECK(st != ATTN_JVP_OK, "a launch of 2^27 workgroups accepted (%d)", st);
  const FwdGeom g = fwd_geom(2, 128, 128);
  CHECK(!grid_fits(((int64_t)1 << 32) / (64 * g.waves) + 1, 64 * g.waves), "grid limit");
  CHECK(grid_fits(((int64_t)1 << 32) / (64 * g.waves) - 1, 64 * g.waves), "grid limit");
  // the small geometry: only unmasked bfloat16 d_qk = d_v = 64, its grid
  // within the launch limits, and the query reports what the launch takes
  {
    const attn_jvp_mask fw = {ATTN_JVP_MASK_FRAME_WINDOW, 4, 64, 2, 1, 1, 1, 0};
    uint64_t y = 0x243f6a8885a308d3ull;
    const int dims[5] = {16, 32, 64, 128, 256};
    int taken = 0;
    for (int i = 0; i < 20000; ++i) {
      y ^= y << 13;
      y ^= y >> 7;
      y ^= y << 17;
      const int d = dims[y % 5], dtype = (int)((y >> 8) % 2);
      const bool masked = (y >> 60) & 1;   // the window holds 256 tokens
      const int bh = 1 + (int)((y >> 16) % 4096);
      const int nq = masked ? 256 : 1 + (int)((y >> 32) % 70000);
      const attn_jvp_shape sh = {1, bh, nq, nq, d, d};
      const bool sm = launch_small(sh, dtype, masked ? &fw : nullptr);
      if (sm) {
        ++taken;
        CHECK(dtype == ATTN_JVP_BF16 && d == 64 && !masked, "small geometry for dtype %d d %d", dtype, d);
        const FwdGeom gs = fwd16_geom_small(2, 64, 64);
        CHECK(grid_fits((int64_t)bh * ((nq + gs.block_m - 1) / gs.block_m), 64 * gs.waves),
              "small grid beyond the launch limits");
      }
      int bm = 0, bn = 0;
      const int gst = attn_jvp_fwd_geometry(&sh, dtype, masked ? &fw : nullptr, &bm, &bn);
      if (fwd_built(dtype == ATTN_JVP_BF16 ? 2 : 4, d, d)) {
        const FwdGeom gd = fwd_geom(dtype == ATTN_JVP_BF16 ? 2 : 4, d, d);
        const FwdGeom ge = sm ? fwd16_geom_small(2, 64, 64) : gd;
        CHECK(gst == ATTN_JVP_OK && bm == ge.block_m && bn == ge.block_n,
              "fwd_geometry %d: (%d, %d)", gst, bm, bn);
      } else {
        CHECK(gst == ATTN_JVP_EUNSUPPORTED, "fwd_geometry of an unbuilt dim: %d", gst);
      }
    }
    CHECK(taken > 0, "the small geometry never taken");
  }
  // pseudo-random calls: every one returns a status, and OK only for calls
  // that satisfy the documented rules this loop can state
  uint64_t x = 0x9e3779b97f4a7c15ull;
  auto rnd = [&x]() {
    x ^= x << 13;
    x ^= x >> 7;
    x ^= x << 17;
    return x;
  };
  const int dims[] = {1, 8, 16, 32, 64, 96, 128, 256, 512};
  for (int i = 0; i < 50000; ++i) {
    attn_jvp_shape r;
    r.batch = (int)(rnd() % 5) - 1 + ((rnd() & 1023) == 0 ? (1 << 30) : 0);
    r.heads = (int)(rnd() % 70) - 1;
    r.seqlen_q = (rnd() & 255) == 0 ? 0x7fff0000 + (int)(rnd() % 0xffff)
                                    : (int)(rnd() % 100000) - 2;
    r.seqlen_kv = (int)(rnd() % 100000) - 2;
    r.head_dim_qk = dims[rnd() % 9];
    r.head_dim_v = dims[rnd() % 9];
    const int dtype = (int)(rnd() % 3);
    attn_jvp_layout Lr = contiguous(r);
    if (rnd() & 1) {
      for (int j = 0; j < 3; ++j) {
        Lr.q[j] = Lr.dq[j] = (int64_t)(rnd() % (1ull << 45)) - 8;
        Lr.o[j] = Lr.dout[j] = (int64_t)(rnd() % 4096);
      }
    }
    attn_jvp_mask mk;
    mk.kind = (int)(rnd() % 3);
    mk.frames = (int)(rnd() % 50) - 1;
    mk.tokens_per_frame = (int)(rnd() % 2000);
    mk.chunk_frames = (int)(rnd() % 7) - 1;
    mk.radius_chunks = (int)(rnd() % 5) - 1;
    mk.anchor_first = (int)(rnd() & 1);
    mk.anchor_last = (int)(rnd() & 1);
    mk.anchor_queries_see_all = (int)(rnd() & 1);
    const int code = check_args(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], lse, dlse, &r,
                                dtype, &Lr, (rnd() & 1) ? &mk : nullptr);
    CHECK(code <= 0 && code >= ATTN_JVP_EHIP, "status %d", code);
    if (code == ATTN_JVP_OK) {
      FwdGeom gg;
      CHECK(r.batch > 0 && r.heads > 0 && r.seqlen_q > 0 && r.seqlen_kv > 0, "sizes");
      CHECK(shape_for(dtype, r.head_dim_qk, r.head_dim_v, &gg), "unbuilt shape accepted");
      const int64_t nqb = (r.seqlen_q + gg.block_m - 1) / gg.block_m;
      CHECK(grid_fits((int64_t)r.batch * r.heads * nqb, 64 * gg.waves), "grid");
    }
    attn_jvp_bwd_layout Lb = contiguous_bwd(r);
    const int cb = check_bwd(p[0], p[1], p[2], p[3], p[4], lse, p[5], p[6], p[7], dlse, &r,
                             dtype, &Lb, nullptr);
    CHECK(cb <= 0 && cb >= ATTN_JVP_EHIP, "bwd status %d", cb);
    MergeParams mp;
    const int cm = check_merge((int)(rnd() % 70) - 1, (const float *)p[0], (const float *)p[1],
                               lse, dlse, p[6], p[7], (const float *)p[2], (const float *)p[3],
                               r.batch, r.heads, r.seqlen_q, r.head_dim_v, dtype, nullptr, &mp);
    CHECK(cm <= 0 && cm >= ATTN_JVP_EHIP, "merge status %d", cm);
  }
}

static void check_splits() {
  for (int b = 1; b <= 4; ++b)
    for (int h = 1; h <= 64; h *= 2)
      for (int nq = 1; nq <= 70000; nq = nq * 3 + 1)
        for (int nkv = 1; nkv <= 300000; nkv = nkv * 5 + 3) {
          const attn_jvp_shape s = {b, h, nq, nkv, 128, 64};
          const int ns = choose_splits(s, ATTN_JVP_BF16, nullptr);
          CHECK(ns >= 1 && ns <= 64, "splits %d", ns);
          const SplitWs w = split_workspace(s, ns);
          const size_t rows = (size_t)ns * b * h * nq;
          CHECK(w.o == 0 && w.dout >= rows * 64 * 4 && w.lse >= w.dout + rows * 64 * 4 &&
                    w.dlse >= w.lse + rows * 4 && w.total >= w.dlse + rows * 4,
                "workspace layout");
          CHECK(w.dout % 256 == 0 && w.lse % 256 == 0 && w.dlse % 256 == 0, "alignment");
        }
  // masked split planning on the long-video window
  const Window lv{42, 1560, 5, 1, 1, 1, 0};
  const attn_jvp_mask desc = lv.desc();
  const attn_jvp_shape s = {1, 1, 65520, 65520, 128, 128};
  const int ns = choose_splits(s, ATTN_JVP_BF16, &desc);
  CHECK(ns >= 1 && ns <= 64, "masked splits %d", ns);
}

static void check_walks() {
  uint32_t s = 12345u;
  auto rnd = [&](int n) {
    s = s * 1664525u + 1013904223u;
    return (int)((s >> 8) % (uint32_t)n);
  };
  for (int trial = 0; trial < 20000; ++trial) {
    TileRanges tr;
    tr.n = 1 + rnd(3);
    int at = rnd(5);
    for (int r = 0; r < 3; ++r) {
      if (r < tr.n) {
        tr.lo[r] = at;
        tr.hi[r] = at + (rnd(4) == 0 ? 0 : 1 + rnd(40));   // some ranges empty
        at = tr.hi[r] + rnd(30);
      } else {
        tr.lo[r] = tr.hi[r] = 0;   // unused ranges are empty
      }
    }
    std::vector<int> want;
    for (int r = 0; r < tr.n; ++r)
      for (int t = tr.lo[r]; t < tr.hi[r]; ++t) want.push_back(t);
    CHECK((int)want.size() == tile_count(tr), "walk: tile_count %d, %zu tiles", tile_count(tr),
          want.size());
    const TileWalk w = tile_walk(tr);
    for (int i = 0; i < (int)want.size(); ++i)
      CHECK(walk_at(w, i) == want[i] && tile_at(tr, i) == want[i],
            "walk: n %d ranges [%d,%d) [%d,%d) [%d,%d) index %d: %d, want %d", tr.n, tr.lo[0],
            tr.hi[0], tr.lo[1], tr.hi[1], tr.lo[2], tr.hi[2], i, walk_at(w, i), want[i]);
  }
}

int main() {
  check_walks();
  check_work_lists();
  check_validation();
  check_splits();
  if (failures) {
    printf("host checks: %d failures\n", failures);
    return 1;
  }
  printf("host checks: ok\n");
  return 0;
}
