// Launch planning shared by the host code and the kernels: the launch
// geometry of every instance, the frame-window mask descriptor and the
// visible-tile work lists, and the kernel parameter blocks.  Plain C++: the
// host unit (host.cpp) is built by the host compiler alone, so that the
// validation and planning code can also be built and exercised under the
// address and undefined-behaviour sanitizers on a machine without a GPU;
// under hipcc the mask functions are also device functions.

#pragma once

#include <limits.h>
#include <stdint.h>

#if defined(__HIPCC__)
#define AJ_HD __host__ __device__
#else
#define AJ_HD
#endif

namespace attn_jvp {

// ---------------------------------------------------------------------------
// Launch geometry of the forward kernel instance (element size es = 2 for
// bfloat16, 4 for float32; head dims d_qk, d_v).  16 query rows per wave.
//  * waves: eight (two per SIMD, <= 256 VGPRs each) while the resident
//    registers -- Q and dQ fragments, O, A, B accumulators -- stay within 128
//    per lane (64 for float32, whose score steps need more working
//    registers), else four (one per SIMD); bfloat16 d_qk = d_v = 64 runs
//    twelve (three per SIMD): its softmax VALU work per MFMA is twice that
//    of d = 128 and the third wave keeps the matrix cores fed.
//  * block_n: 64-key tiles while two LDS stages of K, dK, V, dV fit in
//    128 KiB, else 32.
// ---------------------------------------------------------------------------
struct FwdGeom {
  int waves, block_m, block_n, lds;
  bool rows32;   // the 32-query-row kernel (kernel32.h)
};

constexpr FwdGeom fwd16_geom(int es, int dqk, int dv) {
  const int resident = (es == 2 ? dqk / 4 : dqk / 2) + 3 * dv / 4;
  const int waves = (es == 2 && dqk == 64 && dv == 64) ? 12
                                                       : (resident <= (es == 2 ? 128 : 64) ? 8 : 4);
  const int row_bytes = (dqk + dv) * es;
  const int bn = 4 * 64 * row_bytes <= 128 * 1024 ? 64 : 32;
  return FwdGeom{waves, 16 * waves, bn, 4 * bn * row_bytes, false};
}

// A second geometry of bfloat16 d_qk = d_v = 64 for grids that the twelve-
// wave blocks fill badly: four waves (64 query rows) and 32-key tiles, so
// that three workgroups share a CU (the same three waves per SIMD, 32 KiB of
// LDS each) and the grid comes in thirds of the 192-row blocks.  Its waves
// run a little slower (each workgroup copies every key tile for 64 rows, and
// waits at a barrier every 32 keys): 0.4-4.5 % where both grids end in a
// full round of the chip.  fwd_pick_small takes it when the twelve-wave
// grid's round count exceeds the small grid's by more than 10 %: measured
// 2 x 24 x 4096 (4.1 rounds of 192-row blocks against 4 of 64-row blocks)
// 9.6 % faster, 8 x 24 x 1024 11 %, 1 x 24 x 16384 (8.1 against 8) 3.8 %;
// the text-to-image 4 x 16 x 4352 (6 rounds either way) keeps the twelve
// waves.  Never with a mask or key splits (their tile lists follow the
// default geometry).
constexpr bool fwd_has_small(int es, int dqk, int dv) {
  return es == 2 && dqk == 64 && dv == 64;
}

constexpr FwdGeom fwd16_geom_small(int es, int dqk, int dv) {
  return FwdGeom{4, 64, 32, 4 * 32 * (dqk + dv) * es, false};
}

// bh = batch x heads; cus = compute units (256 on MI355X).
inline bool fwd_pick_small(int es, int dqk, int dv, int64_t bh, int64_t nq, bool masked,
                           int nsplit, int cus = 256) {
  if (!fwd_has_small(es, dqk, dv) || masked || nsplit != 1) return false;
  const int64_t wg12 = bh * ((nq + 191) / 192), wg4 = bh * ((nq + 63) / 64);
  const int64_t r12 = (wg12 + cus - 1) / cus, r4 = (wg4 + 3 * cus - 1) / (3 * cus);
  return (double)r4 * 1.1 < (double)r12;
}

// The 32-query-row kernel for bfloat16 d_qk = d_v, built only when
// ATTN_JVP_ROWS32_D128 or _D64 is defined to 1: four waves of 32 rows (one
// per SIMD), 32-key steps, four LDS stages of K, dK, V, dV, 32x32x16 MFMAs.
// Its resident registers (Q, dQ, O, A, B: about 256 per lane at d = 128)
// allow one wave per SIMD, so the softmax work of a step cannot hide behind
// another wave's MFMAs; measured at 1.18 ms against 0.92 ms for the 16-row
// kernel on 2 x 24 heads x 4096 tokens at d = 128, it stays off by default.
#ifndef ATTN_JVP_ROWS32_D128
#define ATTN_JVP_ROWS32_D128 0
#endif
#ifndef ATTN_JVP_ROWS32_D64
#define ATTN_JVP_ROWS32_D64 0
#endif

constexpr bool use_rows32(int es, int dqk, int dv) {
  return es == 2 && dqk == dv &&
         ((dqk == 128 && ATTN_JVP_ROWS32_D128) || (dqk == 64 && ATTN_JVP_ROWS32_D64));
}

constexpr FwdGeom fwd_geom(int es, int dqk, int dv) {
  return use_rows32(es, dqk, dv) ? FwdGeom{4, 128, 32, 4 * 4 * 32 * dqk * es, true}
                                 : fwd16_geom(es, dqk, dv);
}

// Head dims with a compiled forward instance: d_qk, d_v in {16, 32, 64, 128,
// 256} for bfloat16 and {16, 32, 64} for float32.
constexpr bool fwd_built(int es, int dqk, int dv) {
  auto ok = [](int es_, int d) {
    return d == 16 || d == 32 || d == 64 || (es_ == 2 && (d == 128 || d == 256));
  };
  return (es == 2 || es == 4) && ok(es, dqk) && ok(es, dv);
}

// ---------------------------------------------------------------------------
// Launch geometry of the two backward launches (d_qk = d_v = d): the
// query-owned dQ launch and the key-owned dK/dV launch, 16 rows per wave and
// row block.
//  * resident per lane: two operand fragment sets and one (dQ) or two (dK,
//    dV) accumulator sets; eight waves while that fits 96 (dQ) or 96 / 48
//    (dK/dV, bf16 / float32) registers, else four.
//  * bfloat16 d = 128 and d = 64: waves may own two 16-row blocks (every
//    streamed LDS fragment then feeds both); the dK/dV launch runs four
//    waves there (d = 128: one per SIMD with 192 resident registers; d = 64:
//    two such workgroups per CU), and the d = 64 dQ launch four waves, two
//    workgroups per CU.
//  * block_n: 64-row streamed tiles while two stages of both tensors fit in
//    128 KiB and the transposing reads' largest constant offset (stage,
//    second tensor, row 48 of the tile) fits the 16-bit DS offset field,
//    else 32.
// ---------------------------------------------------------------------------
struct BwdGeom {
  int waves_dq, min_blocks_dq, rb_dq_max;
  int waves_dkv, min_blocks_dkv, rb_dkv_max;
  int block_n, lds;
};

constexpr BwdGeom bwd_geom(int es, int d) {
  const int rb = d * es;
  const int res_dq = (es == 2 ? d / 4 : d / 2) + d / 4;
  const int res_dkv = (es == 2 ? d / 4 : d / 2) + d / 2;
  const bool two = es == 2 && (d == 128 || d == 64);
  const int waves_dq = (es == 2 && d == 64) ? 4 : (res_dq <= 96 ? 8 : 4);
  const int waves_dkv = two ? 4 : (res_dkv <= (es == 2 ? 96 : 48) ? 8 : 4);
  const int bn = (4 * 64 * rb <= 128 * 1024 && 3 * 64 * rb + 48 * rb < 65536) ? 64 : 32;
  return BwdGeom{waves_dq, (es == 2 && d == 64) ? 2 : 1, two ? 2 : 1,
                 waves_dkv, (es == 2 && d == 64) ? 2 : 1, two ? 2 : 1,
                 bn, 4 * bn * rb};
}

constexpr bool bwd_built(int es, int d) { return fwd_built(es, d, d); }

// ---------------------------------------------------------------------------
// Frame-window mask (page "VDN-Minimax-H3 ... Stage A1", yfxerp.com): token i
// is in frame i / tpf, frame f in chunk f / chunk; a key is visible to a
// query when their chunks are at most `radius` apart, or the key lies in the
// first (`first`) or last (`last`) frame; with `see_all` the queries of those
// anchor frames see every key.
// ---------------------------------------------------------------------------
struct MaskDev {
  int kind;        // 0 none, 1 frame window
  int frames, tpf, chunk, radius;
  int first, last, see_all;
  float inv_tpf, inv_chunk;
};

// floor(n / den) for 0 <= n < 2^24 from a float estimate and exact fix-up.
AJ_HD inline int div_fix(int n, int den, float inv) {
  int q = (int)((float)n * inv);
  q -= (q * den > n);
  q -= (q * den > n);
  q += ((q + 1) * den <= n);
  q += ((q + 1) * den <= n);
  return q;
}

struct TileRanges {
  int n;
  int lo[3], hi[3];   // tile index ranges [lo, hi), ascending, disjoint
};

// Append [a, z) to ranges kept in ascending order of start, merging where
// they touch (static indices only, so nothing is spilled to memory).
AJ_HD inline void add_range(TileRanges &tr, int a, int z) {
  if (tr.n == 0) {
    tr.lo[0] = a; tr.hi[0] = z; tr.n = 1;
  } else if (tr.n == 1) {
    if (a <= tr.hi[0]) tr.hi[0] = z > tr.hi[0] ? z : tr.hi[0];
    else { tr.lo[1] = a; tr.hi[1] = z; tr.n = 2; }
  } else {
    if (a <= tr.hi[1]) tr.hi[1] = z > tr.hi[1] ? z : tr.hi[1];
    else { tr.lo[2] = a; tr.hi[2] = z; tr.n = 3; }
  }
}

AJ_HD inline TileRanges all_tiles(int N, int BN) {
  TileRanges tr;
  tr.n = 1;
  tr.lo[0] = 0;
  tr.hi[0] = (N + BN - 1) / BN;
  tr.lo[1] = tr.hi[1] = tr.lo[2] = tr.hi[2] = 0;
  return tr;
}

// Key-tile ranges (tiles of BN keys) that some query of rows [q_lo, q_hi)
// can see: first-frame anchor, chunk window, last-frame anchor.
AJ_HD inline TileRanges visible_tiles(const MaskDev &m, int q_lo, int q_hi, int N, int BN) {
  TileRanges tr = all_tiles(N, BN);
  if (m.kind == 0) return tr;
  const int T = m.tpf, C = m.chunk, F = m.frames, R = m.radius;
  const int qf0 = q_lo / T, qf1 = (q_hi - 1) / T;
  if (m.see_all && ((m.first && qf0 == 0) || (m.last && qf1 == F - 1))) return tr;
  const int c0 = qf0 / C, c1 = qf1 / C;
  const long long f_lo_l = (long long)(c0 - R) * C;
  const int f_lo = f_lo_l < 0 ? 0 : (int)f_lo_l;
  const long long f_hi_l = (long long)(c1 + R + 1) * C;
  const int f_hi = f_hi_l > F ? F : (int)f_hi_l;
  tr.n = 0;
  tr.lo[0] = tr.hi[0] = 0;
  if (m.first) add_range(tr, 0, (T + BN - 1) / BN);
  add_range(tr, f_lo * T / BN, (f_hi * T + BN - 1) / BN);
  if (m.last) add_range(tr, (F - 1) * T / BN, (F * T + BN - 1) / BN);
  return tr;
}

// Query-tile ranges that see some key of rows [k_lo, k_hi): the transpose of
// visible_tiles.  A block holding a key of an anchor frame is seen by every
// query; otherwise the queries of the chunks within the radius of the
// block's chunks, plus (see_all) the anchor query frames.
AJ_HD inline TileRanges visible_query_tiles(const MaskDev &m, int k_lo, int k_hi, int N,
                                            int BN) {
  TileRanges tr = all_tiles(N, BN);
  if (m.kind == 0) return tr;
  const int T = m.tpf, C = m.chunk, F = m.frames, R = m.radius;
  const int kf0 = k_lo / T, kf1 = (k_hi - 1) / T;
  if ((m.first && kf0 == 0) || (m.last && kf1 == F - 1)) return tr;
  const int c0 = kf0 / C, c1 = kf1 / C;
  const long long f_lo_l = (long long)(c0 - R) * C;
  const int f_lo = f_lo_l < 0 ? 0 : (int)f_lo_l;
  const long long f_hi_l = (long long)(c1 + R + 1) * C;
  const int f_hi = f_hi_l > F ? F : (int)f_hi_l;
  tr.n = 0;
  tr.lo[0] = tr.hi[0] = 0;
  if (m.see_all && m.first) add_range(tr, 0, (T + BN - 1) / BN);
  add_range(tr, f_lo * T / BN, (f_hi * T + BN - 1) / BN);
  if (m.see_all && m.last) add_range(tr, (F - 1) * T / BN, (F * T + BN - 1) / BN);
  return tr;
}

// Number of tiles in the ranges, and the tile index of the idx-th of them.
AJ_HD inline int tile_count(const TileRanges &tr) {
  return (tr.hi[0] - tr.lo[0]) + (tr.hi[1] - tr.lo[1]) + (tr.hi[2] - tr.lo[2]);
}

// A walk over the ranges with the steps over the gaps precomputed: the
// idx-th tile (0 <= idx < tile_count) is base + idx, plus d0 once idx >= j0
// (range 1 reached) and d1 once idx >= j1 (range 2 reached); a range that
// does not exist has its j at INT_MAX.  Per tile that is two compares and
// selects of uniform values (no branches in the key loops); for the one
// range of an unmasked walk the steps fold away.
struct TileWalk {
  int base, j0, d0, j1, d1;
};

AJ_HD inline TileWalk tile_walk(const TileRanges &tr) {
  const int len0 = tr.hi[0] - tr.lo[0];
  const int len01 = len0 + (tr.hi[1] - tr.lo[1]);
  TileWalk w;
  w.base = tr.lo[0];
  w.j0 = tr.n > 1 ? len0 : INT_MAX;
  w.d0 = tr.n > 1 ? tr.lo[1] - tr.hi[0] : 0;
  w.j1 = tr.n > 2 ? len01 : INT_MAX;
  w.d1 = tr.n > 2 ? tr.lo[2] - tr.hi[1] : 0;
  return w;
}

AJ_HD inline int walk_at(const TileWalk &w, int idx) {
  int t = w.base + idx;
  t += idx >= w.j0 ? w.d0 : 0;
  t += idx >= w.j1 ? w.d1 : 0;
  return t;
}

AJ_HD inline int tile_at(const TileRanges &tr, int idx) { return walk_at(tile_walk(tr), idx); }

// ---------------------------------------------------------------------------
// Kernel parameter blocks.
// ---------------------------------------------------------------------------
struct Params {
  const void *q, *k, *v, *dq, *dk, *dv;
  void *o, *dout;
  float *lse, *dlse;
  int64_t sq[3], sk[3], sv[3], so[3];   // (b, h, n) element strides
  int B, H, Nq, Nkv;
  int nqb;                              // query blocks per (b, h)
  int nsplit;                           // key splits per query block (1: none)
  int partial;                          // 1: outputs are float32 partials
  int small;                            // 1: the small geometry (fwd16_geom_small)
  float scale, scale_log2;
  MaskDev mask;
};

struct BwdParams {
  const void *q, *k, *v, *o, *g;   // inputs; g = dL/dO
  const float *lse;                // [B, H, Nq], natural log, from the forward
  void *gq, *gk, *gv;              // outputs dL/dQ, dL/dK, dL/dV
  float *delta;                    // [B, H, Nq]: D = rowsum(G (.) O), written by the dQ kernel
  int64_t sq[3], sk[3], sv[3], so[3], sg[3], sgq[3], sgk[3], sgv[3];   // (b, h, n) strides
  int B, H, Nq, Nkv;
  int nqb, nkb;                    // query / key blocks per (b, h)
  float scale, scale_log2;
  MaskDev mask;                    // frame window (kind 0: none); Nq == Nkv when on
  int rbq, rbk;                    // 16-row blocks per dQ / dK-dV wave (1, or 2 where built)
};

// Merge of key-split partials.  Partials are float32, contiguous: O, dO
// [parts, B, H, Nq, dv], LSE, dLSE [parts, B, H, Nq].  Outputs: O, dO in the
// dtype with (b, h, n) element strides so[], LSE and dLSE float32 contiguous
// [B, H, Nq].  One thread per four output elements, 256 threads per block.
struct MergeParams {
  const float *o_parts, *do_parts, *lse_parts, *dlse_parts;
  void *o, *dout;
  float *lse, *dlse;
  int64_t so[3];
  int parts, B, H, Nq, dv;
};

constexpr int kMergeThreads = 256;

}  // namespace attn_jvp
