// Primal backward of attention for gfx950: dQ, dK, dV from the saved
// log-sum-exp (page "带分数正则的一致性蒸馏", gitcode.csdn.net, section 注意力,
// subsection 反向).  With the upstream gradient G = dL/dO:
//   P = exp(s Q K^T - LSE),  dV = P^T G,  dP = G V^T,
//   dS = P (.) (dP - D),  D = rowsum(dP (.) P) = rowsum(G (.) O),
//   dQ = s dS K,  dK = s dS^T Q.
// The pages parallelise dQ over query tokens and dK, dV over key tokens (two
// tilings); so do these two kernels, with no atomics:
//   * bwd_dq_kernel: a workgroup owns query rows (16 per wave; Q and G
//     fragments in registers), streams K and V tiles through LDS, writes D
//     (from its own rows of G and O) and dQ;
//   * bwd_dkv_kernel: a workgroup owns key rows (16 per wave; K and V
//     fragments in registers), streams Q and G tiles through LDS, reads D and
//     LSE per query, writes dK and dV.
// Both recompute S and P; MFMA fragment layouts, LDS staging (asynchronous
// global->LDS copies, two stages, swizzled rows) and transposing reads are
// those of the forward kernel (kernel.h).  d_qk = d_v = D, as the pages
// require for the backward.
//
// The VALU work per score is kept to the exponential, one FMA, one multiply
// and the bf16 packs: the dP accumulators start at -D, so the MFMAs yield
// dP - D; the dK/dV kernel reads each streamed query's -LSE log2 e (-inf for
// rows past the end and for rows with no visible key, which makes P = 0) and
// -D from LDS rows that two waves transform once per tile, a tile ahead of
// use; the dQ kernel masks keys past the end only in the last tile.
//
// With the frame-window mask (page "VDN-Minimax-H3 ... Stage A1", yfxerp.com)
// each launch walks only the streamed tiles its block can see -- key tiles for
// a query block, as in the forward, and for a key block the query tiles that
// see it (anchor keys are seen by every query; with anchor_queries_see_all the
// anchor query frames see every key) -- and applies element masks (P = 0) in
// the tiles that are only partly visible.

#pragma once

#include "kernel.h"

namespace attn_jvp {

// Global->LDS copies of the streamed tiles: SideCopier's scheme (1 KiB per
// wave instruction, lane-chosen swizzled chunk, clamped tail rows) for two
// tensors with their own row strides; KS is the swizzle kind of lds_off.
template <typename T, int RB, int BN, int W, int KS>
struct PairCopier {
  static constexpr int CPR = RB / 16;
  static constexpr int TILE = BN * RB;
  static constexpr int NI = TILE / 1024;
  static constexpr int IPW = (NI + W - 1) / W;
  static_assert(NI * 1024 == TILE, "a tile is whole 1 KiB wave copies");

  const char *base[2];
  int64_t rstride[2];
  uint32_t rs[2];           // below 2^24 bytes, checked on the host
  uint32_t slot[IPW];       // (row << 16) | swizzled chunk, per lane
  int wave;

  __device__ void init(const T *t0, const T *t1, int64_t s0, int64_t s1, int wave_, int lane) {
    wave = wave_;
    base[0] = (const char *)t0;
    base[1] = (const char *)t1;
    rstride[0] = s0 * (int64_t)sizeof(T);
    rstride[1] = s1 * (int64_t)sizeof(T);
    rs[0] = (uint32_t)rstride[0];
    rs[1] = (uint32_t)rstride[1];
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int s = (i * W + wave) * 64 + lane;
      const int r = s / CPR;
      const int c = (s % CPR) ^ swz<RB, KS>(r);
      slot[i] = ((uint32_t)r << 16) | (uint32_t)c;
    }
  }

  __device__ void issue(int k0, int N, char *dst0, int tstride) const {
    const int valid = (N - k0 < BN ? N - k0 : BN) - 1;   // last real row
    const char *tb0 = base[0] + (int64_t)k0 * rstride[0];
    const char *tb1 = base[1] + (int64_t)k0 * rstride[1];
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      if (NI % W != 0 && i * W + wave >= NI) break;   // uniform per wave
      uint32_t r = slot[i] >> 16;
      r = r < (uint32_t)valid ? r : (uint32_t)valid;
      const uint32_t c16 = (slot[i] & 0xffffu) << 4;
      // 32-bit lane offsets from a wave-uniform base: the copies take the
      // scalar-base address form (no 64-bit address arithmetic per lane);
      // r < BN and the strides are below 2^24 bytes, so they fit
      const uint32_t off0 = __umul24(r, rs[0]) + c16;
      const uint32_t off1 = __umul24(r, rs[1]) + c16;
      char *dst = dst0 + (i * W + wave) * 1024;
      __builtin_amdgcn_global_load_lds((const void *)(tb0 + off0), (lds_void *)dst, 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void *)(tb1 + off1), (lds_void *)(dst + tstride),
                                       16, 0, 0);
    }
  }
};

// 16-byte LDS read through inline asm (see lds_read_tr) and a wait for four
// such values (at most N LDS operations left outstanding).
__device__ inline f32x4 lds_read_f4(uint32_t addr) {
  f32x4 v;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}

template <int N>
__device__ inline void lds_quad_wait(f32x4 &a, f32x4 &b, f32x4 &c, f32x4 &d) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt field");
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d) : "n"(N));
}

template <typename T, int D>
struct BwdCfg {
  static constexpr int ES = (int)sizeof(T);
  static constexpr int RB = D * ES;
  static constexpr BwdGeom G = bwd_geom(ES, D);
  static constexpr int kWavesDq = G.waves_dq;
  static constexpr int kMinBlocksDq = G.min_blocks_dq;
  static constexpr int kRbDqMax = G.rb_dq_max;
  static constexpr int kWavesDkv = G.waves_dkv;
  static constexpr int kMinBlocksDkv = G.min_blocks_dkv;
  static constexpr int kRbDkvMax = G.rb_dkv_max;
  static constexpr int kBN = G.block_n;
  static constexpr int kLds = G.lds;   // 2 stages x 2 tensors
};

template <typename T, int D, bool KEYS, bool MASKED, int RBS>
__global__ __launch_bounds__((64 * (KEYS ? BwdCfg<T, D>::kWavesDkv : BwdCfg<T, D>::kWavesDq)),
                             (KEYS ? BwdCfg<T, D>::kMinBlocksDkv : BwdCfg<T, D>::kMinBlocksDq))
void bwd_kernel(BwdParams p) {
  using C = BwdCfg<T, D>;
  using EK = ElemK<T, D>;
  using EV = ElemV<T>;
  using FragK = typename EK::Frag;
  using FragV = typename EV::Frag;
  constexpr bool BF16 = sizeof(T) == 2;
  constexpr int W = KEYS ? C::kWavesDkv : C::kWavesDq;
  constexpr int R = RBS;   // 16-row blocks per wave
  static_assert(R >= 1 && R <= (KEYS ? C::kRbDkvMax : C::kRbDqMax), "row blocks");
  constexpr int BN = C::kBN;
  constexpr int CK = kStepKeys;
  constexpr int NSTEP = BN / CK;
  constexpr int KL = EK::KL, KI = EK::KI;
  constexpr int RB = C::RB;
  constexpr int TL = BN * RB;          // bytes per tensor tile
  constexpr int DS = D / KI;
  constexpr int ND = D / 16;
  constexpr float kLog2e = 1.4426950408889634f;
  constexpr int kRowSlot = 3 * 256;    // bytes of one slot of query-term rows
  // The d = 64 dQ launch (two four-wave workgroups per CU) issues its MFMA
  // blocks at raised priority, so that where both waves of a SIMD are ready
  // the one feeding the matrix core goes first: text-to-image backward
  // 1.2 % faster; at d = 128 (one eight-wave workgroup) and for the key-owned
  // launch it measured the same or slower.
  constexpr bool kPrio = BF16 && !KEYS && D == 64;
  // The streamed tiles are read both along rows (score operands) and
  // transposed (product operands): bfloat16 tiles take the swizzle that is
  // conflict-free for both; the float32 products read single elements,
  // where the operand-row rule does best.
  constexpr int KSW = BF16 ? kSwzB : kSwzK;

  // tiles, then (dK/dV kernel) three slots x 3 rows of 64 floats of query
  // terms: row 0 -LSE log2 e, row 1 -D, row 2 a landing row for the waves
  // that copy neither
  __shared__ __attribute__((aligned(1024))) char smem[C::kLds + (KEYS ? 3 * kRowSlot : 0)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rl = lane & 15;       // this lane's owned row (query or key) within a row block
  const int lg = lane >> 4;

  const int lid = logical_block_id();
  const int nblk = KEYS ? p.nkb : p.nqb;
  const int bh = lid / nblk;
  const int blk = lid - bh * nblk;
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int Nq = p.Nq, Nkv = p.Nkv;
  const int Nown = KEYS ? Nkv : Nq;      // rows this kernel owns
  const int Nstr = KEYS ? Nq : Nkv;      // rows it streams

  // owned: (A, Bt) = (Q, G) for dQ, (K, V) for dK, dV -- B operands in registers
  const T *A0 = KEYS ? (const T *)p.k + b * p.sk[0] + h * p.sk[1]
                     : (const T *)p.q + b * p.sq[0] + h * p.sq[1];
  const T *A1 = KEYS ? (const T *)p.v + b * p.sv[0] + h * p.sv[1]
                     : (const T *)p.g + b * p.sg[0] + h * p.sg[1];
  const int64_t as0 = KEYS ? p.sk[2] : p.sq[2];
  const int64_t as1 = KEYS ? p.sv[2] : p.sg[2];
  // streamed: tensor 0 (K for dQ, Q for dK/dV) and tensor 1 (V for dQ, G for dK/dV)
  const T *S0 = KEYS ? (const T *)p.q + b * p.sq[0] + h * p.sq[1]
                     : (const T *)p.k + b * p.sk[0] + h * p.sk[1];
  const T *S1 = KEYS ? (const T *)p.g + b * p.sg[0] + h * p.sg[1]
                     : (const T *)p.v + b * p.sv[0] + h * p.sv[1];
  const int64_t ss0 = KEYS ? p.sq[2] : p.sk[2];
  const int64_t ss1 = KEYS ? p.sg[2] : p.sv[2];
  const float *LSE = p.lse + (int64_t)bh * Nq;
  float *DEL = p.delta + (int64_t)bh * Nq;

  // owned rows of the lane: one per row block, r0 + 16 (R wave + rb) + rl
  const int r0 = blk * (W * R * kWaveRows);
  int row[R];
  bool rvalid[R];
#pragma unroll
  for (int rb = 0; rb < R; ++rb) {
    row[rb] = r0 + (wave * R + rb) * kWaveRows + rl;
    rvalid[rb] = row[rb] < Nown;
  }
  const int r_hi = r0 + W * R * kWaveRows < Nown ? r0 + W * R * kWaveRows : Nown;

  // streamed tiles this block visits, in ascending order (all of them
  // without a mask); iteration it walks tile walk_at(walk, it)
  TileRanges tr;
  if constexpr (MASKED) {
    tr = KEYS ? visible_query_tiles(p.mask, r0, r_hi, Nq, BN)
              : visible_tiles(p.mask, r0, r_hi, Nkv, BN);
  } else {
    tr = all_tiles(Nstr, BN);
  }
  const int ntile = tile_count(tr);
  const TileWalk walk = tile_walk(tr);

  // Mask terms.  The lane's own row sees the streamed rows [vis_lo, vis_hi)
  // by the chunk rule, plus [0, a_first_hi) and [a_last_lo, Nstr) (anchor
  // key frames for the dQ kernel; anchor query frames with
  // anchor_queries_see_all for the dK/dV kernel; an owned row that is
  // itself in such a frame sees everything).  Streamed rows in
  // [win_lo, win_hi) are seen by every row of the block, and so are those
  // of the anchor intervals, so tiles inside them need no element mask.
  int vis_lo[R], vis_hi[R];
  int a_first_hi = 0, a_last_lo = Nstr, win_lo = 0, win_hi = 0;
  bool blk_all = false;   // dK/dV: every key of the block is an anchor key
#pragma unroll
  for (int rb = 0; rb < R; ++rb) {
    vis_lo[rb] = 0;
    vis_hi[rb] = Nstr;
  }
  if constexpr (MASKED) {
    const long long F = p.mask.frames, TPF = p.mask.tpf, CH = p.mask.chunk, Rd = p.mask.radius;
#pragma unroll
    for (int rb = 0; rb < R; ++rb) {
      const int rf = div_fix(rvalid[rb] ? row[rb] : 0, p.mask.tpf, p.mask.inv_tpf);
      const int rc = div_fix(rf, p.mask.chunk, p.mask.inv_chunk);
      const bool r_anchor = (p.mask.first && rf == 0) || (p.mask.last && rf == p.mask.frames - 1);
      // dQ: an anchor query sees all keys only with see_all; dK/dV: an
      // anchor key is seen by all queries
      const bool r_all = KEYS ? r_anchor : (p.mask.see_all && r_anchor);
      long long flo = (rc - Rd) * CH, fhi = (rc + Rd + 1) * CH;
      flo = flo < 0 ? 0 : flo;
      fhi = fhi > F ? F : fhi;
      if (!r_all) {
        vis_lo[rb] = (int)(flo * TPF);
        vis_hi[rb] = fhi > flo ? (int)(fhi * TPF) : vis_lo[rb];
      }
    }
    const bool a_on = KEYS ? p.mask.see_all : true;
    a_first_hi = (a_on && p.mask.first) ? (int)TPF : 0;
    a_last_lo = (a_on && p.mask.last) ? (int)((F - 1) * TPF) : Nstr;
    const long long c0 = (r0 / TPF) / CH;
    const long long c1 = ((r_hi - 1) / TPF) / CH;
    long long wlo = (c1 - Rd) * CH, whi = (c0 + Rd + 1) * CH;
    wlo = wlo < 0 ? 0 : wlo;
    whi = whi > F ? F : whi;
    if (whi > wlo) {
      win_lo = (int)(wlo * TPF);
      win_hi = (int)(whi * TPF);
    }
    if constexpr (KEYS) {
      const long long f0 = r0 / TPF, f1 = (r_hi - 1) / TPF;
      blk_all = (p.mask.first && f1 == 0) || (p.mask.last && f0 == F - 1);
    }
  }
  // does the tile at streamed row t0 need element masks (frame window)?
  auto needs_mask = [&](int t0) __attribute__((always_inline)) {
    if constexpr (!MASKED) {
      return false;
    } else {
      const int tz = t0 + BN < Nstr ? t0 + BN : Nstr;
      const bool in_win = t0 >= win_lo && tz <= win_hi;
      const bool in_first = tz <= a_first_hi;
      const bool in_last = t0 >= a_last_lo;
      return !(blk_all || in_win || in_first || in_last);
    }
  };

  // streamed tiles: both tensors have rows of D elements, one copier; the
  // same tile is read as operand rows and through transposing loads, so
  // one swizzle (the operand-row rule) serves both
  PairCopier<T, RB, BN, W, KSW> copier;
  copier.init(S0, S1, ss0, ss1, wave, lane);
  // dK/dV kernel: the streamed query rows' LSE and D come as 4-byte
  // global->LDS copies (64 rows per wave instruction) into slot it % 3, two
  // tiles ahead of use: wave 0 copies LSE, wave 1 D, the other waves the
  // landing row (no branch around the copies).  During tile it - 1, waves 0
  // and 1 turn their row of tile it into -LSE log2 e and -D in place.  Rows
  // are clamped to Nq - 1 for the copy; the transform gives them -inf.
  const uint32_t rows_a = lds_addr(smem) + C::kLds;
  auto issue_rows = [&](int it) __attribute__((always_inline)) {
    if constexpr (KEYS) {
      int qr = walk_at(walk, it) * BN + lane;
      qr = qr < Nq ? qr : Nq - 1;
      const int which = wave < 2 ? wave : 2;
      const float *src = (which == 1 ? DEL : LSE) + qr;
      __builtin_amdgcn_global_load_lds(
          (const void *)src, (lds_void *)(smem + C::kLds + (it % 3) * kRowSlot + which * 256), 4,
          0, 0);
    }
  };
  auto transform_rows = [&](int it) __attribute__((always_inline)) {
    if constexpr (KEYS) {
      if (wave < 2) {
        const uint32_t a = rows_a + (it % 3) * kRowSlot + wave * 256 + lane * 4;
        float v;
        asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a));
        const int qr = walk_at(walk, it) * BN + lane;
        float t;
        if (wave == 0) t = (qr < Nq && v != -INFINITY) ? -v * kLog2e : -INFINITY;
        else t = -v;
        asm volatile("ds_write_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(a), "v"(t) : "memory");
      }
    }
  };
  auto issue_tile = [&](int it, int g) __attribute__((always_inline)) {
    copier.issue(walk_at(walk, it) * BN, Nstr, smem + g * TL, 2 * TL);
  };
  if (ntile > 0) {
    issue_tile(0, 0);
    issue_rows(0);
    if (ntile > 1) issue_rows(1);
    if constexpr (KEYS) {
      wait_vmem();
      transform_rows(0);   // visible to all waves after the first tile's barrier
    }
  }

  // owned fragments (B operands): lane holds row rl of each row block,
  // d-slice s KI + lg KL
  FragK af[R][DS], bf[R][DS];
#pragma unroll
  for (int rb = 0; rb < R; ++rb)
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      if (rvalid[rb]) {
        af[rb][s] = *(const FragK *)(A0 + (int64_t)row[rb] * as0 + s * KI + lg * KL);
        bf[rb][s] = *(const FragK *)(A1 + (int64_t)row[rb] * as1 + s * KI + lg * KL);
      } else {
        af[rb][s] = FragK{};
        bf[rb][s] = FragK{};
      }
    }

  // dQ kernel: the lane's query row terms.  D = rowsum(G (.) O) from the
  // lane's quarter of the row (the same d-slices as its G fragments),
  // summed over the row's four lanes; L2 = LSE * log2 e (+inf for a row
  // with no visible key, so that P = 0 there).
  float d_row[R], l2_row[R];
#pragma unroll
  for (int rb = 0; rb < R; ++rb) {
    d_row[rb] = 0.f;
    l2_row[rb] = 0.f;
    if constexpr (!KEYS) {
      const T *Orow = (const T *)p.o + b * p.so[0] + h * p.so[1];
      float part = 0.f;
      if (rvalid[rb]) {
#pragma unroll
        for (int s = 0; s < DS; ++s) {
          const FragK of = *(const FragK *)(Orow + (int64_t)row[rb] * p.so[2] + s * KI + lg * KL);
          if constexpr (BF16) {
#pragma unroll
            for (int j = 0; j < KL; ++j) part = fmaf((float)bf[rb][s][j], (float)of[j], part);
          } else {
            part = fmaf(bf[rb][s], of, part);
          }
        }
      }
      d_row[rb] = row_sum4(part);
      if (rvalid[rb] && lg == 0) DEL[row[rb]] = d_row[rb];
      const float lse = rvalid[rb] ? LSE[row[rb]] : 0.f;
      l2_row[rb] = lse == -INFINITY ? INFINITY : lse * kLog2e;
    }
  }

  // accumulators: dQ^T (dQ kernel) or dK^T and dV^T (dK/dV kernel); lane
  // holds d = 16e + 4 lg + 0..3 of its owned row
  f32x4 acc0[R][ND], acc1[R][KEYS ? ND : 1];
#pragma unroll
  for (int rb = 0; rb < R; ++rb)
#pragma unroll
    for (int e = 0; e < ND; ++e) acc0[rb][e] = f32x4{};
  if constexpr (KEYS) {
#pragma unroll
    for (int rb = 0; rb < R; ++rb)
#pragma unroll
      for (int e = 0; e < ND; ++e) acc1[rb][e] = f32x4{};
  }

  const float c2 = p.scale_log2;
  const uint32_t smem_a = lds_addr(smem);
  uint32_t rdl[DS];                          // operand-row reads, k-step s
#pragma unroll
  for (int s = 0; s < DS; ++s)
    rdl[s] = smem_a + lds_off<RB, KSW>(rl, (s * KI + lg * KL) * (int)sizeof(T));
  uint32_t trl[BF16 ? ND : 1];               // transposing reads, d block e
  if constexpr (BF16) {
#pragma unroll
    for (int e = 0; e < ND; ++e)
      trl[e] = smem_a + lds_off<RB, KSW>(4 * lg + (rl >> 2), (16 * e + 4 * (rl & 3)) * 2);
  }

  // dQ kernel: -LSE log2 e of the lane's query (-inf for a row with no
  // visible key, so that P = 0 there) and the start value of its dP sums
  float nl2_row[R];
  f32x4 nd_row[R];
#pragma unroll
  for (int rb = 0; rb < R; ++rb) {
    nl2_row[rb] = KEYS ? 0.f : -l2_row[rb];
    nd_row[rb] = f32x4{-d_row[rb], -d_row[rb], -d_row[rb], -d_row[rb]};
  }

  // One 32-row step kc of the streamed tile in stage G.
  //  dQ kernel:   X^T = K Q^T (keys x queries), Y^T = V G^T - D; lane: query
  //               rl, keys 4 lg + i (+16 for the second half)
  //  dK/dV kernel: X = Q K^T (queries x keys), Y = G V^T - D; lane: key rl,
  //               queries 4 lg + i (+16)
  // rows: LDS address of the tile's query-term slot (dK/dV kernel); tail:
  // the tile holds streamed rows past the end (dQ kernel masks those keys);
  // need: the tile is partly visible under the frame window
  // after_scores runs once the step's score MFMAs are issued
  auto step = [&](auto G_, auto KC_, int t0, uint32_t rows, bool tail, bool need,
                  auto &&after_scores) __attribute__((always_inline)) {
    constexpr int G = decltype(G_)::value;
    constexpr int kb = decltype(KC_)::value * CK;
    f32x4 nl2[2], y0[2];
    if constexpr (KEYS) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const uint32_t a = rows + (kb + 16 * kb2 + 4 * lg) * 4;
        nl2[kb2] = lds_read_f4(a);
        y0[kb2] = lds_read_f4(a + 256);
      }
    }
    // S (xs) and dP - D (ys) of each row block
    f32x4 xs[R][2], ys[R][2];
    if constexpr (BF16 && D >= 32) {
      // slices j = (kb2, s), kb2-major, each a tensor-0 and a tensor-1 read
      // that feed every row block; PD slices in flight
      constexpr int NP = 2 * DS;
      constexpr int PD0 = D >= 128 ? 3 : 2;
      constexpr int PD = PD0 < NP ? PD0 : NP;
      bf16x8 r0f[NP], r1f[NP];
      auto issue = [&](auto j_) __attribute__((always_inline)) {
        constexpr int j = decltype(j_)::value;
        constexpr int kb2 = j / DS, s = j % DS;
        constexpr int OFF = G * TL + (kb + 16 * kb2) * RB;
        r0f[j] = lds_read_k<OFF>(rdl[s]);
        r1f[j] = lds_read_k<OFF + 2 * TL>(rdl[s]);
      };
      static_for<0, PD - 1>([&](auto j_) __attribute__((always_inline)) { issue(j_); });
      if constexpr (KEYS) lds_quad_wait<2 * (PD - 1)>(nl2[0], nl2[1], y0[0], y0[1]);
      f32x4 x_[R][2], y_[R][2];
#pragma unroll
      for (int rb = 0; rb < R; ++rb)
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          x_[rb][kb2] = f32x4{};
          y_[rb][kb2] = KEYS ? y0[kb2] : nd_row[rb];
        }
      if constexpr (kPrio) __builtin_amdgcn_s_setprio(1);
      static_for<0, NP>([&](auto j_) __attribute__((always_inline)) {
        constexpr int j = decltype(j_)::value;
        constexpr int kb2 = j / DS, s = j % DS;
        if constexpr (j + PD - 1 < NP) issue(std::integral_constant<int, j + PD - 1>{});
        constexpr int newer = (NP - 1 - j) < (PD - 1) ? (NP - 1 - j) : (PD - 1);
        lds_wait<2 * newer>();
#pragma unroll
        for (int rb = 0; rb < R; ++rb) {
          x_[rb][kb2] = EK::mfma(r0f[j], af[rb][s], x_[rb][kb2]);
          y_[rb][kb2] = EK::mfma(r1f[j], bf[rb][s], y_[rb][kb2]);
        }
      });
      if constexpr (kPrio) __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int rb = 0; rb < R; ++rb)
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          xs[rb][kb2] = x_[rb][kb2];
          ys[rb][kb2] = y_[rb][kb2];
        }
    } else {
      if constexpr (KEYS) lds_quad_wait<0>(nl2[0], nl2[1], y0[0], y0[1]);
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        f32x4 x_[R], y_[R];
#pragma unroll
        for (int rb = 0; rb < R; ++rb) {
          x_[rb] = f32x4{};
          y_[rb] = KEYS ? y0[kb2] : nd_row[rb];
        }
#pragma unroll
        for (int s = 0; s < DS; ++s) {
          const char *rp = smem + (rdl[s] - smem_a) + G * TL + (kb + 16 * kb2) * RB;
          const FragK r0f = *(const FragK *)rp;
          const FragK r1f = *(const FragK *)(rp + 2 * TL);
#pragma unroll
          for (int rb = 0; rb < R; ++rb) {
            x_[rb] = EK::mfma(r0f, af[rb][s], x_[rb]);
            y_[rb] = EK::mfma(r1f, bf[rb][s], y_[rb]);
          }
        }
#pragma unroll
        for (int rb = 0; rb < R; ++rb) {
          xs[rb][kb2] = x_[rb];
          ys[rb][kb2] = y_[rb];
        }
      }
    }
    after_scores();
    // P and dS = P (.) (dP - D), unscaled
    f32x4 pv[R][2], dsv[R][2];
#pragma unroll
    for (int rb = 0; rb < R; ++rb)
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          pv[rb][kb2][i] =
              __builtin_amdgcn_exp2f(fmaf(xs[rb][kb2][i], c2, KEYS ? nl2[kb2][i] : nl2_row[rb]));
    if constexpr (!KEYS) {
      if (tail) {
        const int sbase = t0 + kb;   // first key of the step
#pragma unroll
        for (int rb = 0; rb < R; ++rb)
#pragma unroll
          for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              pv[rb][kb2][i] = sbase + 16 * kb2 + 4 * lg + i < Nkv ? pv[rb][kb2][i] : 0.f;
      }
    }
    if constexpr (MASKED) {
      if (need) {
        // bitwise, not short-circuit: no branch per element
        const int sbase = t0 + kb;
#pragma unroll
        for (int rb = 0; rb < R; ++rb)
#pragma unroll
          for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int sr = sbase + 16 * kb2 + 4 * lg + i;
              const bool in_chunks = (unsigned)(sr - vis_lo[rb]) < (unsigned)(vis_hi[rb] - vis_lo[rb]);
              const bool vis = in_chunks | (sr < a_first_hi) | (sr >= a_last_lo);
              pv[rb][kb2][i] = vis ? pv[rb][kb2][i] : 0.f;
            }
      }
    }
#pragma unroll
    for (int rb = 0; rb < R; ++rb)
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int i = 0; i < 4; ++i) dsv[rb][kb2][i] = pv[rb][kb2][i] * ys[rb][kb2][i];
    // products over the 32 streamed rows: acc0 += T0^T (dS or P) ; acc1 ...
    //  dQ kernel:    dQ^T += K^T dS^T        (T0 = K tile, transposed reads,
    //                                         shared by the row blocks)
    //  dK/dV kernel: dK^T += Q^T dS, dV^T += G^T P
    if constexpr (BF16) {
      bf16x8 dsf[R], pf[R];
#pragma unroll
      for (int rb = 0; rb < R; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dsf[rb][i] = (__bf16)dsv[rb][0][i];
          dsf[rb][4 + i] = (__bf16)dsv[rb][1][i];
        }
      if constexpr (KEYS) {
#pragma unroll
        for (int rb = 0; rb < R; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pf[rb][i] = (__bf16)pv[rb][0][i];
            pf[rb][4 + i] = (__bf16)pv[rb][1][i];
          }
      }
      constexpr int VO = G * TL + kb * RB;
      constexpr int NR = KEYS ? 4 : 2;          // transposing reads per d block
      auto issue = [&](auto e_, i16x4 (&r)[4]) __attribute__((always_inline)) {
        constexpr int e = decltype(e_)::value;
        r[0] = lds_read_tr<VO>(trl[e]);
        r[1] = lds_read_tr<VO + 16 * RB>(trl[e]);
        if constexpr (KEYS) {
          r[2] = lds_read_tr<VO + 2 * TL>(trl[e]);
          r[3] = lds_read_tr<VO + 2 * TL + 16 * RB>(trl[e]);
        }
      };
      i16x4 buf[3][4];
      issue(std::integral_constant<int, 0>{}, buf[0]);
      if constexpr (ND > 1) issue(std::integral_constant<int, 1>{}, buf[1]);
      if constexpr (kPrio) __builtin_amdgcn_s_setprio(1);
      static_for<0, ND>([&](auto e_) __attribute__((always_inline)) {
        constexpr int e = decltype(e_)::value;
        i16x4(&cur)[4] = buf[e % 3];
        if constexpr (e + 2 < ND) {
          issue(std::integral_constant<int, e + 2>{}, buf[(e + 2) % 3]);
          lds_wait<2 * NR>();
        } else if constexpr (e + 1 < ND) {
          lds_wait<NR>();
        } else {
          lds_wait<0>();
        }
        const FragV t0f = __builtin_bit_cast(FragV, __builtin_shufflevector(cur[0], cur[1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int rb = 0; rb < R; ++rb) acc0[rb][e] = EV::mfma(t0f, dsf[rb], acc0[rb][e]);
        if constexpr (KEYS) {
          const FragV t1f = __builtin_bit_cast(FragV, __builtin_shufflevector(cur[2], cur[3], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int rb = 0; rb < R; ++rb) acc1[rb][e] = EV::mfma(t1f, pf[rb], acc1[rb][e]);
        }
      });
      if constexpr (kPrio) __builtin_amdgcn_s_setprio(0);
    } else {
      // float32: k-step (kb2, i) takes streamed row 16 kb2 + 4 lg + i
      const char *Ts = smem + G * TL;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = kb + 16 * kb2 + 4 * lg + i;
#pragma unroll
          for (int e = 0; e < ND; ++e) {
            const int o = lds_off<RB, KSW>(r, (16 * e + rl) * 4);
            const FragV t0f = *(const FragV *)(Ts + o);
#pragma unroll
            for (int rb = 0; rb < R; ++rb) acc0[rb][e] = EV::mfma(t0f, dsv[rb][kb2][i], acc0[rb][e]);
            if constexpr (KEYS) {
              const FragV t1f = *(const FragV *)(Ts + 2 * TL + o);
#pragma unroll
              for (int rb = 0; rb < R; ++rb)
                acc1[rb][e] = EV::mfma(t1f, pv[rb][kb2][i], acc1[rb][e]);
            }
          }
        }
    }
  };

  auto tile = [&](auto G_, int it) __attribute__((always_inline)) {
    wait_vmem();
    __syncthreads();   // tile `it` landed; every wave is done with tile it-1
    const uint32_t rows = rows_a + (it % 3) * kRowSlot;
    const int t0 = walk_at(walk, it) * BN;
    const bool tail = t0 + BN > Nstr;
    const bool need = needs_mask(t0);
    // the next tile's copies (and the query-term rows) go out behind the
    // first step's score MFMAs, not at the barrier
    auto next = [&]() __attribute__((always_inline)) {
      if (it + 1 < ntile) issue_tile(it + 1, 1 - decltype(G_)::value);
      if constexpr (KEYS) {
        if (it + 2 < ntile) issue_rows(it + 2);
        if (it + 1 < ntile) transform_rows(it + 1);
      }
    };
    auto none = []() __attribute__((always_inline)) {};
    static_for<0, NSTEP>([&](auto kc) __attribute__((always_inline)) {
      if constexpr (decltype(kc)::value == 0) step(G_, kc, t0, rows, tail, need, next);
      else step(G_, kc, t0, rows, tail, need, none);
    });
  };

  int it = 0;
  for (; it + 1 < ntile; it += 2) {
    tile(std::integral_constant<int, 0>{}, it);
    tile(std::integral_constant<int, 1>{}, it + 1);
  }
  if (it < ntile) tile(std::integral_constant<int, 0>{}, it);

  // epilogue: dQ = s dQ^T, dK = s dK^T, dV = dV^T
  typedef T T4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int rb = 0; rb < R; ++rb) {
    if (!rvalid[rb]) continue;
    T *O0 = KEYS ? (T *)p.gk + b * p.sgk[0] + h * p.sgk[1] + (int64_t)row[rb] * p.sgk[2]
                 : (T *)p.gq + b * p.sgq[0] + h * p.sgq[1] + (int64_t)row[rb] * p.sgq[2];
#pragma unroll
    for (int e = 0; e < ND; ++e) {
      T4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = (T)(acc0[rb][e][i] * p.scale);
      *(T4 *)(O0 + 16 * e + 4 * lg) = o;
    }
    if constexpr (KEYS) {
      T *O1 = (T *)p.gv + b * p.sgv[0] + h * p.sgv[1] + (int64_t)row[rb] * p.sgv[2];
#pragma unroll
      for (int e = 0; e < ND; ++e) {
        T4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = (T)acc1[rb][e][i];
        *(T4 *)(O1 + 16 * e + 4 * lg) = o;
      }
    }
  }
}

// One launch of the dQ (KEYS false) or dK/dV kernel with the row blocks
// per wave the host chose.
template <typename T, int D, bool KEYS, bool MASKED>
hipError_t launch_bwd_one(const BwdParams &p, hipStream_t s) {
  using C = BwdCfg<T, D>;
  constexpr int RMAX = KEYS ? C::kRbDkvMax : C::kRbDqMax;
  const int rb = KEYS ? p.rbk : p.rbq;
  const dim3 grid(p.B * p.H * (KEYS ? p.nkb : p.nqb));
  const dim3 block(64 * (KEYS ? C::kWavesDkv : C::kWavesDq));
  if constexpr (RMAX >= 2) {
    if (rb == 2) {
      hipLaunchKernelGGL((bwd_kernel<T, D, KEYS, MASKED, 2>), grid, block, 0, s, p);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((bwd_kernel<T, D, KEYS, MASKED, 1>), grid, block, 0, s, p);
  return hipGetLastError();
}

// dQ (and D) first, then dK and dV, on one stream.
template <typename T, int D, bool MASKED>
hipError_t launch_bwd_pair(const BwdParams &p, hipStream_t s) {
  const hipError_t err = launch_bwd_one<T, D, false, MASKED>(p, s);
  if (err != hipSuccess) return err;
  return launch_bwd_one<T, D, true, MASKED>(p, s);
}

template <typename T, int D>
hipError_t launch_bwd_instance(const BwdParams &p, hipStream_t s) {
  return p.mask.kind != 0 ? launch_bwd_pair<T, D, true>(p, s) : launch_bwd_pair<T, D, false>(p, s);
}

}  // namespace attn_jvp
