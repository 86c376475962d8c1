// Fused attention JVP for gfx950 with 32 query rows per wave and
// v_mfma_f32_32x32x16_bf16 (bfloat16, d_qk = d_v = 64 or 128).
//
// What is computed is that of kernel.h (page "带分数正则的一致性蒸馏",
// gitcode.csdn.net, section 注意力: O = softmax(s Q K^T) V, its tangent
// dO = P dV + (P (.) dS) V - rowsum(P (.) dS) O with dS = s (dQ K^T + Q dK^T),
// the row log-sum-exp and its tangent, by the streaming form with sum l,
// tangent sum r and accumulators O~, A~ = P~ dV, B~ = (P~ (.) dS) V).
// The execution differs:
//   * a wave owns 32 query rows and computes S^T = K Q^T 32 keys at a time
//     with 32x32x16 MFMAs: half the MFMA and LDS instructions per FLOP of the
//     16x16x32 form.  Lane l holds query l % 32 and keys 8u + 4(l / 32) +
//     0..3 (u = 0..3) of a step, so a row's maximum takes one cross-lane step
//     (v_permlane32_swap) and its sums stay lane-partial until the epilogue;
//   * the value products take the scores' registers as B operands as they
//     are: k-step kk of a step holds keys 16kk + 4(l / 32) + 0..3 and
//     16kk + 8 + 4(l / 32) + 0..3, and the transposing LDS reads of V and dV
//     (ds_read_b64_tr_b16) fetch exactly those keys for the A operands;
//   * O^T, A^T, B^T for 32 rows x d are 3 d / 2 registers per lane, held in
//     AGPRs, so one wave runs per SIMD (four per workgroup, 128 query rows;
//     at d = 64 two workgroups share a CU); the Q, dQ fragments take the
//     remaining AGPRs (MFMAs read A and B operands from either file);
//   * keys move in 32-key steps through four LDS stages (K, dK of every stage
//     in one 64 KiB region, V, dV in another, so every LDS offset fits the
//     instructions' 16-bit field), copies three steps ahead, one barrier per
//     step.  A step's iteration issues the NEXT step's score MFMAs with this
//     step's exponentials placed between their slices, then this step's value
//     MFMAs: every MFMA is inline asm that keeps its place in the program, so
//     the single wave of a SIMD always has independent MFMA and VALU work;
//   * the softmax reference of a row is fixed, so no instruction of the key
//     loop ever reads or scales an accumulator (which would make the
//     register allocator move them between the register files every step).
//     The first pass takes as reference the row's first finite step maximum
//     and tracks the true maximum; float32 and bfloat16 hold P~ up to 2^127,
//     and the pass's results are exact as long as no row's maximum exceeds
//     its reference by more than 2^64.  A block with such a row walks its keys
//     again with each row's true maximum as reference (nothing can overflow
//     then); the first pass's values are discarded.  With the data of the
//     attention workloads the second pass never runs.
// The exp2-domain softmax with float32 row sums taken before the bf16
// rounding of P~ and P~ (.) dS, the scale applied in the epilogue, the
// frame-window walk and element masks, key splits and the epilogue are those
// of kernel.h.

#pragma once

#include "kernel.h"

namespace attn_jvp {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// LDS reads in flight: K/dK slices of the score products, V/dV groups of
// the value products.
#ifndef ATTN_JVP_R32_KPD
#define ATTN_JVP_R32_KPD 2
#endif
#ifndef ATTN_JVP_R32_VPD
#define ATTN_JVP_R32_VPD 2
#endif

// A pass's P~ may reach 2^kRefSlack (log2 units above the reference).
constexpr float kRefSlack = 64.0f;

template <int D>
struct Cfg32 {
  static constexpr FwdGeom G = fwd_geom(2, D, D);
  static_assert(G.rows32, "the 32-row geometry is not selected for this head dim");
  static constexpr int RB = 2 * D;          // bytes per K / V row
  static constexpr int kWaves = G.waves;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kBlockM = G.block_m;
  static constexpr int kStep = G.block_n;   // keys per step and stage
  static constexpr int kStages = 4;
  static constexpr int TS = kStep * RB;     // one tensor's rows of one stage
  static constexpr int kVRegion = kStages * 2 * TS;
  static constexpr int kLds = G.lds;
  static constexpr int kMinBlocks = D == 64 ? 2 : 1;
  static_assert(kBlockM == 32 * kWaves && kStep == 32, "geometry");
  static_assert(kLds == 2 * kVRegion, "two regions of four stages");
  static_assert(kVRegion <= 65536, "LDS offsets within a region fit 16 bits");
};

// ---------------------------------------------------------------------------
// MFMAs as inline asm.  The compiler cannot see hazards inside inline asm, so
// each helper states the ones that concern it:
//  * score MFMAs read K slices (LDS loads) and Q fragments (global loads):
//    no VALU producer; each MFMA reading srcC reads exactly what the one
//    before wrote (forwarded, no wait).  The VALU may touch S, dS only after
//    scores_settle() (20 wait states, above the MFMA result latency);
//  * value MFMAs read P~ and H packs that a VALU wrote: s_nop 1 first (two
//    wait states); the accumulators are read by the compiler's code only
//    after acc_settle() (24 wait states).
// ---------------------------------------------------------------------------
template <bool FIRST>
__device__ inline void mfma32_scores(f32x16 &S, f32x16 &dS, bf16x8 kf, bf16x8 dkf, bf16x8 q,
                                     bf16x8 dq) {
  if constexpr (FIRST) {
    asm volatile(
        "v_mfma_f32_32x32x16_bf16 %0, %2, %4, 0\n"
        "v_mfma_f32_32x32x16_bf16 %1, %2, %5, 0\n"
        "v_mfma_f32_32x32x16_bf16 %1, %3, %4, %1\n"
        : "=&v"(S), "=&v"(dS)
        : "v"(kf), "v"(dkf), "a"(q), "a"(dq));
  } else {
    asm volatile(
        "v_mfma_f32_32x32x16_bf16 %0, %2, %4, %0\n"
        "v_mfma_f32_32x32x16_bf16 %1, %2, %5, %1\n"
        "v_mfma_f32_32x32x16_bf16 %1, %3, %4, %1\n"
        : "+v"(S), "+v"(dS)
        : "v"(kf), "v"(dkf), "a"(q), "a"(dq));
  }
}

__device__ inline void scores_settle(f32x16 &S, f32x16 &dS) {
  asm volatile("s_nop 7\n s_nop 7\n s_nop 3\n" : "+v"(S), "+v"(dS));
}

// O += V P, A += dV P, B += V H for one (d block, k-step).
__device__ inline void mfma32_values(f32x16 &o, f32x16 &a, f32x16 &bb, bf16x8 vf, bf16x8 dvf,
                                     bf16x8 P, bf16x8 H) {
  asm volatile(
      "s_nop 1\n"
      "v_mfma_f32_32x32x16_bf16 %0, %3, %5, %0\n"
      "v_mfma_f32_32x32x16_bf16 %1, %4, %5, %1\n"
      "v_mfma_f32_32x32x16_bf16 %2, %3, %6, %2\n"
      : "+a"(o), "+a"(a), "+a"(bb)
      : "v"(vf), "v"(dvf), "v"(P), "v"(H));
}

__device__ inline void acc_settle(f32x16 &o, f32x16 &a, f32x16 &bb) {
  asm volatile("s_nop 7\n s_nop 7\n s_nop 7\n" : "+a"(o), "+a"(a), "+a"(bb));
}

// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt bits [3:0] and [15:14], expcnt
// and lgkmcnt left at their maxima): at most N vector-memory operations of
// this wave still outstanding.
template <int N>
__device__ inline void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ inline float swap32_max(float x) {
  const unsigned u = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_elementwise_maximum(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ inline float swap32_sum(float x) {
  const unsigned u = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int D, bool MASKED>
__global__ __launch_bounds__(Cfg32<D>::kThreads, Cfg32<D>::kMinBlocks) void attn_jvp_kernel32(
    Params p) {
  using C = Cfg32<D>;
  using T = __bf16;
  constexpr int W = C::kWaves;
  constexpr int RB = C::RB, TS = C::TS;
  constexpr int NSL = D / 16;   // 16-wide d slices of the score products
  constexpr int NDB = D / 32;   // 32-wide d blocks of the value products
  constexpr int VR = C::kVRegion;
  using KCopy = SideCopier<T, RB, 32, W, kSwzK32>;
  using VCopy = SideCopier<T, RB, 32, W, kSwzV32>;
  static_assert(KCopy::NI % W == 0 && VCopy::NI % W == 0, "every wave issues every copy");
  constexpr int kCopies = 2 * KCopy::IPW + 2 * VCopy::IPW;   // per wave and step

  __shared__ __attribute__((aligned(1024))) char smem[C::kLds];
  __shared__ int vote[W];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qj = lane & 31;   // this lane's query within the wave
  const int hh = lane >> 5;   // which keys of a step: 8u + 4 hh + 0..3

  const int lid_all = logical_block_id();
  const int lid = lid_all / p.nsplit;
  const int split = lid_all - lid * p.nsplit;
  const int bh = lid / p.nqb;
  const int qb = lid - bh * p.nqb;
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int Nq = p.Nq, Nkv = p.Nkv;

  const int q0 = qb * C::kBlockM;
  const int q_hi = (q0 + C::kBlockM < Nq) ? q0 + C::kBlockM : Nq;
  TileRanges tr;
  if constexpr (MASKED) tr = visible_tiles(p.mask, q0, q_hi, Nkv, 32);
  else tr = all_tiles(Nkv, 32);
  const int nvis = tile_count(tr);
  const int per_split = (nvis + p.nsplit - 1) / p.nsplit;
  const int t_first = split * per_split;
  const int t_last = t_first + per_split < nvis ? t_first + per_split : nvis;
  const int nstep = t_last > t_first ? t_last - t_first : 0;

  // ---- Q, dQ fragments (B operands of S^T = K Q^T, in AGPRs) ----
  const int qrow = q0 + wave * 32 + qj;
  const bool qvalid = qrow < Nq;
  const T *Q = (const T *)p.q + b * p.sq[0] + h * p.sq[1];
  const T *dQ = (const T *)p.dq + b * p.sq[0] + h * p.sq[1];
  bf16x8 qf[NSL], dqf[NSL];
#pragma unroll
  for (int s = 0; s < NSL; ++s) {
    if (qvalid) {
      const int64_t off = (int64_t)qrow * p.sq[2] + 16 * s + 8 * hh;
      qf[s] = *(const bf16x8 *)(Q + off);
      dqf[s] = *(const bf16x8 *)(dQ + off);
    } else {
      qf[s] = bf16x8{};
      dqf[s] = bf16x8{};
    }
  }
#pragma unroll
  for (int s = 0; s < NSL; ++s) asm volatile("" : "+a"(qf[s]), "+a"(dqf[s]));

  KCopy kcopy;
  VCopy vcopy;
  kcopy.init((const T *)p.k + b * p.sk[0] + h * p.sk[1],
             (const T *)p.dk + b * p.sk[0] + h * p.sk[1], p.sk[2], wave, lane);
  vcopy.init((const T *)p.v + b * p.sv[0] + h * p.sv[1],
             (const T *)p.dv + b * p.sv[0] + h * p.sv[1], p.sv[2], wave, lane);
  // step j (32 keys) into stage g: K, dK at g * 2 TS, V, dV at VR + g * 2 TS
  auto issue_step = [&](int j, int g) __attribute__((always_inline)) {
    const int k0 = tile_at(tr, t_first + j) * 32;
    kcopy.issue(k0, Nkv, smem + g * 2 * TS, TS);
    vcopy.issue(k0, Nkv, smem + VR + g * 2 * TS, TS);
  };

  f32x16 oacc[NDB], aacc[NDB], bacc[NDB];
  float l_run = 0.f, r_run = 0.f;
  float m_ref = -INFINITY;    // softmax reference, log2 units
  float m_true = -INFINITY;   // the row's running maximum, log2 units
  const float scale = p.scale;
  const float c2 = p.scale_log2;

  // Query-side mask terms (as in kernel.h): the chunk rule's key interval
  // [kv_lo, kv_hi) of this lane's query, the anchor frames, and the keys
  // [win_lo, win_hi) every row of the block sees.
  int kv_lo = 0, kv_hi = Nkv, a_first_hi = 0, a_last_lo = Nkv;
  int win_lo = 0, win_hi = 0;
  if constexpr (MASKED) {
    const long long F = p.mask.frames, TPF = p.mask.tpf, CH = p.mask.chunk, R = p.mask.radius;
    const int qf_ = div_fix(qvalid ? qrow : 0, p.mask.tpf, p.mask.inv_tpf);
    const int q_chunk = div_fix(qf_, p.mask.chunk, p.mask.inv_chunk);
    const bool q_all = p.mask.see_all &&
                       ((p.mask.first && qf_ == 0) || (p.mask.last && qf_ == p.mask.frames - 1));
    long long flo = (q_chunk - R) * CH, fhi = (q_chunk + R + 1) * CH;
    flo = flo < 0 ? 0 : flo;
    fhi = fhi > F ? F : fhi;
    if (!q_all) {
      kv_lo = (int)(flo * TPF);
      kv_hi = fhi > flo ? (int)(fhi * TPF) : kv_lo;
    }
    a_first_hi = p.mask.first ? (int)TPF : 0;
    a_last_lo = p.mask.last ? (int)((F - 1) * TPF) : Nkv;
    const long long c0 = (q0 / TPF) / CH;
    const long long c1 = ((q_hi - 1) / TPF) / CH;
    long long wlo = (c1 - R) * CH, whi = (c0 + R + 1) * CH;
    wlo = wlo < 0 ? 0 : wlo;
    whi = whi > F ? F : whi;
    if (whi > wlo) {
      win_lo = (int)(wlo * TPF);
      win_hi = (int)(whi * TPF);
    }
  }

  // Lane parts of the LDS addresses.  K operand of slice s: row qj, bytes
  // (16 s + 8 hh) * 2.  V transposing reads of d block e: in 16-lane group g,
  // lane i addresses row 4 (g / 2) + i / 4 and d 32 e + 16 (g % 2) + 4 (i % 4),
  // so that it receives d = 32 e + 16 (g % 2) + i of rows 4 (g / 2) + 0..3;
  // rows 8 and 16 further (the second read, the second k-step) keep the
  // swizzle, so they and the tensor are constant offsets, the stage a
  // per-step add.
  const uint32_t smem_a = lds_addr(smem);
  uint32_t kl[NSL];
#pragma unroll
  for (int s = 0; s < NSL; ++s) kl[s] = smem_a + lds_off<RB, kSwzK32>(qj, (16 * s + 8 * hh) * 2);
  uint32_t vl[NDB];
  {
    const int g = lane >> 4, i = lane & 15;
#pragma unroll
    for (int e = 0; e < NDB; ++e)
      vl[e] = smem_a + VR +
              lds_off<RB, kSwzV32>(4 * (g >> 1) + (i >> 2), (32 * e + 16 * (g & 1) + 4 * (i & 3)) * 2);
  }

  // ---- S^T, dS^T of the step in stage g (value v of the lane: key
  // 8 (v / 4) + 4 hh + v % 4 of the step, query qj).  The K, dK slices are
  // read PD - 1 ahead of their MFMAs; kread(g, kf, dkf) issues the first
  // PD - 1 (separately, so that they can go out before the step's barrier),
  // scores_from() the rest.  between(s) runs after the MFMAs of slice s and
  // stays there ----
  constexpr int PD = NSL < ATTN_JVP_R32_KPD ? NSL : ATTN_JVP_R32_KPD;   // slices in flight
  auto kread = [&](int g, bf16x8 (&kf)[NSL], bf16x8 (&dkf)[NSL], auto s_)
                   __attribute__((always_inline)) {
    constexpr int s = decltype(s_)::value;
    const uint32_t a = kl[s] + (uint32_t)g * (2 * TS);
    kf[s] = lds_read_k<0>(a);
    dkf[s] = lds_read_k<TS>(a);
  };
  auto kread_first = [&](int g, bf16x8 (&kf)[NSL], bf16x8 (&dkf)[NSL])
                         __attribute__((always_inline)) {
    static_for<0, PD - 1>([&](auto s_) __attribute__((always_inline)) { kread(g, kf, dkf, s_); });
  };
  auto scores_from = [&](int g, bf16x8 (&kf)[NSL], bf16x8 (&dkf)[NSL], f32x16 &S, f32x16 &dS,
                         auto &&between) __attribute__((always_inline)) {
    static_for<0, NSL>([&](auto s_) __attribute__((always_inline)) {
      constexpr int s = decltype(s_)::value;
      if constexpr (s + PD - 1 < NSL) kread(g, kf, dkf, std::integral_constant<int, s + PD - 1>{});
      constexpr int newer = (NSL - 1 - s) < (PD - 1) ? (NSL - 1 - s) : (PD - 1);
      lds_wait<2 * newer>();
      mfma32_scores<s == 0>(S, dS, kf[s], dkf[s], qf[s], dqf[s]);
      between(s_);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // ---- O^T += V^T P^T ; A^T += dV^T P^T ; B^T += V^T H^T, stage g ----
  auto values = [&](int g, const bf16x8 (&P)[2], const bf16x8 (&H)[2], auto &&between)
                    __attribute__((always_inline)) {
    constexpr int NV = 2 * NDB;           // (d block, k-step) groups
    constexpr int VD = NV < ATTN_JVP_R32_VPD ? NV : ATTN_JVP_R32_VPD;   // groups in flight
    const uint32_t goff = (uint32_t)g * (2 * TS);
    auto issue = [&](auto v_, i16x4 (&r)[4]) __attribute__((always_inline)) {
      constexpr int v = decltype(v_)::value;
      constexpr int e = v / 2, kk = v % 2;
      constexpr int O = kk * 16 * RB;
      const uint32_t a = vl[e] + goff;
      r[0] = lds_read_tr<O>(a);
      r[1] = lds_read_tr<O + 8 * RB>(a);
      r[2] = lds_read_tr<O + TS>(a);
      r[3] = lds_read_tr<O + TS + 8 * RB>(a);
    };
    i16x4 buf[VD][4];
    static_for<0, VD - 1>([&](auto v_) __attribute__((always_inline)) {
      issue(v_, buf[decltype(v_)::value]);
    });
    static_for<0, NV>([&](auto v_) __attribute__((always_inline)) {
      constexpr int v = decltype(v_)::value;
      constexpr int e = v / 2, kk = v % 2;
      i16x4(&cur)[4] = buf[v % VD];
      if constexpr (v + VD - 1 < NV)
        issue(std::integral_constant<int, v + VD - 1>{}, buf[(v + VD - 1) % VD]);
      constexpr int newer = (NV - 1 - v) < (VD - 1) ? (NV - 1 - v) : (VD - 1);
      lds_wait<4 * newer>();
      const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(cur[0], cur[1], 0, 1, 2, 3, 4, 5, 6, 7));
      const bf16x8 dvf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(cur[2], cur[3], 0, 1, 2, 3, 4, 5, 6, 7));
      mfma32_values(oacc[e], aacc[e], bacc[e], vf, dvf, P[kk], H[kk]);
      between(v_);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // ---- element masks of a step starting at key ka ----
  auto apply_mask = [&](int ka, f32x16 &S, f32x16 &dS) __attribute__((always_inline)) {
    // the key index comes out of a volatile asm inside the branch, so the
    // selects below cannot be hoisted out of it (if-conversion would run
    // them on every step)
    int kb = ka + 4 * hh;
    asm volatile("" : "+v"(kb));
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = kb + 8 * (v >> 2) + (v & 3);
      bool vis = key < Nkv;
      if constexpr (MASKED) {
        const bool in_chunks = (unsigned)(key - kv_lo) < (unsigned)(kv_hi - kv_lo);
        vis = vis & (in_chunks | (key < a_first_hi) | (key >= a_last_lo));
      }
      S[v] = vis ? S[v] : -INFINITY;
      dS[v] = vis ? dS[v] : 0.f;
    }
  };
  auto needs_mask = [&](int k0) __attribute__((always_inline)) {
    const int kz = k0 + 32;
    bool m = kz > Nkv;
    if constexpr (MASKED) {
      const bool in_win = k0 >= win_lo && kz <= win_hi;
      const bool in_first = p.mask.first && kz <= p.mask.tpf;
      const bool in_last = p.mask.last && k0 >= (p.mask.frames - 1) * p.mask.tpf;
      m = m || !(in_win || in_first || in_last);
    }
    return m;
  };

  // ---- a step's row maximum (log2 units): the running maximum follows it,
  // and a reference still at -inf (no visible key yet: every P~ so far was
  // 0, so the accumulators are zero) takes it ----
  auto track_max = [&](const f32x16 &S) __attribute__((always_inline)) {
    float a0 = __builtin_elementwise_maximum(S[0], S[1]);
    float a1 = __builtin_elementwise_maximum(S[2], S[3]);
    float a2 = __builtin_elementwise_maximum(S[4], S[5]);
    float a3 = __builtin_elementwise_maximum(S[6], S[7]);
    float a4 = __builtin_elementwise_maximum(S[8], S[9]);
    float a5 = __builtin_elementwise_maximum(S[10], S[11]);
    float a6 = __builtin_elementwise_maximum(S[12], S[13]);
    float a7 = __builtin_elementwise_maximum(S[14], S[15]);
    a0 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(a0, a1),
                                       __builtin_elementwise_maximum(a2, a3));
    a4 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(a4, a5),
                                       __builtin_elementwise_maximum(a6, a7));
    const float mx = swap32_max(__builtin_elementwise_maximum(a0, a4)) * c2;
    m_true = __builtin_elementwise_maximum(m_true, mx);
    m_ref = m_ref == -INFINITY ? mx : m_ref;
  };

  // ---- P~ = exp2(S - m), H = P~ dS (float32 row sums before the bf16
  // rounding) for elements [v0, v0 + n) of a step (n even), packed pair by
  // pair into the bf16 B operands of the two k-steps (elements 0..7, 8..15)
  auto softmax_part = [&](const f32x16 &S, const f32x16 &dS, float m_use, bf16x8 (&P)[2],
                          bf16x8 (&H)[2], auto v0_, auto n_) __attribute__((always_inline)) {
    static_assert(decltype(n_)::value % 2 == 0, "pairs");
    static_for<0, decltype(n_)::value / 2>([&](auto i_) __attribute__((always_inline)) {
      constexpr int v = decltype(v0_)::value + 2 * decltype(i_)::value;
      const float p0 = __builtin_amdgcn_exp2f(fmaf(S[v], c2, -m_use));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(S[v + 1], c2, -m_use));
      const float h0 = p0 * dS[v], h1 = p1 * dS[v + 1];
      l_run += p0;
      l_run += p1;
      r_run += h0;
      r_run += h1;
      // keep the sums here, between the MFMAs (the compiler would sink the
      // two chains of adds to the next step, where nothing hides them)
      asm volatile("" : "+v"(l_run), "+v"(r_run));
      P[v >> 3][v & 7] = (__bf16)p0;
      P[v >> 3][(v & 7) + 1] = (__bf16)p1;
      H[v >> 3][v & 7] = (__bf16)h0;
      H[v >> 3][(v & 7) + 1] = (__bf16)h1;
    });
  };

  // One step with the next one's scores beside it: S, dS hold step j;
  // Sn, dSn receive step j + 1 (masked, maximum tracked).  On entry, step
  // j + 1 is in its stage on every wave (the previous barrier said so) and
  // kf, dkf hold the first slices of its K, dK reads, in flight.  The barrier
  // here says that step j + 2 landed on every wave and that every wave is
  // done with step j - 1, whose stage the copies of step j + 3 then take.
  auto step = [&](int j, const f32x16 &S, const f32x16 &dS, f32x16 &Sn, f32x16 &dSn,
                  bf16x8 (&kf)[NSL], bf16x8 (&dkf)[NSL]) __attribute__((always_inline)) {
    if (j + 2 < nstep) wait_vm<0>();
    __builtin_amdgcn_s_barrier();
    const bool copy = j + 3 < nstep;
    const int kc = copy ? tile_at(tr, t_first + j + 3) * 32 : 0;
    const int gc = (j + 3) & 3;
    bf16x8 P[2], H[2];
    const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
    constexpr int PER = 16 / NSL;   // exponentials after each score slice
    scores_from((j + 1) & 3, kf, dkf, Sn, dSn, [&](auto s_) __attribute__((always_inline)) {
      constexpr int s = decltype(s_)::value;
      softmax_part(S, dS, m_use, P, H, std::integral_constant<int, s * PER>{},
                   std::integral_constant<int, PER>{});
      // the copies of step j + 3 go out between the score MFMAs
      if constexpr (s == 1) {
        if (copy) kcopy.issue(kc, Nkv, smem + gc * 2 * TS, TS);
      } else if constexpr (s == 2) {
        if (copy) vcopy.issue(kc, Nkv, smem + VR + gc * 2 * TS, TS);
      }
    });
    const int kn = tile_at(tr, t_first + j + 1) * 32;
    const bool need = needs_mask(kn);
    values(j & 3, P, H, [&](auto v_) __attribute__((always_inline)) {
      constexpr int v = decltype(v_)::value;
      // the next step's row maximum between the value MFMAs
      if constexpr (v == 0) {
        scores_settle(Sn, dSn);
        if (need) apply_mask(kn, Sn, dSn);
      } else if constexpr (v == 1) {
        track_max(Sn);
      }
    });
  };
  auto last = [&](int j, const f32x16 &S, const f32x16 &dS) __attribute__((always_inline)) {
    bf16x8 P[2], H[2];
    const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
    softmax_part(S, dS, m_use, P, H, std::integral_constant<int, 0>{},
                 std::integral_constant<int, 16>{});
    values(j & 3, P, H, [](auto) {});
  };

  // ---- the key walk (one pass, rarely two) ----
  for (int pass = 0;; ++pass) {
#pragma unroll
    for (int e = 0; e < NDB; ++e) {
      oacc[e] = f32x16{};
      aacc[e] = f32x16{};
      bacc[e] = f32x16{};
    }
    l_run = 0.f;
    r_run = 0.f;
    if (nstep > 0) {
      issue_step(0, 0);
      if (nstep > 1) issue_step(1, 1);
      if (nstep > 2) issue_step(2, 2);
      // steps 0 and 1 landed (step 2 may still be in flight)
      if (nstep > 2) wait_vm<kCopies>();
      else wait_vm<0>();
      __builtin_amdgcn_s_barrier();
      f32x16 Sa, dSa, Sb, dSb;
      bf16x8 kf[NSL], dkf[NSL];
      kread_first(0, kf, dkf);
      scores_from(0, kf, dkf, Sa, dSa, [](auto) {});
      if (nstep > 1) kread_first(1, kf, dkf);
      scores_settle(Sa, dSa);
      {
        const int k0 = tile_at(tr, t_first) * 32;
        if (needs_mask(k0)) apply_mask(k0, Sa, dSa);
      }
      track_max(Sa);
      int j = 0;
      for (; j + 2 < nstep; j += 2) {
        step(j, Sa, dSa, Sb, dSb, kf, dkf);
        kread_first((j + 2) & 3, kf, dkf);
        step(j + 1, Sb, dSb, Sa, dSa, kf, dkf);
        if (j + 3 < nstep) kread_first((j + 3) & 3, kf, dkf);
      }
      if (j + 1 < nstep) {
        step(j, Sa, dSa, Sb, dSb, kf, dkf);
        last(j + 1, Sb, dSb);
      } else {
        last(j, Sa, dSa);
      }
    }
    if (pass > 0) break;
    // does any row of the block need the second pass?  (a vote over the
    // waves: all of them walk the keys together)
    const bool mine = __any(m_true > m_ref + kRefSlack);
    if (lane == 0) vote[wave] = mine ? 1 : 0;
    __syncthreads();
    int any = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) any |= vote[w];
    if (!any) break;
    __syncthreads();   // every wave has read the votes and left the stages
    m_ref = m_true;
  }

  // ---- epilogue: lanes l and l + 32 hold halves of query qj's sums ----
  const float l_tot = swap32_sum(l_run);
  const float r_tot = swap32_sum(r_run);
  const bool empty = !(l_tot > 0.f);
  const float inv = empty ? 0.f : 1.f / l_tot;
  const float mu = scale * r_tot * inv;   // dLSE
  const float sinv = scale * inv;
  const float lse = empty ? -INFINITY : (m_ref + log2f(l_tot)) * 0.69314718055994530942f;
  if (qvalid && p.partial) {
    const int64_t row = ((int64_t)split * p.B * p.H + bh) * Nq + qrow;
    float *O = (float *)p.o + row * D;
    float *dO = (float *)p.dout + row * D;
    static_for<0, NDB>([&](auto e_) __attribute__((always_inline)) {
      constexpr int e = decltype(e_)::value;
      __builtin_amdgcn_sched_barrier(0);
      acc_settle(oacc[e], aacc[e], bacc[e]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int d0 = 32 * e + 8 * u + 4 * hh;
        f32x4 ov, dv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ov[i] = oacc[e][4 * u + i] * inv;
          dv[i] = fmaf(bacc[e][4 * u + i], sinv, aacc[e][4 * u + i] * inv) - mu * ov[i];
        }
        *(f32x4 *)(O + d0) = ov;
        *(f32x4 *)(dO + d0) = dv;
      }
    });
    if (hh == 0) {
      p.lse[row] = lse;
      p.dlse[row] = mu;
    }
  } else if (qvalid) {
    T *O = (T *)p.o + b * p.so[0] + h * p.so[1] + (int64_t)qrow * p.so[2];
    T *dO = (T *)p.dout + b * p.so[0] + h * p.so[1] + (int64_t)qrow * p.so[2];
    typedef T T4 __attribute__((ext_vector_type(4)));
    static_for<0, NDB>([&](auto e_) __attribute__((always_inline)) {
      constexpr int e = decltype(e_)::value;
      __builtin_amdgcn_sched_barrier(0);
      acc_settle(oacc[e], aacc[e], bacc[e]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int d0 = 32 * e + 8 * u + 4 * hh;
        T4 ov, dv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float o = oacc[e][4 * u + i] * inv;
          ov[i] = (T)o;
          dv[i] = (T)(fmaf(bacc[e][4 * u + i], sinv, aacc[e][4 * u + i] * inv) - mu * o);
        }
        *(T4 *)(O + d0) = ov;
        *(T4 *)(dO + d0) = dv;
      }
    });
    if (hh == 0) {
      const int64_t ro = (int64_t)bh * Nq + qrow;
      p.lse[ro] = lse;
      p.dlse[ro] = mu;
    }
  }
}

template <int D, bool MASKED>
hipError_t launch_instance32(const Params &p, hipStream_t stream) {
  using C = Cfg32<D>;
  const int grid = p.B * p.H * p.nqb * p.nsplit;
  hipLaunchKernelGGL((attn_jvp_kernel32<D, MASKED>), dim3(grid), dim3(C::kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn_jvp
