// Fused attention forward-mode derivative (JVP) for AMD gfx950 (MI355X):
// the device code, shared by the instantiation units.
//
// What is computed (page "带分数正则的一致性蒸馏", gitcode.csdn.net, section
// 注意力): per query row, O = softmax(s Q K^T) V together with its tangent
// dO = P dV + (P (.) dS) V - rowsum(P (.) dS) O, dS = s (dQ K^T + Q dK^T), the
// natural-log row log-sum-exp and its tangent.  The pages stream K/V blocks
// with an online max m, sum l, tangent sum r and accumulators O~, A~ = P~ dV,
// B~ = H~ V (H~ = P~ (.) dS); the kernel keeps all three and combines A~ and
// B~ only in the epilogue (B~ carries dS without the scale).  Q, dQ are
// [.., Lq, d_qk], K, dK [.., Lkv, d_qk], V, dV [.., Lkv, d_v], O, dO
// [.., Lq, d_v] (the pages' op contract allows Lq != Lkv and d_qk != d_v).
//
// gfx950 design (one workgroup = W waves x 16 query rows of one (b, h)):
//   * every wave owns 16 query rows and computes the TRANSPOSED score tile
//     S^T = K Q^T with 16x16 MFMAs: lane l holds 4 keys of query l % 16, so
//     the row max and row sums need one butterfly over the four lanes of a
//     row (v_permlane16/32_swap), and the rounded scores are directly the B
//     operand of the value products;
//   * Q and dQ stay in registers (B operands) for the whole key loop;
//   * K, dK, V, dV tiles move global -> LDS with asynchronous
//     global_load_lds_dwordx4 copies into two LDS stages (the next tile
//     streams in while the current one is consumed; no register staging),
//     row-major with an XOR swizzle of the 16-byte chunks chosen from the
//     measured LDS bank geometry (K and dK for operand-row reads, V and dV
//     for transposing reads; both conflict-free);
//   * the score products read their K and dK slices two or three slices
//     ahead of the MFMAs that use them, with explicit LDS waits;
//   * the value products need V and dV transposed (keys along the MFMA k
//     dimension): ds_read_b64_tr_b16 transposes on the way out of LDS;
//   * O^T, A^T, B^T accumulate in 16x16 fp32 fragments that belong to the
//     lane's own query, so the online rescale is one multiply by a per-lane
//     factor, skipped unless the row max grew by more than 2^8;
//   * exp2 domain for the scores (scale * log2 e folded into one FMA), the
//     tangent stays in natural units;
//   * workgroup ids are remapped so that all query blocks of one (b, h) land
//     on the same XCD (dispatch round-robins consecutive ids over the 8 XCDs),
//     keeping that head's K/V/dK/dV in one L2;
//   * with a frame-window mask, each query block walks only the key-tile
//     ranges some of its rows can see; element masks run on partial tiles;
//   * at d_qk + d_v >= 256 a step's MFMA blocks run at raised wave priority,
//     so that of the two waves of a SIMD the one feeding the matrix core
//     issues first.
// Eight waves (two per SIMD) when the resident registers allow it, else four;
// twelve (three per SIMD) at bf16 d_qk = d_v = 64; 64-key tiles when two
// stages fit in 128 KiB of LDS, else 32-key tiles.
// float32 inputs use the same structure with v_mfma_f32_16x16x4_f32.

#pragma once

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <type_traits>

#include "plan.h"

namespace attn_jvp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kWaveRows = 16;   // query rows per wave
constexpr int kStepKeys = 32;   // keys per softmax step

// ---------------------------------------------------------------------------
// Launch shape of one (dtype, d_qk, d_v) instance.
// ---------------------------------------------------------------------------
template <typename T, int DQK, int DV, bool SMALL = false>
struct Cfg {
  static constexpr int ES = (int)sizeof(T);
  static constexpr int RBK = DQK * ES;   // bytes per K / dK row
  static constexpr int RBV = DV * ES;    // bytes per V / dV row
  static constexpr FwdGeom G = SMALL ? fwd16_geom_small(ES, DQK, DV) : fwd16_geom(ES, DQK, DV);
  static constexpr int kWaves = G.waves;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kBlockM = G.block_m;
  static constexpr int kBN = G.block_n;
  static constexpr int kLds = G.lds;   // two stages of K, dK, V, dV
  static_assert(kBlockM == kWaveRows * kWaves, "16 query rows per wave");
};

// ---------------------------------------------------------------------------
// MFMA traits.  For an operand tile with 16 rows (or columns) and K along the
// contraction, lane l holds row l % 16 and the K slice of lane group l / 16;
// the 16x16 result puts column l % 16 and rows 4 (l / 16) + 0..3 in lane l.
// ElemK contracts over the head dim (scores), ElemV over keys (values).
// ---------------------------------------------------------------------------
template <typename T, int DQK> struct ElemK;

template <int DQK> struct ElemK<__bf16, DQK> {
  using Frag = bf16x8;            // 8 bf16 along K per lane
  static constexpr int KL = 8;    // K elements per lane
  static constexpr int KI = 32;   // K per instruction (four lane groups)
  __device__ static inline f32x4 mfma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct ElemK<__bf16, 16> {
  using Frag = bf16x4;
  static constexpr int KL = 4;
  static constexpr int KI = 16;
  __device__ static inline f32x4 mfma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
};

template <int DQK> struct ElemK<float, DQK> {
  using Frag = float;
  static constexpr int KL = 1;
  static constexpr int KI = 4;
  __device__ static inline f32x4 mfma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

template <typename T> struct ElemV;

template <> struct ElemV<__bf16> {
  using Frag = bf16x8;
  __device__ static inline f32x4 mfma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct ElemV<float> {
  using Frag = float;
  __device__ static inline f32x4 mfma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// Dispatch places workgroup w on XCD (w mod 8).  Give each XCD a contiguous
// run of logical ids so a head's query blocks share one L2: logical id of
// block w of n.
__device__ inline int logical_id_of(int w, int n) {
  const int per = n / 8, rem = n % 8;
  const int x = w % 8, local = w / 8;
  return x * per + (x < rem ? x : rem) + local;
}

__device__ inline int logical_block_id() { return logical_id_of(blockIdx.x, gridDim.x); }

// ---------------------------------------------------------------------------
// LDS tile layout.  A K or dK tile is BN rows of RB = d_qk * sizeof(T) bytes,
// a V or dV tile BN rows of d_v * sizeof(T), row-major (one key per row).
// The 16-byte chunks of row r are XOR-permuted by a rule chosen for how the
// tile is read.  Bank geometry of gfx950 LDS (measured with two active lanes
// and the bank-conflict counter): 64 four-byte banks; an 8-byte read
// (ds_read_b64, ds_read_b64_tr_b16) serves 32 consecutive lanes per pass; a
// 16-byte read serves 16 lanes per pass, the four-lane groups of a half-wave
// whose 3-bit group index has even parity (lanes 0-3, 12-15, 20-23, 24-27),
// then those with odd parity.
//  * kswz(r), operand rows: the row's sweep index mod the chunks per sweep.
//    The rows of one 16-byte-read pass land on distinct slots.  Used by the
//    float32 tiles.
//  * vswz(r), transposing reads: the four rows one pass reads as 32-byte
//    runs cover distinct banks.
//  * bswz(r), both: bfloat16 tiles read along rows, and backward tiles read
//    both along rows and transposed.  A function of r mod 8 (per row size)
//    that satisfies both conditions above.
// All rules repeat every 16 rows, so a row offset that is a multiple of 16
// keeps a lane's swizzle.
// ---------------------------------------------------------------------------
template <int RB>
struct Sweep {
  static constexpr int CPR = RB / 16;                 // chunks per row
  static constexpr int RPB = RB >= 256 ? 1 : 256 / RB; // rows per bank sweep
  static constexpr int CW = CPR < 16 ? CPR : 16;       // chunks per sweep per row
};

template <int RB>
__device__ inline int kswz(int r) {
  return (r / Sweep<RB>::RPB) % Sweep<RB>::CW;
}

template <int RB>
__device__ inline int vswz(int r) {
  constexpr int H = Sweep<RB>::CW / 2;
  const int m = r / Sweep<RB>::RPB;
  return ((m % H) << 1) | ((m / H) % 2);
}

template <int RB>
__device__ inline int bswz(int r) {
  if constexpr (RB >= 256) return (r % 8) << 1;
  else if constexpr (RB == 128) return r % 8;
  else if constexpr (RB == 64) return (r >> 1) & 3;
  else return kswz<RB>(r);
}

// Rules of the 32-query-row kernel (kernel32.h), whose operand-row reads
// cover 32 consecutive rows (a 16-lane pass reads rows r mod 32 in
// {0-3, 12-15, 20-23, 24-27} or {4-11, 16-19, 28-31}, all at one chunk) and
// whose transposing reads cover 4 consecutive rows x 64 bytes per pass:
//  * k32swz(r): 16 distinct slots over each pass's rows (r mod 16 for
//    256-byte rows; for 128-byte rows two rows share a bank sweep, so
//    (r mod 2, slot) must differ: slot (r / 2) mod 8);
//  * v32swz(r): the four rows' 64-byte runs on distinct quarters of the
//    bank sweep (4 (r mod 4) for 256-byte rows, 4 ((r / 2) mod 2) for
//    128-byte rows).
template <int RB>
__device__ inline int k32swz(int r) {
  static_assert(RB == 256 || RB == 128, "32-row rules are built for d = 128 and 64");
  if constexpr (RB == 256) return r % 16;
  else return (r >> 1) % 8;
}

template <int RB>
__device__ inline int v32swz(int r) {
  static_assert(RB == 256 || RB == 128, "32-row rules are built for d = 128 and 64");
  if constexpr (RB == 256) return 4 * (r % 4);
  else return 4 * ((r >> 1) & 1);
}

// swizzle kinds (template argument KS below)
constexpr int kSwzV = 0;
constexpr int kSwzK = 1;
constexpr int kSwzB = 2;
constexpr int kSwzK32 = 3;
constexpr int kSwzV32 = 4;

template <int RB, int KS>
__device__ inline int swz(int r) {
  if constexpr (KS == kSwzK) return kswz<RB>(r);
  else if constexpr (KS == kSwzV) return vswz<RB>(r);
  else if constexpr (KS == kSwzK32) return k32swz<RB>(r);
  else if constexpr (KS == kSwzV32) return v32swz<RB>(r);
  else return bswz<RB>(r);
}

template <int RB, int KS>
__device__ inline int lds_off(int r, int byte_col) {
  return r * RB + ((((byte_col >> 4) ^ swz<RB, KS>(r))) << 4) + (byte_col & 15);
}

// Read 4 consecutive-key bf16 values of one d column: ds_read_b64_tr_b16.
// In each 16-lane group, lane i receives element (i % 4) of the 8-byte chunks
// addressed by lanes i/4, i/4 + 4, i/4 + 8 and i/4 + 12 (in that order).
//
// Issued through inline asm: the compiler cannot tell that these reads never
// touch the LDS stage an in-flight global->LDS copy is filling, and would
// otherwise wait for every outstanding copy (vmcnt(0)) before the first one,
// serialising the tile prefetch.  The compiler does not count these reads, so
// lds_wait() must run before their results are used; extra LDS operations
// it does not know about only make its own lgkmcnt waits stronger, since LDS
// operations complete in issue order.
template <int OFF>
__device__ inline i16x4 lds_read_tr(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "DS offset field");
  i16x4 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF));
  return v;
}

__device__ inline uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __attribute__((always_inline)) inline void static_for(F &&f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Wait until at most N LDS operations are outstanding (the asm-issued reads
// above and below included), then a scheduling barrier that no instruction
// crosses, so that nothing reading their values is scheduled before the
// wait.  Tying the values through an asm wait instead (an output operand per
// value) orders them as well, but the compiler then takes the asm for the
// values' last VALU writer and puts a wait state (s_nop) between it and the
// MFMA that reads them next: five to eight more s_nop per 32-key step of the
// d = 128 forward, which measured 2-3 % slower there and in the backward.
template <int N>
__device__ inline void lds_wait() {
  static_assert(N >= 0 && N <= 15, "lgkmcnt field");
  // vmcnt 63 and expcnt 7 (no wait on either), lgkmcnt N
  __builtin_amdgcn_s_waitcnt(0xC07F | (N << 8));
  __builtin_amdgcn_sched_barrier(0);
}

// K-side operand read (one 16-byte row slice of K or dK), issued through
// inline asm for the reason given at lds_read_tr; lds_wait<N> waits for it.
// Holding the reads in flight this way lets the score MFMAs of one slice
// run while the next slices are still on their way from LDS.
template <int OFF>
__device__ inline bf16x8 lds_read_k(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "DS offset field");
  bf16x8 v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF));
  return v;
}

// Sum and maximum over the four lanes l, l^16, l^32, l^48 that hold one
// query row.  v_permlane16_swap(x, x) returns rows (x0, x0, x2, x2) and
// (x1, x1, x3, x3) of x's four 16-lane rows, and v_permlane32_swap(x, x)
// returns halves (lo, lo) and (hi, hi): combining the pair is one butterfly
// step, done in the VALU without an LDS round trip.  Every lane of the row
// ends with the same bits (same operand order on both sides).
__device__ inline float row_sum4(float x) {
  const unsigned u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const unsigned v = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ inline float row_max4(float x) {
  const unsigned u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __builtin_elementwise_maximum(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const unsigned v = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __builtin_elementwise_maximum(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Asynchronous global->LDS copies of the key tiles of one side (K and dK, or
// V and dV: two tensors with one row width RB).  Each wave instruction fills
// 1 KiB of LDS contiguously, lane l writing bytes [16 l, 16 l + 16); the
// lane picks the global chunk that the swizzled layout puts there.  The
// per-lane byte offsets inside a tile are fixed, so they are computed once; a
// tile then only moves the (scalar) base pointers.  The NI instructions of a
// tensor tile go round-robin over the W waves.  Rows past the end of the
// sequence re-read row N-1 (their scores are masked to -inf and their
// tangents to 0).
template <typename T, int RB, int BN, int W, int KS>
struct SideCopier {
  static constexpr int CPR = RB / 16;
  static constexpr int TILE = BN * RB;
  static constexpr int NI = TILE / 1024;
  static constexpr int IPW = (NI + W - 1) / W;
  static_assert(NI * 1024 == TILE, "a tile is whole 1 KiB wave copies");

  const char *base[2];      // byte base of the two tensors for this (b, h)
  int64_t rstride;          // row stride in bytes (shared by the two)
  uint32_t rs;              // the same, 32-bit (below 2^24, checked on the host)
  uint32_t slot[IPW];       // (row << 16) | swizzled chunk, per lane
  int wave;                 // wave index (uniform)

  __device__ void init(const T *t0, const T *t1, int64_t stride, int wave_, int lane) {
    wave = wave_;
    base[0] = (const char *)t0;
    base[1] = (const char *)t1;
    rstride = stride * (int64_t)sizeof(T);
    rs = (uint32_t)rstride;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int s = (i * W + wave) * 64 + lane;
      const int r = s / CPR;
      const int c = (s % CPR) ^ swz<RB, KS>(r);
      slot[i] = ((uint32_t)r << 16) | (uint32_t)c;
    }
  }

  // LDS: tensor t of stage g at dst0 + t * tstride (dst0 already holds g)
  __device__ void issue(int k0, int N, char *dst0, int tstride) const {
    const int valid = (N - k0 < BN ? N - k0 : BN) - 1;   // last real row
    const char *tb0 = base[0] + (int64_t)k0 * rstride;
    const char *tb1 = base[1] + (int64_t)k0 * rstride;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      if (NI % W != 0 && i * W + wave >= NI) break;   // uniform per wave
      uint32_t r = slot[i] >> 16;
      r = r < (uint32_t)valid ? r : (uint32_t)valid;
      const uint32_t off = __umul24(r, rs) + ((slot[i] & 0xffffu) << 4);
      char *dst = dst0 + (i * W + wave) * 1024;
      __builtin_amdgcn_global_load_lds((const void *)(tb0 + off), (lds_void *)dst, 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void *)(tb1 + off), (lds_void *)(dst + tstride),
                                       16, 0, 0);
    }
  }
};

// Stores of a wave's 16 rows of DV bfloat16 results held in the MFMA layout
// (lane l holds elements 16 e + 4 (l / 16) + 0..3 of row l % 16) through 16
// rows of LDS private to the wave: each lane writes its 8-byte pieces, then
// reads back and stores 16 bytes of a whole row, so that a store instruction
// writes 4 whole 256-byte rows (d = 128) instead of 32-byte pieces of 16.
// 16-byte chunk c of row r sits at slot c ^ (r / RPB mod CPR), RPB rows per
// 256-byte bank sweep: the writes (16 rows of one chunk per pass) and the
// row reads are free of bank conflicts.  Rows at or past nvalid are not
// stored.  LDS operations of a wave complete in order, so the same rows can
// serve the next call at once.
template <typename T, int DV>
struct RowStager {
  static constexpr int kRow = DV * (int)sizeof(T);
  static constexpr int CPR = kRow / 16;
  static constexpr int RPB = kRow >= 256 ? 1 : 256 / kRow;
  static constexpr int RPI = 64 / CPR;   // rows per store instruction
  static constexpr int kBytes = 16 * kRow;
  static constexpr bool kBuilt = sizeof(T) == 2 && DV >= 64 && CPR <= 64;
  typedef T T4 __attribute__((ext_vector_type(4)));
  typedef unsigned U4 __attribute__((ext_vector_type(4)));

  __device__ static int slot(int r, int c) { return r * kRow + ((c ^ ((r / RPB) % CPR)) << 4); }

  // vals(e): the lane's T4 of 16-wide block e; base: byte address of row 0;
  // stride: bytes between rows
  template <typename F>
  __device__ static void store(char *ws, int lane, F &&vals, char *base, int64_t stride,
                               int nvalid) {
    static_assert(kBuilt && 16 % RPI == 0, "row staging");
    const int rl = lane & 15, lg = lane >> 4;
#pragma unroll
    for (int e = 0; e < DV / 16; ++e) {
      const int bc = (16 * e + 4 * lg) * (int)sizeof(T);
      *(T4 *)(ws + slot(rl, bc >> 4) + (bc & 15)) = vals(e);
    }
#pragma unroll
    for (int j = 0; j < 16 / RPI; ++j) {
      const int r = RPI * j + lane / CPR, c = lane % CPR;
      const U4 v = *(const U4 *)(ws + slot(r, c));
      if (r < nvalid) *(U4 *)(base + r * stride + c * 16) = v;
    }
  }
};

__device__ inline void wait_vmem() {
  // s_waitcnt vmcnt(0): every global->LDS copy this wave issued has landed
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Lazy rescale: the running max only moves when a step's max exceeds it by
// more than 2^8 (P~ then stays below 256); the final normalisation uses the
// same reference, so the result is unchanged.  In the plain step order a
// step first compares each lane's own raw scores with the threshold (no
// cross-lane reduction, no scaling) and forms the row maxima only when some
// lane is above it: a third fewer VALU instructions between the MFMA blocks
// (4-8 % at d = 16 to 64).  The overlapped order of the larger head dims
// hides the row maxima behind MFMAs already (1 % slower with the check), and
// the one-wave-per-SIMD instances (d = 256), at their register limit, spill
// more with it (2 % slower): both keep the plain row maximum.
constexpr float kRescaleThreshold = 8.0f;

// The small geometry runs three workgroups per CU (at most 168 registers).
template <typename T, int DQK, int DV, bool MASKED, bool SMALL = false>
__global__ __launch_bounds__((Cfg<T, DQK, DV, SMALL>::kThreads), (SMALL ? 3 : 1))
void attn_jvp_kernel(Params p) {
  using C = Cfg<T, DQK, DV, SMALL>;
  using EK = ElemK<T, DQK>;
  using EV = ElemV<T>;
  using FragK = typename EK::Frag;
  using FragV = typename EV::Frag;
  constexpr bool BF16 = sizeof(T) == 2;
  constexpr int W = C::kWaves;
  constexpr int BN = C::kBN;
  constexpr int CK = kStepKeys;
  constexpr int NSTEP = BN / CK;              // 32-key steps per tile: 1 or 2
  constexpr int KL = EK::KL;
  constexpr int KI = EK::KI;
  constexpr int RBK = C::RBK, RBV = C::RBV;   // bytes per LDS row
  constexpr int TK = BN * RBK, TV = BN * RBV; // bytes per tensor tile
  constexpr int VB = 4 * TK;                  // V-side region: after K, dK stages
  constexpr int KSK = BF16 ? kSwzB : kSwzK;   // K-side swizzle (layout notes above)
  constexpr int DS = DQK / KI;                // k-steps over d_qk
  constexpr int ND = DV / 16;                 // 16-wide d_v blocks
  static_assert(NSTEP == 1 || NSTEP == 2, "tile shape");
  static_assert(DQK % KI == 0 && DV % 16 == 0, "head dims");

  // Output staging (bfloat16, d_qk = d_v >= 64): each wave's 16 rows of O,
  // then of dO, pass through LDS rows of its own beyond the tile stages, so
  // that the global stores write whole rows (16 bytes per lane, 1 KiB per
  // instruction) instead of 32-byte pieces of 16 rows.  Measured with per-
  // block timestamps, issuing the direct stores took 1.9 us per block.
  using Stager = RowStager<T, DV>;
  constexpr int kOutWave = Stager::kBytes;
  constexpr bool kStageOut =
      Stager::kBuilt && DQK == DV && C::kLds + W * kOutWave <= 160 * 1024;
  __shared__ __attribute__((aligned(1024))) char smem[C::kLds + (kStageOut ? W * kOutWave : 0)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  const int qi = lane & 15;        // this lane's query within the wave
  const int lg = lane >> 4;        // lane group 0..3

  // logical id = (bh * nqb + qb) * nsplit + split
  const int lid_all = logical_block_id();
  const int lid = lid_all / p.nsplit;
  const int split = lid_all - lid * p.nsplit;
  const int bh = lid / p.nqb;
  const int qb = lid - bh * p.nqb;
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int Nq = p.Nq, Nkv = p.Nkv;

  const T *Q = (const T *)p.q + b * p.sq[0] + h * p.sq[1];
  const T *dQ = (const T *)p.dq + b * p.sq[0] + h * p.sq[1];

  const int q0 = qb * C::kBlockM;
  const int q_hi = (q0 + C::kBlockM < Nq) ? q0 + C::kBlockM : Nq;

  TileRanges tr;
  if constexpr (MASKED) tr = visible_tiles(p.mask, q0, q_hi, Nkv, BN);
  else tr = all_tiles(Nkv, BN);
  // unused ranges are empty (lo = hi = 0).  With key splits, this workgroup
  // takes the split-th run of ceil(n / nsplit) of the n visited tiles.
  const int nvis = tile_count(tr);
  const int per_split = (nvis + p.nsplit - 1) / p.nsplit;
  const int t_first = split * per_split;
  const int t_last = t_first + per_split < nvis ? t_first + per_split : nvis;
  const int ntile = t_last > t_first ? t_last - t_first : 0;
  const TileWalk walk = tile_walk(tr);

  // first tile in flight before anything else
  SideCopier<T, RBK, BN, W, KSK> kcopy;
  SideCopier<T, RBV, BN, W, kSwzV> vcopy;
  kcopy.init((const T *)p.k + b * p.sk[0] + h * p.sk[1],
             (const T *)p.dk + b * p.sk[0] + h * p.sk[1], p.sk[2], wave, lane);
  vcopy.init((const T *)p.v + b * p.sv[0] + h * p.sv[1],
             (const T *)p.dv + b * p.sv[0] + h * p.sv[1], p.sv[2], wave, lane);
  auto issue_tile = [&](int it, int g) __attribute__((always_inline)) {
    const int k0 = walk_at(walk, t_first + it) * BN;
    kcopy.issue(k0, Nkv, smem + g * TK, 2 * TK);
    vcopy.issue(k0, Nkv, smem + VB + g * TV, 2 * TV);
  };
  auto issue_k = [&](int it, int g) __attribute__((always_inline)) {
    kcopy.issue(walk_at(walk, t_first + it) * BN, Nkv, smem + g * TK, 2 * TK);
  };
  auto issue_v = [&](int it, int g) __attribute__((always_inline)) {
    vcopy.issue(walk_at(walk, t_first + it) * BN, Nkv, smem + VB + g * TV, 2 * TV);
  };
  if (ntile > 0) issue_tile(0, 0);

  const int qrow = q0 + wave * kWaveRows + qi;
  const bool qvalid = qrow < Nq;

  // ---- Q, dQ fragments (B operands of S^T = K Q^T), resident ----
  FragK qf[DS], dqf[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    if (qvalid) {
      const int64_t off = (int64_t)qrow * p.sq[2] + s * KI + lg * KL;
      qf[s] = *(const FragK *)(Q + off);
      dqf[s] = *(const FragK *)(dQ + off);
    } else {
      qf[s] = FragK{};
      dqf[s] = FragK{};
    }
  }

  // O^T, A^T = (P~ dV)^T and B^T = ((P~ . dS) V)^T blocks (dS without the
  // scale, applied once in the epilogue): lane holds d = 16e + 4 lg + 0..3 of
  // query qi.  The row sums l (of P~) and r (of P~ . dS) are taken in fp32
  // before the bf16 rounding, lane-partial until the epilogue.
  f32x4 oacc[ND], aacc[ND], bacc[ND];
#pragma unroll
  for (int e = 0; e < ND; ++e) {
    oacc[e] = f32x4{};
    aacc[e] = f32x4{};
    bacc[e] = f32x4{};
  }
  float l_run = 0.f, r_run = 0.f;
  float m_run = -INFINITY;   // reference max, log2 units
  float s_thr = -INFINITY;   // raw score above which m_run must move

  const float scale = p.scale;
  const float c2 = p.scale_log2;

  // Query-side mask terms.  Chunks are runs of whole frames, so the keys
  // this lane's query sees by the chunk rule form one interval
  // [kv_lo, kv_hi); the anchor frames add [0, a_first_hi) and
  // [a_last_lo, N).  Keys in [win_lo, win_hi) and the anchor frames are
  // visible to every row of the block, so tiles inside them need no mask.
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
    // the rows of the whole block: chunks c0..c1
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

  // Lane-dependent parts of the LDS addresses, fixed for the whole loop.
  // Rows kb + 16 kb2 + qi (K operand) and kb + 16 u + 4 lg + qi / 4
  // (transpose reads of V) have the swizzle of their row mod 16, so adding
  // the step's row offset and the stage/tensor offset is a constant that goes
  // into the instructions' offset field.
  const uint32_t smem_a = lds_addr(smem);
  uint32_t kl[DS];                          // K operand, k-step s
#pragma unroll
  for (int s = 0; s < DS; ++s)
    kl[s] = smem_a + lds_off<RBK, KSK>(qi, (s * KI + lg * KL) * (int)sizeof(T));
  uint32_t vl[BF16 ? ND : 1];               // V transpose reads, d block e
  if constexpr (BF16) {
#pragma unroll
    for (int e = 0; e < ND; ++e)
      vl[e] = smem_a + VB + lds_off<RBV, kSwzV>(4 * lg + (qi >> 2), (16 * e + 4 * (qi & 3)) * 2);
  }

  // ---- S^T and dS^T of 32-key step KC of the tile in stage G ----
  // sacc[kb2][i] is the score of key kb + 16 kb2 + 4 lg + i for query qi
  auto scores = [&](auto G_, auto KC_, f32x4 (&sacc)[2], f32x4 (&dsacc)[2])
                    __attribute__((always_inline)) {
    constexpr int G = decltype(G_)::value;
    constexpr int kb = decltype(KC_)::value * CK;
    if constexpr (BF16 && DQK >= 32) {
      // slices j = (kb2, s), kb2-major, each a K and a dK read; PD slices in
      // flight (the wait before slice j leaves the later ones outstanding)
      constexpr int NP = 2 * DS;
      constexpr int PD0 = DQK >= 128 ? 3 : 2;
      constexpr int PD = PD0 < NP ? PD0 : NP;
      bf16x8 kf[NP], dkf[NP];
      auto issue = [&](auto j_) __attribute__((always_inline)) {
        constexpr int j = decltype(j_)::value;
        constexpr int kb2 = j / DS, s = j % DS;
        constexpr int OFF = G * TK + (kb + 16 * kb2) * RBK;
        kf[j] = lds_read_k<OFF>(kl[s]);
        dkf[j] = lds_read_k<OFF + 2 * TK>(kl[s]);
      };
      static_for<0, PD - 1>([&](auto j_) __attribute__((always_inline)) { issue(j_); });
      f32x4 s_[2] = {f32x4{}, f32x4{}}, ds_[2] = {f32x4{}, f32x4{}};
      static_for<0, NP>([&](auto j_) __attribute__((always_inline)) {
        constexpr int j = decltype(j_)::value;
        constexpr int kb2 = j / DS, s = j % DS;
        if constexpr (j + PD - 1 < NP) issue(std::integral_constant<int, j + PD - 1>{});
        constexpr int newer = (NP - 1 - j) < (PD - 1) ? (NP - 1 - j) : (PD - 1);
        lds_wait<2 * newer>();
        s_[kb2] = EK::mfma(kf[j], qf[s], s_[kb2]);
        ds_[kb2] = EK::mfma(kf[j], dqf[s], ds_[kb2]);
        ds_[kb2] = EK::mfma(dkf[j], qf[s], ds_[kb2]);
      });
      sacc[0] = s_[0];
      sacc[1] = s_[1];
      dsacc[0] = ds_[0];
      dsacc[1] = ds_[1];
    } else {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        f32x4 s_ = f32x4{}, ds_ = f32x4{};
#pragma unroll
        for (int s = 0; s < DS; ++s) {
          const char *kp = smem + (kl[s] - smem_a) + G * TK + (kb + 16 * kb2) * RBK;
          const FragK kf = *(const FragK *)kp;
          const FragK dkf = *(const FragK *)(kp + 2 * TK);
          s_ = EK::mfma(kf, qf[s], s_);
          ds_ = EK::mfma(kf, dqf[s], ds_);
          ds_ = EK::mfma(dkf, qf[s], ds_);
        }
        sacc[kb2] = s_;
        dsacc[kb2] = ds_;
      }
    }
  };

  // ---- element masks (key tail, partial frame-window tiles) ----
  // ka is the first key of the step.  Straight-line selects: the visibility
  // of every element is computed, with no per-lane branch.
  auto apply_mask = [&](int ka, f32x4 (&sacc)[2], f32x4 (&dsacc)[2])
                        __attribute__((always_inline)) {
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = ka + 16 * kb2 + 4 * lg + i;
        bool vis = key < Nkv;
        if constexpr (MASKED) {
          // bitwise, not short-circuit: no branch per element
          const bool in_chunks = (unsigned)(key - kv_lo) < (unsigned)(kv_hi - kv_lo);
          vis = vis & (in_chunks | (key < a_first_hi) | (key >= a_last_lo));
        }
        sacc[kb2][i] = vis ? sacc[kb2][i] : -INFINITY;
        dsacc[kb2][i] = vis ? dsacc[kb2][i] : 0.f;
      }
    }
  };

  // ---- running max (log2 domain) and lazy rescale of the accumulators ----
  // IEEE maximum (NaN-propagating): v_maximum3_f32, no canonicalisation
  constexpr bool kOverlap = BF16 && NSTEP == 2 && DQK + DV >= 256;
  // s_nop words between the 64-byte boundary and the key loop (see the
  // loop): the masked bf16 d = 128 loop measured best four words in
  // (long video 42.7 ms, against 44.8 at the boundary and 42.7-44.0 at the
  // other offsets), every other instance on the boundary
  //
  // At bf16 d = 64 the rescale and element-mask branches are also marked
  // unlikely, so that their blocks sit after the loop and a tile's common
  // path falls through; with the loop at its best offset for that layout
  // (two words in for the twelve-wave blocks, six for the small geometry)
  // text-to-image measured 1.5 % and the small geometry 0.8 % faster, while
  // the d = 128 loops gained nothing (within noise) and keep their layout.
  constexpr bool kHintRare = BF16 && DQK == 64 && DV == 64 && !MASKED;
  constexpr int kLoopPad = (MASKED && BF16 && DQK == 128 && DV == 128) ? 4
                           : kHintRare                                 ? (SMALL ? 6 : 2)
                                                                       : 0;
  constexpr bool kLaneCheck = !kOverlap && (W >= 8 || SMALL);   // two or more waves per SIMD
  auto update_max = [&](const f32x4 (&sacc)[2]) __attribute__((always_inline)) {
    // eight scores in a tree of three-input maxima
    auto mx3 = [](float a, float b, float c) __attribute__((always_inline)) {
      return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
    };
    const float t0 = mx3(sacc[0][0], sacc[0][1], sacc[0][2]);
    const float t1 = mx3(sacc[0][3], sacc[1][0], sacc[1][1]);
    const float lane_mx =
        __builtin_elementwise_maximum(mx3(sacc[1][2], sacc[1][3], t0), t1);
    // c2 > 0: lane_mx > s_thr iff lane_mx * c2 > m_run + threshold (up to
    // the rounding of s_thr, which only moves the decision by an ulp)
    if (!kLaneCheck || (kHintRare ? __builtin_expect(__any(lane_mx > s_thr), 0) : __any(lane_mx > s_thr))) {
      const float mx = row_max4(lane_mx) * c2;
      if ((kHintRare ? __builtin_expect(__any(mx > m_run + kRescaleThreshold), 0)
                     : __any(mx > m_run + kRescaleThreshold))) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
        r_run *= alpha;
#pragma unroll
        for (int e = 0; e < ND; ++e) {
          oacc[e] *= alpha;
          aacc[e] *= alpha;
          bacc[e] *= alpha;
        }
        m_run = m_new;
        s_thr = (m_run + kRescaleThreshold) / c2;
      }
    }
  };

  // ---- P~ = exp2(S - m) and H = P~ . dS (in place), row sums l and r ----
  auto softmax = [&](f32x4 (&sacc)[2], f32x4 (&dsacc)[2]) __attribute__((always_inline)) {
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[kb2][i], c2, -m_use));
        const float hv = pv * dsacc[kb2][i];
        l_run += pv;
        r_run += hv;
        sacc[kb2][i] = pv;
        dsacc[kb2][i] = hv;
      }
    }
  };

  // ---- O^T += V^T P^T ; A^T += dV^T P^T ; B^T += V^T H^T, step KC, stage G ----
  auto accumulate = [&](auto G_, auto KC_, const f32x4 (&sacc)[2], const f32x4 (&dsacc)[2])
                        __attribute__((always_inline)) {
    constexpr int G = decltype(G_)::value;
    constexpr int kb = decltype(KC_)::value * CK;
    if constexpr (BF16) {
      // B operand: lane (query qi, group lg) gives keys 4lg + 0..3 and
      // 16 + 4lg + 0..3 of the step, in that order
      bf16x8 pf, hf;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pf[i] = (__bf16)sacc[0][i];
        pf[4 + i] = (__bf16)sacc[1][i];
        hf[i] = (__bf16)dsacc[0][i];
        hf[4 + i] = (__bf16)dsacc[1][i];
      }
      // A operand for d block e: lane (d = 16e + qi, group lg) needs the same
      // keys of V and dV -- four transpose reads.  Groups e+1 and e+2 are in
      // flight while group e feeds its MFMAs.
      constexpr int VO = G * TV + kb * RBV;          // stage and step rows
      auto issue = [&](auto e_, i16x4 (&r)[4]) __attribute__((always_inline)) {
        constexpr int e = decltype(e_)::value;
        r[0] = lds_read_tr<VO>(vl[e]);
        r[1] = lds_read_tr<VO + 16 * RBV>(vl[e]);
        r[2] = lds_read_tr<VO + 2 * TV>(vl[e]);
        r[3] = lds_read_tr<VO + 2 * TV + 16 * RBV>(vl[e]);
      };
      i16x4 buf[3][4];
      issue(std::integral_constant<int, 0>{}, buf[0]);
      if constexpr (ND > 1) issue(std::integral_constant<int, 1>{}, buf[1]);
      static_for<0, ND>([&](auto e_) __attribute__((always_inline)) {
        constexpr int e = decltype(e_)::value;
        i16x4(&cur)[4] = buf[e % 3];
        if constexpr (e + 2 < ND) {
          issue(std::integral_constant<int, e + 2>{}, buf[(e + 2) % 3]);
          lds_wait<8>();
        } else if constexpr (e + 1 < ND) {
          lds_wait<4>();
        } else {
          lds_wait<0>();
        }
        const FragV vf = __builtin_bit_cast(FragV, __builtin_shufflevector(cur[0], cur[1], 0, 1, 2, 3, 4, 5, 6, 7));
        const FragV dvf = __builtin_bit_cast(FragV, __builtin_shufflevector(cur[2], cur[3], 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[e] = EV::mfma(vf, pf, oacc[e]);
        aacc[e] = EV::mfma(dvf, pf, aacc[e]);
        bacc[e] = EV::mfma(vf, hf, bacc[e]);
      });
    } else {
      // float32: k-step (kb2, i) takes key 16 kb2 + 4 lg + i from lane group lg
      const char *Vs = smem + VB + G * TV;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kb + 16 * kb2 + 4 * lg + i;
#pragma unroll
          for (int e = 0; e < ND; ++e) {
            const int o = lds_off<RBV, kSwzV>(key, (16 * e + qi) * 4);
            const FragV vf = *(const FragV *)(Vs + o);
            const FragV dvf = *(const FragV *)(Vs + 2 * TV + o);
            oacc[e] = EV::mfma(vf, sacc[kb2][i], oacc[e]);
            aacc[e] = EV::mfma(dvf, sacc[kb2][i], aacc[e]);
            bacc[e] = EV::mfma(vf, dsacc[kb2][i], bacc[e]);
          }
        }
    }
  };

  // Does the tile at key k0 need element masks?  Only the key tail, and in
  // the frame-window case a tile not wholly inside the block's common window
  // or an anchor frame.
  auto needs_mask = [&](int k0) __attribute__((always_inline)) {
    const int kz = k0 + BN;
    bool m = kz > Nkv;
    if constexpr (MASKED) {
      const bool in_win = k0 >= win_lo && kz <= win_hi;
      const bool in_first = p.mask.first && kz <= p.mask.tpf;
      const bool in_last = p.mask.last && k0 >= (p.mask.frames - 1) * p.mask.tpf;
      m = m || !(in_win || in_first || in_last);
    }
    return m;
  };

  // One tile in stage G: wait for it, release the other stage to the copy of
  // the next tile, then its steps.  With two steps a, b and the larger head
  // dims the order puts independent work side by side: the scores of b next
  // to the exponentials of a, the products of a next to the running max of
  // b; otherwise the plain order measures faster.  The element masks sit
  // behind a branch that is uniform over the tile, placed where the order
  // already ends a block.
  // In the overlapped schedule a wave issues its MFMA blocks at raised
  // priority: where both waves of a SIMD have an instruction ready, the one
  // feeding the matrix core goes first and the other's VALU and LDS work
  // fills the MFMAs' shadow (3-5 % at d = 128; at d = 64 and 32, with three
  // and two waves per SIMD and the plain order, it did not help).
  auto mfma_block = [&](auto &&body) __attribute__((always_inline)) {
    if constexpr (kOverlap) __builtin_amdgcn_s_setprio(1);
    body();
    if constexpr (kOverlap) __builtin_amdgcn_s_setprio(0);
  };
  auto tile = [&](auto G_, int it) __attribute__((always_inline)) {
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    const int k0 = walk_at(walk, t_first + it) * BN;
    const bool need = needs_mask(k0);
    wait_vmem();
    __syncthreads();   // tile `it` landed; every wave is done with tile it-1
    f32x4 sa[2], dsa[2];
    mfma_block([&]() __attribute__((always_inline)) { scores(G_, C0{}, sa, dsa); });
    // the next tile's copies go out behind MFMA work (K and dK after the
    // first scores, V and dV after the second step's scores where the order
    // overlaps), not at the barrier where every wave would issue them while
    // the matrix cores idle
    if (it + 1 < ntile) issue_k(it + 1, 1 - decltype(G_)::value);
    if constexpr (!kOverlap) {
      if (it + 1 < ntile) issue_v(it + 1, 1 - decltype(G_)::value);
    }
    if (kHintRare ? __builtin_expect(need, 0) : need) apply_mask(k0, sa, dsa);
    update_max(sa);
    if constexpr (NSTEP == 1) {
      softmax(sa, dsa);
      mfma_block([&]() __attribute__((always_inline)) { accumulate(G_, C0{}, sa, dsa); });
    } else {
      f32x4 sb[2], dsb[2];
      if constexpr (kOverlap) {
        mfma_block([&]() __attribute__((always_inline)) { scores(G_, C1{}, sb, dsb); });
        softmax(sa, dsa);
        // the exponentials of a are computed here, beside the scores of b,
        // not sunk past the mask branch below
        asm volatile("" ::"v"(sa[0]), "v"(sa[1]), "v"(dsa[0]), "v"(dsa[1]));
        if (it + 1 < ntile) issue_v(it + 1, 1 - decltype(G_)::value);
        if (kHintRare ? __builtin_expect(need, 0) : need) apply_mask(k0 + CK, sb, dsb);
        mfma_block([&]() __attribute__((always_inline)) { accumulate(G_, C0{}, sa, dsa); });
      } else {
        softmax(sa, dsa);
        mfma_block([&]() __attribute__((always_inline)) { accumulate(G_, C0{}, sa, dsa); });
        mfma_block([&]() __attribute__((always_inline)) { scores(G_, C1{}, sb, dsb); });
        if (kHintRare ? __builtin_expect(need, 0) : need) apply_mask(k0 + CK, sb, dsb);
      }
      update_max(sb);
      softmax(sb, dsb);
      mfma_block([&]() __attribute__((always_inline)) { accumulate(G_, C1{}, sb, dsb); });
    }
  };

  // The key loop's code starts kLoopPad 4-byte words past a 64-byte
  // boundary (the assembler pads with s_nop here, once per block).  Where
  // the same loop lands modulo 32 bytes moved the time of the 1 x 40 x 32760
  // d = 128 launch by up to 9 % (over the eight 4-byte offsets of this loop:
  // 47.3 to 52.7 ms; image-DiT 0.918 to 0.950 ms; text-to-image at d = 64
  // 0.768 to 0.781 ms) and that of the masked long-video launch by 5 %;
  // pinning it keeps that from changing with unrelated code ahead of the
  // loop, at the offset that measured best.  A change to the loop's own
  // code calls for measuring the offsets again.
  asm volatile(".p2align 6\n\t.rept %0\n\ts_nop 0\n\t.endr" ::"n"(kLoopPad));
  int it = 0;
  for (; it + 1 < ntile; it += 2) {
    tile(std::integral_constant<int, 0>{}, it);
    tile(std::integral_constant<int, 1>{}, it + 1);
  }
  if (it < ntile) tile(std::integral_constant<int, 0>{}, it);

  // ---- epilogue ----
  const float l_tot = row_sum4(l_run);
  const bool empty = !(l_tot > 0.f);
  const float inv = empty ? 0.f : 1.f / l_tot;
  const float mu = scale * row_sum4(r_run) * inv;   // dLSE
  const float sinv = scale * inv;
  if (qvalid && p.partial) {
    // float32 partial of this key split: O, dO [split, B, H, Lq, d_v] and
    // LSE, dLSE [split, B, H, Lq], contiguous
    const int64_t row = ((int64_t)split * p.B * p.H + bh) * Nq + qrow;
    float *O = (float *)p.o + row * DV;
    float *dO = (float *)p.dout + row * DV;
#pragma unroll
    for (int e = 0; e < ND; ++e) {
      const int d0 = 16 * e + 4 * lg;
      f32x4 ov, dv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ov[i] = oacc[e][i] * inv;
        dv[i] = fmaf(bacc[e][i], sinv, aacc[e][i] * inv) - mu * ov[i];
      }
      *(f32x4 *)(O + d0) = ov;
      *(f32x4 *)(dO + d0) = dv;
    }
    if (lg == 0) {
      p.lse[row] = empty ? -INFINITY : (m_run + log2f(l_tot)) * 0.69314718055994530942f;
      p.dlse[row] = mu;
    }
  } else if (kStageOut && !p.partial) {
    if constexpr (kStageOut) {
      char *ws = smem + C::kLds + wave * kOutWave;
      const int row0 = q0 + wave * kWaveRows;
      const int64_t stride = p.so[2] * (int64_t)sizeof(T);
      char *Ob = (char *)((T *)p.o + b * p.so[0] + h * p.so[1]) + row0 * stride;
      char *dOb = (char *)((T *)p.dout + b * p.so[0] + h * p.so[1]) + row0 * stride;
      typedef typename Stager::T4 T4;
      Stager::store(ws, lane, [&](int e) __attribute__((always_inline)) {
        T4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (T)(oacc[e][i] * inv);
        return v;
      }, Ob, stride, Nq - row0);
      Stager::store(ws, lane, [&](int e) __attribute__((always_inline)) {
        T4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float o = oacc[e][i] * inv;
          v[i] = (T)(fmaf(bacc[e][i], sinv, aacc[e][i] * inv) - mu * o);
        }
        return v;
      }, dOb, stride, Nq - row0);
      if (qvalid && lg == 0) {
        const int64_t ro = (int64_t)bh * Nq + qrow;
        p.lse[ro] = empty ? -INFINITY : (m_run + log2f(l_tot)) * 0.69314718055994530942f;
        p.dlse[ro] = mu;
      }
    }
  } else if (qvalid) {
    T *O = (T *)p.o + b * p.so[0] + h * p.so[1] + (int64_t)qrow * p.so[2];
    T *dO = (T *)p.dout + b * p.so[0] + h * p.so[1] + (int64_t)qrow * p.so[2];
    // each lane owns 4 consecutive d of its row per d block: one packed
    // 8-byte (bf16) or 16-byte (float32) store per block and tensor
    typedef T T4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int e = 0; e < ND; ++e) {
      const int d0 = 16 * e + 4 * lg;
      T4 ov, dv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float o = oacc[e][i] * inv;
        ov[i] = (T)o;
        dv[i] = (T)(fmaf(bacc[e][i], sinv, aacc[e][i] * inv) - mu * o);
      }
      *(T4 *)(O + d0) = ov;
      *(T4 *)(dO + d0) = dv;
    }
    if (lg == 0) {
      const int64_t ro = (int64_t)bh * Nq + qrow;
      p.lse[ro] = empty ? -INFINITY : (m_run + log2f(l_tot)) * 0.69314718055994530942f;
      p.dlse[ro] = mu;
    }
  }
}

// Launch one instance: grid = B * H * ceil(Nq / block_m) * nsplit workgroups.
template <typename T, int DQK, int DV, bool MASKED, bool SMALL = false>
hipError_t launch_instance(const Params &p, hipStream_t stream) {
  using C = Cfg<T, DQK, DV, SMALL>;
  const int grid = p.B * p.H * p.nqb * p.nsplit;
  hipLaunchKernelGGL((attn_jvp_kernel<T, DQK, DV, MASKED, SMALL>), dim3(grid), dim3(C::kThreads),
                     0, stream, p);
  return hipGetLastError();
}

}  // namespace attn_jvp
