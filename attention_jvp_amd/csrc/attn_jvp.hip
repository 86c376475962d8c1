// Host side of the attn_jvp C ABI: argument checks, launch shapes and
// dispatch to the kernel instances (kernel.h, instantiated per head dim in
// the inst_*.hip units).  The op contract (shape rules, tangents sharing the
// primals' strides, default scale d_qk^-1/2, outputs allocated by the
// caller, O and dO in the input dtype, LSE in float32) follows the page
// "带分数正则的一致性蒸馏" (gitcode.csdn.net), section 注意力, 前向 kernel.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include "attn_jvp.h"
#include "bwd.h"
#include "dispatch.h"

namespace attn_jvp {

namespace {
template <typename T, int DQK>
bool shape_dv(int dv, Shape *out) {
  switch (dv) {
    case 16: *out = shape_of<T, DQK, 16>(); return true;
    case 32: *out = shape_of<T, DQK, 32>(); return true;
    case 64: *out = shape_of<T, DQK, 64>(); return true;
    case 128: if (sizeof(T) == 2) { *out = shape_of<T, DQK, 128>(); return true; } return false;
    case 256: if (sizeof(T) == 2) { *out = shape_of<T, DQK, 256>(); return true; } return false;
    default: return false;
  }
}
}  // namespace

bool shape_for(bool bf16, int dqk, int dv, Shape *out) {
  if (bf16) {
    switch (dqk) {
      case 16: return shape_dv<__bf16, 16>(dv, out);
      case 32: return shape_dv<__bf16, 32>(dv, out);
      case 64: return shape_dv<__bf16, 64>(dv, out);
      case 128: return shape_dv<__bf16, 128>(dv, out);
      case 256: return shape_dv<__bf16, 256>(dv, out);
      default: return false;
    }
  }
  switch (dqk) {
    case 16: return shape_dv<float, 16>(dv, out);
    case 32: return shape_dv<float, 32>(dv, out);
    case 64: return shape_dv<float, 64>(dv, out);
    default: return false;
  }
}

}  // namespace attn_jvp

namespace {

using attn_jvp::MaskDev;
using attn_jvp::Params;
using attn_jvp::Shape;

struct Extent {
  uintptr_t lo, hi;
};

Extent extent_of(const void *ptr, const int64_t s[3], int B, int H, int N, int d,
                 int esize) {
  const int64_t last = (int64_t)(B - 1) * s[0] + (int64_t)(H - 1) * s[1] +
                       (int64_t)(N - 1) * s[2] + d;
  return Extent{(uintptr_t)ptr, (uintptr_t)ptr + (uintptr_t)(last * esize)};
}

bool overlaps(Extent a, Extent b) { return a.lo < b.hi && b.lo < a.hi; }

bool same3(const int64_t a[3], const int64_t b[3]) {
  return a[0] == b[0] && a[1] == b[1] && a[2] == b[2];
}

bool mask_on(const attn_jvp_mask *mask) {
  return mask != nullptr && mask->kind != ATTN_JVP_MASK_NONE;
}

// The frame window is a self-attention mask: queries and keys are the same
// frames * tokens_per_frame tokens.
int check_mask(const attn_jvp_mask *mask, int Nq, int Nkv) {
  if (!mask_on(mask)) return ATTN_JVP_OK;
  if (mask->kind != ATTN_JVP_MASK_FRAME_WINDOW) return ATTN_JVP_EMASK;
  if (mask->frames < 1 || mask->tokens_per_frame < 1 || mask->chunk_frames < 1 ||
      mask->radius_chunks < 0)
    return ATTN_JVP_EMASK;
  if (Nq != Nkv) return ATTN_JVP_EMASK;
  if ((int64_t)mask->frames * mask->tokens_per_frame != Nq) return ATTN_JVP_EMASK;
  if (Nq >= (1 << 24)) return ATTN_JVP_EMASK;   // frame arithmetic range
  return ATTN_JVP_OK;
}

MaskDev to_dev(const attn_jvp_mask *mask) {
  MaskDev m;
  memset(&m, 0, sizeof(m));
  if (!mask_on(mask)) return m;
  m.kind = 1;
  m.frames = mask->frames;
  m.tpf = mask->tokens_per_frame;
  m.chunk = mask->chunk_frames;
  // a radius of `frames` already reaches every chunk
  m.radius = mask->radius_chunks > mask->frames ? mask->frames : mask->radius_chunks;
  m.first = mask->anchor_first != 0;
  m.last = mask->anchor_last != 0;
  m.see_all = mask->anchor_queries_see_all != 0;
  m.inv_tpf = 1.0f / (float)m.tpf;
  m.inv_chunk = 1.0f / (float)m.chunk;
  return m;
}

// Contiguous [B, H, N, d] strides of every tensor of a shape.
attn_jvp_layout contiguous(const attn_jvp_shape &s) {
  attn_jvp_layout L;
  const int64_t nq = s.seqlen_q, nkv = s.seqlen_kv, dqk = s.head_dim_qk, dv = s.head_dim_v;
  const int64_t q[3] = {s.heads * nq * dqk, nq * dqk, dqk};
  const int64_t k[3] = {s.heads * nkv * dqk, nkv * dqk, dqk};
  const int64_t v[3] = {s.heads * nkv * dv, nkv * dv, dv};
  const int64_t o[3] = {s.heads * nq * dv, nq * dv, dv};
  for (int i = 0; i < 3; ++i) {
    L.q[i] = L.dq[i] = q[i];
    L.k[i] = L.dk[i] = k[i];
    L.v[i] = L.dv[i] = v[i];
    L.o[i] = L.dout[i] = o[i];
  }
  return L;
}

// out_esize: bytes per O / dO element (the dtype's, or 4 for float32
// partials); the o / dout strides of L are in those elements.
int check_args(const void *Q, const void *K, const void *V, const void *dQ,
               const void *dK, const void *dV, void *O, void *dO, float *LSE,
               float *dLSE, const attn_jvp_shape *shape, int dtype,
               const attn_jvp_layout *L, const attn_jvp_mask *mask, int out_esize = 0) {
  if (!Q || !K || !V || !dQ || !dK || !dV || !O || !dO || !LSE || !dLSE || !shape || !L)
    return ATTN_JVP_EINVAL;
  const int B = shape->batch, H = shape->heads, Nq = shape->seqlen_q, Nkv = shape->seqlen_kv;
  const int dqk = shape->head_dim_qk, dv = shape->head_dim_v;
  if (B <= 0 || H <= 0 || Nq <= 0 || Nkv <= 0 || dqk <= 0 || dv <= 0) return ATTN_JVP_EINVAL;
  if (dtype != ATTN_JVP_BF16 && dtype != ATTN_JVP_FP32) return ATTN_JVP_EINVAL;
  Shape sh;
  if (!attn_jvp::shape_for(dtype == ATTN_JVP_BF16, dqk, dv, &sh)) return ATTN_JVP_EUNSUPPORTED;
  if (mask_on(mask) && dqk != dv) return ATTN_JVP_EUNSUPPORTED;
  if ((int64_t)B * H * ((Nq + sh.block_m - 1) / sh.block_m) > 0x7fffffffLL) return ATTN_JVP_EINVAL;
  if (!same3(L->q, L->dq) || !same3(L->k, L->dk) || !same3(L->v, L->dv) ||
      !same3(L->o, L->dout))
    return ATTN_JVP_ESTRIDE;
  const int esize = dtype == ATTN_JVP_BF16 ? 2 : 4;
  const int oes = out_esize ? out_esize : esize;
  const int64_t *all[4] = {L->q, L->k, L->v, L->o};
  for (int i = 0; i < 4; ++i) {
    const int64_t align = 16 / (i == 3 ? oes : esize);
    for (int j = 0; j < 3; ++j)
      if (all[i][j] < 0 || all[i][j] % align != 0) return ATTN_JVP_ESTRIDE;
  }
  // key-tile offsets use 24-bit row strides (in bytes)
  if (L->k[2] * esize >= (1 << 24) || L->v[2] * esize >= (1 << 24)) return ATTN_JVP_ESTRIDE;
  const void *ptrs[8] = {Q, K, V, dQ, dK, dV, O, dO};
  for (int i = 0; i < 8; ++i)
    if ((uintptr_t)ptrs[i] % 16 != 0) return ATTN_JVP_ESTRIDE;
  if ((uintptr_t)LSE % 4 != 0 || (uintptr_t)dLSE % 4 != 0) return ATTN_JVP_ESTRIDE;
  // outputs must not overlap inputs or each other
  const Extent in[6] = {
      extent_of(Q, L->q, B, H, Nq, dqk, esize),   extent_of(K, L->k, B, H, Nkv, dqk, esize),
      extent_of(V, L->v, B, H, Nkv, dv, esize),   extent_of(dQ, L->q, B, H, Nq, dqk, esize),
      extent_of(dK, L->k, B, H, Nkv, dqk, esize), extent_of(dV, L->v, B, H, Nkv, dv, esize)};
  const int64_t rows = (int64_t)B * H * Nq;
  const Extent out[4] = {extent_of(O, L->o, B, H, Nq, dv, oes),
                         extent_of(dO, L->o, B, H, Nq, dv, oes),
                         Extent{(uintptr_t)LSE, (uintptr_t)LSE + (uintptr_t)(rows * 4)},
                         Extent{(uintptr_t)dLSE, (uintptr_t)dLSE + (uintptr_t)(rows * 4)}};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(out[i], in[j])) return ATTN_JVP_ESTRIDE;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(out[i], out[j])) return ATTN_JVP_ESTRIDE;
  }
  return check_mask(mask, Nq, Nkv);
}

hipError_t dispatch(const Params &p, int dtype, int dqk, int dv, bool masked, hipStream_t s) {
  if (dtype == ATTN_JVP_FP32) return attn_jvp::launch_fp32(p, dqk, dv, masked, s);
  switch (dqk) {
    case 16: return attn_jvp::launch_bf16_qk16(p, dv, masked, s);
    case 32: return attn_jvp::launch_bf16_qk32(p, dv, masked, s);
    case 64: return attn_jvp::launch_bf16_qk64(p, dv, masked, s);
    case 128: return attn_jvp::launch_bf16_qk128(p, dv, masked, s);
    case 256: return attn_jvp::launch_bf16_qk256(p, dv, masked, s);
    default: return hipErrorInvalidValue;
  }
}

Params make_params(const void *Q, const void *K, const void *V, const void *dQ,
                   const void *dK, const void *dV, void *O, void *dO, float *LSE,
                   float *dLSE, const attn_jvp_shape &shape, float scale, int dtype,
                   const attn_jvp_layout &L, const attn_jvp_mask *mask) {
  Shape sh;
  attn_jvp::shape_for(dtype == ATTN_JVP_BF16, shape.head_dim_qk, shape.head_dim_v, &sh);
  Params p;
  memset(&p, 0, sizeof(p));
  p.q = Q; p.k = K; p.v = V; p.dq = dQ; p.dk = dK; p.dv = dV;
  p.o = O; p.dout = dO; p.lse = LSE; p.dlse = dLSE;
  for (int i = 0; i < 3; ++i) {
    p.sq[i] = L.q[i];
    p.sk[i] = L.k[i];
    p.sv[i] = L.v[i];
    p.so[i] = L.o[i];
  }
  p.B = shape.batch;
  p.H = shape.heads;
  p.Nq = shape.seqlen_q;
  p.Nkv = shape.seqlen_kv;
  p.nqb = (p.Nq + sh.block_m - 1) / sh.block_m;
  p.nsplit = 1;
  p.partial = 0;
  p.scale = (scale > 0.f && isfinite(scale)) ? scale : 1.0f / sqrtf((float)shape.head_dim_qk);
  p.scale_log2 = p.scale * 1.4426950408889634f;
  p.mask = to_dev(mask);
  return p;
}

// float32 partial outputs of a call: contiguous [B, H, Lq, d_v] in floats
void partial_out_strides(const attn_jvp_shape &s, attn_jvp_layout *L) {
  const int64_t o[3] = {(int64_t)s.heads * s.seqlen_q * s.head_dim_v,
                        (int64_t)s.seqlen_q * s.head_dim_v, (int64_t)s.head_dim_v};
  for (int i = 0; i < 3; ++i) L->o[i] = L->dout[i] = o[i];
}

// Split-KV workspace: O, dO partials [ns, B, H, Lq, d_v] then LSE, dLSE
// partials [ns, B, H, Lq], float32, each region 256-byte aligned.
struct SplitWs {
  size_t o, dout, lse, dlse, total;
};

SplitWs split_workspace(const attn_jvp_shape &s, int ns) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t rows = (size_t)ns * s.batch * s.heads * s.seqlen_q;
  SplitWs w;
  w.o = 0;
  w.dout = up(rows * s.head_dim_v * 4);
  w.lse = w.dout + up(rows * s.head_dim_v * 4);
  w.dlse = w.lse + up(rows * 4);
  w.total = w.dlse + up(rows * 4);
  return w;
}

// Key splits for one call: enough workgroups to fill the chip about twice
// over (more splits only add partial traffic for the merge), each split
// keeping at least two key tiles, at most 64.
int choose_splits(const attn_jvp_shape &s, int dtype, const attn_jvp_mask *mask) {
  Shape sh;
  if (!attn_jvp::shape_for(dtype == ATTN_JVP_BF16, s.head_dim_qk, s.head_dim_v, &sh)) return 1;
  const int64_t nqb = (s.seqlen_q + sh.block_m - 1) / sh.block_m;
  const int64_t wgs = (int64_t)s.batch * s.heads * nqb;
  int64_t tiles = (s.seqlen_kv + sh.block_n - 1) / sh.block_n;
  if (mask_on(mask) && check_mask(mask, s.seqlen_q, s.seqlen_kv) == ATTN_JVP_OK) {
    const MaskDev m = to_dev(mask);
    int64_t mx = 0;
    for (int64_t qb = 0; qb < nqb; ++qb) {
      const int q0 = (int)(qb * sh.block_m);
      const int q1 = q0 + sh.block_m < s.seqlen_q ? q0 + sh.block_m : s.seqlen_q;
      const attn_jvp::TileRanges tr = attn_jvp::visible_tiles(m, q0, q1, s.seqlen_kv, sh.block_n);
      int64_t c = 0;
      for (int i = 0; i < tr.n; ++i) c += tr.hi[i] - tr.lo[i];
      mx = c > mx ? c : mx;
    }
    tiles = mx;
  }
  const int64_t target = 2 * 256;
  if (wgs >= target / 2) return 1;
  int64_t ns = (target + wgs - 1) / wgs;
  const int64_t cap = tiles / 2 > 1 ? tiles / 2 : 1;
  ns = ns < cap ? ns : cap;
  return (int)(ns < 64 ? ns : 64);
}

attn_jvp_bwd_layout contiguous_bwd(const attn_jvp_shape &s) {
  const attn_jvp_layout f = contiguous(s);
  attn_jvp_bwd_layout L;
  for (int i = 0; i < 3; ++i) {
    L.q[i] = L.gq[i] = f.q[i];
    L.k[i] = L.gk[i] = f.k[i];
    L.v[i] = L.gv[i] = f.v[i];
    L.o[i] = L.go[i] = f.o[i];
  }
  return L;
}

int check_bwd(const void *Q, const void *K, const void *V, const void *O, const void *gO,
              const float *LSE, void *gQ, void *gK, void *gV, float *delta,
              const attn_jvp_shape *shape, int dtype, const attn_jvp_bwd_layout *L,
              const attn_jvp_mask *mask) {
  if (!Q || !K || !V || !O || !gO || !LSE || !gQ || !gK || !gV || !delta || !shape || !L)
    return ATTN_JVP_EINVAL;
  const int B = shape->batch, H = shape->heads, Nq = shape->seqlen_q, Nkv = shape->seqlen_kv;
  const int d = shape->head_dim_qk;
  if (B <= 0 || H <= 0 || Nq <= 0 || Nkv <= 0 || d <= 0 || shape->head_dim_v <= 0)
    return ATTN_JVP_EINVAL;
  if (dtype != ATTN_JVP_BF16 && dtype != ATTN_JVP_FP32) return ATTN_JVP_EINVAL;
  if (shape->head_dim_v != d) return ATTN_JVP_EUNSUPPORTED;   // the pages: one head dim
  int bq, bk, rbq_max, rbk_max;
  if (!attn_jvp::bwd_shape_for(dtype == ATTN_JVP_BF16, d, &bq, &bk, &rbq_max, &rbk_max))
    return ATTN_JVP_EUNSUPPORTED;
  if ((int64_t)B * H * ((Nq + bq - 1) / bq) > 0x7fffffffLL ||
      (int64_t)B * H * ((Nkv + bk - 1) / bk) > 0x7fffffffLL)
    return ATTN_JVP_EINVAL;
  const int esize = dtype == ATTN_JVP_BF16 ? 2 : 4;
  const int64_t align = 16 / esize;
  const int64_t *all[8] = {L->q, L->k, L->v, L->o, L->go, L->gq, L->gk, L->gv};
  for (int i = 0; i < 8; ++i)
    for (int j = 0; j < 3; ++j)
      if (all[i][j] < 0 || all[i][j] % align != 0) return ATTN_JVP_ESTRIDE;
  // streamed tiles use 24-bit row strides (in bytes)
  const int64_t *streamed[4] = {L->q, L->k, L->v, L->go};
  for (int i = 0; i < 4; ++i)
    if (streamed[i][2] * esize >= (1 << 24)) return ATTN_JVP_ESTRIDE;
  const void *ptrs[8] = {Q, K, V, O, gO, gQ, gK, gV};
  for (int i = 0; i < 8; ++i)
    if ((uintptr_t)ptrs[i] % 16 != 0) return ATTN_JVP_ESTRIDE;
  if ((uintptr_t)LSE % 4 != 0 || (uintptr_t)delta % 4 != 0) return ATTN_JVP_ESTRIDE;
  const int64_t rows = (int64_t)B * H * Nq;
  const Extent in[6] = {extent_of(Q, L->q, B, H, Nq, d, esize),
                        extent_of(K, L->k, B, H, Nkv, d, esize),
                        extent_of(V, L->v, B, H, Nkv, d, esize),
                        extent_of(O, L->o, B, H, Nq, d, esize),
                        extent_of(gO, L->go, B, H, Nq, d, esize),
                        {(uintptr_t)LSE, (uintptr_t)LSE + (uintptr_t)(rows * 4)}};
  const Extent out[4] = {extent_of(gQ, L->gq, B, H, Nq, d, esize),
                         extent_of(gK, L->gk, B, H, Nkv, d, esize),
                         extent_of(gV, L->gv, B, H, Nkv, d, esize),
                         {(uintptr_t)delta, (uintptr_t)delta + (uintptr_t)(rows * 4)}};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(out[i], in[j])) return ATTN_JVP_ESTRIDE;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(out[i], out[j])) return ATTN_JVP_ESTRIDE;
  }
  return check_mask(mask, Nq, Nkv);
}

attn_jvp_shape square(int B, int H, int N, int d) {
  attn_jvp_shape s;
  s.batch = B;
  s.heads = H;
  s.seqlen_q = s.seqlen_kv = N;
  s.head_dim_qk = s.head_dim_v = d;
  return s;
}

}  // namespace

extern "C" {

int attn_jvp_check_ex(const void *Q, const void *K, const void *V, const void *dQ,
                      const void *dK, const void *dV, void *O, void *dO, float *LSE,
                      float *dLSE, const attn_jvp_shape *shape, int dtype,
                      const attn_jvp_layout *layout, const attn_jvp_mask *mask) {
  if (!shape) return ATTN_JVP_EINVAL;
  const attn_jvp_layout L = layout ? *layout : contiguous(*shape);
  return check_args(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE, shape, dtype, &L, mask);
}

int attn_jvp_fwd_ex(const void *Q, const void *K, const void *V, const void *dQ,
                    const void *dK, const void *dV, void *O, void *dO, float *LSE,
                    float *dLSE, const attn_jvp_shape *shape, float scale, int dtype,
                    const attn_jvp_layout *layout, const attn_jvp_mask *mask,
                    void *stream) {
  if (!shape) return ATTN_JVP_EINVAL;
  const attn_jvp_layout L = layout ? *layout : contiguous(*shape);
  const int st = check_args(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE, shape, dtype, &L, mask);
  if (st != ATTN_JVP_OK) return st;
  const Params p = make_params(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE, *shape, scale, dtype, L,
                               mask);
  const hipError_t err = dispatch(p, dtype, shape->head_dim_qk, shape->head_dim_v,
                                  mask_on(mask), (hipStream_t)stream);
  return err == hipSuccess ? ATTN_JVP_OK : ATTN_JVP_EHIP;
}

int attn_jvp_fwd_partial(const void *Q, const void *K, const void *V, const void *dQ,
                         const void *dK, const void *dV, float *O, float *dO, float *LSE,
                         float *dLSE, const attn_jvp_shape *shape, float scale, int dtype,
                         const attn_jvp_layout *layout, void *stream) {
  if (!shape) return ATTN_JVP_EINVAL;
  attn_jvp_layout L = layout ? *layout : contiguous(*shape);
  partial_out_strides(*shape, &L);
  const int st = check_args(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE, shape, dtype, &L, nullptr, 4);
  if (st != ATTN_JVP_OK) return st;
  Params p = make_params(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE, *shape, scale, dtype, L, nullptr);
  p.partial = 1;
  const hipError_t err = dispatch(p, dtype, shape->head_dim_qk, shape->head_dim_v, false,
                                  (hipStream_t)stream);
  return err == hipSuccess ? ATTN_JVP_OK : ATTN_JVP_EHIP;
}

int attn_jvp_merge(int num_parts, const float *O_parts, const float *dO_parts,
                   const float *LSE_parts, const float *dLSE_parts, void *O, void *dO,
                   float *LSE, float *dLSE, int B, int H, int Lq, int d_v, int dtype,
                   const int64_t *o_strides, void *stream) {
  if (!O_parts || !dO_parts || !LSE_parts || !dLSE_parts || !O || !dO || !LSE || !dLSE)
    return ATTN_JVP_EINVAL;
  if (num_parts < 1 || B <= 0 || H <= 0 || Lq <= 0 || d_v <= 0) return ATTN_JVP_EINVAL;
  if (dtype != ATTN_JVP_BF16 && dtype != ATTN_JVP_FP32) return ATTN_JVP_EINVAL;
  if (d_v % 4 != 0) return ATTN_JVP_EUNSUPPORTED;
  const int esize = dtype == ATTN_JVP_BF16 ? 2 : 4;
  const int64_t rows = (int64_t)B * H * Lq;
  if (rows * (d_v / 4) / 256 > 0x7fffffffLL) return ATTN_JVP_EINVAL;
  const int64_t so[3] = {o_strides ? o_strides[0] : (int64_t)H * Lq * d_v,
                         o_strides ? o_strides[1] : (int64_t)Lq * d_v,
                         o_strides ? o_strides[2] : (int64_t)d_v};
  for (int j = 0; j < 3; ++j)
    if (so[j] < 0 || so[j] % 4 != 0) return ATTN_JVP_ESTRIDE;   // 4-wide stores
  if ((uintptr_t)O_parts % 16 || (uintptr_t)dO_parts % 16 || (uintptr_t)O % (4 * esize) ||
      (uintptr_t)dO % (4 * esize) || (uintptr_t)LSE_parts % 4 || (uintptr_t)dLSE_parts % 4 ||
      (uintptr_t)LSE % 4 || (uintptr_t)dLSE % 4)
    return ATTN_JVP_ESTRIDE;
  const uintptr_t pe = (uintptr_t)(num_parts * rows * d_v * 4);
  const uintptr_t le = (uintptr_t)(num_parts * rows * 4);
  const Extent in[4] = {{(uintptr_t)O_parts, (uintptr_t)O_parts + pe},
                        {(uintptr_t)dO_parts, (uintptr_t)dO_parts + pe},
                        {(uintptr_t)LSE_parts, (uintptr_t)LSE_parts + le},
                        {(uintptr_t)dLSE_parts, (uintptr_t)dLSE_parts + le}};
  const Extent out[4] = {extent_of(O, so, B, H, Lq, d_v, esize),
                         extent_of(dO, so, B, H, Lq, d_v, esize),
                         {(uintptr_t)LSE, (uintptr_t)LSE + (uintptr_t)(rows * 4)},
                         {(uintptr_t)dLSE, (uintptr_t)dLSE + (uintptr_t)(rows * 4)}};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 4; ++j)
      if (overlaps(out[i], in[j])) return ATTN_JVP_ESTRIDE;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(out[i], out[j])) return ATTN_JVP_ESTRIDE;
  }
  attn_jvp::MergeParams m;
  m.o_parts = O_parts; m.do_parts = dO_parts; m.lse_parts = LSE_parts; m.dlse_parts = dLSE_parts;
  m.o = O; m.dout = dO; m.lse = LSE; m.dlse = dLSE;
  for (int j = 0; j < 3; ++j) m.so[j] = so[j];
  m.parts = num_parts; m.B = B; m.H = H; m.Nq = Lq; m.dv = d_v;
  const hipError_t err = attn_jvp::launch_merge(m, dtype == ATTN_JVP_BF16, (hipStream_t)stream);
  return err == hipSuccess ? ATTN_JVP_OK : ATTN_JVP_EHIP;
}

int attn_jvp_splitkv_plan(const attn_jvp_shape *shape, int dtype, const attn_jvp_mask *mask,
                          int *num_splits, size_t *workspace_bytes) {
  if (!shape || !num_splits || !workspace_bytes) return ATTN_JVP_EINVAL;
  if (shape->batch <= 0 || shape->heads <= 0 || shape->seqlen_q <= 0 || shape->seqlen_kv <= 0)
    return ATTN_JVP_EINVAL;
  if (dtype != ATTN_JVP_BF16 && dtype != ATTN_JVP_FP32) return ATTN_JVP_EINVAL;
  Shape sh;
  if (!attn_jvp::shape_for(dtype == ATTN_JVP_BF16, shape->head_dim_qk, shape->head_dim_v, &sh))
    return ATTN_JVP_EUNSUPPORTED;
  if (*num_splits < 0 || *num_splits > 1024) return ATTN_JVP_EINVAL;
  const int ns = *num_splits ? *num_splits : choose_splits(*shape, dtype, mask);
  *num_splits = ns;
  *workspace_bytes = ns > 1 ? split_workspace(*shape, ns).total : 0;
  return ATTN_JVP_OK;
}

int attn_jvp_fwd_splitkv(const void *Q, const void *K, const void *V, const void *dQ,
                         const void *dK, const void *dV, void *O, void *dO, float *LSE,
                         float *dLSE, const attn_jvp_shape *shape, float scale, int dtype,
                         const attn_jvp_layout *layout, const attn_jvp_mask *mask,
                         int num_splits, void *workspace, size_t workspace_bytes,
                         void *stream) {
  if (!shape) return ATTN_JVP_EINVAL;
  int ns = num_splits;
  size_t need = 0;
  int st = attn_jvp_splitkv_plan(shape, dtype, mask, &ns, &need);
  if (st != ATTN_JVP_OK) return st;
  if (ns == 1)
    return attn_jvp_fwd_ex(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE, shape, scale, dtype, layout,
                           mask, stream);
  const attn_jvp_layout L = layout ? *layout : contiguous(*shape);
  st = check_args(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE, shape, dtype, &L, mask);
  if (st != ATTN_JVP_OK) return st;
  if (!workspace || (uintptr_t)workspace % 256 != 0) return ATTN_JVP_EINVAL;
  if (workspace_bytes < need) return ATTN_JVP_EINVAL;
  Shape sh;
  attn_jvp::shape_for(dtype == ATTN_JVP_BF16, shape->head_dim_qk, shape->head_dim_v, &sh);
  const int64_t nqb = (shape->seqlen_q + sh.block_m - 1) / sh.block_m;
  if ((int64_t)shape->batch * shape->heads * nqb * ns > 0x7fffffffLL) return ATTN_JVP_EINVAL;
  // the workspace must not overlap the call's tensors
  const Extent ws{(uintptr_t)workspace, (uintptr_t)workspace + need};
  const int esize = dtype == ATTN_JVP_BF16 ? 2 : 4;
  const int B = shape->batch, H = shape->heads, Nq = shape->seqlen_q, Nkv = shape->seqlen_kv;
  const int dqk = shape->head_dim_qk, dv = shape->head_dim_v;
  const Extent all[10] = {
      extent_of(Q, L.q, B, H, Nq, dqk, esize),   extent_of(K, L.k, B, H, Nkv, dqk, esize),
      extent_of(V, L.v, B, H, Nkv, dv, esize),   extent_of(dQ, L.q, B, H, Nq, dqk, esize),
      extent_of(dK, L.k, B, H, Nkv, dqk, esize), extent_of(dV, L.v, B, H, Nkv, dv, esize),
      extent_of(O, L.o, B, H, Nq, dv, esize),    extent_of(dO, L.o, B, H, Nq, dv, esize),
      {(uintptr_t)LSE, (uintptr_t)LSE + (uintptr_t)((int64_t)B * H * Nq * 4)},
      {(uintptr_t)dLSE, (uintptr_t)dLSE + (uintptr_t)((int64_t)B * H * Nq * 4)}};
  for (int i = 0; i < 10; ++i)
    if (overlaps(ws, all[i])) return ATTN_JVP_ESTRIDE;

  const SplitWs w = split_workspace(*shape, ns);
  char *base = (char *)workspace;
  float *op = (float *)(base + w.o), *dop = (float *)(base + w.dout);
  float *lp = (float *)(base + w.lse), *dlp = (float *)(base + w.dlse);
  Params p = make_params(Q, K, V, dQ, dK, dV, op, dop, lp, dlp, *shape, scale, dtype, L, mask);
  p.partial = 1;
  p.nsplit = ns;
  hipError_t err = dispatch(p, dtype, dqk, dv, mask_on(mask), (hipStream_t)stream);
  if (err != hipSuccess) return ATTN_JVP_EHIP;
  attn_jvp::MergeParams m;
  m.o_parts = op; m.do_parts = dop; m.lse_parts = lp; m.dlse_parts = dlp;
  m.o = O; m.dout = dO; m.lse = LSE; m.dlse = dLSE;
  for (int j = 0; j < 3; ++j) m.so[j] = L.o[j];
  m.parts = ns; m.B = B; m.H = H; m.Nq = Nq; m.dv = dv;
  err = attn_jvp::launch_merge(m, dtype == ATTN_JVP_BF16, (hipStream_t)stream);
  return err == hipSuccess ? ATTN_JVP_OK : ATTN_JVP_EHIP;
}

int attn_jvp_bwd_check(const void *Q, const void *K, const void *V, const void *O,
                       const void *gO, const float *LSE, void *gQ, void *gK, void *gV,
                       float *delta, const attn_jvp_shape *shape, int dtype,
                       const attn_jvp_bwd_layout *layout, const attn_jvp_mask *mask) {
  if (!shape) return ATTN_JVP_EINVAL;
  const attn_jvp_bwd_layout L = layout ? *layout : contiguous_bwd(*shape);
  return check_bwd(Q, K, V, O, gO, LSE, gQ, gK, gV, delta, shape, dtype, &L, mask);
}

int attn_jvp_bwd(const void *Q, const void *K, const void *V, const void *O, const void *gO,
                 const float *LSE, void *gQ, void *gK, void *gV, float *delta,
                 const attn_jvp_shape *shape, float scale, int dtype,
                 const attn_jvp_bwd_layout *layout, const attn_jvp_mask *mask,
                 void *stream) {
  if (!shape) return ATTN_JVP_EINVAL;
  const attn_jvp_bwd_layout L = layout ? *layout : contiguous_bwd(*shape);
  const int st = check_bwd(Q, K, V, O, gO, LSE, gQ, gK, gV, delta, shape, dtype, &L, mask);
  if (st != ATTN_JVP_OK) return st;
  int bq, bk, rbq_max, rbk_max;
  attn_jvp::bwd_shape_for(dtype == ATTN_JVP_BF16, shape->head_dim_qk, &bq, &bk, &rbq_max,
                          &rbk_max);
  // two row blocks per wave halve a launch's LDS traffic per MFMA but also
  // its workgroups: taken while at least two rounds of workgroups (512 on
  // 256 CUs) remain
  const int64_t bh = (int64_t)shape->batch * shape->heads;
  const int rbq =
      (rbq_max >= 2 && bh * ((shape->seqlen_q + 2 * bq - 1) / (2 * bq)) >= 512) ? 2 : 1;
  const int rbk =
      (rbk_max >= 2 && bh * ((shape->seqlen_kv + 2 * bk - 1) / (2 * bk)) >= 512) ? 2 : 1;
  attn_jvp::BwdParams p;
  memset(&p, 0, sizeof(p));
  p.q = Q; p.k = K; p.v = V; p.o = O; p.g = gO; p.lse = LSE;
  p.gq = gQ; p.gk = gK; p.gv = gV; p.delta = delta;
  for (int i = 0; i < 3; ++i) {
    p.sq[i] = L.q[i]; p.sk[i] = L.k[i]; p.sv[i] = L.v[i]; p.so[i] = L.o[i];
    p.sg[i] = L.go[i]; p.sgq[i] = L.gq[i]; p.sgk[i] = L.gk[i]; p.sgv[i] = L.gv[i];
  }
  p.B = shape->batch;
  p.H = shape->heads;
  p.Nq = shape->seqlen_q;
  p.Nkv = shape->seqlen_kv;
  p.rbq = rbq;
  p.rbk = rbk;
  p.nqb = (p.Nq + rbq * bq - 1) / (rbq * bq);
  p.nkb = (p.Nkv + rbk * bk - 1) / (rbk * bk);
  p.scale = (scale > 0.f && isfinite(scale)) ? scale : 1.0f / sqrtf((float)shape->head_dim_qk);
  p.scale_log2 = p.scale * 1.4426950408889634f;
  p.mask = to_dev(mask);
  const hipError_t err = attn_jvp::launch_bwd(p, dtype == ATTN_JVP_BF16, shape->head_dim_qk,
                                              (hipStream_t)stream);
  return err == hipSuccess ? ATTN_JVP_OK : ATTN_JVP_EHIP;
}

int attn_jvp_check(const void *Q, const void *K, const void *V, const void *dQ,
                   const void *dK, const void *dV, void *O, void *dO, float *LSE,
                   float *dLSE, int B, int H, int N, int d, int dtype,
                   const attn_jvp_layout *layout, const attn_jvp_mask *mask) {
  if (!layout) return ATTN_JVP_EINVAL;
  const attn_jvp_shape s = square(B, H, N, d);
  return check_args(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE, &s, dtype, layout, mask);
}

int attn_jvp_fwd_strided(const void *Q, const void *K, const void *V,
                         const void *dQ, const void *dK, const void *dV, void *O,
                         void *dO, float *LSE, float *dLSE, int B, int H, int N,
                         int d, float scale, int dtype,
                         const attn_jvp_layout *layout, const attn_jvp_mask *mask,
                         void *stream) {
  if (!layout) return ATTN_JVP_EINVAL;
  const attn_jvp_shape s = square(B, H, N, d);
  return attn_jvp_fwd_ex(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE, &s, scale, dtype, layout,
                         mask, stream);
}

int attn_jvp_fwd(const void *Q, const void *K, const void *V, const void *dQ,
                 const void *dK, const void *dV, void *O, void *dO, float *LSE,
                 float *dLSE, int B, int H, int N, int d, float scale, int dtype,
                 const attn_jvp_mask *mask, void *stream) {
  const attn_jvp_shape s = square(B, H, N, d);
  return attn_jvp_fwd_ex(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE, &s, scale, dtype, nullptr,
                         mask, stream);
}

int attn_jvp_tile_shape_ex(int dtype, int d_qk, int d_v, int *block_m, int *block_n) {
  if (!block_m || !block_n) return ATTN_JVP_EINVAL;
  if (dtype != ATTN_JVP_BF16 && dtype != ATTN_JVP_FP32) return ATTN_JVP_EINVAL;
  Shape sh;
  if (!attn_jvp::shape_for(dtype == ATTN_JVP_BF16, d_qk, d_v, &sh)) return ATTN_JVP_EUNSUPPORTED;
  *block_m = sh.block_m;
  *block_n = sh.block_n;
  return ATTN_JVP_OK;
}

int attn_jvp_tile_shape(int dtype, int d, int *block_m, int *block_n) {
  return attn_jvp_tile_shape_ex(dtype, d, d, block_m, block_n);
}

int attn_jvp_visible_tiles(int N, int dtype, int d, const attn_jvp_mask *mask,
                           int64_t *tiles_per_block) {
  int bm, bn;
  const int st = attn_jvp_tile_shape(dtype, d, &bm, &bn);
  if (st != ATTN_JVP_OK) return st;
  if (N <= 0 || !tiles_per_block) return ATTN_JVP_EINVAL;
  const int mst = check_mask(mask, N, N);
  if (mst != ATTN_JVP_OK) return mst;
  const MaskDev m = to_dev(mask);
  const int nqb = (N + bm - 1) / bm;
  for (int qb = 0; qb < nqb; ++qb) {
    const int q0 = qb * bm;
    const int q1 = q0 + bm < N ? q0 + bm : N;
    const attn_jvp::TileRanges tr = attn_jvp::visible_tiles(m, q0, q1, N, bn);
    int64_t c = 0;
    for (int i = 0; i < tr.n; ++i) c += tr.hi[i] - tr.lo[i];
    tiles_per_block[qb] = c;
  }
  return ATTN_JVP_OK;
}

int attn_jvp_bwd_visible_tiles(int N, int block_rows, int tile_rows, int keys,
                               const attn_jvp_mask *mask, int64_t *tiles_per_block) {
  if (N <= 0 || block_rows <= 0 || tile_rows <= 0 || !tiles_per_block) return ATTN_JVP_EINVAL;
  const int mst = check_mask(mask, N, N);
  if (mst != ATTN_JVP_OK) return mst;
  const MaskDev m = to_dev(mask);
  const int nb = (N + block_rows - 1) / block_rows;
  for (int b = 0; b < nb; ++b) {
    const int r0 = b * block_rows;
    const int r1 = r0 + block_rows < N ? r0 + block_rows : N;
    const attn_jvp::TileRanges tr = keys ? attn_jvp::visible_query_tiles(m, r0, r1, N, tile_rows)
                                         : attn_jvp::visible_tiles(m, r0, r1, N, tile_rows);
    int64_t c = 0;
    for (int i = 0; i < tr.n; ++i) c += tr.hi[i] - tr.lo[i];
    tiles_per_block[b] = c;
  }
  return ATTN_JVP_OK;
}

const char *attn_jvp_status_string(int status) {
  switch (status) {
    case ATTN_JVP_OK: return "ok";
    case ATTN_JVP_EINVAL: return "invalid argument (null pointer, size or dtype)";
    case ATTN_JVP_EUNSUPPORTED: return "unsupported head dimensions for this dtype";
    case ATTN_JVP_ESTRIDE:
      return "bad layout (tangent strides differ from the primal's, misaligned "
             "pointer or stride, or outputs overlapping inputs)";
    case ATTN_JVP_EMASK: return "inconsistent mask descriptor";
    case ATTN_JVP_EHIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}

}  // extern "C"
