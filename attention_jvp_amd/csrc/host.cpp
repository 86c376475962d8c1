// Host side of the attn_jvp C ABI without the HIP runtime: argument checks,
// launch shapes, split planning and the entry points that launch nothing.
// The op contract (shape rules, tangents sharing the primals' strides,
// default scale d_qk^-1/2, outputs allocated by the caller, O and dO in the
// input dtype, LSE in float32) follows the page "带分数正则的一致性蒸馏"
// (gitcode.csdn.net), section 注意力, 前向 kernel; the backward's (dQ, dK, dV
// from the saved log-sum-exp) its subsection 反向.

#include "host.h"

#include <math.h>
#include <string.h>

namespace attn_jvp {

namespace {

struct Extent {
  uintptr_t lo, hi;
};

// The byte extent of a [B, H, N, d] view (all sizes >= 1, strides >= 0)
// stays below 2^48, so that the int64 offsets of the host and the kernels
// cannot overflow.
bool view_fits(const int64_t s[3], int B, int H, int N, int d, int esize) {
  const __int128 last = (__int128)(B - 1) * s[0] + (__int128)(H - 1) * s[1] +
                        (__int128)(N - 1) * s[2] + d;
  return last * esize < ((__int128)1 << 48);
}

// Byte range of a [B, H, N, d] view that passed view_fits.
Extent extent_of(const void *ptr, const int64_t s[3], int B, int H, int N, int d, int esize) {
  const int64_t last = (int64_t)(B - 1) * s[0] + (int64_t)(H - 1) * s[1] +
                       (int64_t)(N - 1) * s[2] + d;
  return Extent{(uintptr_t)ptr, (uintptr_t)ptr + (uintptr_t)(last * esize)};
}

Extent rows_extent(const void *ptr, int64_t rows, int esize) {
  return Extent{(uintptr_t)ptr, (uintptr_t)ptr + (uintptr_t)(rows * esize)};
}

bool overlaps(Extent a, Extent b) { return a.lo < b.hi && b.lo < a.hi; }

bool same3(const int64_t a[3], const int64_t b[3]) {
  return a[0] == b[0] && a[1] == b[1] && a[2] == b[2];
}

// Every stride non-negative and a multiple of `align` elements, and the
// largest element offset of the view representable.
bool strides_ok(const int64_t s[3], int64_t align) {
  for (int j = 0; j < 3; ++j)
    if (s[j] < 0 || s[j] % align != 0 || s[j] > (INT64_C(1) << 40)) return false;
  return true;
}

int esize_of(int dtype) { return dtype == ATTN_JVP_BF16 ? 2 : 4; }

bool dtype_ok(int dtype) { return dtype == ATTN_JVP_BF16 || dtype == ATTN_JVP_FP32; }

}  // namespace

bool grid_fits(int64_t workgroups, int threads) {
  return workgroups >= 1 && workgroups <= INT64_C(0x7fffffff) &&
         workgroups * threads <= INT64_C(0xffffffff);
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

bool shape_for(int dtype, int dqk, int dv, FwdGeom *out) {
  if (!dtype_ok(dtype) || !fwd_built(esize_of(dtype), dqk, dv)) return false;
  *out = fwd_geom(esize_of(dtype), dqk, dv);
  return true;
}

bool launch_small(const attn_jvp_shape &s, int dtype, const attn_jvp_mask *mask) {
  if (!dtype_ok(dtype)) return false;
  const int es = esize_of(dtype), dqk = s.head_dim_qk, dv = s.head_dim_v;
  if (!fwd_pick_small(es, dqk, dv, (int64_t)s.batch * s.heads, s.seqlen_q, mask_on(mask), 1))
    return false;
  const FwdGeom g = fwd16_geom_small(es, dqk, dv);
  return grid_fits((int64_t)s.batch * s.heads * ((s.seqlen_q + g.block_m - 1) / g.block_m),
                   64 * g.waves);
}

void set_small(Params *p, int dtype, const attn_jvp_shape &s) {
  const FwdGeom g = fwd16_geom_small(esize_of(dtype), s.head_dim_qk, s.head_dim_v);
  p->small = 1;
  p->nqb = (p->Nq + g.block_m - 1) / g.block_m;
}

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

attn_jvp_shape square(int B, int H, int N, int d) {
  attn_jvp_shape s;
  s.batch = B;
  s.heads = H;
  s.seqlen_q = s.seqlen_kv = N;
  s.head_dim_qk = s.head_dim_v = d;
  return s;
}

int check_args(const void *Q, const void *K, const void *V, const void *dQ, const void *dK,
               const void *dV, const void *O, const void *dO, const float *LSE,
               const float *dLSE, const attn_jvp_shape *shape, int dtype,
               const attn_jvp_layout *L, const attn_jvp_mask *mask, int out_esize, int nsplit) {
  if (!Q || !K || !V || !dQ || !dK || !dV || !O || !dO || !LSE || !dLSE || !shape || !L)
    return ATTN_JVP_EINVAL;
  const int B = shape->batch, H = shape->heads, Nq = shape->seqlen_q, Nkv = shape->seqlen_kv;
  const int dqk = shape->head_dim_qk, dv = shape->head_dim_v;
  if (B <= 0 || H <= 0 || Nq <= 0 || Nkv <= 0 || dqk <= 0 || dv <= 0) return ATTN_JVP_EINVAL;
  if (!dtype_ok(dtype)) return ATTN_JVP_EINVAL;
  FwdGeom g;
  if (!shape_for(dtype, dqk, dv, &g)) return ATTN_JVP_EUNSUPPORTED;
  if (mask_on(mask) && dqk != dv) return ATTN_JVP_EUNSUPPORTED;
  const int64_t nqb = (Nq + g.block_m - 1) / g.block_m;
  if (nsplit < 1 || !grid_fits((int64_t)B * H * nqb * nsplit, 64 * g.waves))
    return ATTN_JVP_EINVAL;
  if (!same3(L->q, L->dq) || !same3(L->k, L->dk) || !same3(L->v, L->dv) ||
      !same3(L->o, L->dout))
    return ATTN_JVP_ESTRIDE;
  const int esize = esize_of(dtype);
  const int oes = out_esize ? out_esize : esize;
  const int64_t *all[4] = {L->q, L->k, L->v, L->o};
  for (int i = 0; i < 4; ++i)
    if (!strides_ok(all[i], 16 / (i == 3 ? oes : esize))) return ATTN_JVP_ESTRIDE;
  // key-tile offsets use 24-bit row strides (in bytes)
  if (L->k[2] * esize >= (1 << 24) || L->v[2] * esize >= (1 << 24)) return ATTN_JVP_ESTRIDE;
  if (!view_fits(L->q, B, H, Nq, dqk, esize) || !view_fits(L->k, B, H, Nkv, dqk, esize) ||
      !view_fits(L->v, B, H, Nkv, dv, esize) || !view_fits(L->o, B, H, Nq, dv, oes))
    return ATTN_JVP_ESTRIDE;
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
                         extent_of(dO, L->o, B, H, Nq, dv, oes), rows_extent(LSE, rows, 4),
                         rows_extent(dLSE, rows, 4)};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(out[i], in[j])) return ATTN_JVP_ESTRIDE;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(out[i], out[j])) return ATTN_JVP_ESTRIDE;
  }
  return check_mask(mask, Nq, Nkv);
}

Params make_params(const void *Q, const void *K, const void *V, const void *dQ, const void *dK,
                   const void *dV, void *O, void *dO, float *LSE, float *dLSE,
                   const attn_jvp_shape &shape, float scale, int dtype,
                   const attn_jvp_layout &L, const attn_jvp_mask *mask) {
  FwdGeom g;
  shape_for(dtype, shape.head_dim_qk, shape.head_dim_v, &g);
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
  p.nqb = (p.Nq + g.block_m - 1) / g.block_m;
  p.nsplit = 1;
  p.partial = 0;
  p.scale = (scale > 0.f && isfinite(scale)) ? scale : 1.0f / sqrtf((float)shape.head_dim_qk);
  p.scale_log2 = p.scale * 1.4426950408889634f;
  p.mask = to_dev(mask);
  return p;
}

void partial_out_strides(const attn_jvp_shape &s, attn_jvp_layout *L) {
  const int64_t o[3] = {(int64_t)s.heads * s.seqlen_q * s.head_dim_v,
                        (int64_t)s.seqlen_q * s.head_dim_v, (int64_t)s.head_dim_v};
  for (int i = 0; i < 3; ++i) L->o[i] = L->dout[i] = o[i];
}

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
  FwdGeom g;
  if (!shape_for(dtype, s.head_dim_qk, s.head_dim_v, &g)) return 1;
  const int64_t nqb = (s.seqlen_q + g.block_m - 1) / g.block_m;
  const int64_t wgs = (int64_t)s.batch * s.heads * nqb;
  int64_t tiles = (s.seqlen_kv + g.block_n - 1) / g.block_n;
  if (mask_on(mask) && check_mask(mask, s.seqlen_q, s.seqlen_kv) == ATTN_JVP_OK) {
    const MaskDev m = to_dev(mask);
    int64_t mx = 0;
    for (int64_t qb = 0; qb < nqb; ++qb) {
      const int q0 = (int)(qb * g.block_m);
      const int q1 = q0 + g.block_m < s.seqlen_q ? q0 + g.block_m : s.seqlen_q;
      const int64_t c = tile_count(visible_tiles(m, q0, q1, s.seqlen_kv, g.block_n));
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

int check_workspace(const void *workspace, size_t workspace_bytes, size_t need,
                    const void *const tensors[10], const attn_jvp_shape &s, int dtype,
                    const attn_jvp_layout &L) {
  if (!workspace || (uintptr_t)workspace % 256 != 0) return ATTN_JVP_EINVAL;
  if (workspace_bytes < need) return ATTN_JVP_EINVAL;
  const Extent ws{(uintptr_t)workspace, (uintptr_t)workspace + need};
  const int es = esize_of(dtype);
  const int B = s.batch, H = s.heads, Nq = s.seqlen_q, Nkv = s.seqlen_kv;
  const int dqk = s.head_dim_qk, dv = s.head_dim_v;
  const int64_t rows = (int64_t)B * H * Nq;
  const Extent all[10] = {
      extent_of(tensors[0], L.q, B, H, Nq, dqk, es), extent_of(tensors[1], L.k, B, H, Nkv, dqk, es),
      extent_of(tensors[2], L.v, B, H, Nkv, dv, es), extent_of(tensors[3], L.q, B, H, Nq, dqk, es),
      extent_of(tensors[4], L.k, B, H, Nkv, dqk, es), extent_of(tensors[5], L.v, B, H, Nkv, dv, es),
      extent_of(tensors[6], L.o, B, H, Nq, dv, es), extent_of(tensors[7], L.o, B, H, Nq, dv, es),
      rows_extent(tensors[8], rows, 4), rows_extent(tensors[9], rows, 4)};
  for (int i = 0; i < 10; ++i)
    if (overlaps(ws, all[i])) return ATTN_JVP_ESTRIDE;
  return ATTN_JVP_OK;
}

int check_bwd(const void *Q, const void *K, const void *V, const void *O, const void *gO,
              const float *LSE, const void *gQ, const void *gK, const void *gV,
              const float *delta, const attn_jvp_shape *shape, int dtype,
              const attn_jvp_bwd_layout *L, const attn_jvp_mask *mask) {
  if (!Q || !K || !V || !O || !gO || !LSE || !gQ || !gK || !gV || !delta || !shape || !L)
    return ATTN_JVP_EINVAL;
  const int B = shape->batch, H = shape->heads, Nq = shape->seqlen_q, Nkv = shape->seqlen_kv;
  const int d = shape->head_dim_qk;
  if (B <= 0 || H <= 0 || Nq <= 0 || Nkv <= 0 || d <= 0 || shape->head_dim_v <= 0)
    return ATTN_JVP_EINVAL;
  if (!dtype_ok(dtype)) return ATTN_JVP_EINVAL;
  if (shape->head_dim_v != d) return ATTN_JVP_EUNSUPPORTED;   // the pages: one head dim
  const int esize = esize_of(dtype);
  if (!bwd_built(esize, d)) return ATTN_JVP_EUNSUPPORTED;
  const BwdGeom g = bwd_geom(esize, d);
  // one 16-row block per wave is the launch with the most workgroups
  if (!grid_fits((int64_t)B * H * ((Nq + 16 * g.waves_dq - 1) / (16 * g.waves_dq)),
                 64 * g.waves_dq) ||
      !grid_fits((int64_t)B * H * ((Nkv + 16 * g.waves_dkv - 1) / (16 * g.waves_dkv)),
                 64 * g.waves_dkv))
    return ATTN_JVP_EINVAL;
  const int64_t align = 16 / esize;
  const int64_t *all[8] = {L->q, L->k, L->v, L->o, L->go, L->gq, L->gk, L->gv};
  for (int i = 0; i < 8; ++i)
    if (!strides_ok(all[i], align)) return ATTN_JVP_ESTRIDE;
  // streamed tiles use 24-bit row strides (in bytes)
  const int64_t *streamed[4] = {L->q, L->k, L->v, L->go};
  for (int i = 0; i < 4; ++i)
    if (streamed[i][2] * esize >= (1 << 24)) return ATTN_JVP_ESTRIDE;
  const int rows_of[8] = {Nq, Nkv, Nkv, Nq, Nq, Nq, Nkv, Nkv};
  for (int i = 0; i < 8; ++i)
    if (!view_fits(all[i], B, H, rows_of[i], d, esize)) return ATTN_JVP_ESTRIDE;
  const void *ptrs[8] = {Q, K, V, O, gO, gQ, gK, gV};
  for (int i = 0; i < 8; ++i)
    if ((uintptr_t)ptrs[i] % 16 != 0) return ATTN_JVP_ESTRIDE;
  if ((uintptr_t)LSE % 4 != 0 || (uintptr_t)delta % 4 != 0) return ATTN_JVP_ESTRIDE;
  const int64_t rows = (int64_t)B * H * Nq;
  const Extent in[6] = {extent_of(Q, L->q, B, H, Nq, d, esize),
                        extent_of(K, L->k, B, H, Nkv, d, esize),
                        extent_of(V, L->v, B, H, Nkv, d, esize),
                        extent_of(O, L->o, B, H, Nq, d, esize),
                        extent_of(gO, L->go, B, H, Nq, d, esize), rows_extent(LSE, rows, 4)};
  const Extent out[4] = {extent_of(gQ, L->gq, B, H, Nq, d, esize),
                         extent_of(gK, L->gk, B, H, Nkv, d, esize),
                         extent_of(gV, L->gv, B, H, Nkv, d, esize), rows_extent(delta, rows, 4)};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(out[i], in[j])) return ATTN_JVP_ESTRIDE;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(out[i], out[j])) return ATTN_JVP_ESTRIDE;
  }
  return check_mask(mask, Nq, Nkv);
}

BwdParams make_bwd_params(const void *Q, const void *K, const void *V, const void *O,
                          const void *gO, const float *LSE, void *gQ, void *gK, void *gV,
                          float *delta, const attn_jvp_shape &shape, float scale, int dtype,
                          const attn_jvp_bwd_layout &L, const attn_jvp_mask *mask) {
  const BwdGeom g = bwd_geom(esize_of(dtype), shape.head_dim_qk);
  const int bq = 16 * g.waves_dq, bk = 16 * g.waves_dkv;
  // two row blocks per wave halve a launch's LDS traffic per MFMA but also
  // its workgroups: taken while at least two rounds of workgroups (512 on
  // 256 CUs) remain
  const int64_t bh = (int64_t)shape.batch * shape.heads;
  const int rbq =
      (g.rb_dq_max >= 2 && bh * ((shape.seqlen_q + 2 * bq - 1) / (2 * bq)) >= 512) ? 2 : 1;
  const int rbk =
      (g.rb_dkv_max >= 2 && bh * ((shape.seqlen_kv + 2 * bk - 1) / (2 * bk)) >= 512) ? 2 : 1;
  BwdParams p;
  memset(&p, 0, sizeof(p));
  p.q = Q; p.k = K; p.v = V; p.o = O; p.g = gO; p.lse = LSE;
  p.gq = gQ; p.gk = gK; p.gv = gV; p.delta = delta;
  for (int i = 0; i < 3; ++i) {
    p.sq[i] = L.q[i]; p.sk[i] = L.k[i]; p.sv[i] = L.v[i]; p.so[i] = L.o[i];
    p.sg[i] = L.go[i]; p.sgq[i] = L.gq[i]; p.sgk[i] = L.gk[i]; p.sgv[i] = L.gv[i];
  }
  p.B = shape.batch;
  p.H = shape.heads;
  p.Nq = shape.seqlen_q;
  p.Nkv = shape.seqlen_kv;
  p.rbq = rbq;
  p.rbk = rbk;
  p.nqb = (p.Nq + rbq * bq - 1) / (rbq * bq);
  p.nkb = (p.Nkv + rbk * bk - 1) / (rbk * bk);
  p.scale = (scale > 0.f && isfinite(scale)) ? scale : 1.0f / sqrtf((float)shape.head_dim_qk);
  p.scale_log2 = p.scale * 1.4426950408889634f;
  p.mask = to_dev(mask);
  return p;
}

int check_merge(int num_parts, const float *O_parts, const float *dO_parts,
                const float *LSE_parts, const float *dLSE_parts, const void *O, const void *dO,
                const float *LSE, const float *dLSE, int B, int H, int Lq, int d_v, int dtype,
                const int64_t *o_strides, MergeParams *m) {
  if (!O_parts || !dO_parts || !LSE_parts || !dLSE_parts || !O || !dO || !LSE || !dLSE || !m)
    return ATTN_JVP_EINVAL;
  if (num_parts < 1 || B <= 0 || H <= 0 || Lq <= 0 || d_v <= 0) return ATTN_JVP_EINVAL;
  if (!dtype_ok(dtype)) return ATTN_JVP_EINVAL;
  if (d_v % 4 != 0) return ATTN_JVP_EUNSUPPORTED;
  const int esize = esize_of(dtype);
  const int64_t rows = (int64_t)B * H * Lq;
  const int64_t threads = rows * (d_v / 4);
  if (!grid_fits((threads + kMergeThreads - 1) / kMergeThreads, kMergeThreads))
    return ATTN_JVP_EINVAL;
  if ((int64_t)num_parts * rows * d_v > (INT64_C(1) << 40)) return ATTN_JVP_EINVAL;
  const int64_t so[3] = {o_strides ? o_strides[0] : (int64_t)H * Lq * d_v,
                         o_strides ? o_strides[1] : (int64_t)Lq * d_v,
                         o_strides ? o_strides[2] : (int64_t)d_v};
  if (!strides_ok(so, 4) || !view_fits(so, B, H, Lq, d_v, esize))
    return ATTN_JVP_ESTRIDE;   // 4-wide stores
  if ((uintptr_t)O_parts % 16 || (uintptr_t)dO_parts % 16 || (uintptr_t)O % (4 * esize) ||
      (uintptr_t)dO % (4 * esize) || (uintptr_t)LSE_parts % 4 || (uintptr_t)dLSE_parts % 4 ||
      (uintptr_t)LSE % 4 || (uintptr_t)dLSE % 4)
    return ATTN_JVP_ESTRIDE;
  const Extent in[4] = {rows_extent(O_parts, num_parts * rows * d_v, 4),
                        rows_extent(dO_parts, num_parts * rows * d_v, 4),
                        rows_extent(LSE_parts, num_parts * rows, 4),
                        rows_extent(dLSE_parts, num_parts * rows, 4)};
  const Extent out[4] = {extent_of(O, so, B, H, Lq, d_v, esize),
                         extent_of(dO, so, B, H, Lq, d_v, esize), rows_extent(LSE, rows, 4),
                         rows_extent(dLSE, rows, 4)};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 4; ++j)
      if (overlaps(out[i], in[j])) return ATTN_JVP_ESTRIDE;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(out[i], out[j])) return ATTN_JVP_ESTRIDE;
  }
  memset(m, 0, sizeof(*m));
  m->o_parts = O_parts; m->do_parts = dO_parts; m->lse_parts = LSE_parts;
  m->dlse_parts = dLSE_parts;
  m->o = (void *)O; m->dout = (void *)dO; m->lse = (float *)LSE; m->dlse = (float *)dLSE;
  for (int j = 0; j < 3; ++j) m->so[j] = so[j];
  m->parts = num_parts; m->B = B; m->H = H; m->Nq = Lq; m->dv = d_v;
  return ATTN_JVP_OK;
}

}  // namespace attn_jvp

using namespace attn_jvp;

extern "C" {

int attn_jvp_check_ex(const void *Q, const void *K, const void *V, const void *dQ,
                      const void *dK, const void *dV, void *O, void *dO, float *LSE,
                      float *dLSE, const attn_jvp_shape *shape, int dtype,
                      const attn_jvp_layout *layout, const attn_jvp_mask *mask) {
  if (!shape) return ATTN_JVP_EINVAL;
  const attn_jvp_layout L = layout ? *layout : contiguous(*shape);
  return check_args(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE, shape, dtype, &L, mask);
}

int attn_jvp_check(const void *Q, const void *K, const void *V, const void *dQ,
                   const void *dK, const void *dV, void *O, void *dO, float *LSE,
                   float *dLSE, int B, int H, int N, int d, int dtype,
                   const attn_jvp_layout *layout, const attn_jvp_mask *mask) {
  if (!layout) return ATTN_JVP_EINVAL;
  const attn_jvp_shape s = square(B, H, N, d);
  return check_args(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE, &s, dtype, layout, mask);
}

int attn_jvp_splitkv_plan(const attn_jvp_shape *shape, int dtype, const attn_jvp_mask *mask,
                          int *num_splits, size_t *workspace_bytes) {
  if (!shape || !num_splits || !workspace_bytes) return ATTN_JVP_EINVAL;
  if (shape->batch <= 0 || shape->heads <= 0 || shape->seqlen_q <= 0 || shape->seqlen_kv <= 0)
    return ATTN_JVP_EINVAL;
  if (!dtype_ok(dtype)) return ATTN_JVP_EINVAL;
  FwdGeom g;
  if (!shape_for(dtype, shape->head_dim_qk, shape->head_dim_v, &g)) return ATTN_JVP_EUNSUPPORTED;
  if (*num_splits < 0 || *num_splits > 1024) return ATTN_JVP_EINVAL;
  const int ns = *num_splits ? *num_splits : choose_splits(*shape, dtype, mask);
  *num_splits = ns;
  *workspace_bytes = ns > 1 ? split_workspace(*shape, ns).total : 0;
  return ATTN_JVP_OK;
}

int attn_jvp_bwd_check(const void *Q, const void *K, const void *V, const void *O,
                       const void *gO, const float *LSE, void *gQ, void *gK, void *gV,
                       float *delta, const attn_jvp_shape *shape, int dtype,
                       const attn_jvp_bwd_layout *layout, const attn_jvp_mask *mask) {
  if (!shape) return ATTN_JVP_EINVAL;
  const attn_jvp_bwd_layout L = layout ? *layout : contiguous_bwd(*shape);
  return check_bwd(Q, K, V, O, gO, LSE, gQ, gK, gV, delta, shape, dtype, &L, mask);
}

int attn_jvp_tile_shape_ex(int dtype, int d_qk, int d_v, int *block_m, int *block_n) {
  if (!block_m || !block_n) return ATTN_JVP_EINVAL;
  if (!dtype_ok(dtype)) return ATTN_JVP_EINVAL;
  FwdGeom g;
  if (!shape_for(dtype, d_qk, d_v, &g)) return ATTN_JVP_EUNSUPPORTED;
  *block_m = g.block_m;
  *block_n = g.block_n;
  return ATTN_JVP_OK;
}

int attn_jvp_tile_shape(int dtype, int d, int *block_m, int *block_n) {
  return attn_jvp_tile_shape_ex(dtype, d, d, block_m, block_n);
}

int attn_jvp_fwd_geometry(const attn_jvp_shape *shape, int dtype, const attn_jvp_mask *mask,
                          int *block_m, int *block_n) {
  if (!shape || !block_m || !block_n) return ATTN_JVP_EINVAL;
  const attn_jvp_shape &s = *shape;
  if (s.batch <= 0 || s.heads <= 0 || s.seqlen_q <= 0 || s.seqlen_kv <= 0) return ATTN_JVP_EINVAL;
  if (!dtype_ok(dtype)) return ATTN_JVP_EINVAL;
  FwdGeom g;
  if (!shape_for(dtype, s.head_dim_qk, s.head_dim_v, &g)) return ATTN_JVP_EUNSUPPORTED;
  if (launch_small(s, dtype, mask)) g = fwd16_geom_small(esize_of(dtype), s.head_dim_qk, s.head_dim_v);
  *block_m = g.block_m;
  *block_n = g.block_n;
  return ATTN_JVP_OK;
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
    tiles_per_block[qb] = tile_count(visible_tiles(m, q0, q1, N, bn));
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
    const TileRanges tr = keys ? visible_query_tiles(m, r0, r1, N, tile_rows)
                               : visible_tiles(m, r0, r1, N, tile_rows);
    tiles_per_block[b] = tile_count(tr);
  }
  return ATTN_JVP_OK;
}

const char *attn_jvp_status_string(int status) {
  switch (status) {
    case ATTN_JVP_OK: return "ok";
    case ATTN_JVP_EINVAL: return "invalid argument (null pointer, size, dtype or launch too large)";
    case ATTN_JVP_EUNSUPPORTED: return "unsupported head dimensions for this dtype";
    case ATTN_JVP_ESTRIDE:
      return "bad layout (tangent strides differ from the primal's, misaligned "
             "pointer or stride, or outputs overlapping inputs)";
    case ATTN_JVP_EMASK: return "inconsistent mask descriptor";
    case ATTN_JVP_EHIP: return "HIP runtime error at launch";
    case ATTN_JVP_ENOSCRATCH:
      return "the split partials exceed the static scratch of the allocation-free entry point";
    default: return "unknown status";
  }
}

}  // extern "C"
