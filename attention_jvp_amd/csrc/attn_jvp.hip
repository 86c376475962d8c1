// The launching entry points of the attn_jvp C ABI: each validates its call
// with the host code (host.cpp; nothing is launched on error) and dispatches
// to the kernel instances (kernel.h and bwd.h, instantiated per head dim in
// the inst_*.hip units; merge.hip).  Op contract: page "带分数正则的一致性蒸馏"
// (gitcode.csdn.net), section 注意力, 前向 kernel and subsection 反向.

#include <hip/hip_runtime.h>

#include <mutex>

#include "attn_jvp.h"
#include "dispatch.h"
#include "host.h"

namespace {

using attn_jvp::Params;

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

int status_of(hipError_t err) { return err == hipSuccess ? ATTN_JVP_OK : ATTN_JVP_EHIP; }

// Split-KV forward with ns splits whose float32 partials go to `workspace`
// (need bytes of the plan): the split launch, then the merge.
int run_splitkv(const void *Q, const void *K, const void *V, const void *dQ, const void *dK,
                const void *dV, void *O, void *dO, float *LSE, float *dLSE,
                const attn_jvp_shape &shape, float scale, int dtype,
                const attn_jvp_layout *layout, const attn_jvp_mask *mask, int ns, size_t need,
                void *workspace, size_t workspace_bytes, hipStream_t stream) {
  using namespace attn_jvp;
  if (ns == 1)
    return attn_jvp_fwd_ex(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE, &shape, scale, dtype, layout,
                           mask, stream);
  const attn_jvp_layout L = layout ? *layout : contiguous(shape);
  int st = check_args(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE, &shape, dtype, &L, mask, 0, ns);
  if (st != ATTN_JVP_OK) return st;
  const void *const tensors[10] = {Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE};
  st = check_workspace(workspace, workspace_bytes, need, tensors, shape, dtype, L);
  if (st != ATTN_JVP_OK) return st;

  const SplitWs w = split_workspace(shape, ns);
  char *base = (char *)workspace;
  float *op = (float *)(base + w.o), *dop = (float *)(base + w.dout);
  float *lp = (float *)(base + w.lse), *dlp = (float *)(base + w.dlse);
  MergeParams m;
  st = check_merge(ns, op, dop, lp, dlp, O, dO, LSE, dLSE, shape.batch, shape.heads,
                   shape.seqlen_q, shape.head_dim_v, dtype, L.o, &m);
  if (st != ATTN_JVP_OK) return st;
  Params p = make_params(Q, K, V, dQ, dK, dV, op, dop, lp, dlp, shape, scale, dtype, L, mask);
  p.partial = 1;
  p.nsplit = ns;
  const hipError_t err = dispatch(p, dtype, shape.head_dim_qk, shape.head_dim_v, mask_on(mask),
                                  stream);
  if (err != hipSuccess) return ATTN_JVP_EHIP;
  return status_of(launch_merge(m, dtype == ATTN_JVP_BF16, stream));
}

// ---- Static scratch of the allocation-free split-KV entry point ----------
// Each GPU the library runs on holds one copy of this array (placed with the
// code object, kept until the process ends).  Host code never passes the
// array's name to a kernel: that is a host-side stand-in, not the device
// address.  Each device's address comes from hipGetSymbolAddress, taken once
// per device with that device current, and only that address is used.
constexpr size_t kScratchBytes = size_t(ATTN_JVP_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_ptr[kMaxDevices];

// The scratch address on the device of `stream` (which must be the current
// device).
int scratch_of_stream(hipStream_t stream, void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return ATTN_JVP_EHIP;
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return ATTN_JVP_EHIP;
    if ((int)sdev != dev) return ATTN_JVP_EINVAL;
  }
  if (dev < 0 || dev >= kMaxDevices) return ATTN_JVP_EINVAL;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ATTN_JVP_EHIP;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return ATTN_JVP_OK;
}

}  // namespace

using namespace attn_jvp;

extern "C" {

int attn_jvp_fwd_ex(const void *Q, const void *K, const void *V, const void *dQ,
                    const void *dK, const void *dV, void *O, void *dO, float *LSE,
                    float *dLSE, const attn_jvp_shape *shape, float scale, int dtype,
                    const attn_jvp_layout *layout, const attn_jvp_mask *mask,
                    void *stream) {
  if (!shape) return ATTN_JVP_EINVAL;
  const attn_jvp_layout L = layout ? *layout : contiguous(*shape);
  const int st = check_args(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE, shape, dtype, &L, mask);
  if (st != ATTN_JVP_OK) return st;
  Params p = make_params(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE, *shape, scale, dtype, L, mask);
  if (launch_small(*shape, dtype, mask)) set_small(&p, dtype, *shape);
  return status_of(dispatch(p, dtype, shape->head_dim_qk, shape->head_dim_v, mask_on(mask),
                            (hipStream_t)stream));
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
  return status_of(dispatch(p, dtype, shape->head_dim_qk, shape->head_dim_v, false,
                            (hipStream_t)stream));
}

int attn_jvp_merge(int num_parts, const float *O_parts, const float *dO_parts,
                   const float *LSE_parts, const float *dLSE_parts, void *O, void *dO,
                   float *LSE, float *dLSE, int B, int H, int Lq, int d_v, int dtype,
                   const int64_t *o_strides, void *stream) {
  MergeParams m;
  const int st = check_merge(num_parts, O_parts, dO_parts, LSE_parts, dLSE_parts, O, dO, LSE,
                             dLSE, B, H, Lq, d_v, dtype, o_strides, &m);
  if (st != ATTN_JVP_OK) return st;
  return status_of(launch_merge(m, dtype == ATTN_JVP_BF16, (hipStream_t)stream));
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
  const int st = attn_jvp_splitkv_plan(shape, dtype, mask, &ns, &need);
  if (st != ATTN_JVP_OK) return st;
  return run_splitkv(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE, *shape, scale, dtype, layout, mask,
                     ns, need, workspace, workspace_bytes, (hipStream_t)stream);
}

int attn_jvp_fwd_splitkv_noalloc(const void *Q, const void *K, const void *V, const void *dQ,
                                 const void *dK, const void *dV, void *O, void *dO, float *LSE,
                                 float *dLSE, const attn_jvp_shape *shape, float scale,
                                 int dtype, const attn_jvp_layout *layout,
                                 const attn_jvp_mask *mask, int num_splits, void *stream) {
  if (!shape) return ATTN_JVP_EINVAL;
  int ns = num_splits;
  size_t need = 0;
  int st = attn_jvp_splitkv_plan(shape, dtype, mask, &ns, &need);
  if (st != ATTN_JVP_OK) return st;
  if (need > kScratchBytes) {
    if (num_splits != 0) return ATTN_JVP_ENOSCRATCH;
    // the plan's own choice: the most splits whose partials fit (one split
    // needs no scratch at all)
    while (ns > 1 && split_workspace(*shape, ns).total > kScratchBytes) --ns;
    need = ns > 1 ? split_workspace(*shape, ns).total : 0;
  }
  void *ws = nullptr;
  if (ns > 1) {
    st = scratch_of_stream((hipStream_t)stream, &ws);
    if (st != ATTN_JVP_OK) return st;
  }
  return run_splitkv(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE, *shape, scale, dtype, layout, mask,
                     ns, need, ws, kScratchBytes, (hipStream_t)stream);
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
  const BwdParams p = make_bwd_params(Q, K, V, O, gO, LSE, gQ, gK, gV, delta, *shape, scale,
                                      dtype, L, mask);
  return status_of(launch_bwd(p, dtype == ATTN_JVP_BF16, shape->head_dim_qk, (hipStream_t)stream));
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

}  // extern "C"
