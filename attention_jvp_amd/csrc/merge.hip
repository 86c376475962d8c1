// Merge of key-split partials of the attention JVP.
//
// A softmax over a union of disjoint key sets is the softmax over each set,
// reweighted by that set's share of the total mass: with per-set outputs
// (O_k, dO_k, LSE_k, dLSE_k) over the same query rows,
//   LSE  = log sum_k exp(LSE_k)            w_k = exp(LSE_k - LSE)
//   O    = sum_k w_k O_k
//   dLSE = sum_k w_k dLSE_k                (dw_k = w_k (dLSE_k - dLSE))
//   dO   = sum_k w_k (dO_k + (dLSE_k - dLSE) O_k)
// (the product rule on O = sum_k w_k O_k).  The per-set quantities are those
// of the page "带分数正则的一致性蒸馏" (gitcode.csdn.net), section 注意力; the
// identity itself follows from the definition and is not on the pages.
//
// Memory-bound: each thread owns 4 consecutive d_v columns of one row and
// reads 2 * num_parts float4 values plus the row's per-part scalars, once.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "dispatch.h"

namespace attn_jvp {
namespace {

template <typename T>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeParams m) {
  const int cpr = m.dv / 4;                               // threads per row
  const int64_t t = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
  const int64_t rows = (int64_t)m.B * m.H * m.Nq;
  if (t >= rows * cpr) return;
  const int64_t row = t / cpr;
  const int c = (int)(t - row * cpr) * 4;
  const int64_t bh = row / m.Nq;
  const int n = (int)(row - bh * m.Nq);
  const int b = (int)(bh / m.H), h = (int)(bh - (int64_t)b * m.H);

  T *O = (T *)m.o + b * m.so[0] + h * m.so[1] + (int64_t)n * m.so[2] + c;
  T *dO = (T *)m.dout + b * m.so[0] + h * m.so[1] + (int64_t)n * m.so[2] + c;
  typedef T T4 __attribute__((ext_vector_type(4)));
  typedef float f4 __attribute__((ext_vector_type(4)));

  // One pass over the parts with a running maximum mx (online log-sum-exp):
  // with u_k = exp(LSE_k - mx), accumulate su = sum u_k, sd = sum u_k dLSE_k,
  // ob = sum u_k O_k and ub = sum u_k (dO_k + dLSE_k O_k).  Then w_k = u_k/su,
  // and dO = sum w_k (dO_k + dLSE_k O_k) - dLSE O, the identity above with
  // the dLSE term taken out of the sum.
  float mx = -INFINITY, su = 0.f, sd = 0.f;
  f4 ob = {0.f, 0.f, 0.f, 0.f}, ub = {0.f, 0.f, 0.f, 0.f};
  auto fold = [&](float lk, float dk, f4 ok, f4 gk) {
    // IEEE maximum: a NaN in any part propagates to the row, as in one pass
    const float mn = __builtin_elementwise_maximum(mx, lk);
    if (mn == -INFINITY) return;                      // nothing seen yet
    const float alpha = expf(mx - mn);                // 0 on the first seen part
    const float u = expf(lk - mn);                    // 0 for an empty part
    su = su * alpha + u;
    sd = sd * alpha + u * dk;
    ob = ob * alpha + u * ok;
    ub = ub * alpha + u * (gk + dk * ok);
    mx = mn;
  };
  // four parts' loads in flight before they are folded in order
  constexpr int G = 4;
  int k = 0;
  for (; k + G <= m.parts; k += G) {
    float lk[G], dk[G];
    f4 ok[G], gk[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int64_t r = (int64_t)(k + j) * rows + row;
      lk[j] = m.lse_parts[r];
      dk[j] = m.dlse_parts[r];
      ok[j] = *(const f4 *)(m.o_parts + r * m.dv + c);
      gk[j] = *(const f4 *)(m.do_parts + r * m.dv + c);
    }
#pragma unroll
    for (int j = 0; j < G; ++j) fold(lk[j], dk[j], ok[j], gk[j]);
  }
  for (; k < m.parts; ++k) {
    const int64_t r = (int64_t)k * rows + row;
    fold(m.lse_parts[r], m.dlse_parts[r], *(const f4 *)(m.o_parts + r * m.dv + c),
         *(const f4 *)(m.do_parts + r * m.dv + c));
  }
  if (mx == -INFINITY) {                 // no part saw a key: the empty-row convention
    T4 z;
    for (int i = 0; i < 4; ++i) z[i] = (T)0.f;
    *(T4 *)O = z;
    *(T4 *)dO = z;
    if (c == 0) {
      m.lse[row] = -INFINITY;
      m.dlse[row] = 0.f;
    }
    return;
  }
  const float inv = 1.f / su;
  const float dlse = sd * inv;
  T4 ov, dv;
  for (int i = 0; i < 4; ++i) {
    const float o = ob[i] * inv;
    ov[i] = (T)o;
    dv[i] = (T)(ub[i] * inv - dlse * o);
  }
  *(T4 *)O = ov;
  *(T4 *)dO = dv;
  if (c == 0) {
    m.lse[row] = mx + logf(su);
    m.dlse[row] = dlse;
  }
}

}  // namespace

hipError_t launch_merge(const MergeParams &m, bool bf16, hipStream_t s) {
  const int64_t threads = (int64_t)m.B * m.H * m.Nq * (m.dv / 4);
  const int64_t blocks = (threads + kMergeThreads - 1) / kMergeThreads;
  if (blocks > 0x7fffffffLL || blocks * kMergeThreads > 0xffffffffLL) return hipErrorInvalidValue;
  if (bf16)
    hipLaunchKernelGGL(merge_kernel<__bf16>, dim3((unsigned)blocks), dim3(kMergeThreads), 0, s, m);
  else
    hipLaunchKernelGGL(merge_kernel<float>, dim3((unsigned)blocks), dim3(kMergeThreads), 0, s, m);
  return hipGetLastError();
}

}  // namespace attn_jvp
