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
// reads 2 * num_parts float4 values plus the row's per-part scalars.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "dispatch.h"

namespace attn_jvp {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams m) {
  const int cpr = m.dv / 4;                               // threads per row
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rows = (int64_t)m.B * m.H * m.Nq;
  if (t >= rows * cpr) return;
  const int64_t row = t / cpr;
  const int c = (int)(t - row * cpr) * 4;
  const int64_t bh = row / m.Nq;
  const int n = (int)(row - bh * m.Nq);
  const int b = (int)(bh / m.H), h = (int)(bh - (int64_t)b * m.H);

  // row scalars: LSE, dLSE
  // IEEE maximum: a NaN in any part propagates to the row, as in one pass
  float mx = -INFINITY;
  for (int k = 0; k < m.parts; ++k)
    mx = __builtin_elementwise_maximum(mx, m.lse_parts[k * rows + row]);
  T *O = (T *)m.o + b * m.so[0] + h * m.so[1] + (int64_t)n * m.so[2] + c;
  T *dO = (T *)m.dout + b * m.so[0] + h * m.so[1] + (int64_t)n * m.so[2] + c;
  typedef T T4 __attribute__((ext_vector_type(4)));
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
  float sum = 0.f;
  for (int k = 0; k < m.parts; ++k) sum += expf(m.lse_parts[k * rows + row] - mx);
  const float lse = mx + logf(sum);
  float dlse = 0.f;
  for (int k = 0; k < m.parts; ++k) {
    const float w = expf(m.lse_parts[k * rows + row] - lse);
    dlse += w * m.dlse_parts[k * rows + row];
  }

  // columns c..c+3
  typedef float f4 __attribute__((ext_vector_type(4)));
  f4 o = {0.f, 0.f, 0.f, 0.f}, d = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < m.parts; ++k) {
    const float lk = m.lse_parts[k * rows + row];
    const float w = expf(lk - lse);                      // 0 for an empty part
    const float g = m.dlse_parts[k * rows + row] - dlse;
    const int64_t off = (k * rows + row) * m.dv + c;
    const f4 ok = *(const f4 *)(m.o_parts + off);
    const f4 dk = *(const f4 *)(m.do_parts + off);
    o += w * ok;                      // an empty part has w = 0, O_k = dO_k = 0
    d += w * (dk + g * ok);
  }
  T4 ov, dv;
  for (int i = 0; i < 4; ++i) {
    ov[i] = (T)o[i];
    dv[i] = (T)d[i];
  }
  *(T4 *)O = ov;
  *(T4 *)dO = dv;
  if (c == 0) {
    m.lse[row] = lse;
    m.dlse[row] = dlse;
  }
}

}  // namespace

hipError_t launch_merge(const MergeParams &m, bool bf16, hipStream_t s) {
  const int64_t threads = (int64_t)m.B * m.H * m.Nq * (m.dv / 4);
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (bf16)
    hipLaunchKernelGGL(merge_kernel<__bf16>, dim3((unsigned)blocks), dim3(256), 0, s, m);
  else
    hipLaunchKernelGGL(merge_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, s, m);
  return hipGetLastError();
}

}  // namespace attn_jvp
