// Per-d_qk launch entry points; each is defined in its own translation unit
// (inst_*.hip) so the kernel instances compile in parallel.
#pragma once

#include <hip/hip_runtime.h>

#include "kernel.h"

namespace attn_jvp {

// bfloat16, d_qk fixed by the unit, d_v in {16, 32, 64, 128, 256}; a frame-
// window mask needs d_v == d_qk.  Returns hipErrorInvalidValue for a shape
// the unit does not hold.
hipError_t launch_bf16_qk16(const Params &p, int dv, bool masked, hipStream_t s);
hipError_t launch_bf16_qk32(const Params &p, int dv, bool masked, hipStream_t s);
hipError_t launch_bf16_qk64(const Params &p, int dv, bool masked, hipStream_t s);
hipError_t launch_bf16_qk128(const Params &p, int dv, bool masked, hipStream_t s);
hipError_t launch_bf16_qk256(const Params &p, int dv, bool masked, hipStream_t s);
// float32, d_qk and d_v in {16, 32, 64}.
hipError_t launch_fp32(const Params &p, int dqk, int dv, bool masked, hipStream_t s);

// Block shape of (bf16?, d_qk, d_v); false if the shape is not built.
bool shape_for(bool bf16, int dqk, int dv, Shape *out);

// Merge of key-split partials (merge.hip).  Partials are float32,
// contiguous: O, dO [parts, B, H, Nq, dv], LSE, dLSE [parts, B, H, Nq].
// Outputs: O, dO in the dtype with (b, h, n) element strides so[], LSE and
// dLSE float32 contiguous [B, H, Nq].
struct MergeParams {
  const float *o_parts, *do_parts, *lse_parts, *dlse_parts;
  void *o, *dout;
  float *lse, *dlse;
  int64_t so[3];
  int parts, B, H, Nq, dv;
};
hipError_t launch_merge(const MergeParams &m, bool bf16, hipStream_t s);

// Primal backward (inst_bwd.hip, kernels in bwd.h): d_qk = d_v = d.
struct BwdParams;
hipError_t launch_bwd(const BwdParams &p, bool bf16, int d, hipStream_t s);
// Query rows per dQ workgroup and key rows per dK/dV workgroup with one
// 16-row block per wave, and the most 16-row blocks a wave of each launch may
// own (its workgroup then covers that many times the rows); false if
// (dtype, d) is not built.
bool bwd_shape_for(bool bf16, int d, int *block_q, int *block_k, int *rbq_max,
                   int *rbk_max);

}  // namespace attn_jvp
