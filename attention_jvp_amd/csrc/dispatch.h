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

// Merge of key-split partials (merge.hip).
hipError_t launch_merge(const MergeParams &m, bool bf16, hipStream_t s);

// Primal backward (inst_bwd.hip, kernels in bwd.h): d_qk = d_v = d.
hipError_t launch_bwd(const BwdParams &p, bool bf16, int d, hipStream_t s);
}  // namespace attn_jvp
