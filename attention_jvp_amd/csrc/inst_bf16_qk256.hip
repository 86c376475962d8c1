// Kernel instances: bfloat16, d_qk = 256, every d_v.
#include "inst.h"

namespace attn_jvp {

hipError_t launch_bf16_qk256(const Params &p, int dv, bool masked, hipStream_t s) {
  return launch_dv<__bf16, 256>(p, dv, masked, s);
}

}  // namespace attn_jvp
