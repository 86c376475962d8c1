// Kernel instances: float32, d_qk and d_v in {16, 32, 64}.
#include "inst.h"

namespace attn_jvp {

hipError_t launch_fp32(const Params &p, int dqk, int dv, bool masked, hipStream_t s) {
  switch (dqk) {
    case 16: return launch_dv<float, 16>(p, dv, masked, s);
    case 32: return launch_dv<float, 32>(p, dv, masked, s);
    case 64: return launch_dv<float, 64>(p, dv, masked, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn_jvp
