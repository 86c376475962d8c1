// Backward kernel instances: d_qk = d_v = D in {16, 32, 64, 128, 256}
// (bfloat16) and {16, 32, 64} (float32).
#include "bwd.h"
#include "dispatch.h"

namespace attn_jvp {

hipError_t launch_bwd(const BwdParams &p, bool bf16, int d, hipStream_t s) {
  if (bf16) {
    switch (d) {
      case 16: return launch_bwd_instance<__bf16, 16>(p, s);
      case 32: return launch_bwd_instance<__bf16, 32>(p, s);
      case 64: return launch_bwd_instance<__bf16, 64>(p, s);
      case 128: return launch_bwd_instance<__bf16, 128>(p, s);
      case 256: return launch_bwd_instance<__bf16, 256>(p, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (d) {
    case 16: return launch_bwd_instance<float, 16>(p, s);
    case 32: return launch_bwd_instance<float, 32>(p, s);
    case 64: return launch_bwd_instance<float, 64>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn_jvp
