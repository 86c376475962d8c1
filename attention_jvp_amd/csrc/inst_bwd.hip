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

bool bwd_shape_for(bool bf16, int d, int *block_q, int *block_k) {
  auto set = [&](int wq, int wk) {
    *block_q = 16 * wq;
    *block_k = 16 * wk;
    return true;
  };
  if (bf16) {
    switch (d) {
      case 16: return set(BwdCfg<__bf16, 16>::kWavesDq, BwdCfg<__bf16, 16>::kWavesDkv);
      case 32: return set(BwdCfg<__bf16, 32>::kWavesDq, BwdCfg<__bf16, 32>::kWavesDkv);
      case 64: return set(BwdCfg<__bf16, 64>::kWavesDq, BwdCfg<__bf16, 64>::kWavesDkv);
      case 128: return set(BwdCfg<__bf16, 128>::kWavesDq, BwdCfg<__bf16, 128>::kWavesDkv);
      case 256: return set(BwdCfg<__bf16, 256>::kWavesDq, BwdCfg<__bf16, 256>::kWavesDkv);
      default: return false;
    }
  }
  switch (d) {
    case 16: return set(BwdCfg<float, 16>::kWavesDq, BwdCfg<float, 16>::kWavesDkv);
    case 32: return set(BwdCfg<float, 32>::kWavesDq, BwdCfg<float, 32>::kWavesDkv);
    case 64: return set(BwdCfg<float, 64>::kWavesDq, BwdCfg<float, 64>::kWavesDkv);
    default: return false;
  }
}

}  // namespace attn_jvp
