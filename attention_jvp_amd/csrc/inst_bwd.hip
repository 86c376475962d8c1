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

template <typename T, int D>
bool bwd_rows(int *block_q, int *block_k, int *rbq_max, int *rbk_max) {
  using C = BwdCfg<T, D>;
  *block_q = 16 * C::kWavesDq;
  *block_k = 16 * C::kWavesDkv;
  *rbq_max = C::kRbDqMax;
  *rbk_max = C::kRbDkvMax;
  return true;
}

bool bwd_shape_for(bool bf16, int d, int *block_q, int *block_k, int *rbq_max,
                   int *rbk_max) {
  if (bf16) {
    switch (d) {
      case 16: return bwd_rows<__bf16, 16>(block_q, block_k, rbq_max, rbk_max);
      case 32: return bwd_rows<__bf16, 32>(block_q, block_k, rbq_max, rbk_max);
      case 64: return bwd_rows<__bf16, 64>(block_q, block_k, rbq_max, rbk_max);
      case 128: return bwd_rows<__bf16, 128>(block_q, block_k, rbq_max, rbk_max);
      case 256: return bwd_rows<__bf16, 256>(block_q, block_k, rbq_max, rbk_max);
      default: return false;
    }
  }
  switch (d) {
    case 16: return bwd_rows<float, 16>(block_q, block_k, rbq_max, rbk_max);
    case 32: return bwd_rows<float, 32>(block_q, block_k, rbq_max, rbk_max);
    case 64: return bwd_rows<float, 64>(block_q, block_k, rbq_max, rbk_max);
    default: return false;
  }
}

}  // namespace attn_jvp
