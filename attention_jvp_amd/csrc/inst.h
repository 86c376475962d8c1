// Dispatch over d_v for one (dtype, d_qk); included by the inst_*.hip units.
#pragma once

#include "dispatch.h"
#if ATTN_JVP_ROWS32_D128 || ATTN_JVP_ROWS32_D64
#include "kernel32.h"
#endif

namespace attn_jvp {

// A frame-window mask is built for d_qk == d_v only.
template <typename T, int DQK, int DV>
hipError_t launch_pair(const Params &p, bool masked, hipStream_t s) {
#if ATTN_JVP_ROWS32_D128 || ATTN_JVP_ROWS32_D64
  if constexpr (use_rows32((int)sizeof(T), DQK, DV)) {
    return masked ? launch_instance32<DQK, true>(p, s) : launch_instance32<DQK, false>(p, s);
  }
#endif
  if (masked) {
    if constexpr (DQK == DV) return launch_instance<T, DQK, DV, true>(p, s);
    else return hipErrorInvalidValue;
  }
  if constexpr (fwd_has_small((int)sizeof(T), DQK, DV)) {
    if (p.small) return launch_instance<T, DQK, DV, false, true>(p, s);
  }
  if (p.small) return hipErrorInvalidValue;
  return launch_instance<T, DQK, DV, false>(p, s);
}

template <typename T, int DQK>
hipError_t launch_dv(const Params &p, int dv, bool masked, hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    switch (dv) {
      case 16: return launch_pair<T, DQK, 16>(p, masked, s);
      case 32: return launch_pair<T, DQK, 32>(p, masked, s);
      case 64: return launch_pair<T, DQK, 64>(p, masked, s);
      case 128: return launch_pair<T, DQK, 128>(p, masked, s);
      case 256: return launch_pair<T, DQK, 256>(p, masked, s);
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (dv) {
      case 16: return launch_pair<T, DQK, 16>(p, masked, s);
      case 32: return launch_pair<T, DQK, 32>(p, masked, s);
      case 64: return launch_pair<T, DQK, 64>(p, masked, s);
      default: return hipErrorInvalidValue;
    }
  }
}

}  // namespace attn_jvp
