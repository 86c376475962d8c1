// Host-side validation and launch planning of the attn_jvp C ABI (host.cpp):
// plain C++, no HIP runtime.  The launching entry points (attn_jvp.hip)
// validate every call here first and launch nothing on error.

#pragma once

#include <stddef.h>
#include <stdint.h>

#include "attn_jvp.h"
#include "plan.h"

namespace attn_jvp {

// Launches are one-dimensional: the work-item count (workgroups x threads)
// must fit in 32 bits and the workgroup count in 31.
bool grid_fits(int64_t workgroups, int threads);

bool mask_on(const attn_jvp_mask *mask);
int check_mask(const attn_jvp_mask *mask, int Nq, int Nkv);
MaskDev to_dev(const attn_jvp_mask *mask);

// Geometry of a built forward instance; false if (dtype, d_qk, d_v) is not
// built.
bool shape_for(int dtype, int dqk, int dv, FwdGeom *out);

// Does an unsplit forward launch of this call take the small geometry
// (fwd16_geom_small)?  set_small switches a launch's parameters to it.
bool launch_small(const attn_jvp_shape &s, int dtype, const attn_jvp_mask *mask);
void set_small(Params *p, int dtype, const attn_jvp_shape &s);

attn_jvp_layout contiguous(const attn_jvp_shape &s);
attn_jvp_bwd_layout contiguous_bwd(const attn_jvp_shape &s);
attn_jvp_shape square(int B, int H, int N, int d);

// Validate a forward call.  out_esize: bytes per O / dO element (0: the
// dtype's; 4 for float32 partials).  nsplit: key splits of the launch.
int check_args(const void *Q, const void *K, const void *V, const void *dQ, const void *dK,
               const void *dV, const void *O, const void *dO, const float *LSE,
               const float *dLSE, const attn_jvp_shape *shape, int dtype,
               const attn_jvp_layout *L, const attn_jvp_mask *mask, int out_esize = 0,
               int nsplit = 1);

Params make_params(const void *Q, const void *K, const void *V, const void *dQ, const void *dK,
                   const void *dV, void *O, void *dO, float *LSE, float *dLSE,
                   const attn_jvp_shape &shape, float scale, int dtype,
                   const attn_jvp_layout &L, const attn_jvp_mask *mask);

// float32 partial outputs of a call: contiguous [B, H, Lq, d_v] in floats.
void partial_out_strides(const attn_jvp_shape &s, attn_jvp_layout *L);

// Split-KV workspace: O, dO partials [ns, B, H, Lq, d_v] then LSE, dLSE
// partials [ns, B, H, Lq], float32, each region 256-byte aligned.
struct SplitWs {
  size_t o, dout, lse, dlse, total;
};
SplitWs split_workspace(const attn_jvp_shape &s, int ns);

// Key splits for one call (1: no split).
int choose_splits(const attn_jvp_shape &s, int dtype, const attn_jvp_mask *mask);

// The workspace of a split call: 256-byte aligned, at least `need` bytes,
// overlapping none of the call's tensors.
int check_workspace(const void *workspace, size_t workspace_bytes, size_t need,
                    const void *const tensors[10], const attn_jvp_shape &s, int dtype,
                    const attn_jvp_layout &L);

int check_bwd(const void *Q, const void *K, const void *V, const void *O, const void *gO,
              const float *LSE, const void *gQ, const void *gK, const void *gV,
              const float *delta, const attn_jvp_shape *shape, int dtype,
              const attn_jvp_bwd_layout *L, const attn_jvp_mask *mask);

BwdParams make_bwd_params(const void *Q, const void *K, const void *V, const void *O,
                          const void *gO, const float *LSE, void *gQ, void *gK, void *gV,
                          float *delta, const attn_jvp_shape &shape, float scale, int dtype,
                          const attn_jvp_bwd_layout &L, const attn_jvp_mask *mask);

int check_merge(int num_parts, const float *O_parts, const float *dO_parts,
                const float *LSE_parts, const float *dLSE_parts, const void *O, const void *dO,
                const float *LSE, const float *dLSE, int B, int H, int Lq, int d_v, int dtype,
                const int64_t *o_strides, MergeParams *m);

}  // namespace attn_jvp
