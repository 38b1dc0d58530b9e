// vfm_k_attn.hip -- the large-batch attention kernel (k_attn_m), compiled
// on its own so that its build flags (MFMA accumulators in VGPRs) do not
// reach the other kernels.
#define VFM_ATTN_M_INSTANTIATE
#include "vfm_phases.h"

namespace vfm {
template __global__ void k_attn_m<bf16, 64>(VP, int, int);
template __global__ void k_attn_m<bf16, 128>(VP, int, int);
template __global__ void k_attn_m<bf16, 256>(VP, int, int);
}  // namespace vfm
