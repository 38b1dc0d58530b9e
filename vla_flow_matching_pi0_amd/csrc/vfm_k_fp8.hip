// vfm_k_fp8.hip -- kernel set: FP8 e4m3 weights, bf16 activations quantised at the GEMM input.
#include "vfm_phases.h"

namespace vfm {
VFM_DEFINE_KERNEL_SET(ks_fp8, bf16, WF_FP8, false, 64, 128, 256)
}  // namespace vfm
