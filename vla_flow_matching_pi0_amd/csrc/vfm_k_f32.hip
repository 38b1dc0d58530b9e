// vfm_k_f32.hip -- kernel set: fp32 weights and activations (head_dim 64, 128).
#include "vfm_phases.h"

namespace vfm {
VFM_DEFINE_KERNEL_SET(ks_f32, float, WF_NATIVE, false, 64, 128)
}  // namespace vfm
