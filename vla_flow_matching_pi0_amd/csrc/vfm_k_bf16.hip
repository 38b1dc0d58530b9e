// vfm_k_bf16.hip -- kernel set: bf16 weights and activations.
#include "vfm_phases.h"

namespace vfm {
VFM_DEFINE_KERNEL_SET(ks_bf16, bf16, WF_NATIVE, false, 64, 128, 256)
}  // namespace vfm
