// vfm_k_i8.hip -- kernel set: int8 weights with fp32 per-column scales, bf16 activations (W8A16).
#include "vfm_phases.h"

namespace vfm {
VFM_DEFINE_KERNEL_SET(ks_i8, bf16, WF_I8, false, 64, 128, 256)
}  // namespace vfm
