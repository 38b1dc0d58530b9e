// vfm_k_w4.hip -- kernel set: int4 weights with fp16 group scales, bf16 activations.
#include "vfm_phases.h"

namespace vfm {
VFM_DEFINE_KERNEL_SET(ks_w4, bf16, WF_W4, false, 64, 128, 256)
}  // namespace vfm
