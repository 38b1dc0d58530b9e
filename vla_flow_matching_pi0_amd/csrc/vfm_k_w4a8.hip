// vfm_k_w4a8.hip -- kernel set: int4 weights with fp16 group scales, e4m3 activations (W4A8).
#include "vfm_phases.h"

namespace vfm {
VFM_DEFINE_KERNEL_SET(ks_w4a8, bf16, WF_W4A8, false, 64, 128, 256)
}  // namespace vfm
