// vfm_k_cal.hip -- kernel set: the FP8 calibration pass: bf16 phase kernels whose GEMMs record the largest |input|.
#include "vfm_phases.h"

namespace vfm {
VFM_DEFINE_KERNEL_SET(ks_cal, bf16, WF_NATIVE, true, 64, 128, 256)
}  // namespace vfm
