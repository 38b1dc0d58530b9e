// vfm_launch.cpp -- picks the kernel set of an expert (activation type,
// weight format, calibration) and sizes the persistent grid.
#include "vfm_params.h"

namespace vfm {

#define VFM_DECLARE_KERNEL_SET(NAME)                                                                              \
  hipError_t NAME##_launch(const VP& p, int mode, int phase, int k, int l, int grid, size_t lds, hipStream_t st); \
  hipError_t NAME##_prepare(int d, int lds);                                                                      \
  hipError_t NAME##_occupancy(int d, size_t lds, int* per_cu);
VFM_DECLARE_KERNEL_SET(ks_f32)
VFM_DECLARE_KERNEL_SET(ks_bf16)
VFM_DECLARE_KERNEL_SET(ks_cal)
VFM_DECLARE_KERNEL_SET(ks_fp8)
VFM_DECLARE_KERNEL_SET(ks_w4)
VFM_DECLARE_KERNEL_SET(ks_i8)
VFM_DECLARE_KERNEL_SET(ks_w4a8)

// LDS of the row phases (norms, step boundary): the boundary's reduction
// slots, row, per-thread partials and action row, which covers the norms'
// reduction slots too.
static size_t row_lds_bytes(const VP& p) { return (NTHREADS / 64 + p.W + 4 * NTHREADS + MAX_A_HOST) * 4; }

size_t lds_bytes(const VP& p, int act_bytes) {
  const size_t nwaves = NTHREADS / 64;
  const size_t gemm = nwaves * 2 * 4 * 64 * 16;
  const size_t epc = 16 / act_bytes;
  const size_t attn = ((size_t)ATT_KEYS_HOST * (p.d + epc) + (size_t)p.d * (ATT_KEYS_HOST + epc)) * act_bytes;
  const size_t row = row_lds_bytes(p);
  size_t m = gemm > attn ? gemm : attn;
  return m > row ? m : row;
}

hipError_t prepare_kernels(int kset, int d, int lds) {
  switch (kset) {
    case KS_F32: return ks_f32_prepare(d, lds);
    case KS_BF16: return ks_bf16_prepare(d, lds);
    case KS_CAL: return ks_cal_prepare(d, lds);
    case KS_FP8: return ks_fp8_prepare(d, lds);
    case KS_W4: return ks_w4_prepare(d, lds);
    case KS_I8: return ks_i8_prepare(d, lds);
    case KS_W4A8: return ks_w4a8_prepare(d, lds);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_phase(const VP& p, int kset, int mode, int phase, int k, int l, int grid, size_t lds,
                        hipStream_t st) {
  // A phase launched on its own takes only the LDS its own kernel uses: the
  // row phases then fit several workgroups per compute unit (one row each)
  // instead of the two that the GEMM phases' allocation would allow.
  if (mode != 0 && mode != 3 &&
      (phase == PH_RN_ATTN || phase == PH_RN_MLP || phase == PH_BOUNDARY || phase == PH_COMBINE)) {
    const size_t row = row_lds_bytes(p);
    if (row < lds) lds = row;
  }
  switch (kset) {
    case KS_F32: return ks_f32_launch(p, mode, phase, k, l, grid, lds, st);
    case KS_BF16: return ks_bf16_launch(p, mode, phase, k, l, grid, lds, st);
    case KS_CAL: return ks_cal_launch(p, mode, phase, k, l, grid, lds, st);
    case KS_FP8: return ks_fp8_launch(p, mode, phase, k, l, grid, lds, st);
    case KS_W4: return ks_w4_launch(p, mode, phase, k, l, grid, lds, st);
    case KS_I8: return ks_i8_launch(p, mode, phase, k, l, grid, lds, st);
    case KS_W4A8: return ks_w4a8_launch(p, mode, phase, k, l, grid, lds, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t max_cooperative_grid(int kset, int d, size_t lds, int* grid) {
  int per_cu = 0;
  hipError_t e;
  switch (kset) {
    case KS_F32: e = ks_f32_occupancy(d, lds, &per_cu); break;
    case KS_BF16: e = ks_bf16_occupancy(d, lds, &per_cu); break;
    case KS_FP8: e = ks_fp8_occupancy(d, lds, &per_cu); break;
    case KS_W4: e = ks_w4_occupancy(d, lds, &per_cu); break;
    case KS_I8: e = ks_i8_occupancy(d, lds, &per_cu); break;
    case KS_W4A8: e = ks_w4a8_occupancy(d, lds, &per_cu); break;
    default: e = hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  int dev = 0, cus = 0;
  e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  *grid = per_cu >= 1 ? cus : 0;
  return hipSuccess;
}

}  // namespace vfm
