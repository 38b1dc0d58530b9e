// vfm_stage_io.h -- what a plan (vfm_plan.cpp) needs to know of the objects
// its stages run: the device byte ranges a denoise call or a prefix pass
// reads and writes, and whether the launch holds every compute unit.
#pragma once
#include <stddef.h>

#include <vector>

#include "vfm.h"

namespace vfm {

// Error text for vfm_last_error() (defined with the expert's runtime).
vfm_status report(vfm_status s, const char* fmt, ...);

struct IoRange {
  const void* ptr;
  size_t bytes;
};

struct StageIO {
  std::vector<IoRange> reads, writes;
  const void* owner = nullptr;   // the producer or expert whose private workspace the stage uses
  bool device_wide = false;      // a persistent kernel with device-wide barriers
};

// Ranges of vfm_denoise(x, noise, state, actions) with the expert's current
// bindings (NULL pointers: the bound buffers). VFM_E_UNBOUND when a needed
// buffer is not bound.
vfm_status expert_stage_io(const vfm_expert* x, const float* noise, const float* state, const float* actions,
                           StageIO* io);

// Ranges of vfm_prefix_run(p, embeds, B, P, prefix_k, prefix_v). VFM_E_SHAPE
// when B or P is outside the producer's limits.
vfm_status prefix_stage_io(const vfm_prefix* p, const void* embeds, int B, int P, const void* prefix_k,
                           const void* prefix_v, StageIO* io);

}  // namespace vfm
