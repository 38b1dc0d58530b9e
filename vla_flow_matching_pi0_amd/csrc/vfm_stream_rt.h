// vfm_stream_rt.h -- host side of the streaming batch-1 kernel: work plans,
// workspace, create-time tables and the launch (used by vfm_runtime.cpp).
#pragma once
#include <hip/hip_runtime.h>

#include <string>
#include <vector>

#include "vfm.h"
#include "vfm_stream_params.h"

namespace vfm {
namespace sk {

struct StreamShape {
  int L, W, Hq, Hkv, d, F, H, A, S, N, maxP;
  float eps;
};

// One GEMM's plan: tile t runs on XCD t % 8; the workgroups of an XCD are
// grouped by K split so that the units of one workgroup share their split.
struct GemmPlanH {
  int T = 0, S = 1, nkb = 0, nkbs = 0, U = 0;
  std::vector<uint32_t> units;   // [G][U]
};

// Plans and sizes that depend only on shapes and the device (testable on the host).
struct StreamPlan {
  int G = 0, per_xcd = 0;
  GemmPlanH g[4];
  GemmPlanH in;                  // in projection: W/16 tiles, no split
  int regions[4] = {0, 0, 0, 0}, scratch = 0, ctl = 0, lds = 0;
};

// Build the plan; returns false with a reason when the shape does not fit the
// kernel (then the expert keeps the other launch modes).
bool stream_plan(const StreamShape& s, int G, const int splits[4], StreamPlan* out, std::string* why);
// Attention plan for prefix length P: unit (head j, 32-key split c) on XCD j % 8.
bool stream_attn_plan(const StreamShape& s, int G, int per_xcd, int P, std::vector<uint32_t>* units, int* AU, int* KS,
                      int* KSp, std::string* why);

struct StreamState;

// Launch settings that do not change results.
struct StreamTune {
  int stop_after = 0;        // diagnostics: leave after this barrier (0: the whole loop)
  int dma_cap = DMA_CAP;     // loader: most direct-to-LDS loads in flight, 1 .. 63
  int fail_epoch = 0;        // diagnostics: barrier made unreachable (0: none)
  long spin_limit = SPIN_LIMIT;   // polls before a device-wide or head wait gives up
};

vfm_status stream_create(const StreamShape& shape, const uint8_t* const* wq, const uint8_t* const* wo,
                         const uint8_t* const* wg, const uint8_t* const* wd, const float* mod, hipStream_t st,
                         StreamState** out, std::string* why);
void stream_destroy(StreamState* s);
// Whether a call with prefix length P fits (P <= maxP and the attention plan fits).
bool stream_accepts(const StreamState* s, int P, std::string* why);
vfm_status stream_run(StreamState* s, int P, const void* pk, const void* pv, const float* noise, const float* state,
                      float* x, const float* in_w, const float* in_b, const float* st_w, const float* st_b,
                      const float* out_w, const float* out_b, const float* rope, bool cooperative,
                      unsigned long long* trace, const StreamTune& tune, hipStream_t st);
// Device-side failure flagged by an earlier launch (host-mapped word; no synchronisation).
bool stream_failed(const StreamState* s);
// Clear the failure and every counter a failed launch may have left behind (enqueued on st).
hipError_t stream_reset(StreamState* s, hipStream_t st);
// Barriers per launch (trace layout: word triples (arrive, counters complete, workgroup ready) per barrier
// after the start triple).
int stream_barriers(const StreamState* s);
const StreamPlan& stream_plan_of(const StreamState* s);
// Diagnostics: raw bytes of an internal buffer ("slab" of step/layer index k L + l, "h", "s_emb", "vt",
// "apart", "aml", "shw_q", "shw_g"), synchronous.
vfm_status stream_debug_copy(const StreamState* s, const std::string& name, int index, void* dst, size_t bytes);
// Byte offsets within a slab of y_attn, ss_attn, q, k, v^T, attn, y_mlp, ss_mlp, act; returns the slab size.
size_t stream_slab_layout(const StreamState* s, size_t* offs);

}  // namespace sk
}  // namespace vfm
