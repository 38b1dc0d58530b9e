// vfm_plan.cpp -- C ABI of plans (include/vfm.h, vfm_plan_*): stages with
// update rates, dependencies derived per tick from the device ranges each due
// stage reads and writes, one stream per stage, and every tick forked from and
// joined back into the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <vector>

#include "vfm.h"
#include "vfm_stage_io.h"

using namespace vfm;

namespace {

constexpr int MAX_STAGES = 256;

enum Kind { K_PREFIX = 0, K_DENOISE = 1, K_GRAPH = 2 };

struct Stage {
  int kind = K_GRAPH;
  vfm_prefix* pre = nullptr;
  vfm_expert* ex = nullptr;
  hipGraphExec_t graph = nullptr;
  const void* in0 = nullptr;   // prefix: embeddings; denoise: noise (NULL: bound)
  const void* in1 = nullptr;   // denoise: state (NULL: bound)
  void* out0 = nullptr;        // prefix: prefix_k; denoise: actions (NULL: bound)
  void* out1 = nullptr;        // prefix: prefix_v
  int B = 0, P = 0;
  int every = 1, offset = 0;
  std::vector<IoRange> g_reads, g_writes;   // an adopted graph's declared ranges
  std::vector<int> edges_from;              // declared dependencies on earlier stages
  hipStream_t stream = nullptr;
  hipEvent_t done = nullptr;
};

bool due(const Stage& s, int64_t t) { return t >= s.offset && (t - s.offset) % s.every == 0; }

bool overlap(const IoRange& a, const IoRange& b) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.ptr), b0 = reinterpret_cast<uintptr_t>(b.ptr);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

bool any_overlap(const std::vector<IoRange>& x, const std::vector<IoRange>& y) {
  for (const IoRange& a : x)
    for (const IoRange& b : y)
      if (overlap(a, b)) return true;
  return false;
}

// Must the later stage j wait for the earlier stage i? Read-after-write,
// write-after-read and write-after-write on any range, a shared producer or
// expert (its private workspace), or a launch that holds the whole device.
bool conflict(const StageIO& i, const StageIO& j) {
  if (i.device_wide || j.device_wide) return true;
  if (i.owner && i.owner == j.owner) return true;
  return any_overlap(i.writes, j.reads) || any_overlap(i.writes, j.writes) || any_overlap(i.reads, j.writes);
}

vfm_status stage_io(const Stage& s, StageIO* io) {
  switch (s.kind) {
    case K_PREFIX:
      return prefix_stage_io(s.pre, s.in0, s.B, s.P, s.out0, s.out1, io);
    case K_DENOISE:
      return expert_stage_io(s.ex, static_cast<const float*>(s.in0), static_cast<const float*>(s.in1),
                             static_cast<const float*>(s.out0), io);
    default:
      io->reads = s.g_reads;
      io->writes = s.g_writes;
      io->owner = s.graph;   // one executable graph is never launched twice at once
      io->device_wide = false;
      return VFM_OK;
  }
}

vfm_status check_rate(int32_t every, int32_t offset) {
  if (every < 1) return report(VFM_E_INVALID_ARG, "every must be >= 1 (got %d)", every);
  if (offset < 0 || offset >= every) return report(VFM_E_INVALID_ARG, "offset %d outside [0, every)", offset);
  return VFM_OK;
}

bool misaligned(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 != 0; }

}  // namespace

struct vfm_plan {
  std::vector<Stage> st;
  hipEvent_t entry = nullptr;

  // The due stages of tick t (ascending) and their ranges; for each, the
  // positions in `run` of the stages it waits for.
  vfm_status schedule(int64_t t, std::vector<int>* run, std::vector<std::vector<int>>* waits) const {
    run->clear();
    for (int j = 0; j < (int)st.size(); ++j)
      if (due(st[j], t)) run->push_back(j);
    std::vector<StageIO> io(run->size());
    for (size_t k = 0; k < run->size(); ++k) {
      const vfm_status s = stage_io(st[(*run)[k]], &io[k]);
      if (s != VFM_OK) return s;
    }
    waits->assign(run->size(), {});
    for (size_t k = 0; k < run->size(); ++k) {
      const Stage& sj = st[(*run)[k]];
      for (size_t k2 = 0; k2 < k; ++k2) {
        const int i = (*run)[k2];
        const bool edge = std::find(sj.edges_from.begin(), sj.edges_from.end(), i) != sj.edges_from.end();
        if (edge || conflict(io[k2], io[k])) (*waits)[k].push_back((int)k2);
      }
    }
    return VFM_OK;
  }

  vfm_status add(Stage s, int32_t* id) {
    if ((int)st.size() >= MAX_STAGES) return report(VFM_E_INVALID_ARG, "a plan holds at most %d stages", MAX_STAGES);
    st.push_back(std::move(s));
    if (id) *id = (int32_t)st.size() - 1;
    return VFM_OK;
  }
};

extern "C" {

vfm_status vfm_plan_create(vfm_plan** out) {
  if (!out) return report(VFM_E_INVALID_ARG, "out is NULL");
  *out = new vfm_plan();
  return VFM_OK;
}

vfm_status vfm_plan_add_prefix(vfm_plan* pl, vfm_prefix* pre, const void* embeds, int32_t batch, int32_t prefix_len,
                               void* prefix_k, void* prefix_v, int32_t every, int32_t offset, int32_t* stage) {
  if (!pl || !pre || !embeds || !prefix_k || !prefix_v) return report(VFM_E_INVALID_ARG, "NULL argument");
  if (misaligned(embeds) || misaligned(prefix_k) || misaligned(prefix_v))
    return report(VFM_E_INVALID_ARG, "buffers must be 16-byte aligned");
  vfm_status s = check_rate(every, offset);
  if (s != VFM_OK) return s;
  StageIO io;
  if ((s = prefix_stage_io(pre, embeds, batch, prefix_len, prefix_k, prefix_v, &io)) != VFM_OK) return s;
  Stage g;
  g.kind = K_PREFIX;
  g.pre = pre;
  g.in0 = embeds;
  g.out0 = prefix_k;
  g.out1 = prefix_v;
  g.B = batch;
  g.P = prefix_len;
  g.every = every;
  g.offset = offset;
  return pl->add(std::move(g), stage);
}

vfm_status vfm_plan_add_denoise(vfm_plan* pl, vfm_expert* ex, const float* noise, const float* state, float* actions,
                                int32_t every, int32_t offset, int32_t* stage) {
  if (!pl || !ex) return report(VFM_E_INVALID_ARG, "NULL argument");
  if (misaligned(noise) || misaligned(state) || misaligned(actions))
    return report(VFM_E_INVALID_ARG, "noise / state / actions must be 16-byte aligned");
  const vfm_status s = check_rate(every, offset);
  if (s != VFM_OK) return s;
  Stage g;
  g.kind = K_DENOISE;
  g.ex = ex;
  g.in0 = noise;
  g.in1 = state;
  g.out0 = actions;
  g.every = every;
  g.offset = offset;
  return pl->add(std::move(g), stage);
}

vfm_status vfm_plan_add_graph(vfm_plan* pl, void* graph_exec, const vfm_range* reads, int32_t n_reads,
                              const vfm_range* writes, int32_t n_writes, int32_t every, int32_t offset,
                              int32_t* stage) {
  if (!pl || !graph_exec) return report(VFM_E_INVALID_ARG, "NULL argument");
  if (n_reads < 0 || n_writes < 0 || (n_reads > 0 && !reads) || (n_writes > 0 && !writes))
    return report(VFM_E_INVALID_ARG, "range lists do not match their counts");
  const vfm_status s = check_rate(every, offset);
  if (s != VFM_OK) return s;
  Stage g;
  g.kind = K_GRAPH;
  g.graph = static_cast<hipGraphExec_t>(graph_exec);
  for (int i = 0; i < n_reads + n_writes; ++i) {
    const vfm_range& r = i < n_reads ? reads[i] : writes[i - n_reads];
    if (!r.ptr || r.bytes == 0) return report(VFM_E_INVALID_ARG, "range %d has a NULL pointer or 0 bytes", i);
    (i < n_reads ? g.g_reads : g.g_writes).push_back({r.ptr, r.bytes});
  }
  g.every = every;
  g.offset = offset;
  return pl->add(std::move(g), stage);
}

vfm_status vfm_plan_add_edge(vfm_plan* pl, int32_t from, int32_t to) {
  if (!pl) return report(VFM_E_INVALID_ARG, "plan is NULL");
  const int n = (int)pl->st.size();
  if (from < 0 || to < 0 || from >= n || to >= n || from >= to)
    return report(VFM_E_INVALID_ARG, "edge %d -> %d: need 0 <= from < to < %d", from, to, n);
  std::vector<int>& e = pl->st[to].edges_from;
  if (std::find(e.begin(), e.end(), from) == e.end()) e.push_back(from);
  return VFM_OK;
}

vfm_status vfm_plan_deps(vfm_plan* pl, int64_t tick, int32_t stage, int32_t* deps, int32_t cap, int32_t* n) {
  if (!pl || !n || cap < 0 || (cap > 0 && !deps)) return report(VFM_E_INVALID_ARG, "NULL argument");
  if (tick < 0) return report(VFM_E_INVALID_ARG, "tick must be >= 0");
  if (stage < 0 || stage >= (int)pl->st.size()) return report(VFM_E_INVALID_ARG, "stage %d out of range", stage);
  std::vector<int> run;
  std::vector<std::vector<int>> waits;
  const vfm_status s = pl->schedule(tick, &run, &waits);
  if (s != VFM_OK) return s;
  const auto it = std::find(run.begin(), run.end(), stage);
  if (it == run.end()) {
    *n = -1;
    return VFM_OK;
  }
  const std::vector<int>& w = waits[it - run.begin()];
  *n = (int32_t)w.size();
  for (int k = 0; k < (int)w.size() && k < cap; ++k) deps[k] = run[w[k]];
  return VFM_OK;
}

vfm_status vfm_plan_run(vfm_plan* pl, int64_t tick, void* stream) {
  if (!pl) return report(VFM_E_INVALID_ARG, "plan is NULL");
  if (tick < 0) return report(VFM_E_INVALID_ARG, "tick must be >= 0");
  std::vector<int> run;
  std::vector<std::vector<int>> waits;
  vfm_status result = pl->schedule(tick, &run, &waits);
  if (result != VFM_OK || run.empty()) return result;

  // Streams and events on first use (default priority, no blocking on the
  // legacy stream).
  hipError_t e = hipSuccess;
  if (!pl->entry) e = hipEventCreateWithFlags(&pl->entry, hipEventDisableTiming);
  for (int j : run) {
    Stage& g = pl->st[j];
    if (e == hipSuccess && !g.stream) e = hipStreamCreateWithFlags(&g.stream, hipStreamNonBlocking);
    if (e == hipSuccess && !g.done) e = hipEventCreateWithFlags(&g.done, hipEventDisableTiming);
  }
  if (e != hipSuccess) return report(VFM_E_HIP, "plan streams: %s", hipGetErrorString(e));

  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((e = hipEventRecord(pl->entry, s)) != hipSuccess) return report(VFM_E_HIP, "hipEventRecord: %s", hipGetErrorString(e));
  std::vector<int> enqueued;
  for (size_t k = 0; k < run.size() && result == VFM_OK; ++k) {
    Stage& g = pl->st[run[k]];
    e = hipStreamWaitEvent(g.stream, pl->entry, 0);
    for (int k2 : waits[k])
      if (e == hipSuccess) e = hipStreamWaitEvent(g.stream, pl->st[run[k2]].done, 0);
    if (e != hipSuccess) {
      result = report(VFM_E_HIP, "hipStreamWaitEvent: %s", hipGetErrorString(e));
      break;
    }
    switch (g.kind) {
      case K_PREFIX:
        result = vfm_prefix_run(g.pre, g.in0, g.B, g.P, g.out0, g.out1, g.stream);
        break;
      case K_DENOISE:
        result = vfm_denoise(g.ex, static_cast<const float*>(g.in0), static_cast<const float*>(g.in1),
                             static_cast<float*>(g.out0), g.stream);
        break;
      default:
        e = hipGraphLaunch(g.graph, g.stream);
        if (e != hipSuccess) result = report(VFM_E_HIP, "hipGraphLaunch: %s", hipGetErrorString(e));
        break;
    }
    // Joined even after a failure, so that whatever the stage did enqueue
    // stays ordered before later work on the caller's stream.
    e = hipEventRecord(g.done, g.stream);
    if (e != hipSuccess) {
      if (result == VFM_OK) result = report(VFM_E_HIP, "hipEventRecord: %s", hipGetErrorString(e));
      break;
    }
    enqueued.push_back(run[k]);
  }
  for (int j : enqueued) {
    e = hipStreamWaitEvent(s, pl->st[j].done, 0);
    if (e != hipSuccess && result == VFM_OK) result = report(VFM_E_HIP, "hipStreamWaitEvent: %s", hipGetErrorString(e));
  }
  return result;
}

vfm_status vfm_plan_destroy(vfm_plan* pl) {
  if (!pl) return VFM_OK;
  for (Stage& g : pl->st) {
    if (g.stream) {
      (void)hipStreamSynchronize(g.stream);
      (void)hipStreamDestroy(g.stream);
    }
    if (g.done) (void)hipEventDestroy(g.done);
  }
  if (pl->entry) (void)hipEventDestroy(pl->entry);
  delete pl;
  return VFM_OK;
}

}  // extern "C"
