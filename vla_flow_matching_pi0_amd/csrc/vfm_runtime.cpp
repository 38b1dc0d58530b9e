// vfm_runtime.cpp -- host runtime behind the C ABI in include/vfm.h:
// config and weight validation, create-time packing, the named-buffer
// registry, launch modes (persistent / graph / eager) and error reporting.
//
// Named device buffers as the only state and replay of a captured launch
// sequence keyed by its shape follow the FlashRT walk-through (exec/: Buffer
// and Graph objects; component 7, graph capture with pointer-only inputs).
#include "vfm.h"
#include "vfm_params.h"
#include "vfm_stage_io.h"
#include "vfm_stream_rt.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <cstring>
#include <map>
#include <string>
#include <vector>

using vfm::VP;

namespace {

thread_local std::string g_err;

vfm_status fail(vfm_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

#define HIPCHK(call)                                                                          \
  do {                                                                                        \
    hipError_t e_ = (call);                                                                   \
    if (e_ != hipSuccess) return fail(VFM_E_HIP, "%s failed: %s", #call, hipGetErrorString(e_)); \
  } while (0)

struct BoundBuf {
  void* ptr = nullptr;
  int dtype = -1;
  int ndim = 0;
  int64_t shape[5] = {0, 0, 0, 0, 0};
  bool bound = false;
};

// Column map of one fused, packed weight: packed column -> (source, column).
struct ColMap {
  std::vector<int> src, idx;
};

}  // namespace

struct vfm_expert {
  vfm_config cfg{};
  int act_bf16 = 0;       // activations are bf16 (else f32)
  int src_bf16 = 0;       // master weights are bf16 (else f32)
  int wprec = VFM_W_FP32; // storage of the per-layer GEMM weights
  int kset = vfm::KS_F32; // kernel set of the hot path
  int KW = 16;            // K per 16-byte weight block of a lane (16 f32, 32 bf16, 64 fp8, 128 int4)
  unsigned* wamax = nullptr;        // FP8: [L][4] largest |weight| of each fused tensor (device, float bits)
  std::vector<float> wscale;        // FP8: [L][4] weight scales
  std::vector<float> act_scale;     // FP8: [L][4] activation scales (empty until calibrated or set)
  float* qs = nullptr;              // FP8: device [L][4][alpha, 1/act_scale]
  int L = 0, W = 0, Hq = 0, Hkv = 0, d = 0, F = 0, H = 0, A = 0, S = 0, E = 0, N = 0;
  int pi0 = 0;            // variant pi0: a state token before the action tokens
  int T = 0;              // suffix tokens per sample: H (+1 for pi0)
  uint8_t* w_tmlp = nullptr;   // pi0: packed time-MLP output weight
  float *tbias = nullptr, *tmlp_b = nullptr;
  int maxB = 0, maxP = 0, KSmax = 0;
  std::vector<void*> allocs;
  std::vector<uint8_t*> w_qkv, w_o, w_gu, w_down;
  ColMap map_qkv, map_o, map_gu, map_down;
  float *in_w = nullptr, *in_b = nullptr, *st_w = nullptr, *st_b = nullptr, *out_w = nullptr, *out_b = nullptr;
  float* mod = nullptr;
  float* rope = nullptr;
  int rope_P = -1;
  float* s_emb = nullptr;
  float* h = nullptr;
  float *part_o = nullptr, *part_d = nullptr;
  uint8_t* ring = nullptr;     // write-once activation slabs, one per (step, layer)
  size_t slab = 0, off_xna = 0, off_q = 0, off_k = 0, off_v = 0, off_attn = 0, off_xnm = 0, off_act = 0, off_u = 0;
  float *opart = nullptr, *ml = nullptr;
  unsigned* bar = nullptr;
  unsigned long long* trace = nullptr;   // phase timeline (option "trace")
  size_t trace_words = 0;
  unsigned* herr = nullptr;        // pinned, host-mapped: set by a persistent launch whose barrier wait gave up
  unsigned* herr_dev = nullptr;    // its device address
  BoundBuf prefix_k, prefix_v, noise, state, actions;
  int mode = 3;                    // 0 persistent, 1 graph, 2 eager, 3 auto, 4 stream (see launch_mode_of)
  vfm::sk::StreamState* ss = nullptr;   // streaming batch-1 kernel (bf16 pi0.5 experts whose shapes fit it)
  std::string ss_why;                    // why there is none
  int ss_P = -1;                         // prefix length of the last stream-eligibility check
  bool ss_P_ok = false;
  vfm::sk::StreamTune ss_tune;          // streaming kernel launch settings (diagnostics, loader depth)
  long spin_limit = vfm::BARRIER_SPIN_LIMIT_HOST;   // polls before a device-wide wait gives up
  int fail_barrier = 0;                  // diagnostics: barrier made unreachable (0: none)
  size_t lds = 0;
  int coop_grid = 0;
  bool coop_launch = true;   // persistent kernel: cooperative launch (else an ordinary one of the same grid)
  int gemm_tiles = 0;        // large-M GEMMs: 0 auto, 1 128-column tiles only, 2 256-column tiles where they apply
  // norms folded into the persistent kernel's GEMMs (bf16 pi0.5 experts, W a multiple of 256 up to 1024)
  bool can_fuse = false;
  // option "fused_norms": -1 auto (fold where the call has at most
  // FOLD_AUTO_ROWS rows), 1 at any size, 0 never
  int fuse_norms = -1;
  float *shw_q = nullptr, *shw_g = nullptr;   // [N][L][columns] shift W per step, layer and norm
  size_t off_ssa = 0, off_ssm = 0;            // slab offsets of the per-tile sums of squares [Mpad][W/16]
  unsigned* fcnt = nullptr;                   // [2][FCNT_MAX] split arrival counters
  // XCD-local split exchange of the fused kernel (option "xcd_local"): its
  // counters are never cleared by the kernel, so the host clears them when
  // the split plan changes (xl_plan: S and column groups of o and down) or a
  // launch failed
  bool xcd_local = true;
  bool xcd_attn = true;                       // ... and the attention splits with their merge
  bool attn_merge = true;                     // option "attn_merge": the persistent kernels' in-place merge
  unsigned* xcnt = nullptr;                   // [2][FCNT_MAX] counters, XCNT_STRIDE words apart
  unsigned* hcnt = nullptr;                   // [HCNT_MAX] attention head counters, HCNT_STRIDE words apart
  long long xl_plan = -1;
  // graph variants, most recently used first: key = shape + pointers
  struct GraphEntry {
    std::vector<uintptr_t> key;
    hipGraphExec_t exec;
  };
  std::vector<GraphEntry> graphs;
  int graph_cap = 8;
  hipStream_t cap_stream = nullptr;

  void drop_graphs() {
    for (GraphEntry& g : graphs) (void)hipGraphExecDestroy(g.exec);
    graphs.clear();
  }

  void* dalloc(size_t bytes) {
    void* p = nullptr;
    if (bytes == 0) bytes = 16;
    if (hipMalloc(&p, bytes) != hipSuccess) return nullptr;
    allocs.push_back(p);
    return p;
  }
};

namespace {

// GEMM inputs are e4m3 with calibrated activation scales (FP8 and W4A8).
bool fp8_act(const vfm_expert* x) { return x->wprec == VFM_W_FP8 || x->wprec == VFM_W_W4A8; }

// Launch mode of a call with M = B x T rows. "auto" takes graph launch where
// the large-batch kernels apply (bf16 weights, M >= 256 rows: large-M GEMM
// tiles and single-pass attention), else the persistent kernel, which is the
// faster one while the GEMMs are skinny.
bool stream_fits(const vfm_expert* x, int B, int P) {
  if (!x->ss || B != 1) return false;
  vfm_expert* m = const_cast<vfm_expert*>(x);
  if (P != m->ss_P) {
    std::string why;
    m->ss_P_ok = vfm::sk::stream_accepts(x->ss, P, &why);
    m->ss_P = P;
  }
  return m->ss_P_ok;
}

int launch_mode_of(const vfm_expert* x, int B, int P) {
  if (x->mode != 3) return x->mode;
  return (x->kset == vfm::KS_BF16 && B * x->T >= 256) ? 1 : 0;
}

// Host decoders of the packed formats (export only).
float e4m3_value(uint8_t c) {
  const int e = (c >> 3) & 15, m = c & 7;
  const float v = e == 0 ? (float)m * 0.001953125f : std::ldexp(1.0f + (float)m * 0.125f, e - 7);
  return (c & 0x80) ? -v : v;
}
float half_value(uint16_t h) {
  const int e = (h >> 10) & 31, m = h & 1023;
  float v;
  if (e == 0) v = std::ldexp((float)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = std::ldexp(1.0f + (float)m / 1024.0f, e - 15);
  return (h & 0x8000) ? -v : v;
}

int elem_bytes(int dt) { return dt == VFM_F32 ? 4 : dt == VFM_BF16 || dt == VFM_F16 ? 2 : 1; }

vfm_status validate_config(const vfm_config* c) {
  if (!c) return fail(VFM_E_INVALID_ARG, "config is NULL");
  if (c->abi_version != VFM_ABI_VERSION)
    return fail(VFM_E_INVALID_ARG, "abi_version %d != %d", c->abi_version, VFM_ABI_VERSION);
  if (c->num_layers < 0 || c->num_layers > vfm::MAX_LAYERS)
    return fail(VFM_E_INVALID_ARG, "num_layers %d outside [0, %d]", c->num_layers, vfm::MAX_LAYERS);
  if (c->width < 256 || c->width % 256 != 0 || c->width > 2048)
    return fail(VFM_E_INVALID_ARG, "width %d must be a multiple of 256 in [256, 2048]", c->width);
  if (c->num_kv_heads < 1 || c->num_q_heads < 1 || c->num_q_heads % c->num_kv_heads != 0)
    return fail(VFM_E_INVALID_ARG, "num_q_heads %d must be a positive multiple of num_kv_heads %d", c->num_q_heads,
                c->num_kv_heads);
  if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256)
    return fail(VFM_E_INVALID_ARG, "head_dim %d must be 64, 128 or 256", c->head_dim);
  if (c->act_dtype == VFM_F32 && c->head_dim > 128)
    return fail(VFM_E_INVALID_ARG, "fp32 experts support head_dim <= 128");
  if ((c->num_q_heads * c->head_dim) % 256 != 0)
    return fail(VFM_E_INVALID_ARG, "num_q_heads * head_dim must be a multiple of 256");
  if (c->mlp_dim < 256 || c->mlp_dim % 256 != 0 || c->mlp_dim > 65536)
    return fail(VFM_E_INVALID_ARG, "mlp_dim %d must be a multiple of 256 in [256, 65536]", c->mlp_dim);
  if (c->action_horizon < 1 || c->action_horizon > 64)
    return fail(VFM_E_INVALID_ARG, "action_horizon %d outside [1, 64]", c->action_horizon);
  if (c->action_dim != 4 && c->action_dim != 8 && c->action_dim != 16 && c->action_dim != 32 && c->action_dim != 64)
    return fail(VFM_E_INVALID_ARG, "action_dim %d must be 4, 8, 16, 32 or 64", c->action_dim);
  if (c->state_dim < 0 || c->state_dim > 4096) return fail(VFM_E_INVALID_ARG, "state_dim %d out of range", c->state_dim);
  if (c->time_emb_dim < 4 || c->time_emb_dim % 2 != 0 || c->time_emb_dim > 8192)
    return fail(VFM_E_INVALID_ARG, "time_emb_dim %d must be even in [4, 8192]", c->time_emb_dim);
  if (c->max_prefix_len < 1 || c->max_prefix_len > 4000)
    return fail(VFM_E_INVALID_ARG, "max_prefix_len %d outside [1, 4000]", c->max_prefix_len);
  if (c->max_batch < 1 || c->max_batch > 1024) return fail(VFM_E_INVALID_ARG, "max_batch %d outside [1, 1024]", c->max_batch);
  if (c->num_steps < 1 || c->num_steps > 1000) return fail(VFM_E_INVALID_ARG, "num_steps %d outside [1, 1000]", c->num_steps);
  if (!(c->rope_base > 0.f)) return fail(VFM_E_INVALID_ARG, "rope_base must be > 0");
  if (!(c->rms_eps > 0.f)) return fail(VFM_E_INVALID_ARG, "rms_eps must be > 0");
  if (c->weight_precision < VFM_W_FP32 || c->weight_precision > VFM_W_W4A8)
    return fail(VFM_E_INVALID_ARG, "weight_precision %d unknown", c->weight_precision);
  if (c->variant != VFM_VARIANT_PI05 && c->variant != VFM_VARIANT_PI0)
    return fail(VFM_E_INVALID_ARG, "variant %d unknown", c->variant);
  if (c->variant == VFM_VARIANT_PI0) {
    if (c->weight_precision != VFM_W_FP32 && c->weight_precision != VFM_W_BF16)
      return fail(VFM_E_UNSUPPORTED, "the pi0 variant is built for fp32 and bf16 weights");
    if (c->state_dim < 1) return fail(VFM_E_INVALID_ARG, "the pi0 variant needs a state input (state_dim >= 1)");
    if (c->time_emb_dim != c->width) return fail(VFM_E_INVALID_ARG, "the pi0 variant needs time_emb_dim == width");
    if (c->action_horizon > 63) return fail(VFM_E_INVALID_ARG, "the pi0 variant takes at most 63 action tokens");
    if (c->num_layers < 1) return fail(VFM_E_INVALID_ARG, "the pi0 variant needs at least one layer");
  }
  if (c->weight_precision == VFM_W_FP32 && c->act_dtype != VFM_F32)
    return fail(VFM_E_INVALID_ARG, "fp32 weights need act_dtype VFM_F32");
  if (c->weight_precision != VFM_W_FP32 && c->act_dtype != VFM_BF16)
    return fail(VFM_E_INVALID_ARG, "16-bit and quantised weights need act_dtype VFM_BF16");
  if (c->weight_precision >= VFM_W_FP8) {
    // every wave of a GEMM workgroup takes at least one 16-byte weight block
    const bool w4 = c->weight_precision == VFM_W_W4A16 || c->weight_precision == VFM_W_W4A8;
    const int span = (w4 ? 128 : 64) * (vfm::NTHREADS / 64);
    if (c->width % span || (c->num_q_heads * c->head_dim) % span || c->mlp_dim % span)
      return fail(VFM_E_INVALID_ARG, "quantised weights need width, num_q_heads * head_dim and mlp_dim to be "
                  "multiples of %d", span);
    if (w4 && c->w4_group_size != 128)
      return fail(VFM_E_UNSUPPORTED, "w4_group_size %d: only 128 is built", c->w4_group_size);
  }
  return VFM_OK;
}

// Whether the persistent kernel can fold the norms into its GEMMs: bf16
// pi0.5 experts whose width is a multiple of 256 up to 1024 (a GEMM lane
// reads at most 16 per-tile sums of squares of a row).
// The folded norms' shift W tables over the weights the GEMMs multiply by
// (bf16, dequantised int4, or int8 codes times their column scales).
hipError_t shift_tables(vfm_expert* x, int L, int W, int Nq, int F, int n_norms, hipStream_t s) {
  if (x->kset == vfm::KS_BF16) {
    hipError_t e = vfm::sk::shift_proj(x->shw_q, x->w_qkv.data(), L, W, Nq, x->mod, n_norms, 0, W, x->N, s);
    if (e == hipSuccess) e = vfm::sk::shift_proj(x->shw_g, x->w_gu.data(), L, W, 2 * F, x->mod, n_norms, 1, W, x->N, s);
    return e;
  }
  const int fmt = x->kset == vfm::KS_W4 ? 1 : 2;
  hipError_t e = vfm::sk::shift_proj_q(x->shw_q, x->w_qkv.data(), L, W, Nq, x->mod, n_norms, 0, W, x->N, fmt, s);
  if (e == hipSuccess) e = vfm::sk::shift_proj_q(x->shw_g, x->w_gu.data(), L, W, 2 * F, x->mod, n_norms, 1, W, x->N, fmt, s);
  return e;
}

// fused_norms "auto": fold the norms into the GEMMs where the call has at
// most this many rows (two 64-row tiles: batch 1 and 2 of pi0.5)
constexpr long FOLD_AUTO_ROWS = 128;

bool can_fold_norms(const vfm_config* c) {
  const int w = c->weight_precision;
  return (w == VFM_W_BF16 || w == VFM_W_W4A16 || w == VFM_W_W8A16) && c->variant != VFM_VARIANT_PI0 &&
         c->num_layers > 0 && c->width % 256 == 0 && c->width <= 1024;
}

// The kernels address every buffer through 32-bit byte offsets from its
// base (buffer resources of up to 2 GiB): refuse configurations whose largest
// buffer would not fit.
constexpr size_t WORKSPACE_MAX = 64ull << 30;   // largest workspace an expert may allocate

vfm_status check_extents(const vfm_config* c) {
  const size_t ab = c->act_dtype == VFM_F32 ? 4 : 2;
  const size_t L = c->num_layers, W = c->width, Hq = c->num_q_heads, Hkv = c->num_kv_heads, d = c->head_dim;
  const size_t F = c->mlp_dim, H = c->action_horizon + (c->variant == VFM_VARIANT_PI0), N = c->num_steps;
  const size_t B = c->max_batch, P = c->max_prefix_len;
  const size_t M = B * H, Mpad = (M + 63) / 64 * 64;
  const size_t KS = (P + vfm::ATT_KEYS_HOST - 1) / vfm::ATT_KEYS_HOST + (H + vfm::ATT_KEYS_HOST - 1) / vfm::ATT_KEYS_HOST;
  struct { const char* what; size_t bytes; } ext[] = {
      {"modulation table", N * (2 * L + 1) * 3 * W * 4},
      {"residual stream", M * W * 4},
      {"K-split partial sums", (size_t)vfm::MAX_KSPLIT * M * W * 4},
      {"one layer of the prefix K/V", B * P * Hkv * d * ab},
      {"gate/up GEMM input or output", std::max(Mpad * W, F * Mpad) * ab},
      {"attention output", Mpad * Hq * d * ab},
      {"attention split outputs", B * Hq * KS * 64 * d * 4},
      {"packed gate/up weight", W * 2 * F * 4},
  };
  for (const auto& e : ext)
    if (e.bytes > 0x7FFFFFF0ull)
      return fail(VFM_E_UNSUPPORTED, "the %s would take %zu bytes, beyond the 2 GiB one buffer offset addresses "
                  "(reduce max_batch, max_prefix_len, num_steps or the widths)", e.what, e.bytes);
  // total workspace: the write-once activation ring (one slab per step and
  // layer, the slab of create's layout) plus the per-call buffers
  auto al = [](size_t b) { return (b + 4095) / 4096 * 4096; };
  const size_t slab = al(Mpad * W * ab) + al(B * Hq * d * 64 * ab) + 2 * al(B * Hkv * d * 64 * ab) +
                      al(Mpad * Hq * d * ab) + al(Mpad * W * ab) + al(F * Mpad * ab) +
                      (c->variant == VFM_VARIANT_PI0 ? al(Mpad * W * ab) : 0) +
                      (can_fold_norms(c) ? 2 * al(Mpad * (W / 16) * 4) : 0);
  const size_t ring = slab * N * std::max<size_t>(L, 1);
  const size_t other = M * W * 4 * (2 + 2 * (size_t)vfm::MAX_KSPLIT) + B * Hq * KS * 64 * (d + 2) * 4;
  if (ring + other > WORKSPACE_MAX)
    return fail(VFM_E_UNSUPPORTED, "the workspace would take %zu bytes (activation ring %zu = slab %zu x %zu steps x "
                "%zu layers), beyond the %zu the library accepts (reduce max_batch or num_steps)",
                ring + other, ring, slab, N, std::max<size_t>(L, 1), WORKSPACE_MAX);
  return VFM_OK;
}

struct WeightSpec {
  std::string name;
  std::vector<int64_t> shape;
};

std::vector<WeightSpec> weight_specs(const vfm_expert& x) {
  std::vector<WeightSpec> v;
  const int64_t W = x.W, E = x.E, A = x.A, S = x.S, F = x.F, qd = (int64_t)x.Hq * x.d, kd = (int64_t)x.Hkv * x.d;
  if (x.pi0) {
    // action-time MLP on [action ; time] (2W -> W -> W), state token, plain (1 + w) norms
    v.push_back({"time_mlp_in.w", {2 * W, W}});
    v.push_back({"time_mlp_in.b", {W}});
    v.push_back({"time_mlp_out.w", {W, W}});
    v.push_back({"time_mlp_out.b", {W}});
    v.push_back({"in_proj.w", {A, W}});
    v.push_back({"in_proj.b", {W}});
    v.push_back({"state_proj.w", {S, W}});
    v.push_back({"state_proj.b", {W}});
    for (int l = 0; l < x.L; ++l) {
      const std::string p = "layers." + std::to_string(l) + ".";
      v.push_back({p + "attn_norm.w", {W}});
      v.push_back({p + "q.w", {W, qd}});
      v.push_back({p + "k.w", {W, kd}});
      v.push_back({p + "v.w", {W, kd}});
      v.push_back({p + "o.w", {qd, W}});
      v.push_back({p + "mlp_norm.w", {W}});
      v.push_back({p + "gate.w", {W, F}});
      v.push_back({p + "up.w", {W, F}});
      v.push_back({p + "down.w", {F, W}});
    }
    v.push_back({"final_norm.w", {W}});
    v.push_back({"out_proj.w", {W, A}});
    v.push_back({"out_proj.b", {A}});
    return v;
  }
  v.push_back({"time_mlp_in.w", {E, W}});
  v.push_back({"time_mlp_in.b", {W}});
  v.push_back({"time_mlp_out.w", {W, W}});
  v.push_back({"time_mlp_out.b", {W}});
  v.push_back({"in_proj.w", {A, W}});
  v.push_back({"in_proj.b", {W}});
  if (S > 0) {
    v.push_back({"state_proj.w", {S, W}});
    v.push_back({"state_proj.b", {W}});
  }
  for (int l = 0; l < x.L; ++l) {
    const std::string p = "layers." + std::to_string(l) + ".";
    v.push_back({p + "attn_norm.mod.w", {W, 3 * W}});
    v.push_back({p + "attn_norm.mod.b", {3 * W}});
    v.push_back({p + "q.w", {W, qd}});
    v.push_back({p + "k.w", {W, kd}});
    v.push_back({p + "v.w", {W, kd}});
    v.push_back({p + "o.w", {qd, W}});
    v.push_back({p + "mlp_norm.mod.w", {W, 3 * W}});
    v.push_back({p + "mlp_norm.mod.b", {3 * W}});
    v.push_back({p + "gate.w", {W, F}});
    v.push_back({p + "up.w", {W, F}});
    v.push_back({p + "down.w", {F, W}});
  }
  v.push_back({"final_norm.mod.w", {W, 3 * W}});
  v.push_back({"final_norm.mod.b", {3 * W}});
  v.push_back({"out_proj.w", {W, A}});
  v.push_back({"out_proj.b", {A}});
  return v;
}

// Packed column orders (see the GEMM epilogues in vfm_kernels.hip).
ColMap qkv_map(int Hq, int Hkv, int d) {
  ColMap m;
  const int heads = Hq + 2 * Hkv, hd = d / 2;
  for (int head = 0; head < heads; ++head) {
    const int sid = head < Hq ? 0 : head < Hq + Hkv ? 1 : 2;
    const int base = (head < Hq ? head : head < Hq + Hkv ? head - Hq : head - Hq - Hkv) * d;
    for (int tt = 0; tt < d / 16; ++tt)
      for (int g = 0; g < 4; ++g)
        for (int r = 0; r < 4; ++r) {
          int col;
          if (sid < 2) col = tt * 8 + 2 * g + (r & 1) + (r >> 1) * hd;   // rotary pairs in one lane
          else col = tt * 16 + 4 * g + r;
          m.src.push_back(sid);
          m.idx.push_back(base + col);
        }
  }
  return m;
}
ColMap gu_map(int F) {
  ColMap m;
  for (int t = 0; t < F / 8; ++t)
    for (int g = 0; g < 4; ++g)
      for (int r = 0; r < 4; ++r) {
        m.src.push_back(r & 1);              // gate, up, gate, up
        m.idx.push_back(t * 8 + 2 * g + (r >> 1));
      }
  return m;
}
ColMap ident_map(int N) {
  ColMap m;
  for (int c = 0; c < N; ++c) {
    m.src.push_back(0);
    m.idx.push_back(c);
  }
  return m;
}

void free_all(vfm_expert* x) {
  x->drop_graphs();
  vfm::sk::stream_destroy(x->ss);
  x->ss = nullptr;
  if (x->cap_stream) (void)hipStreamDestroy(x->cap_stream);
  if (x->herr) (void)hipHostFree(x->herr);
  for (void* p : x->allocs) (void)hipFree(p);
  x->allocs.clear();
}

// A persistent launch whose barrier wait gave up raised the host-mapped
// error word (and the sticky device word bar[1]); report it once, and clear
// both and the arrival counters that launch left behind (ordered on `s`).
// No synchronisation: a failure not yet visible is reported by a later call
// or by vfm_check, which synchronises first.
vfm_status check_host_err(vfm_expert* x, hipStream_t s) {
  if (!x->herr || __atomic_load_n(x->herr, __ATOMIC_ACQUIRE) == 0u) return VFM_OK;
  *x->herr = 0u;
  (void)vfm::zero_words(x->bar, vfm::BAR_WORDS, s);
  if (x->fcnt) (void)vfm::zero_words(x->fcnt, 2 * vfm::FCNT_MAX, s);
  if (x->xcnt) (void)vfm::zero_words(x->xcnt, vfm::XCNT_WORDS, s);
  if (x->hcnt) (void)vfm::zero_words(x->hcnt, (vfm::HCNT_MAX + 2 * vfm::QCNT_KV) * vfm::HCNT_STRIDE, s);
  x->xl_plan = -1;
  (void)hipStreamSynchronize(s);
  return fail(VFM_E_HIP, "a device-wide phase barrier timed out in an earlier denoise call");
}

// A streaming launch that failed (a barrier that timed out) raised the
// host-mapped error word; report it once and clear every counter it may have
// left behind.
vfm_status check_stream_flag(vfm_expert* x, hipStream_t s) {
  if (!x->ss || !vfm::sk::stream_failed(x->ss)) return VFM_OK;
  (void)vfm::sk::stream_reset(x->ss, s);
  return fail(VFM_E_HIP, "a device-wide barrier of the streaming kernel timed out in an earlier denoise call");
}

vfm_status check_buf(const char* name, const BoundBuf& b, int dtype, std::initializer_list<int64_t> shape) {
  if (!b.bound) return fail(VFM_E_UNBOUND, "buffer '%s' is not bound", name);
  if (b.dtype != dtype) return fail(VFM_E_DTYPE, "buffer '%s' has dtype %d, expected %d", name, b.dtype, dtype);
  if (b.ndim != (int)shape.size()) return fail(VFM_E_SHAPE, "buffer '%s' has %d dims, expected %d", name, b.ndim, (int)shape.size());
  int i = 0;
  for (int64_t s : shape) {
    if (b.shape[i] != s)
      return fail(VFM_E_SHAPE, "buffer '%s' dim %d is %lld, expected %lld", name, i, (long long)b.shape[i], (long long)s);
    ++i;
  }
  return VFM_OK;
}

int phase_grid(const VP& p, int phase) {
  auto cdiv = [](long a, long b) { return (int)((a + b - 1) / b); };
  const int mt = cdiv(p.M, 64);
  long units = 1;
  if (p.bigm) {
    // large-M GEMM kernels: one workgroup per 128 x 128 tile and K split, rounded up to whole XCD rounds
    // (wide tiles, 224 or 256 tokens: 256 columns)
    auto mtl = [&](int i) { return cdiv(p.M, p.gp_bm[i]); };
    auto ncol = [&](int i) { return p.gp_bm[i] > 128 ? 256 : 128; };
    long tiles = -1;
    switch (phase) {
      case vfm::PH_QKV: tiles = (long)(p.Hq + 2 * p.Hkv) * p.d / ncol(0) * mtl(0) * p.gp_s[0]; break;
      case vfm::PH_O: tiles = (long)p.W / ncol(1) * mtl(1) * p.gp_s[1]; break;
      case vfm::PH_GU: tiles = (long)2 * p.F / ncol(2) * mtl(2) * p.gp_s[2]; break;
      case vfm::PH_DOWN: tiles = (long)p.W / ncol(3) * mtl(3) * p.gp_s[3]; break;
      case vfm::PH_TMLP: tiles = (long)p.W / ncol(4) * mtl(4) * p.gp_s[4]; break;
      // single-pass attention: one workgroup per (sample, head), samples in groups of 8 (one per XCD)
      case vfm::PH_ATTN: tiles = (long)cdiv(p.B, 8) * 8 * p.Hq; break;
      default: break;
    }
    if (tiles > 0) return (int)((tiles + 7) / 8 * 8);
  }
  switch (phase) {
    case vfm::PH_BOUNDARY: units = p.M; break;
    case vfm::PH_RN_ATTN:
    case vfm::PH_RN_MLP: units = p.bigm && p.W <= 2 * vfm::NTHREADS ? cdiv(p.M, 2) : p.M; break;
    case vfm::PH_QKV: units = (long)(p.Hq + 2 * p.Hkv) * p.d / (16 * p.gp_nt[0]) * p.gp_s[0] * mt; break;
    case vfm::PH_O: units = (long)p.W / (16 * p.gp_nt[1]) * p.gp_s[1] * mt; break;
    case vfm::PH_GU: units = (long)2 * p.F / (16 * p.gp_nt[2]) * p.gp_s[2] * mt; break;
    case vfm::PH_DOWN: units = (long)p.W / (16 * p.gp_nt[3]) * p.gp_s[3] * mt; break;
    case vfm::PH_TMLP: units = (long)p.W / (16 * p.gp_nt[4]) * p.gp_s[4] * mt; break;
    case vfm::PH_ATTN: units = (long)p.B * p.Hq * p.KS; break;
    case vfm::PH_COMBINE: units = cdiv((long)p.M * p.Hq, vfm::NTHREADS / 64); break;
  }
  if (units < 1) units = 1;
  if (units > 8192) units = 8192;
  return (int)units;
}

hipError_t enqueue_phases(vfm_expert* x, const VP& p, int kset, hipStream_t st) {
  hipError_t e;
  auto run = [&](int ph, int k, int l) { return vfm::launch_phase(p, kset, 1, ph, k, l, phase_grid(p, ph), x->lds, st); };
  if ((e = run(vfm::PH_BOUNDARY, 0, 0)) != hipSuccess) return e;
  for (int k = 0; k < p.N; ++k) {
    if (p.pi0 && ((e = run(vfm::PH_TMLP, k, 0)) != hipSuccess || (e = run(vfm::PH_RN_ATTN, k, 0)) != hipSuccess)) return e;
    for (int l = 0; l < p.L; ++l) {
      if (l > 0 && (e = run(vfm::PH_RN_ATTN, k, l)) != hipSuccess) return e;
      const int seq[] = {vfm::PH_QKV, vfm::PH_ATTN, vfm::PH_COMBINE, vfm::PH_O, vfm::PH_RN_MLP, vfm::PH_GU, vfm::PH_DOWN};
      for (int ph : seq) {
        if (ph == vfm::PH_COMBINE && p.bigm) continue;   // the single-pass attention writes the o input itself
        if ((e = run(ph, k, l)) != hipSuccess) return e;
      }
    }
    if ((e = run(vfm::PH_BOUNDARY, k + 1, 0)) != hipSuccess) return e;
  }
  return hipSuccess;
}

// GEMM plan: nt 16-column tiles per work unit and S splits of K, so that a
// phase has about one unit per workgroup. Only linear epilogues split K.
void plan_gemm(int M, int N, int K, int KB, int nwg, bool linear, int* nt, int* S) {
  const int tiles = N / 16, mt = (M + 63) / 64, waves = vfm::NTHREADS / 64;
  int smax = 1;
  if (linear)
    while (smax * 2 <= vfm::MAX_KSPLIT && K % (smax * 2 * KB * waves) == 0) smax *= 2;
  // one 16-column tile per unit unless there are at least two tiles per
  // workgroup; then the fewest K splits that give every workgroup a unit
  // (measured on the pi0.5 shapes: o and down run fastest as 64 tiles x 4
  // splits, gate/up as 256 pairs of tiles)
  *nt = (tiles % 2 == 0 && (long)tiles * mt >= 2L * nwg) ? 2 : 1;
  int s = 1;
  while (s * 2 <= smax && (long)(tiles / *nt) * mt * s < nwg) s *= 2;
  *S = s;
}

}  // namespace

namespace vfm {
vfm_status report(vfm_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

vfm_status expert_stage_io(const vfm_expert* x, const float* noise, const float* state, const float* actions,
                           StageIO* io) {
  if (!x || !io) return report(VFM_E_INVALID_ARG, "NULL argument");
  if (!x->prefix_k.bound || !x->prefix_v.bound) return report(VFM_E_UNBOUND, "prefix_k / prefix_v are not bound");
  const size_t B = (size_t)x->prefix_k.shape[1], P = (size_t)x->prefix_k.shape[2];
  const size_t kv = (size_t)x->L * B * P * x->Hkv * x->d * (x->act_bf16 ? 2 : 4);
  const size_t xa = B * x->H * x->A * 4;
  if (!noise && !x->noise.bound) return report(VFM_E_UNBOUND, "buffer 'noise' is not bound");
  if (!actions && !x->actions.bound) return report(VFM_E_UNBOUND, "buffer 'actions' is not bound");
  if (x->S > 0 && !state && !x->state.bound) return report(VFM_E_UNBOUND, "buffer 'state' is not bound");
  io->reads = {{x->prefix_k.ptr, kv}, {x->prefix_v.ptr, kv}, {noise ? noise : x->noise.ptr, xa}};
  if (x->S > 0) io->reads.push_back({state ? state : x->state.ptr, B * x->S * 4});
  io->writes = {{actions ? actions : x->actions.ptr, xa}};
  io->owner = x;
  const int lm = launch_mode_of(x, (int)B, (int)P);
  io->device_wide = lm == 0 || lm == 4;
  return VFM_OK;
}
}  // namespace vfm

// Whether large-M GEMM i (qkv, o, gate/up, down, time MLP) of N columns runs
// the 256-column tiles: gate/up by default, any GEMM when asked for. At batch
// 32 (pi0.5 widths) the others measured no faster: qkv's 2560 columns make
// too few tiles, and o and down need twice the K splits, whose partial sums
// the next row phase then reads.
static bool wide_tiles(const vfm_expert* x, int i, int N) {
  if (N % 256 != 0 || x->gemm_tiles == 1) return false;
  return x->gemm_tiles == 2 || i == 2;
}

// The launch parameter block of one call: shapes, weights, workspace,
// buffers and the GEMM plan for the expert's weight format.
vfm_status fill_vp(vfm_expert* x, VP& p, int B, int P, const float* noise, const float* state, float* actions) {
  p.L = x->L; p.W = x->W; p.Hq = x->Hq; p.Hkv = x->Hkv; p.d = x->d; p.F = x->F; p.H = x->T; p.A = x->A;
  p.S = x->S; p.N = x->N; p.B = B; p.P = P; p.M = B * x->T; p.n_norms = 2 * x->L + 1;
  p.pi0 = x->pi0;
  p.w_tmlp = x->w_tmlp; p.tbias = x->tbias; p.tmlp_b = x->tmlp_b; p.off_u = x->off_u;
  constexpr int AK = vfm::ATT_KEYS_HOST;   // keys per attention split
  p.kps = AK;
  p.KS = (P + AK - 1) / AK + (x->T + AK - 1) / AK;   // prefix splits, then chunk splits
  p.eps = x->cfg.rms_eps;
  for (int l = 0; l < x->L; ++l) {
    p.w_qkv[l] = x->w_qkv[l]; p.w_o[l] = x->w_o[l]; p.w_gu[l] = x->w_gu[l]; p.w_down[l] = x->w_down[l];
  }
  p.in_w = x->in_w; p.in_b = x->in_b; p.st_w = x->st_w; p.st_b = x->st_b; p.out_w = x->out_w; p.out_b = x->out_b;
  p.mod = x->mod; p.rope = x->rope;
  p.prefix_k = x->prefix_k.ptr; p.prefix_v = x->prefix_v.ptr;
  p.noise = noise; p.state = state; p.x = actions;
  p.s_emb = x->s_emb; p.h = x->h; p.part_o = x->part_o; p.part_d = x->part_d; p.opart = x->opart; p.ml = x->ml;
  p.ring = x->ring; p.slab = x->slab; p.off_xna = x->off_xna; p.off_q = x->off_q; p.off_k = x->off_k; p.off_v = x->off_v;
  p.off_attn = x->off_attn; p.off_xnm = x->off_xnm; p.off_act = x->off_act; p.bar = x->bar;
  const int mode = launch_mode_of(x, B, P);
  p.trace = mode == 0 ? x->trace : nullptr;
  p.spin_limit = x->spin_limit;
  p.fail_epoch = mode == 0 ? x->fail_barrier : 0;
  p.herr = mode == 0 ? x->herr_dev : nullptr;

  {
    int nwg = x->coop_grid;
    if (nwg == 0) {
      HIPCHK(vfm::max_cooperative_grid(x->kset, x->d, x->lds, &x->coop_grid));
      if (x->coop_grid == 0) return fail(VFM_E_HIP, "persistent kernel does not fit on a compute unit");
      nwg = x->coop_grid;
    }
    const int KB = x->KW;
    const int Ks[5] = {x->W, x->Hq * x->d, x->W, x->F, x->W};
    const int Ns[5] = {(x->Hq + 2 * x->Hkv) * x->d, x->W, 2 * x->F, x->W, x->W};
    for (int i = 0; i < 5; ++i) plan_gemm(p.M, Ns[i], Ks[i], KB, nwg, i != 0 && i != 2, &p.gp_nt[i], &p.gp_s[i]);
    // many rows in the per-phase launch modes: 128 x 128 tiles of the large-M GEMM kernel, and K splits of
    // the linear GEMMs until there are 256 tiles, each split a whole number of 64-K stages
    p.bigm = mode != 0 && x->kset == vfm::KS_BF16 && p.M >= 256;
    if (p.bigm) {
      const int mt = (p.M + 127) / 128;
      for (int i = 0; i < 5; ++i) {
        int sp = 1;
        if (i != 0 && i != 2)
          while (sp < vfm::MAX_KSPLIT && (long)(Ns[i] / 128) * mt * sp < 256 && Ks[i] % (sp * 2 * 64) == 0) sp *= 2;
        p.gp_nt[i] = 8;
        p.gp_s[i] = sp;
        // 128-token tiles just past one per compute unit (256 < tiles <= 384) would run a second round on a
        // few units: 64-token tiles spread the same work about two per unit, both resident at once
        const long t128 = (long)(Ns[i] / 128) * mt * sp;
        p.gp_bm[i] = (t128 > 256 && t128 <= 384) ? 64 : 128;
        if (wide_tiles(x, i, Ns[i])) {
          // 256 columns x 224 or 256 tokens, one tile per compute unit: the token count with the fewer
          // tokens per unit over the whole grid, and for the linear GEMMs K splits (whole 32-K stages)
          // until the tiles fill the 256 units
          int best_bm = 224, best_sp = 1;
          long best_cost = -1;
          for (int bmw : {224, 256}) {
            const long mtw = (p.M + bmw - 1) / bmw;
            int spw = 1;
            if (i != 0 && i != 2)
              while (spw < vfm::MAX_KSPLIT && (long)(Ns[i] / 256) * mtw * spw < 256 && Ks[i] % (spw * 2 * 32) == 0)
                spw *= 2;
            // the kernel's pipeline takes an even number of 32-K stages, at least its ring depth less one
            const int nst = Ks[i] / spw / 32, ring = bmw == 224 ? vfm::GW_RING_224 : vfm::GW_RING_256;
            if (Ks[i] % (spw * 32) != 0 || nst % 2 != 0 || nst < ring - 1) continue;
            const long tiles = (long)(Ns[i] / 256) * mtw * spw;
            const long cost = (tiles + 255) / 256 * bmw * (Ks[i] / spw);
            if (best_cost < 0 || cost < best_cost) best_cost = cost, best_bm = bmw, best_sp = spw;
          }
          if (best_cost >= 0) {
            p.gp_bm[i] = best_bm;
            p.gp_s[i] = best_sp;
          }
        }
      }
    }
    p.S_o = p.gp_s[1];
    p.S_down = p.gp_s[3];
  }
  // the persistent kernel's in-place attention merge with counter-scoped
  // attention start (every persistent kernel whose shapes its counters take)
  const bool merge = mode == 0 && x->attn_merge && (long)B * p.Hq <= vfm::HCNT_MAX && p.Hq <= vfm::QCNT_KV &&
                     p.Hkv <= vfm::QCNT_KV && p.d % (16 * p.gp_nt[0]) == 0;
  p.hcnt = x->hcnt;
  p.qcnt = x->hcnt + (size_t)vfm::HCNT_MAX * vfm::HCNT_STRIDE;
  // separate-norm kernel: a head's attention splits on one XCD (bit 1) and
  // the in-place merge (XL_MERGE)
  p.xl = (mode == 0 && x->xcd_local && x->xcd_attn && x->coop_grid % 8 == 0 ? 2 : 0) | (merge ? vfm::XL_MERGE : 0);
  p.fuse = 0;
  // auto: the folded kernel saves four barriers per layer, which is what a
  // call of one or two samples waits on; from four samples (200 rows) on
  // the split-sum exchanges and the per-row scaling cost more than that
  // (0.4 % slower at 4 samples, 5 % at 32)
  const bool fold = x->fuse_norms > 0 || (x->fuse_norms < 0 && p.M <= FOLD_AUTO_ROWS);
  if (mode == 0 && x->can_fuse && fold && merge) {
    const long mt = (p.M + 63) / 64;
    const long go = (long)p.W / (16 * p.gp_nt[1]) * mt, gd = (long)p.W / (16 * p.gp_nt[3]) * mt;
    if (go <= vfm::FCNT_MAX && gd <= vfm::FCNT_MAX) {
      p.fuse = 1;
      p.shw_q = x->shw_q; p.shw_g = x->shw_g; p.off_ssa = x->off_ssa; p.off_ssm = x->off_ssm; p.fcnt = x->fcnt;
      // XCD-local split sums: every unit of a column group on one XCD (the
      // column-group count and the grid multiples of 8) and a power-of-two
      // split count (the never-cleared counters stay multiples of S, also
      // across a 32-bit wrap)
      // (the folded-norm kernel: any non-zero p.xl selects the XCD-local sums, bit 1
      // the attention placement too; it always merges in place)
      const long ngo = (long)p.W / (16 * p.gp_nt[1]), ngd = (long)p.W / (16 * p.gp_nt[3]);
      auto pow2 = [](int v) { return v > 0 && (v & (v - 1)) == 0; };
      p.xl = x->xcd_local && x->coop_grid % 8 == 0 && ngo % 8 == 0 && ngd % 8 == 0 && pow2(p.gp_s[1]) &&
             pow2(p.gp_s[3]) ? (x->xcd_attn ? 3 : 1) : 0;
      p.xcnt = x->xcnt;
    }
  }
  p.qs = x->qs;
  p.amax = nullptr;
  return VFM_OK;
}

extern "C" {

int vfm_abi_version(void) { return VFM_ABI_VERSION; }

const char* vfm_last_error(void) { return g_err.c_str(); }

vfm_status vfm_expert_create(const vfm_config* cfg, const vfm_tensor* weights, int32_t n_weights, void* stream,
                             vfm_expert** out) {
  if (!out) return fail(VFM_E_INVALID_ARG, "out is NULL");
  *out = nullptr;
  vfm_status st = validate_config(cfg);
  if (st != VFM_OK) return st;
  if ((st = check_extents(cfg)) != VFM_OK) return st;
  if (!weights || n_weights <= 0) return fail(VFM_E_INVALID_ARG, "no weights given");

  vfm_expert tmp;
  tmp.cfg = *cfg;
  tmp.act_bf16 = cfg->act_dtype == VFM_BF16;
  tmp.src_bf16 = cfg->weight_precision != VFM_W_FP32;
  tmp.wprec = cfg->weight_precision;
  tmp.kset = tmp.wprec == VFM_W_FP32 ? vfm::KS_F32 : tmp.wprec == VFM_W_BF16 ? vfm::KS_BF16
           : tmp.wprec == VFM_W_FP8 ? vfm::KS_FP8 : tmp.wprec == VFM_W_W8A16 ? vfm::KS_I8
           : tmp.wprec == VFM_W_W4A8 ? vfm::KS_W4A8 : vfm::KS_W4;
  tmp.KW = tmp.wprec == VFM_W_FP32 ? 16 : tmp.wprec == VFM_W_BF16 ? 32
         : (tmp.wprec == VFM_W_W4A16 || tmp.wprec == VFM_W_W4A8) ? 128 : 64;
  tmp.L = cfg->num_layers; tmp.W = cfg->width; tmp.Hq = cfg->num_q_heads; tmp.Hkv = cfg->num_kv_heads;
  tmp.d = cfg->head_dim; tmp.F = cfg->mlp_dim; tmp.H = cfg->action_horizon; tmp.A = cfg->action_dim;
  tmp.S = cfg->state_dim; tmp.E = cfg->time_emb_dim; tmp.N = cfg->num_steps;
  tmp.maxB = cfg->max_batch; tmp.maxP = cfg->max_prefix_len;
  tmp.pi0 = cfg->variant == VFM_VARIANT_PI0;
  tmp.T = tmp.H + tmp.pi0;

  // ---- weights: every expected name exactly once, right dtype and shape, nothing else
  const int master_dt = tmp.src_bf16 ? VFM_BF16 : VFM_F32;
  std::map<std::string, const vfm_tensor*> byname;
  for (int i = 0; i < n_weights; ++i) {
    const vfm_tensor& t = weights[i];
    if (!t.name) return fail(VFM_E_INVALID_ARG, "weight %d has no name", i);
    if (byname.count(t.name)) return fail(VFM_E_INVALID_ARG, "weight '%s' given twice", t.name);
    byname[t.name] = &t;
  }
  const std::vector<WeightSpec> specs = weight_specs(tmp);
  std::map<std::string, const void*> ptr;
  for (const WeightSpec& sp : specs) {
    auto it = byname.find(sp.name);
    if (it == byname.end()) return fail(VFM_E_INVALID_ARG, "weight '%s' is missing", sp.name.c_str());
    const vfm_tensor& t = *it->second;
    if (!t.dev_ptr) return fail(VFM_E_INVALID_ARG, "weight '%s' has a NULL pointer", sp.name.c_str());
    if (t.dtype != master_dt) return fail(VFM_E_DTYPE, "weight '%s' has dtype %d, expected %d", sp.name.c_str(), t.dtype, master_dt);
    if (t.ndim != (int)sp.shape.size()) return fail(VFM_E_SHAPE, "weight '%s' has %d dims, expected %d", sp.name.c_str(), t.ndim, (int)sp.shape.size());
    for (size_t j = 0; j < sp.shape.size(); ++j)
      if (t.shape[j] != sp.shape[j])
        return fail(VFM_E_SHAPE, "weight '%s' dim %zu is %lld, expected %lld", sp.name.c_str(), j, (long long)t.shape[j], (long long)sp.shape[j]);
    ptr[sp.name] = t.dev_ptr;
  }
  if (byname.size() != specs.size()) {
    for (auto& kv : byname) {
      bool known = false;
      for (const WeightSpec& sp : specs) known |= sp.name == kv.first;
      if (!known) return fail(VFM_E_INVALID_ARG, "unknown weight name '%s'", kv.first.c_str());
    }
  }

  // ---- device work
  vfm_expert* x = new vfm_expert(tmp);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  auto bail = [&](vfm_status code) { free_all(x); delete x; return code; };
  const int ab = x->act_bf16 ? 2 : 4;
  const int L = x->L, W = x->W, Hq = x->Hq, Hkv = x->Hkv, d = x->d, F = x->F, H = x->H, A = x->A, S = x->S;
  const int n_norms = 2 * L + 1;
  const int nqkv = (Hq + 2 * Hkv) * d;

  x->map_qkv = qkv_map(Hq, Hkv, d);
  x->map_o = ident_map(W);
  x->map_gu = gu_map(F);
  x->map_down = ident_map(W);

  // upload column maps
  auto upload_map = [&](const ColMap& m, int** dsrc, int** didx) -> bool {
    *dsrc = (int*)x->dalloc(m.src.size() * 4);
    *didx = (int*)x->dalloc(m.idx.size() * 4);
    if (!*dsrc || !*didx) return false;
    return hipMemcpy(*dsrc, m.src.data(), m.src.size() * 4, hipMemcpyHostToDevice) == hipSuccess &&
           hipMemcpy(*didx, m.idx.data(), m.idx.size() * 4, hipMemcpyHostToDevice) == hipSuccess;
  };
  int *qs, *qi, *os, *oi, *gs, *gi, *ds, *di;
  if (!upload_map(x->map_qkv, &qs, &qi) || !upload_map(x->map_o, &os, &oi) || !upload_map(x->map_gu, &gs, &gi) ||
      !upload_map(x->map_down, &ds, &di)) {
    fail(VFM_E_OOM, "column map upload failed");
    return bail(VFM_E_OOM);
  }
  // packed bytes of a K x N weight (W4: codes then fp16 group scales; W8A16:
  // codes then fp32 column scales)
  auto wbytes = [&](size_t K, size_t N) -> size_t {
    if (x->wprec == VFM_W_FP8) return K * N;
    if (x->wprec == VFM_W_W8A16) return K * N + N * 4;
    if (x->wprec == VFM_W_W4A16 || x->wprec == VFM_W_W4A8) return K * N / 2 + (K / 128) * N * 2;
    return K * N * ab;
  };
  if (x->wprec == VFM_W_FP8) {
    x->wamax = (unsigned*)x->dalloc((size_t)std::max(L, 1) * 4 * 4);
    if (!x->wamax) { fail(VFM_E_OOM, "allocation failed"); return bail(VFM_E_OOM); }
    if (hipMemsetAsync(x->wamax, 0, (size_t)std::max(L, 1) * 16, s) != hipSuccess) { fail(VFM_E_HIP, "memset"); return bail(VFM_E_HIP); }
  }
  for (int l = 0; l < L; ++l) {
    const std::string p = "layers." + std::to_string(l) + ".";
    uint8_t* wq = (uint8_t*)x->dalloc(wbytes(W, nqkv));
    uint8_t* wo = (uint8_t*)x->dalloc(wbytes((size_t)Hq * d, W));
    uint8_t* wg = (uint8_t*)x->dalloc(wbytes(W, 2 * (size_t)F));
    uint8_t* wd = (uint8_t*)x->dalloc(wbytes(F, W));
    if (!wq || !wo || !wg || !wd) { fail(VFM_E_OOM, "weight allocation failed"); return bail(VFM_E_OOM); }
    hipError_t e = hipSuccess;
    if (x->wprec == VFM_W_FP32 || x->wprec == VFM_W_BF16) {
      if ((e = vfm::pack_weight(wq, W, nqkv, qs, qi, ptr[p + "q.w"], Hq * d, ptr[p + "k.w"], Hkv * d, ptr[p + "v.w"], Hkv * d,
                                x->src_bf16, x->act_bf16, s)) != hipSuccess ||
          (e = vfm::pack_weight(wo, Hq * d, W, os, oi, ptr[p + "o.w"], W, nullptr, 0, nullptr, 0, x->src_bf16, x->act_bf16, s)) != hipSuccess ||
          (e = vfm::pack_weight(wg, W, 2 * F, gs, gi, ptr[p + "gate.w"], F, ptr[p + "up.w"], F, nullptr, 0, x->src_bf16, x->act_bf16, s)) != hipSuccess ||
          (e = vfm::pack_weight(wd, F, W, ds, di, ptr[p + "down.w"], W, nullptr, 0, nullptr, 0, x->src_bf16, x->act_bf16, s)) != hipSuccess) {
        fail(VFM_E_HIP, "weight packing failed: %s", hipGetErrorString(e));
        return bail(VFM_E_HIP);
      }
    } else {
      const int fmt = x->wprec == VFM_W_FP8 ? 0 : x->wprec == VFM_W_W8A16 ? 2 : 1;
      unsigned* am = x->wamax ? x->wamax + 4 * l : nullptr;
      if (fmt == 0) {
        // one scale per fused tensor: [q | k | v] and [gate | up] share theirs
        const size_t qn = (size_t)W * Hq * d, kn = (size_t)W * Hkv * d;
        if ((e = vfm::amax_into(am + 0, ptr[p + "q.w"], qn, 1, s)) != hipSuccess ||
            (e = vfm::amax_into(am + 0, ptr[p + "k.w"], kn, 1, s)) != hipSuccess ||
            (e = vfm::amax_into(am + 0, ptr[p + "v.w"], kn, 1, s)) != hipSuccess ||
            (e = vfm::amax_into(am + 1, ptr[p + "o.w"], (size_t)Hq * d * W, 1, s)) != hipSuccess ||
            (e = vfm::amax_into(am + 2, ptr[p + "gate.w"], (size_t)W * F, 1, s)) != hipSuccess ||
            (e = vfm::amax_into(am + 2, ptr[p + "up.w"], (size_t)W * F, 1, s)) != hipSuccess ||
            (e = vfm::amax_into(am + 3, ptr[p + "down.w"], (size_t)F * W, 1, s)) != hipSuccess) {
          fail(VFM_E_HIP, "weight amax failed: %s", hipGetErrorString(e));
          return bail(VFM_E_HIP);
        }
      }
      if ((e = vfm::pack_weight_q(wq, fmt, W, nqkv, qs, qi, ptr[p + "q.w"], Hq * d, ptr[p + "k.w"], Hkv * d, ptr[p + "v.w"],
                                  Hkv * d, am ? am + 0 : nullptr, s)) != hipSuccess ||
          (e = vfm::pack_weight_q(wo, fmt, Hq * d, W, os, oi, ptr[p + "o.w"], W, nullptr, 0, nullptr, 0, am ? am + 1 : nullptr,
                                  s)) != hipSuccess ||
          (e = vfm::pack_weight_q(wg, fmt, W, 2 * F, gs, gi, ptr[p + "gate.w"], F, ptr[p + "up.w"], F, nullptr, 0,
                                  am ? am + 2 : nullptr, s)) != hipSuccess ||
          (e = vfm::pack_weight_q(wd, fmt, F, W, ds, di, ptr[p + "down.w"], W, nullptr, 0, nullptr, 0, am ? am + 3 : nullptr,
                                  s)) != hipSuccess) {
        fail(VFM_E_HIP, "weight packing failed: %s", hipGetErrorString(e));
        return bail(VFM_E_HIP);
      }
    }
    x->w_qkv.push_back(wq); x->w_o.push_back(wo); x->w_gu.push_back(wg); x->w_down.push_back(wd);
  }
  if (x->pi0) {
    x->w_tmlp = (uint8_t*)x->dalloc(wbytes(W, W));
    if (!x->w_tmlp) { fail(VFM_E_OOM, "weight allocation failed"); return bail(VFM_E_OOM); }
    hipError_t e = vfm::pack_weight(x->w_tmlp, W, W, os, oi, ptr["time_mlp_out.w"], W, nullptr, 0, nullptr, 0,
                                    x->src_bf16, x->act_bf16, s);
    if (e != hipSuccess) { fail(VFM_E_HIP, "weight packing failed: %s", hipGetErrorString(e)); return bail(VFM_E_HIP); }
  }
  if (x->wprec == VFM_W_FP8) {
    std::vector<float> am((size_t)L * 4);
    if (L > 0 && (hipMemcpyAsync(am.data(), x->wamax, am.size() * 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
                  hipStreamSynchronize(s) != hipSuccess)) {
      fail(VFM_E_HIP, "weight scales readback failed");
      return bail(VFM_E_HIP);
    }
    x->wscale.resize(am.size());
    for (size_t i = 0; i < am.size(); ++i) x->wscale[i] = am[i] > 0.f ? am[i] / 448.0f : 1.0f;
  }
  if (fp8_act(x)) {
    // W4A8: the group scales are inside the GEMM, so alpha is the activation scale alone
    if (x->wprec == VFM_W_W4A8) x->wscale.assign((size_t)L * 4, 1.0f);
    x->qs = (float*)x->dalloc((size_t)std::max(L, 1) * 8 * 4);
    if (!x->qs) { fail(VFM_E_OOM, "allocation failed"); return bail(VFM_E_OOM); }
  }
  // small f32 weights
  struct Cv { float** dst; const char* name; size_t n; };
  std::vector<Cv> cvs = {{&x->in_b, "in_proj.b", (size_t)W}, {&x->out_w, "out_proj.w", (size_t)W * A},
                         {&x->out_b, "out_proj.b", (size_t)A}};
  if (x->pi0) cvs.push_back({&x->tmlp_b, "time_mlp_out.b", (size_t)W});
  else cvs.push_back({&x->in_w, "in_proj.w", (size_t)A * W});
  if (S > 0) {
    cvs.push_back({&x->st_w, "state_proj.w", (size_t)S * W});
    cvs.push_back({&x->st_b, "state_proj.b", (size_t)W});
  }
  for (const Cv& c : cvs) {
    *c.dst = (float*)x->dalloc(c.n * 4);
    if (!*c.dst) { fail(VFM_E_OOM, "allocation failed"); return bail(VFM_E_OOM); }
    hipError_t e = vfm::to_f32(*c.dst, ptr[c.name], c.n, x->src_bf16, s);
    if (e != hipSuccess) { fail(VFM_E_HIP, "convert %s: %s", c.name, hipGetErrorString(e)); return bail(VFM_E_HIP); }
  }
  // modulation table
  x->mod = (float*)x->dalloc((size_t)x->N * n_norms * 3 * W * 4);
  double* scratch = (double*)x->dalloc(((size_t)x->N * x->E + 2 * (size_t)x->N * W) * 8);
  if (!x->mod || !scratch) { fail(VFM_E_OOM, "allocation failed"); return bail(VFM_E_OOM); }
  if (x->pi0) {
    // plain norms as constant modulation rows; the action half of the time MLP's
    // first layer folded into the action projection; its time half per step
    x->in_w = (float*)x->dalloc((size_t)A * W * 4);
    x->tbias = (float*)x->dalloc((size_t)x->N * W * 4);
    if (!x->in_w || !x->tbias) { fail(VFM_E_OOM, "allocation failed"); return bail(VFM_E_OOM); }
    std::vector<const void*> nw;
    for (int l = 0; l < L; ++l) {
      const std::string p = "layers." + std::to_string(l) + ".";
      nw.push_back(ptr[p + "attn_norm.w"]);
      nw.push_back(ptr[p + "mlp_norm.w"]);
    }
    nw.push_back(ptr["final_norm.w"]);
    hipError_t e = vfm::build_pi0_tables(x->mod, nw.data(), n_norms, x->in_w, x->tbias, ptr["in_proj.w"], ptr["in_proj.b"],
                                         ptr["time_mlp_in.w"], ptr["time_mlp_in.b"], A, W, x->N, x->src_bf16, scratch, s);
    if (e != hipSuccess) { fail(VFM_E_HIP, "pi0 tables: %s", hipGetErrorString(e)); return bail(VFM_E_HIP); }
  } else {
    std::vector<const void*> mw, mb;
    for (int l = 0; l < L; ++l) {
      const std::string p = "layers." + std::to_string(l) + ".";
      mw.push_back(ptr[p + "attn_norm.mod.w"]); mb.push_back(ptr[p + "attn_norm.mod.b"]);
      mw.push_back(ptr[p + "mlp_norm.mod.w"]); mb.push_back(ptr[p + "mlp_norm.mod.b"]);
    }
    mw.push_back(ptr["final_norm.mod.w"]); mb.push_back(ptr["final_norm.mod.b"]);
    hipError_t e = vfm::build_mod_table(x->mod, mw.data(), mb.data(), n_norms, ptr["time_mlp_in.w"], ptr["time_mlp_in.b"],
                                        ptr["time_mlp_out.w"], ptr["time_mlp_out.b"], x->N, x->E, W, x->src_bf16, scratch, s);
    if (e != hipSuccess) { fail(VFM_E_HIP, "modulation table: %s", hipGetErrorString(e)); return bail(VFM_E_HIP); }
  }
  // workspace for max_batch / max_prefix_len (T suffix tokens per sample)
  const int T = x->T;
  const size_t Mmax = (size_t)x->maxB * T;
  x->KSmax = (x->maxP + vfm::ATT_KEYS_HOST - 1) / vfm::ATT_KEYS_HOST + (T + vfm::ATT_KEYS_HOST - 1) / vfm::ATT_KEYS_HOST;
  x->rope = (float*)x->dalloc((size_t)T * d * 4);
  x->s_emb = (float*)x->dalloc(Mmax * W * 4);
  x->part_o = (float*)x->dalloc((size_t)vfm::MAX_KSPLIT * Mmax * W * 4);
  x->part_d = (float*)x->dalloc((size_t)vfm::MAX_KSPLIT * Mmax * W * 4);
  x->h = (float*)x->dalloc(Mmax * W * 4);
  {
    auto al = [](size_t b) { return (b + 4095) / 4096 * 4096; };
    const size_t Mpad = (Mmax + 63) / 64 * 64;
    size_t off = 0;
    x->off_xna = off; off += al(Mpad * W * ab);
    x->off_q = off; off += al((size_t)x->maxB * Hq * d * 64 * ab);
    x->off_k = off; off += al((size_t)x->maxB * Hkv * d * 64 * ab);
    x->off_v = off; off += al((size_t)x->maxB * Hkv * d * 64 * ab);
    x->off_attn = off; off += al(Mpad * Hq * d * ab);
    x->off_xnm = off; off += al(Mpad * W * ab);
    x->off_act = off; off += al((size_t)F * Mpad * ab);
    if (x->pi0) { x->off_u = off; off += al(Mpad * W * ab); }
    if (can_fold_norms(cfg)) {
      x->off_ssa = off; off += al(Mpad * (W / 16) * 4);
      x->off_ssm = off; off += al(Mpad * (W / 16) * 4);
    }
    x->slab = off;
    x->ring = (uint8_t*)x->dalloc(x->slab * (size_t)x->N * std::max(L, 1));
  }
  x->opart = (float*)x->dalloc((size_t)x->maxB * Hq * x->KSmax * 64 * d * 4);
  x->ml = (float*)x->dalloc((size_t)x->maxB * Hq * x->KSmax * 64 * 2 * 4);
  x->bar = (unsigned*)x->dalloc(vfm::BAR_WORDS * 4);
  if (!x->rope || !x->s_emb || !x->part_o || !x->part_d || !x->h || !x->ring || !x->opart || !x->ml || !x->bar) {
    fail(VFM_E_OOM, "workspace allocation failed");
    return bail(VFM_E_OOM);
  }
  if (vfm::zero_words(x->bar, vfm::BAR_WORDS, s) != hipSuccess) { fail(VFM_E_HIP, "barrier clear"); return bail(VFM_E_HIP); }
  if (hipHostMalloc((void**)&x->herr, 4, hipHostMallocMapped) != hipSuccess) { fail(VFM_E_OOM, "pinned allocation failed"); return bail(VFM_E_OOM); }
  *x->herr = 0u;
  if (hipHostGetDevicePointer((void**)&x->herr_dev, x->herr, 0) != hipSuccess) { fail(VFM_E_HIP, "mapped error word"); return bail(VFM_E_HIP); }
  {
    VP shape{};
    shape.d = d;
    shape.W = W;
    x->lds = vfm::lds_bytes(shape, ab);
    hipError_t e = vfm::prepare_kernels(x->kset, d, (int)x->lds);
    if (e == hipSuccess && fp8_act(x)) e = vfm::prepare_kernels(vfm::KS_CAL, d, (int)x->lds);
    if (e != hipSuccess) { fail(VFM_E_HIP, "kernel attribute: %s", hipGetErrorString(e)); return bail(VFM_E_HIP); }
  }
  // norms folded into the persistent kernel's GEMMs: shift W tables (fp64
  // sums over the packed bf16 weights), sums-of-squares rows, split counters
  if (can_fold_norms(cfg)) {
    const int Nq = (Hq + 2 * Hkv) * d, n_norms = 2 * L + 1;
    x->shw_q = (float*)x->dalloc((size_t)x->N * L * Nq * 4);
    x->shw_g = (float*)x->dalloc((size_t)x->N * L * 2 * F * 4);
    x->fcnt = (unsigned*)x->dalloc((size_t)2 * vfm::FCNT_MAX * 4);
    x->xcnt = (unsigned*)x->dalloc((size_t)vfm::XCNT_WORDS * 4);
    x->hcnt = (unsigned*)x->dalloc((size_t)(vfm::HCNT_MAX + 2 * vfm::QCNT_KV) * vfm::HCNT_STRIDE * 4);
    if (!x->shw_q || !x->shw_g || !x->fcnt || !x->xcnt || !x->hcnt) {
      fail(VFM_E_OOM, "workspace allocation failed");
      return bail(VFM_E_OOM);
    }
    if (vfm::zero_words(x->fcnt, 2 * vfm::FCNT_MAX, s) != hipSuccess ||
        vfm::zero_words(x->xcnt, vfm::XCNT_WORDS, s) != hipSuccess ||
        shift_tables(x, L, W, Nq, F, n_norms, s) != hipSuccess) {
      fail(VFM_E_HIP, "shift projection tables");
      return bail(VFM_E_HIP);
    }
    x->can_fuse = true;
  } else {
    x->hcnt = (unsigned*)x->dalloc((size_t)(vfm::HCNT_MAX + 2 * vfm::QCNT_KV) * vfm::HCNT_STRIDE * 4);
    if (!x->hcnt) { fail(VFM_E_OOM, "workspace allocation failed"); return bail(VFM_E_OOM); }
  }
  // the persistent kernel's attention arrival counters (every expert; for a
  // folded-norm expert allocated with its tables above)
  if (vfm::zero_words(x->hcnt, (vfm::HCNT_MAX + 2 * vfm::QCNT_KV) * vfm::HCNT_STRIDE, s) != hipSuccess) {
    fail(VFM_E_HIP, "counter clear");
    return bail(VFM_E_HIP);
  }
  // the streaming batch-1 kernel: bf16 pi0.5 experts whose shapes fit it
  if (x->kset == vfm::KS_BF16 && !x->pi0) {
    const vfm::sk::StreamShape sh{L, W, Hq, Hkv, d, F, H, A, S, x->N, x->maxP, cfg->rms_eps};
    const vfm_status sst = vfm::sk::stream_create(sh, x->w_qkv.data(), x->w_o.data(), x->w_gu.data(), x->w_down.data(),
                                                  x->mod, s, &x->ss, &x->ss_why);
    if (sst != VFM_OK) return bail(sst);
  } else {
    x->ss_why = "the streaming kernel is built for bf16 pi0.5 experts";
  }
  if (hipStreamSynchronize(s) != hipSuccess || hipGetLastError() != hipSuccess) {
    fail(VFM_E_HIP, "create-time device work failed");
    return bail(VFM_E_HIP);
  }
  *out = x;
  return VFM_OK;
}

vfm_status vfm_bind(vfm_expert* x, const char* name, void* dev_ptr, int32_t dtype, int32_t ndim, const int64_t* shape) {
  if (!x) return fail(VFM_E_INVALID_ARG, "expert is NULL");
  if (!name) return fail(VFM_E_INVALID_ARG, "name is NULL");
  if (ndim < 1 || ndim > 5 || !shape) return fail(VFM_E_SHAPE, "buffer '%s': bad ndim %d", name, ndim);
  int64_t numel = 1;
  for (int i = 0; i < ndim; ++i) numel *= shape[i];
  // an empty buffer (a zero-layer expert's prefix) may have a NULL pointer
  if (!dev_ptr && numel != 0) return fail(VFM_E_INVALID_ARG, "buffer '%s': NULL pointer", name);
  if (reinterpret_cast<uintptr_t>(dev_ptr) % 16 != 0) return fail(VFM_E_INVALID_ARG, "buffer '%s': pointer not 16-byte aligned", name);
  BoundBuf* b = nullptr;
  const std::string n = name;
  if (n == "prefix_k") b = &x->prefix_k;
  else if (n == "prefix_v") b = &x->prefix_v;
  else if (n == "noise") b = &x->noise;
  else if (n == "state") b = &x->state;
  else if (n == "actions") b = &x->actions;
  else return fail(VFM_E_INVALID_ARG, "unknown buffer name '%s'", name);
  const int act_dt = x->act_bf16 ? VFM_BF16 : VFM_F32;
  if (b == &x->prefix_k || b == &x->prefix_v) {
    if (dtype != act_dt) return fail(VFM_E_DTYPE, "buffer '%s' must have dtype %d", name, act_dt);
    if (ndim != 5) return fail(VFM_E_SHAPE, "buffer '%s' must be [L][B][P][Hkv][d]", name);
    if (shape[0] != x->L || shape[3] != x->Hkv || shape[4] != x->d)
      return fail(VFM_E_SHAPE, "buffer '%s' must be [%d][B][P][%d][%d]", name, x->L, x->Hkv, x->d);
    if (shape[1] < 1 || shape[1] > x->maxB) return fail(VFM_E_SHAPE, "buffer '%s': batch %lld outside [1, %d]", name, (long long)shape[1], x->maxB);
    if (shape[2] < 1 || shape[2] > x->maxP) return fail(VFM_E_SHAPE, "buffer '%s': prefix %lld outside [1, %d]", name, (long long)shape[2], x->maxP);
  } else {
    if (dtype != VFM_F32) return fail(VFM_E_DTYPE, "buffer '%s' must be f32", name);
    if (b == &x->state) {
      if (x->S == 0) return fail(VFM_E_INVALID_ARG, "this expert has no state input");
      if (ndim != 2 || shape[1] != x->S || shape[0] < 1 || shape[0] > x->maxB)
        return fail(VFM_E_SHAPE, "buffer 'state' must be [B][%d]", x->S);
    } else if (ndim != 3 || shape[1] != x->H || shape[2] != x->A || shape[0] < 1 || shape[0] > x->maxB) {
      return fail(VFM_E_SHAPE, "buffer '%s' must be [B][%d][%d]", name, x->H, x->A);
    }
  }
  b->ptr = dev_ptr;
  b->dtype = dtype;
  b->ndim = ndim;
  for (int i = 0; i < 5; ++i) b->shape[i] = i < ndim ? shape[i] : 0;
  b->bound = true;
  return VFM_OK;
}

vfm_status vfm_set_option(vfm_expert* x, const char* key, const char* value) {
  if (!x || !key || !value) return fail(VFM_E_INVALID_ARG, "NULL argument");
  const std::string k = key, v = value;
  if (k == "trace") {
    if (v == "1" && !x->trace) {
      x->trace_words = 2 * (size_t)(x->N * (8 * (size_t)x->L + 1 + 2 * x->pi0) + 4);
      if (x->ss) x->trace_words = std::max(x->trace_words, 3 * (size_t)(vfm::sk::stream_barriers(x->ss) + 2));
      x->trace = (unsigned long long*)x->dalloc(x->trace_words * 8);
      if (!x->trace) return fail(VFM_E_OOM, "trace buffer");
    } else if (v == "0") {
      x->trace = nullptr;   // the buffer stays owned by the expert
    } else if (v != "1") {
      return fail(VFM_E_INVALID_ARG, "trace must be 0 or 1");
    }
    return VFM_OK;
  }
  if (k == "stream_stop_after") {
    char* end = nullptr;
    const long n = std::strtol(value, &end, 10);
    if (end == value || *end || n < 0) return fail(VFM_E_INVALID_ARG, "stream_stop_after must be a barrier count >= 0");
    x->ss_tune.stop_after = (int)n;
    return VFM_OK;
  }
  if (k == "barrier_spin_limit") {
    char* end = nullptr;
    const long long n = std::strtoll(value, &end, 10);
    if (end == value || *end || n < 1024 || n > (1LL << 40))
      return fail(VFM_E_INVALID_ARG, "barrier_spin_limit must be an integer in [1024, 2^40]");
    x->spin_limit = (long)n;
    x->ss_tune.spin_limit = (long)n;
    return VFM_OK;
  }
  if (k == "fail_barrier") {
    char* end = nullptr;
    const long n = std::strtol(value, &end, 10);
    if (end == value || *end || n < 0) return fail(VFM_E_INVALID_ARG, "fail_barrier must be a barrier index >= 0");
    x->fail_barrier = (int)n;
    x->ss_tune.fail_epoch = (int)n;
    return VFM_OK;
  }
  if (k == "stream_dma_cap") {
    char* end = nullptr;
    const long n = std::strtol(value, &end, 10);
    if (end == value || *end || n < 1 || n > 63) return fail(VFM_E_INVALID_ARG, "stream_dma_cap must be an integer in [1, 63]");
    x->ss_tune.dma_cap = (int)n;
    return VFM_OK;
  }
  if (k == "large_m_tiles") {
    // diagnostics: the large-M GEMM tiles of the per-phase launch modes
    if (v == "auto") x->gemm_tiles = 0;
    else if (v == "narrow") x->gemm_tiles = 1;
    else if (v == "wide") x->gemm_tiles = 2;
    else return fail(VFM_E_INVALID_ARG, "large_m_tiles must be 'auto', 'narrow' or 'wide'");
    x->drop_graphs();
    return VFM_OK;
  }
  if (k == "fused_norms") {
    // the persistent kernel with the norms folded into its GEMMs: "auto"
    // (default) where the call has at most FOLD_AUTO_ROWS rows, "1" at any
    // size, "0" never (separate norm phases)
    if (v == "1") {
      if (!x->can_fuse)
        return fail(VFM_E_UNSUPPORTED, "fused_norms applies to pi0.5 experts with bf16, W4A16 or W8A16 weights and a width that is a multiple of 256 up to 1024");
      x->fuse_norms = 1;
    } else if (v == "0") {
      x->fuse_norms = 0;
    } else if (v == "auto") {
      x->fuse_norms = -1;
    } else {
      return fail(VFM_E_INVALID_ARG, "fused_norms must be 'auto', 0 or 1");
    }
    return VFM_OK;
  }
  if (k == "attn_merge") {
    // the persistent kernels merge the attention key splits in the attention
    // phase, whose units start on per-head counters (1, the default), or run
    // a combine phase between device-wide barriers (0; the folded-norm
    // kernel needs the in-place merge, so "0" also selects separate norms)
    if (v == "1") x->attn_merge = true;
    else if (v == "0") x->attn_merge = false;
    else return fail(VFM_E_INVALID_ARG, "attn_merge must be 0 or 1");
    return VFM_OK;
  }
  if (k == "xcd_local") {
    // the fused kernel's o / down split sums through one XCD's L2 (1, the
    // default where the plan allows it) or through the device coherence point (0)
    if (v == "1") x->xcd_local = true, x->xcd_attn = true;
    else if (v == "0") x->xcd_local = false;
    else if (v == "splits") x->xcd_local = true, x->xcd_attn = false;   // diagnostics: o / down sums only
    else return fail(VFM_E_INVALID_ARG, "xcd_local must be 0, 1 or 'splits'");
    return VFM_OK;
  }
  if (k == "persistent_launch") {
    if (v == "cooperative") x->coop_launch = true;
    else if (v == "plain") x->coop_launch = false;
    else return fail(VFM_E_INVALID_ARG, "persistent_launch must be 'cooperative' or 'plain'");
    return VFM_OK;
  }
  if (k == "graph_cache") {
    char* end = nullptr;
    const long n = std::strtol(value, &end, 10);
    if (end == value || *end || n < 1 || n > 64) return fail(VFM_E_INVALID_ARG, "graph_cache must be an integer in [1, 64]");
    x->graph_cap = (int)n;
    while ((int)x->graphs.size() > x->graph_cap) {
      (void)hipGraphExecDestroy(x->graphs.back().exec);
      x->graphs.pop_back();
    }
    return VFM_OK;
  }
  if (k == "launch_mode") {
    if (v == "persistent") x->mode = 0;
    else if (v == "graph") x->mode = 1;
    else if (v == "eager") x->mode = 2;
    else if (v == "auto") x->mode = 3;
    else if (v == "stream") {
      if (!x->ss) return fail(VFM_E_UNSUPPORTED, "launch_mode 'stream' unavailable: %s", x->ss_why.c_str());
      x->mode = 4;
    }
    else return fail(VFM_E_INVALID_ARG, "launch_mode '%s' unknown", value);
    return VFM_OK;
  }
  return fail(VFM_E_INVALID_ARG, "unknown option '%s'", key);
}

vfm_status vfm_denoise(vfm_expert* x, const float* noise, const float* state, float* actions, void* stream) {
  if (!x) return fail(VFM_E_INVALID_ARG, "expert is NULL");
  vfm_status st = check_host_err(x, reinterpret_cast<hipStream_t>(stream));
  if (st != VFM_OK) return st;
  if (!x->prefix_k.bound) return fail(VFM_E_UNBOUND, "buffer 'prefix_k' is not bound");
  const int B = (int)x->prefix_k.shape[1], P = (int)x->prefix_k.shape[2];
  const int act_dt = x->act_bf16 ? VFM_BF16 : VFM_F32;
  if ((st = check_buf("prefix_v", x->prefix_v, act_dt, {x->L, B, P, x->Hkv, x->d})) != VFM_OK) return st;
  if (!noise) {
    if ((st = check_buf("noise", x->noise, VFM_F32, {B, x->H, x->A})) != VFM_OK) return st;
    noise = (const float*)x->noise.ptr;
  }
  if (!actions) {
    if ((st = check_buf("actions", x->actions, VFM_F32, {B, x->H, x->A})) != VFM_OK) return st;
    actions = (float*)x->actions.ptr;
  }
  if (x->S > 0 && !state) {
    if ((st = check_buf("state", x->state, VFM_F32, {B, x->S})) != VFM_OK) return st;
    state = (const float*)x->state.ptr;
  }
  if ((reinterpret_cast<uintptr_t>(noise) | reinterpret_cast<uintptr_t>(actions) | reinterpret_cast<uintptr_t>(state)) % 16)
    return fail(VFM_E_INVALID_ARG, "noise / state / actions must be 16-byte aligned");

  if (fp8_act(x) && x->act_scale.empty())
    return fail(VFM_E_STATE, "FP8-activation expert: run vfm_calibrate or vfm_set_act_scales first");
  VP p{};
  if ((st = fill_vp(x, p, B, P, noise, state, actions)) != VFM_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (x->rope_P != P) {
    // The table (positions P .. P + T - 1) is rebuilt in place; graphs of
    // other P read it at the same address and see it rebuilt before replay.
    HIPCHK(vfm::build_rope(x->rope, x->T, x->d, P, x->cfg.rope_base, s));
    x->rope_P = P;
  }
  const int mode = launch_mode_of(x, B, P);
  if (mode == 4) {
    if (!stream_fits(x, B, P))
      return fail(VFM_E_UNSUPPORTED, "launch_mode 'stream' runs batch 1 with a prefix the attention plan fits (B = %d, P = %d)", B, P);
    if ((st = check_stream_flag(x, s)) != VFM_OK) return st;
    return vfm::sk::stream_run(x->ss, P, x->prefix_k.ptr, x->prefix_v.ptr, noise, state, actions, x->in_w, x->in_b,
                               x->st_w, x->st_b, x->out_w, x->out_b, x->rope, x->coop_launch, x->trace,
                               x->ss_tune, s);
  }
  if (mode == 0) {
    // one launch per call: the kernel's last workgroup clears the arrival
    // counters, and a failure raises the host-mapped word read by the checks
    if (p.xl & 1) {
      const int mt = (p.M + 63) / 64;
      const long long plan = (((long long)p.gp_s[1] * 64 + p.gp_s[3]) * 4096 + (long long)(p.W / (16 * p.gp_nt[1])) * mt) *
                                 4096 + (long long)(p.W / (16 * p.gp_nt[3])) * mt;
      if (plan != x->xl_plan) {
        HIPCHK(vfm::zero_words(x->xcnt, vfm::XCNT_WORDS, s));
        x->xl_plan = plan;
      }
    }
    HIPCHK(vfm::launch_phase(p, x->kset, x->coop_launch ? 0 : 3, 0, 0, 0, x->coop_grid, x->lds, s));
    return VFM_OK;
  }
  if (mode == 2) {
    HIPCHK(enqueue_phases(x, p, x->kset, s));
    return VFM_OK;
  }
  // graph mode
  std::vector<uintptr_t> key = {(uintptr_t)B, (uintptr_t)P, (uintptr_t)noise, (uintptr_t)state, (uintptr_t)actions,
                                (uintptr_t)p.prefix_k, (uintptr_t)p.prefix_v};
  auto hit = std::find_if(x->graphs.begin(), x->graphs.end(), [&](const vfm_expert::GraphEntry& g) { return g.key == key; });
  if (hit != x->graphs.end()) {
    std::rotate(x->graphs.begin(), hit, hit + 1);
  } else {
    while ((int)x->graphs.size() >= x->graph_cap) {
      (void)hipGraphExecDestroy(x->graphs.back().exec);
      x->graphs.pop_back();
    }
    if (!x->cap_stream) HIPCHK(hipStreamCreateWithFlags(&x->cap_stream, hipStreamNonBlocking));
    hipGraph_t g = nullptr;
    HIPCHK(hipStreamBeginCapture(x->cap_stream, hipStreamCaptureModeThreadLocal));
    hipError_t e = enqueue_phases(x, p, x->kset, x->cap_stream);
    hipError_t e2 = hipStreamEndCapture(x->cap_stream, &g);
    if (e != hipSuccess || e2 != hipSuccess) {
      if (g) (void)hipGraphDestroy(g);
      return fail(VFM_E_HIP, "graph capture failed: %s", hipGetErrorString(e != hipSuccess ? e : e2));
    }
    hipGraphExec_t ge = nullptr;
    e = hipGraphInstantiate(&ge, g, nullptr, nullptr, 0);
    (void)hipGraphDestroy(g);
    if (e != hipSuccess) return fail(VFM_E_HIP, "graph instantiate: %s", hipGetErrorString(e));
    x->graphs.insert(x->graphs.begin(), vfm_expert::GraphEntry{key, ge});
  }
  HIPCHK(hipGraphLaunch(x->graphs.front().exec, s));
  return VFM_OK;
}

vfm_status vfm_calibrate(vfm_expert* x, void* stream) {
  if (!x) return fail(VFM_E_INVALID_ARG, "expert is NULL");
  if (!fp8_act(x)) return fail(VFM_E_STATE, "calibrate applies to FP8 and W4A8 experts only");
  vfm_status st = check_host_err(x, reinterpret_cast<hipStream_t>(stream));
  if (st != VFM_OK) return st;
  if (!x->prefix_k.bound) return fail(VFM_E_UNBOUND, "buffer 'prefix_k' is not bound");
  const int B = (int)x->prefix_k.shape[1], P = (int)x->prefix_k.shape[2];
  if ((st = check_buf("prefix_v", x->prefix_v, VFM_BF16, {x->L, B, P, x->Hkv, x->d})) != VFM_OK) return st;
  if ((st = check_buf("noise", x->noise, VFM_F32, {B, x->H, x->A})) != VFM_OK) return st;
  if ((st = check_buf("actions", x->actions, VFM_F32, {B, x->H, x->A})) != VFM_OK) return st;
  if (x->S > 0 && (st = check_buf("state", x->state, VFM_F32, {B, x->S})) != VFM_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int L = x->L, W = x->W, F = x->F, nqkv = (x->Hq + 2 * x->Hkv) * x->d, qd = x->Hq * x->d;
  // One bf16 pass with the dequantised FP8 weights (materialised for the
  // pass only) records the largest |input| of every GEMM over all steps.
  std::vector<void*> tmp;
  auto release = [&]() { for (void* q : tmp) (void)hipFree(q); tmp.clear(); };
  auto talloc = [&](size_t bytes) -> void* {
    void* q = nullptr;
    if (hipMalloc(&q, bytes) != hipSuccess) return nullptr;
    tmp.push_back(q);
    return q;
  };
  float* amax = (float*)talloc((size_t)std::max(L, 1) * 16);
  if (!amax) { release(); return fail(VFM_E_OOM, "calibration buffers"); }
  VP p{};
  const int kw = x->KW;
  x->KW = 32;   // the bf16 pass plans its GEMMs for 32-K blocks
  st = fill_vp(x, p, B, P, (const float*)x->noise.ptr, (const float*)x->state.ptr, (float*)x->actions.ptr);
  x->KW = kw;
  if (st != VFM_OK) { release(); return st; }
  p.trace = nullptr;
  p.spin_limit = x->spin_limit;
  p.fail_epoch = 0;
  p.herr = nullptr;
  p.amax = amax;
  hipError_t e = hipMemsetAsync(amax, 0, (size_t)std::max(L, 1) * 16, s);
  for (int l = 0; l < L && e == hipSuccess; ++l) {
    uint8_t* bq = (uint8_t*)talloc((size_t)W * nqkv * 2);
    uint8_t* bo = (uint8_t*)talloc((size_t)qd * W * 2);
    uint8_t* bg = (uint8_t*)talloc((size_t)W * 2 * F * 2);
    uint8_t* bd = (uint8_t*)talloc((size_t)F * W * 2);
    if (!bq || !bo || !bg || !bd) { release(); return fail(VFM_E_OOM, "calibration weights"); }
    if (x->wprec == VFM_W_FP8) {
      unsigned* am = x->wamax + 4 * l;
      if ((e = vfm::fp8_to_bf16_packed(bq, x->w_qkv[l], W, nqkv, am + 0, s)) != hipSuccess ||
          (e = vfm::fp8_to_bf16_packed(bo, x->w_o[l], qd, W, am + 1, s)) != hipSuccess ||
          (e = vfm::fp8_to_bf16_packed(bg, x->w_gu[l], W, 2 * F, am + 2, s)) != hipSuccess ||
          (e = vfm::fp8_to_bf16_packed(bd, x->w_down[l], F, W, am + 3, s)) != hipSuccess)
        break;
    } else if ((e = vfm::w4_to_bf16_packed(bq, x->w_qkv[l], W, nqkv, s)) != hipSuccess ||
               (e = vfm::w4_to_bf16_packed(bo, x->w_o[l], qd, W, s)) != hipSuccess ||
               (e = vfm::w4_to_bf16_packed(bg, x->w_gu[l], W, 2 * F, s)) != hipSuccess ||
               (e = vfm::w4_to_bf16_packed(bd, x->w_down[l], F, W, s)) != hipSuccess) {
      break;
    }
    p.w_qkv[l] = bq; p.w_o[l] = bo; p.w_gu[l] = bg; p.w_down[l] = bd;
  }
  if (e == hipSuccess && x->rope_P != P) {
    e = vfm::build_rope(x->rope, x->T, x->d, P, x->cfg.rope_base, s);
    if (e == hipSuccess) x->rope_P = P;
  }
  if (e == hipSuccess) e = enqueue_phases(x, p, vfm::KS_CAL, s);
  std::vector<float> am((size_t)L * 4);
  if (e == hipSuccess && L > 0) e = hipMemcpyAsync(am.data(), amax, am.size() * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  release();
  if (e != hipSuccess) return fail(VFM_E_HIP, "calibration pass failed: %s", hipGetErrorString(e));
  std::vector<float> sc(am.size());
  for (size_t i = 0; i < am.size(); ++i) sc[i] = am[i] > 0.f ? am[i] / 448.0f : 1.0f;
  return vfm_set_act_scales(x, sc.data(), (int32_t)sc.size());
}

vfm_status vfm_set_act_scales(vfm_expert* x, const float* scales, int32_t n) {
  if (!x) return fail(VFM_E_INVALID_ARG, "expert is NULL");
  if (!fp8_act(x)) return fail(VFM_E_STATE, "activation scales apply to FP8 and W4A8 experts only");
  if (n != 4 * x->L) return fail(VFM_E_SHAPE, "expected %d scales", 4 * x->L);
  if (n > 0 && !scales) return fail(VFM_E_INVALID_ARG, "scales is NULL");
  for (int i = 0; i < n; ++i)
    if (!(scales[i] > 0.f) || !std::isfinite(scales[i])) return fail(VFM_E_INVALID_ARG, "scale %d is not a positive number", i);
  std::vector<float> q((size_t)n * 2);
  for (int i = 0; i < n; ++i) {
    q[2 * i] = scales[i] * x->wscale[i];      // alpha of the GEMM epilogue
    q[2 * i + 1] = 1.0f / scales[i];          // the activation quantiser multiplies by this
  }
  HIPCHK(hipDeviceSynchronize());
  if (n > 0) HIPCHK(hipMemcpy(x->qs, q.data(), q.size() * 4, hipMemcpyHostToDevice));
  x->act_scale.assign(scales, scales + n);
  x->drop_graphs();
  return VFM_OK;
}

vfm_status vfm_export(vfm_expert* x, const char* name, void* dst, size_t bytes) {
  if (!x || !name || !dst) return fail(VFM_E_INVALID_ARG, "NULL argument");
  const std::string n = name;
  if (n == "mod_table") {
    const size_t cnt = (size_t)x->N * (2 * x->L + 1) * 3 * x->W;
    if (bytes != cnt * 4) return fail(VFM_E_SHAPE, "mod_table needs %zu bytes", cnt * 4);
    HIPCHK(hipDeviceSynchronize());
    HIPCHK(hipMemcpy(dst, x->mod, bytes, hipMemcpyDeviceToHost));
    return VFM_OK;
  }
  // workspace tensors as left by the last denoise call (diagnostics)
  {
    const int B = x->prefix_k.bound ? (int)x->prefix_k.shape[1] : x->maxB;
    const size_t M = (size_t)B * x->T;
    struct Ws { const char* name; const void* ptr; size_t count; bool act; };
    const Ws ws[] = {{"ws.h", x->h, M * x->W, false}};
    for (const Ws& w : ws) {
      if (n != w.name) continue;
      if (bytes != w.count * 4) return fail(VFM_E_SHAPE, "'%s' needs %zu bytes", name, w.count * 4);
      HIPCHK(hipDeviceSynchronize());
      float* out = static_cast<float*>(dst);
      if (!w.act || !x->act_bf16) {
        HIPCHK(hipMemcpy(dst, w.ptr, bytes, hipMemcpyDeviceToHost));
      } else {
        std::vector<uint16_t> tmp(w.count);
        HIPCHK(hipMemcpy(tmp.data(), w.ptr, w.count * 2, hipMemcpyDeviceToHost));
        for (size_t i = 0; i < w.count; ++i) {
          const uint32_t u = (uint32_t)tmp[i] << 16;
          memcpy(&out[i], &u, 4);
        }
      }
      return VFM_OK;
    }
  }
  if (n == "act_scales" || n == "weight_scales") {
    if (n == "weight_scales" && x->wprec != VFM_W_FP8) return fail(VFM_E_STATE, "'%s' exists for FP8 experts only", name);
    if (!fp8_act(x)) return fail(VFM_E_STATE, "'%s' exists for FP8 and W4A8 experts only", name);
    const std::vector<float>& v = n == "act_scales" ? x->act_scale : x->wscale;
    if (v.empty()) return fail(VFM_E_STATE, "activation scales are not set");
    if (bytes != v.size() * 4) return fail(VFM_E_SHAPE, "'%s' needs %zu bytes", name, v.size() * 4);
    memcpy(dst, v.data(), bytes);
    return VFM_OK;
  }
  if (n == "persistent_plan") {
    // int32 [fused norms (0 / 1), device-wide barriers per call, o splits,
    // down splits, XCD-local split sums (0 / 1), in-place attention merge
    // (0 / 1)] of the persistent kernel at the bound batch and prefix
    if (bytes != 6 * 4) return fail(VFM_E_SHAPE, "'persistent_plan' needs 24 bytes");
    if (!x->prefix_k.bound) return fail(VFM_E_UNBOUND, "buffer 'prefix_k' is not bound");
    const int B = (int)x->prefix_k.shape[1], P = (int)x->prefix_k.shape[2];
    if (launch_mode_of(x, B, P) != 0) return fail(VFM_E_STATE, "the expert does not run the persistent kernel");
    VP p{};
    const vfm_status st = fill_vp(x, p, B, P, nullptr, nullptr, nullptr);
    if (st != VFM_OK) return st;
    int32_t* o = static_cast<int32_t*>(dst);
    o[0] = p.fuse;
    const bool merged = p.fuse || (p.xl & vfm::XL_MERGE);
    o[1] = p.fuse ? 1 + x->N * (4 * x->L + 1) : 1 + x->N * ((merged ? 6 : 8) * x->L + 2 * x->pi0);
    o[2] = p.S_o;
    o[3] = p.S_down;
    o[4] = p.fuse ? (p.xl & 1) : 0;
    o[5] = merged ? 1 : 0;
    return VFM_OK;
  }
  if (n == "trace") {
    // microseconds since kernel start of (arrive, release) of every phase barrier of the last call
    if (!x->trace) return fail(VFM_E_STATE, "trace is off");
    if (bytes != x->trace_words * 4) return fail(VFM_E_SHAPE, "'trace' needs %zu bytes", x->trace_words * 4);
    std::vector<unsigned long long> t(x->trace_words);
    HIPCHK(hipDeviceSynchronize());
    HIPCHK(hipMemcpy(t.data(), x->trace, x->trace_words * 8, hipMemcpyDeviceToHost));
    float* out = static_cast<float*>(dst);
    for (size_t i = 0; i < x->trace_words; ++i) out[i] = t[i] >= t[0] ? (float)((t[i] - t[0]) / 100.0) : -1.0f;
    return VFM_OK;
  }
  // layers.{l}.{q,k,v,o,gate,up,down}.w
  int l = -1;
  char what[16] = {0};
  if (sscanf(name, "layers.%d.%15[a-z].w", &l, what) != 2 || l < 0 || l >= x->L)
    return fail(VFM_E_INVALID_ARG, "unknown tensor '%s'", name);
  const std::string w = what;
  const uint8_t* packed;
  const ColMap* map;
  int K, Npk, sid, ncols;
  if (w == "q" || w == "k" || w == "v") {
    packed = x->w_qkv[l]; map = &x->map_qkv; K = x->W; Npk = (x->Hq + 2 * x->Hkv) * x->d;
    sid = w == "q" ? 0 : w == "k" ? 1 : 2; ncols = (w == "q" ? x->Hq : x->Hkv) * x->d;
  } else if (w == "o") {
    packed = x->w_o[l]; map = &x->map_o; K = x->Hq * x->d; Npk = x->W; sid = 0; ncols = x->W;
  } else if (w == "gate" || w == "up") {
    packed = x->w_gu[l]; map = &x->map_gu; K = x->W; Npk = 2 * x->F; sid = w == "gate" ? 0 : 1; ncols = x->F;
  } else if (w == "down") {
    packed = x->w_down[l]; map = &x->map_down; K = x->F; Npk = x->W; sid = 0; ncols = x->W;
  } else {
    return fail(VFM_E_INVALID_ARG, "unknown tensor '%s'", name);
  }
  if (bytes != (size_t)K * ncols * 4) return fail(VFM_E_SHAPE, "'%s' needs %zu bytes", name, (size_t)K * ncols * 4);
  const int gi = (w == "q" || w == "k" || w == "v") ? 0 : w == "o" ? 1 : (w == "gate" || w == "up") ? 2 : 3;
  size_t nbytes;
  if (x->wprec == VFM_W_FP8) nbytes = (size_t)K * Npk;
  else if (x->wprec == VFM_W_W8A16) nbytes = (size_t)K * Npk + (size_t)Npk * 4;
  else if (x->wprec == VFM_W_W4A16 || x->wprec == VFM_W_W4A8) nbytes = (size_t)K * Npk / 2 + (size_t)(K / 128) * Npk * 2;
  else nbytes = (size_t)K * Npk * (x->act_bf16 ? 2 : 4);
  std::vector<uint8_t> host(nbytes);
  HIPCHK(hipDeviceSynchronize());
  HIPCHK(hipMemcpy(host.data(), packed, host.size(), hipMemcpyDeviceToHost));
  float* out = static_cast<float*>(dst);
  const int KW = x->KW, nkb = K / KW;
  for (int pc = 0; pc < Npk; ++pc) {
    if (map->src[pc] != sid) continue;
    const int col = map->idx[pc];
    const int t = pc / 16, c16 = pc % 16;
    for (int k = 0; k < K; ++k) {
      const int kb = k / KW, rem = k % KW;
      float v;
      if (x->wprec == VFM_W_FP8) {
        // byte 8r + e of lane (g, c16) holds k = 64 kb + 32 r + 8 g + e
        const int r = rem / 32, g = (rem % 32) / 8, e = rem % 8;
        const uint8_t c = host[(((size_t)t * nkb + kb) * 64 + g * 16 + c16) * 16 + r * 8 + e];
        v = e4m3_value(c) * x->wscale[(size_t)l * 4 + gi];
      } else if (x->wprec == VFM_W_W8A16) {
        // byte 8r + e of lane (g, c16) holds k = 64 kb + 32 r + 8 g + e; column scales after the codes
        const int r = rem / 32, g = (rem % 32) / 8, e = rem % 8;
        const int8_t q = (int8_t)host[(((size_t)t * nkb + kb) * 64 + g * 16 + c16) * 16 + r * 8 + e];
        float sc;
        memcpy(&sc, &host[(size_t)K * Npk + (size_t)pc * 4], 4);
        v = (float)q * sc;
      } else if (x->wprec == VFM_W_W4A16 || x->wprec == VFM_W_W4A8) {
        // nibble 8r + e of lane (g, c16) holds k = 128 kb + 32 r + 8 g + e
        const int r = rem / 32, g = (rem % 32) / 8, e = rem % 8;
        const size_t lane_off = (((size_t)t * nkb + kb) * 64 + g * 16 + c16) * 16;
        uint32_t wd;
        memcpy(&wd, &host[lane_off + 4 * r], 4);
        const int q = (int)(wd << (28 - 4 * e)) >> 28;
        uint16_t sb;
        memcpy(&sb, &host[(size_t)K * Npk / 2 + (((size_t)t * nkb + kb) * 16 + c16) * 2], 2);
        v = (float)q * half_value(sb);
      } else if (!x->act_bf16) {
        const int g = rem / 4, e = rem % 4;
        memcpy(&v, &host[(((size_t)t * nkb + kb) * 64 + g * 16 + c16) * 16 + (size_t)e * 4], 4);
      } else {
        const int g = rem / 8, e = rem % 8;
        uint16_t hb;
        memcpy(&hb, &host[(((size_t)t * nkb + kb) * 64 + g * 16 + c16) * 16 + (size_t)e * 2], 2);
        const uint32_t u = (uint32_t)hb << 16;
        memcpy(&v, &u, 4);
      }
      out[(size_t)k * ncols + col] = v;
    }
  }
  return VFM_OK;
}

vfm_status vfm_stream_debug(vfm_expert* x, const char* name, int32_t index, void* dst, size_t bytes) {
  if (!x || !name || !dst) return fail(VFM_E_INVALID_ARG, "NULL argument");
  if (!x->ss) return fail(VFM_E_STATE, "no streaming kernel state: %s", x->ss_why.c_str());
  if (std::string(name) == "slab_layout") {
    if (bytes != 10 * sizeof(uint64_t)) return fail(VFM_E_SHAPE, "'slab_layout' needs 10 uint64");
    size_t offs[9];
    const size_t slab = vfm::sk::stream_slab_layout(x->ss, offs);
    uint64_t* o = static_cast<uint64_t*>(dst);
    for (int i = 0; i < 9; ++i) o[i] = offs[i];
    o[9] = slab;
    return VFM_OK;
  }
  return vfm::sk::stream_debug_copy(x->ss, name, index, dst, bytes);
}

vfm_status vfm_copy_probe(const void* src, void* dst, size_t bytes, int32_t policy, void* stream) {
  if (!src || !dst) return fail(VFM_E_INVALID_ARG, "NULL buffer");
  if (bytes == 0 || bytes % 16 || bytes >= (1ull << 31)) return fail(VFM_E_INVALID_ARG, "bytes must be a positive multiple of 16 below 2 GiB");
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16) return fail(VFM_E_INVALID_ARG, "buffers must be 16-byte aligned");
  if (policy != 0 && policy != 1 && policy != 16) return fail(VFM_E_INVALID_ARG, "policy must be 0 (plain), 1 (sc0) or 16 (sc1)");
  HIPCHK(vfm::copy_probe(src, dst, bytes, policy, reinterpret_cast<hipStream_t>(stream)));
  return VFM_OK;
}

vfm_status vfm_check(vfm_expert* x, void* stream) {
  if (!x) return fail(VFM_E_INVALID_ARG, "expert is NULL");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  HIPCHK(hipStreamSynchronize(s));
  HIPCHK(hipGetLastError());
  vfm_status st = check_stream_flag(x, s);
  if (st != VFM_OK) return st;
  return check_host_err(x, s);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Execution-state capsules: device copies of the bound buffers (and the FP8
// activation scales), taken and put back with stream-ordered D2D copies.
// ---------------------------------------------------------------------------

struct vfm_capsule {
  // layout the state belongs to
  int L = 0, Hkv = 0, d = 0, H = 0, A = 0, S = 0, act_bf16 = 0, B = 0, P = 0;
  struct Slot {
    int which = 0;          // 0 prefix_k, 1 prefix_v, 2 noise, 3 state, 4 actions
    size_t bytes = 0;
    void* dev = nullptr;    // owned by the capsule
  };
  std::vector<Slot> slots;
  bool from_fp8 = false;
  std::vector<float> act_scale;   // FP8 source: its activation scales at save time (may be empty)
  bool saved = false;
};

namespace {

const char* const kBufNames[5] = {"prefix_k", "prefix_v", "noise", "state", "actions"};

BoundBuf* buf_slot(vfm_expert* x, int which) {
  switch (which) {
    case 0: return &x->prefix_k;
    case 1: return &x->prefix_v;
    case 2: return &x->noise;
    case 3: return &x->state;
    default: return &x->actions;
  }
}

size_t buf_bytes(const BoundBuf& b) {
  size_t n = b.dtype == VFM_BF16 ? 2 : 4;
  for (int i = 0; i < b.ndim; ++i) n *= (size_t)b.shape[i];
  return n;
}

// The expert's bindings match the layout the capsule was made for.
vfm_status capsule_matches(vfm_expert* x, const vfm_capsule* c) {
  if (c->L != x->L || c->Hkv != x->Hkv || c->d != x->d || c->H != x->H || c->A != x->A || c->S != x->S ||
      c->act_bf16 != x->act_bf16)
    return fail(VFM_E_SHAPE, "capsule was made for a different expert layout");
  if (!x->prefix_k.bound) return fail(VFM_E_UNBOUND, "buffer 'prefix_k' is not bound");
  if (x->prefix_k.shape[1] != c->B || x->prefix_k.shape[2] != c->P)
    return fail(VFM_E_SHAPE, "capsule holds batch %d, prefix %d; the expert has %lld, %lld bound", c->B, c->P,
                (long long)x->prefix_k.shape[1], (long long)x->prefix_k.shape[2]);
  for (const vfm_capsule::Slot& sl : c->slots) {
    const BoundBuf* b = buf_slot(x, sl.which);
    if (!b->bound) return fail(VFM_E_UNBOUND, "buffer '%s' is in the capsule but not bound", kBufNames[sl.which]);
    if (buf_bytes(*b) != sl.bytes) return fail(VFM_E_SHAPE, "buffer '%s' has another shape than in the capsule",
                                               kBufNames[sl.which]);
  }
  return VFM_OK;
}

}  // namespace

extern "C" {

vfm_status vfm_capsule_create(vfm_expert* x, vfm_capsule** out) {
  if (!out) return fail(VFM_E_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (!x) return fail(VFM_E_INVALID_ARG, "expert is NULL");
  if (!x->prefix_k.bound) return fail(VFM_E_UNBOUND, "buffer 'prefix_k' is not bound");
  vfm_capsule* c = new vfm_capsule();
  c->L = x->L; c->Hkv = x->Hkv; c->d = x->d; c->H = x->H; c->A = x->A; c->S = x->S; c->act_bf16 = x->act_bf16;
  c->B = (int)x->prefix_k.shape[1];
  c->P = (int)x->prefix_k.shape[2];
  c->from_fp8 = fp8_act(x);
  for (int w = 0; w < 5; ++w) {
    const BoundBuf* b = buf_slot(x, w);
    if (!b->bound) continue;
    vfm_capsule::Slot sl;
    sl.which = w;
    sl.bytes = buf_bytes(*b);
    if (sl.bytes > 0 && hipMalloc(&sl.dev, sl.bytes) != hipSuccess) {
      vfm_capsule_destroy(c);
      return fail(VFM_E_OOM, "capsule buffer '%s' (%zu bytes)", kBufNames[w], sl.bytes);
    }
    c->slots.push_back(sl);
  }
  *out = c;
  return VFM_OK;
}

vfm_status vfm_capsule_save(vfm_expert* x, vfm_capsule* c, void* stream) {
  if (!x || !c) return fail(VFM_E_INVALID_ARG, "NULL argument");
  vfm_status st = capsule_matches(x, c);
  if (st != VFM_OK) return st;
  if (c->from_fp8 != fp8_act(x)) return fail(VFM_E_STATE, "capsule and expert differ in FP8 activations");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  for (const vfm_capsule::Slot& sl : c->slots)
    if (sl.bytes) HIPCHK(hipMemcpyAsync(sl.dev, buf_slot(x, sl.which)->ptr, sl.bytes, hipMemcpyDeviceToDevice, s));
  c->act_scale = x->act_scale;
  c->saved = true;
  return VFM_OK;
}

vfm_status vfm_capsule_restore(vfm_expert* x, const vfm_capsule* c, void* stream) {
  if (!x || !c) return fail(VFM_E_INVALID_ARG, "NULL argument");
  if (!c->saved) return fail(VFM_E_STATE, "capsule holds no saved state");
  vfm_status st = capsule_matches(x, c);
  if (st != VFM_OK) return st;
  const bool fp8 = fp8_act(x) && c->from_fp8;
  if (fp8 && c->act_scale != x->act_scale) {
    if (c->act_scale.empty()) {
      x->act_scale.clear();
    } else if ((st = vfm_set_act_scales(x, c->act_scale.data(), (int32_t)c->act_scale.size())) != VFM_OK) {
      return st;
    }
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  for (const vfm_capsule::Slot& sl : c->slots)
    if (sl.bytes) HIPCHK(hipMemcpyAsync(buf_slot(x, sl.which)->ptr, sl.dev, sl.bytes, hipMemcpyDeviceToDevice, s));
  return VFM_OK;
}

vfm_status vfm_capsule_bytes(const vfm_capsule* c, size_t* bytes) {
  if (!c || !bytes) return fail(VFM_E_INVALID_ARG, "NULL argument");
  size_t n = 0;
  for (const vfm_capsule::Slot& sl : c->slots) n += sl.bytes;
  *bytes = n;
  return VFM_OK;
}

vfm_status vfm_capsule_destroy(vfm_capsule* c) {
  if (!c) return VFM_OK;
  (void)hipDeviceSynchronize();
  for (vfm_capsule::Slot& sl : c->slots)
    if (sl.dev) (void)hipFree(sl.dev);
  delete c;
  return VFM_OK;
}

vfm_status vfm_expert_destroy(vfm_expert* x) {
  if (!x) return VFM_OK;
  (void)hipDeviceSynchronize();
  vfm_status st = check_host_err(x, nullptr);
  free_all(x);
  delete x;
  return st;
}

}  // extern "C"
