// vfm_prefix_rt.cpp -- C ABI of the prefix producer (include/vfm.h,
// vfm_prefix_*): config and weight validation, create-time packing, and the
// per-call launch sequence (per layer: norm, fused QKV + rotary + K/V store,
// attention, o projection, norm, fused gate/up + GeGLU, down projection).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "vfm.h"
#include "vfm_params.h"
#include "vfm_prefix.h"
#include "vfm_stage_io.h"

using namespace vfm;

// Static workspace of vfm_prefix_run_noalloc: one array per device (each GPU
// the library runs on holds it until the process ends), its device address
// taken once per device with hipGetSymbolAddress; host code never passes the
// array's name to a kernel.
constexpr size_t NOALLOC_BYTES = 64ull << 20;
static __device__ __align__(256) unsigned char scratch[NOALLOC_BYTES];

struct vfm_prefix {
  vfm_prefix_config cfg{};
  int L = 0, W = 0, Hq = 0, Hkv = 0, d = 0, F = 0, maxB = 0, maxP = 0;
  std::vector<void*> allocs;
  std::vector<uint8_t*> w_qkv, w_o, w_gu, w_down;
  std::vector<float*> g_attn, g_mlp;
  float* x = nullptr;        // [Mpad][W] residual stream
  float* part = nullptr;     // [MAX_SPLIT][Mpad][W]
  uint8_t* xn = nullptr;     // packed [Mpad/16][W/32][64][16 B]
  uint8_t* attn = nullptr;   // packed [Mpad/16][Hq d/32][64][16 B]
  uint8_t* act = nullptr;    // packed [Mpad/16][F/32][64][16 B]
  uint16_t* q = nullptr;     // [maxB maxP][Hq][d]
  uint16_t* vt = nullptr;    // [maxB][Hkv][d][Ppad max]
  float* rope = nullptr;     // [maxP][d/2][2]
  int rope_P = -1;
  bool wide_gu = true;       // option "gate_up_tiles"
  bool wide_down = true;     // option "down_tiles"
  bool half_qkv = true;      // option "qkv_tiles"
  bool half_o = true;        // option "o_tiles"

  void* dalloc(size_t bytes) {
    void* p = nullptr;
    if (bytes == 0) bytes = 16;
    if (hipMalloc(&p, bytes) != hipSuccess) return nullptr;
    allocs.push_back(p);
    return p;
  }
};

namespace {

#define PCHK(call)                                                                                     \
  do {                                                                                                 \
    hipError_t e_ = (call);                                                                            \
    if (e_ != hipSuccess) return report(VFM_E_HIP, "%s failed: %s", #call, hipGetErrorString(e_));     \
  } while (0)

size_t round_up(size_t a, size_t b) { return (a + b - 1) / b * b; }

void free_prefix(vfm_prefix* x) {
  for (void* p : x->allocs) (void)hipFree(p);
  x->allocs.clear();
}

vfm_status validate(const vfm_prefix_config* c) {
  if (!c) return report(VFM_E_INVALID_ARG, "config is NULL");
  if (c->abi_version != VFM_ABI_VERSION) return report(VFM_E_INVALID_ARG, "abi_version %d != %d", c->abi_version, VFM_ABI_VERSION);
  if (c->num_layers < 1 || c->num_layers > 256) return report(VFM_E_INVALID_ARG, "num_layers %d outside [1, 256]", c->num_layers);
  if (c->width < 128 || c->width > 4096 || c->width % 128) return report(VFM_E_INVALID_ARG, "width %d: multiple of 128 in [128, 4096]", c->width);
  if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256) return report(VFM_E_INVALID_ARG, "head_dim %d not in {64, 128, 256}", c->head_dim);
  if (c->num_kv_heads < 1 || c->num_q_heads < 1 || c->num_q_heads % c->num_kv_heads || c->num_q_heads > 64)
    return report(VFM_E_INVALID_ARG, "num_q_heads %d must be a multiple of num_kv_heads %d (at most 64)", c->num_q_heads, c->num_kv_heads);
  if ((c->num_q_heads * c->head_dim) % 128) return report(VFM_E_INVALID_ARG, "num_q_heads * head_dim must be a multiple of 128");
  if (c->mlp_dim < 64 || c->mlp_dim % 64 || c->mlp_dim > 65536) return report(VFM_E_INVALID_ARG, "mlp_dim %d: multiple of 64 in [64, 65536]", c->mlp_dim);
  if (c->max_prefix_len < 1 || c->max_prefix_len > 8192) return report(VFM_E_INVALID_ARG, "max_prefix_len %d outside [1, 8192]", c->max_prefix_len);
  if (c->max_batch < 1 || c->max_batch > 256) return report(VFM_E_INVALID_ARG, "max_batch %d outside [1, 256]", c->max_batch);
  if (!(c->rope_base > 0.f) || !(c->rms_eps > 0.f)) return report(VFM_E_INVALID_ARG, "rope_base and rms_eps must be positive");
  const size_t Mpad = round_up((size_t)c->max_batch * c->max_prefix_len, pfx::TM);
  const size_t W = c->width, F = c->mlp_dim, qd = (size_t)c->num_q_heads * c->head_dim;
  const size_t Ppad = round_up(c->max_prefix_len, pfx::AK);
  struct { const char* what; size_t bytes; } ext[] = {
      {"gate/up activations", Mpad * F * 2},
      {"packed gate/up weight", W * 2 * F * 2},
      {"K-split partial sums", (size_t)pfx::MAX_SPLIT * Mpad * W * 4},
      {"query workspace", Mpad * qd * 2},
      {"transposed values", (size_t)c->max_batch * c->num_kv_heads * c->head_dim * Ppad * 2},
  };
  for (const auto& e : ext)
    if (e.bytes > 0x7FFFFFF0ull)
      return report(VFM_E_UNSUPPORTED, "the %s would take %zu bytes, beyond the 2 GiB one buffer offset addresses", e.what, e.bytes);
  return VFM_OK;
}

struct Spec {
  std::string name;
  std::vector<int64_t> shape;
};

std::vector<Spec> prefix_specs(const vfm_prefix* x) {
  std::vector<Spec> s;
  const int64_t W = x->W, qd = (int64_t)x->Hq * x->d, kd = (int64_t)x->Hkv * x->d, F = x->F;
  for (int l = 0; l < x->L; ++l) {
    const std::string p = "layers." + std::to_string(l) + ".";
    s.push_back({p + "attn_norm.w", {W}});
    s.push_back({p + "q.w", {W, qd}});
    s.push_back({p + "k.w", {W, kd}});
    s.push_back({p + "v.w", {W, kd}});
    s.push_back({p + "o.w", {qd, W}});
    s.push_back({p + "mlp_norm.w", {W}});
    s.push_back({p + "gate.w", {W, F}});
    s.push_back({p + "up.w", {W, F}});
    s.push_back({p + "down.w", {F, W}});
  }
  return s;
}

// Packed column order of the fused QKV weight: [k heads | v heads | q heads];
// inside a k or q head, 4 consecutive columns hold dims (2j, 2j+1, 2j+d/2, 2j+1+d/2).
void qkv_columns(const vfm_prefix* x, std::vector<int>& src, std::vector<int>& idx) {
  const int d = x->d, half = d / 2;
  auto head_cols = [&](int sid, int head, bool rot) {
    for (int p = 0; p < d; ++p) {
      src.push_back(sid);
      idx.push_back(head * d + (rot ? 2 * (p / 4) + (p & 1) + ((p >> 1) & 1) * half : p));
    }
  };
  for (int h = 0; h < x->Hkv; ++h) head_cols(1, h, true);
  for (int h = 0; h < x->Hkv; ++h) head_cols(2, h, false);
  for (int h = 0; h < x->Hq; ++h) head_cols(0, h, true);
}

int plan_split(int tiles, int K) {
  int s = 1;
  while (s < pfx::MAX_SPLIT && tiles * s < 256 && (K / (2 * s)) % pfx::TK == 0 && K % (2 * s) == 0) s *= 2;
  return s;
}

// The buffers one pass reads and writes besides its inputs and outputs.
struct PrefixWork {
  float* x;        // [Mpad][W] residual stream
  float* part;     // [S][Mpad][W] K-split partial sums
  uint8_t* xn;     // normalised stream, operand order
  uint8_t* attn;   // attention output, operand order
  uint8_t* act;    // GeGLU activations, operand order
  uint16_t* q;     // rotated queries
  uint16_t* vt;    // transposed values [B][Hkv][d][Ppad]
  float* rope;     // [P][d/2][2]
};

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;

hipError_t scratch_of_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    it = g_scratch_ptr.emplace(dev, ptr).first;
  }
  *out = it->second;
  return hipSuccess;
}

}  // namespace

namespace vfm {

vfm_status prefix_stage_io(const vfm_prefix* p, const void* embeds, int B, int P, const void* prefix_k,
                           const void* prefix_v, StageIO* io) {
  if (!p || !io) return report(VFM_E_INVALID_ARG, "NULL argument");
  if (B < 1 || B > p->maxB) return report(VFM_E_SHAPE, "batch %d outside [1, %d]", B, p->maxB);
  if (P < 1 || P > p->maxP) return report(VFM_E_SHAPE, "prefix length %d outside [1, %d]", P, p->maxP);
  const size_t kv = (size_t)p->L * B * P * p->Hkv * p->d * 2;
  io->reads = {{embeds, (size_t)B * P * p->W * 2}};
  io->writes = {{prefix_k, kv}, {prefix_v, kv}};
  io->owner = p;
  io->device_wide = false;
  return VFM_OK;
}

}  // namespace vfm

extern "C" {

vfm_status vfm_prefix_create(const vfm_prefix_config* cfg, const vfm_tensor* weights, int32_t n_weights, void* stream,
                             vfm_prefix** out) {
  if (!out) return report(VFM_E_INVALID_ARG, "out is NULL");
  *out = nullptr;
  vfm_status st = validate(cfg);
  if (st != VFM_OK) return st;
  if (!weights || n_weights <= 0) return report(VFM_E_INVALID_ARG, "no weights given");
  vfm_prefix tmp;
  tmp.cfg = *cfg;
  tmp.L = cfg->num_layers; tmp.W = cfg->width; tmp.Hq = cfg->num_q_heads; tmp.Hkv = cfg->num_kv_heads;
  tmp.d = cfg->head_dim; tmp.F = cfg->mlp_dim; tmp.maxB = cfg->max_batch; tmp.maxP = cfg->max_prefix_len;

  std::map<std::string, const vfm_tensor*> byname;
  for (int i = 0; i < n_weights; ++i) {
    const vfm_tensor& t = weights[i];
    if (!t.name) return report(VFM_E_INVALID_ARG, "weight %d has no name", i);
    if (byname.count(t.name)) return report(VFM_E_INVALID_ARG, "weight '%s' given twice", t.name);
    byname[t.name] = &t;
  }
  const std::vector<Spec> specs = prefix_specs(&tmp);
  std::map<std::string, const void*> ptr;
  for (const Spec& sp : specs) {
    auto it = byname.find(sp.name);
    if (it == byname.end()) return report(VFM_E_INVALID_ARG, "weight '%s' is missing", sp.name.c_str());
    const vfm_tensor& t = *it->second;
    if (!t.dev_ptr) return report(VFM_E_INVALID_ARG, "weight '%s' has a NULL pointer", sp.name.c_str());
    if (t.dtype != VFM_BF16) return report(VFM_E_DTYPE, "weight '%s' must be bf16", sp.name.c_str());
    if (t.ndim != (int)sp.shape.size()) return report(VFM_E_SHAPE, "weight '%s' has %d dims, expected %d", sp.name.c_str(), t.ndim, (int)sp.shape.size());
    for (size_t j = 0; j < sp.shape.size(); ++j)
      if (t.shape[j] != sp.shape[j])
        return report(VFM_E_SHAPE, "weight '%s' dim %zu is %lld, expected %lld", sp.name.c_str(), j, (long long)t.shape[j], (long long)sp.shape[j]);
    ptr[sp.name] = t.dev_ptr;
  }
  if (byname.size() != specs.size())
    for (auto& kv : byname)
      if (!ptr.count(kv.first)) return report(VFM_E_INVALID_ARG, "unknown weight name '%s'", kv.first.c_str());

  vfm_prefix* x = new vfm_prefix(tmp);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  auto bail = [&](vfm_status code) { free_prefix(x); delete x; return code; };
  const int L = x->L, W = x->W, Hq = x->Hq, Hkv = x->Hkv, d = x->d, F = x->F;
  const int nqkv = (Hq + 2 * Hkv) * d;

  std::vector<int> qsrc, qidx, osrc, oidx, gsrc, gidx;
  qkv_columns(x, qsrc, qidx);
  for (int c = 0; c < W; ++c) { osrc.push_back(0); oidx.push_back(c); }
  for (int c = 0; c < 2 * F; ++c) { gsrc.push_back(c & 1); gidx.push_back(2 * (c / 4) + ((c >> 1) & 1)); }
  auto upload = [&](const std::vector<int>& v) -> int* {
    int* p = (int*)x->dalloc(v.size() * 4);
    if (p && hipMemcpy(p, v.data(), v.size() * 4, hipMemcpyHostToDevice) != hipSuccess) return nullptr;
    return p;
  };
  int *qs = upload(qsrc), *qi = upload(qidx), *os = upload(osrc), *oi = upload(oidx), *gs = upload(gsrc), *gi = upload(gidx);
  if (!qs || !qi || !os || !oi || !gs || !gi) { report(VFM_E_OOM, "column map upload failed"); return bail(VFM_E_OOM); }
  for (int l = 0; l < L; ++l) {
    const std::string p = "layers." + std::to_string(l) + ".";
    uint8_t* wq = (uint8_t*)x->dalloc((size_t)W * nqkv * 2);
    uint8_t* wo = (uint8_t*)x->dalloc((size_t)Hq * d * W * 2);
    uint8_t* wg = (uint8_t*)x->dalloc((size_t)W * 2 * F * 2);
    uint8_t* wd = (uint8_t*)x->dalloc((size_t)F * W * 2);
    float* ga = (float*)x->dalloc((size_t)W * 4);
    float* gm = (float*)x->dalloc((size_t)W * 4);
    if (!wq || !wo || !wg || !wd || !ga || !gm) { report(VFM_E_OOM, "weight allocation failed"); return bail(VFM_E_OOM); }
    hipError_t e;
    if ((e = pack_weight(wq, W, nqkv, qs, qi, ptr[p + "q.w"], Hq * d, ptr[p + "k.w"], Hkv * d, ptr[p + "v.w"], Hkv * d, 1, 1, s)) != hipSuccess ||
        (e = pack_weight(wo, Hq * d, W, os, oi, ptr[p + "o.w"], W, nullptr, 0, nullptr, 0, 1, 1, s)) != hipSuccess ||
        (e = pack_weight(wg, W, 2 * F, gs, gi, ptr[p + "gate.w"], F, ptr[p + "up.w"], F, nullptr, 0, 1, 1, s)) != hipSuccess ||
        (e = pack_weight(wd, F, W, os, oi, ptr[p + "down.w"], W, nullptr, 0, nullptr, 0, 1, 1, s)) != hipSuccess ||
        (e = to_f32(ga, ptr[p + "attn_norm.w"], W, 1, s)) != hipSuccess ||
        (e = to_f32(gm, ptr[p + "mlp_norm.w"], W, 1, s)) != hipSuccess) {
      report(VFM_E_HIP, "weight packing failed: %s", hipGetErrorString(e));
      return bail(VFM_E_HIP);
    }
    x->w_qkv.push_back(wq); x->w_o.push_back(wo); x->w_gu.push_back(wg); x->w_down.push_back(wd);
    x->g_attn.push_back(ga); x->g_mlp.push_back(gm);
  }
  const size_t Mpad = round_up((size_t)x->maxB * x->maxP, pfx::TM);
  const size_t Ppad = round_up(x->maxP, pfx::AK);
  x->x = (float*)x->dalloc(Mpad * W * 4);
  x->part = (float*)x->dalloc((size_t)pfx::MAX_SPLIT * Mpad * W * 4);
  x->xn = (uint8_t*)x->dalloc(Mpad * W * 2);
  x->attn = (uint8_t*)x->dalloc(Mpad * Hq * d * 2);
  x->act = (uint8_t*)x->dalloc(Mpad * F * 2);
  x->q = (uint16_t*)x->dalloc(Mpad * Hq * d * 2);
  const size_t vt_bytes = (size_t)x->maxB * Hkv * d * Ppad * 2;
  x->vt = (uint16_t*)x->dalloc(vt_bytes);
  x->rope = (float*)x->dalloc((size_t)x->maxP * d * 4);
  if (!x->x || !x->part || !x->xn || !x->attn || !x->act || !x->q || !x->vt || !x->rope) {
    report(VFM_E_OOM, "workspace allocation failed");
    return bail(VFM_E_OOM);
  }
  // every workspace starts at zero: padded token rows and padded key columns
  // are read (and multiplied by zero weights) but never written
  if (hipMemsetAsync(x->attn, 0, Mpad * Hq * d * 2, s) != hipSuccess || hipMemsetAsync(x->act, 0, Mpad * F * 2, s) != hipSuccess ||
      hipMemsetAsync(x->vt, 0, vt_bytes, s) != hipSuccess || hipMemsetAsync(x->xn, 0, Mpad * W * 2, s) != hipSuccess ||
      pfx::prepare() != hipSuccess || hipStreamSynchronize(s) != hipSuccess || hipGetLastError() != hipSuccess) {
    report(VFM_E_HIP, "create-time device work failed");
    return bail(VFM_E_HIP);
  }
  *out = x;
  return VFM_OK;
}

namespace {

vfm_status check_run_args(vfm_prefix* x, const void* embeds, int32_t B, int32_t P, void* prefix_k, void* prefix_v) {
  if (!x) return report(VFM_E_INVALID_ARG, "producer is NULL");
  if (B < 1 || B > x->maxB) return report(VFM_E_SHAPE, "batch %d outside [1, %d]", B, x->maxB);
  if (P < 1 || P > x->maxP) return report(VFM_E_SHAPE, "prefix length %d outside [1, %d]", P, x->maxP);
  if (!embeds || !prefix_k || !prefix_v) return report(VFM_E_INVALID_ARG, "NULL buffer");
  if ((reinterpret_cast<uintptr_t>(embeds) | reinterpret_cast<uintptr_t>(prefix_k) | reinterpret_cast<uintptr_t>(prefix_v)) % 16)
    return report(VFM_E_INVALID_ARG, "buffers must be 16-byte aligned");
  return VFM_OK;
}

// The layer sequence over workspace `ws` (rope already holds positions 0 .. P-1).
vfm_status run_pass(vfm_prefix* x, const PrefixWork& ws, const void* embeds, int32_t B, int32_t P, void* prefix_k,
                    void* prefix_v, hipStream_t s) {
  const int L = x->L, W = x->W, Hq = x->Hq, Hkv = x->Hkv, d = x->d, F = x->F;
  const int M = B * P, Mpad = (int)round_up(M, pfx::TM), Ppad = (int)round_up(P, pfx::AK);
  const size_t kv_layer = (size_t)B * P * Hkv * d;
  const int MT = Mpad / pfx::TM;
  // o: 128 x 64 tiles with half the K splits where 128 x 128 tiles would
  // split K (the same units, half the partial sums for the next norm)
  int S_o = plan_split(MT * (W / pfx::TN), Hq * d);
  const bool o_half = x->half_o && S_o > 1 && W % 64 == 0;
  if (o_half) S_o /= 2;
  const pfx::PartPlan pd = pfx::part_plan(M, Mpad, W, F, plan_split(MT * (W / pfx::TN), F), x->wide_down);
  const int S_d = pd.S;

  pfx::NormArgs na{};
  na.embeds = static_cast<const uint16_t*>(embeds);
  na.x = ws.x; na.part = ws.part; na.xn = ws.xn; na.M = M; na.Mpad = Mpad; na.W = W; na.eps = x->cfg.rms_eps;
  pfx::GemmArgs ga{};
  ga.M = M; ga.Mpad = Mpad; ga.P = P; ga.Ppad = Ppad; ga.Hq = Hq; ga.Hkv = Hkv; ga.d = d;
  ga.part = ws.part; ga.act = ws.act; ga.q = ws.q; ga.vt = ws.vt; ga.rope = ws.rope;
  ga.qkv_half = x->half_qkv ? 1 : 0;
  pfx::AttnArgs aa{};
  aa.q = ws.q; aa.vt = ws.vt; aa.out = ws.attn; aa.P = P; aa.Ppad = Ppad; aa.Hq = Hq; aa.Hkv = Hkv;
  aa.scale_log2 = 1.4426950408889634f / sqrtf((float)d);

  for (int l = 0; l < L; ++l) {
    const bool last = l == L - 1;
    uint16_t* kl = static_cast<uint16_t*>(prefix_k) + (size_t)l * kv_layer;
    uint16_t* vl = static_cast<uint16_t*>(prefix_v) + (size_t)l * kv_layer;
    na.gain = x->g_attn[l];
    na.S = l == 0 ? 0 : S_d;
    PCHK(pfx::norm(l == 0, na, s));
    ga.A = x->w_qkv[l]; ga.B = ws.xn; ga.K = W; ga.S = 1;
    ga.N = last ? 2 * Hkv * d : (Hq + 2 * Hkv) * d;   // the last layer needs its keys and values only
    ga.k_out = kl; ga.v_out = vl;
    PCHK(pfx::gemm(pfx::EPI_QKV, ga, s));
    if (last) break;
    aa.k = kl;
    PCHK(pfx::attention(d, aa, B, s));
    ga.A = x->w_o[l]; ga.B = ws.attn; ga.N = W; ga.K = Hq * d; ga.S = S_o; ga.bm = 0; ga.part_half = o_half ? 1 : 0;
    PCHK(pfx::gemm(pfx::EPI_PART, ga, s));
    na.gain = x->g_mlp[l]; na.S = S_o;
    PCHK(pfx::norm(false, na, s));
    ga.A = x->w_gu[l]; ga.B = ws.xn; ga.N = 2 * F; ga.K = W; ga.S = 1;
    PCHK(pfx::gemm(pfx::EPI_GU, ga, s, x->wide_gu));
    ga.A = x->w_down[l]; ga.B = ws.act; ga.N = W; ga.K = F; ga.S = S_d; ga.bm = pd.bm; ga.part_half = 0;
    PCHK(pfx::gemm(pfx::EPI_PART, ga, s));
  }
  return VFM_OK;
}

}  // namespace

vfm_status vfm_prefix_run(vfm_prefix* x, const void* embeds, int32_t B, int32_t P, void* prefix_k, void* prefix_v,
                          void* stream) {
  vfm_status st = check_run_args(x, embeds, B, P, prefix_k, prefix_v);
  if (st != VFM_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (x->rope_P != P) {
    PCHK(build_rope(x->rope, P, x->d, 0, x->cfg.rope_base, s));
    x->rope_P = P;
  }
  const PrefixWork ws{x->x, x->part, x->xn, x->attn, x->act, x->q, x->vt, x->rope};
  return run_pass(x, ws, embeds, B, P, prefix_k, prefix_v, s);
}

vfm_status vfm_prefix_run_noalloc(vfm_prefix* x, const void* embeds, int32_t B, int32_t P, void* prefix_k,
                                  void* prefix_v, void* stream) {
  vfm_status st = check_run_args(x, embeds, B, P, prefix_k, prefix_v);
  if (st != VFM_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t W = x->W, F = x->F, qd = (size_t)x->Hq * x->d;
  const size_t Mpad = round_up((size_t)B * P, pfx::TM), Ppad = round_up(P, pfx::AK);
  const int MT = (int)(Mpad / pfx::TM);
  const pfx::PartPlan pd = pfx::part_plan(B * P, (int)Mpad, (int)W, (int)F, plan_split(MT * ((int)W / pfx::TN), (int)F),
                                          x->wide_down);
  const size_t S = (size_t)std::max(plan_split(MT * ((int)W / pfx::TN), (int)qd), pd.S);
  // this call's workspace, carved from the static array (256-byte aligned pieces)
  const size_t sz[8] = {Mpad * W * 4, S * Mpad * W * 4, Mpad * W * 2, Mpad * qd * 2, Mpad * F * 2, Mpad * qd * 2,
                        (size_t)B * x->Hkv * x->d * Ppad * 2, (size_t)P * x->d * 4};
  size_t off[8], total = 0;
  for (int i = 0; i < 8; ++i) {
    off[i] = total;
    total += round_up(sz[i], 256);
  }
  if (total > NOALLOC_BYTES)
    return report(VFM_E_UNSUPPORTED, "batch %d x prefix %d needs %zu bytes of workspace; the static workspace holds %zu",
                  B, P, total, NOALLOC_BYTES);
  void* base = nullptr;
  PCHK(scratch_of_device(&base));
  unsigned char* b = static_cast<unsigned char*>(base);
  const PrefixWork ws{reinterpret_cast<float*>(b + off[0]), reinterpret_cast<float*>(b + off[1]),
                      b + off[2], b + off[3], b + off[4], reinterpret_cast<uint16_t*>(b + off[5]),
                      reinterpret_cast<uint16_t*>(b + off[6]), reinterpret_cast<float*>(b + off[7])};
  // the array keeps the last call's contents: the buffers whose padding is
  // read (padded token rows, padded key columns) start at zero again, and the
  // rotary table is rebuilt (with fill and table kernels, no memset nodes)
  PCHK(zero_words(reinterpret_cast<unsigned*>(ws.xn), (int)(sz[2] / 4), s));
  PCHK(zero_words(reinterpret_cast<unsigned*>(ws.attn), (int)(sz[3] / 4), s));
  PCHK(zero_words(reinterpret_cast<unsigned*>(ws.act), (int)(sz[4] / 4), s));
  PCHK(zero_words(reinterpret_cast<unsigned*>(ws.vt), (int)(sz[6] / 4), s));
  PCHK(build_rope(ws.rope, P, x->d, 0, x->cfg.rope_base, s));
  return run_pass(x, ws, embeds, B, P, prefix_k, prefix_v, s);
}

vfm_status vfm_prefix_set_option(vfm_prefix* x, const char* key, const char* value) {
  if (!x || !key || !value) return report(VFM_E_INVALID_ARG, "NULL argument");
  const std::string k = key, v = value;
  if (k == "gate_up_tiles") {
    if (v == "wide") x->wide_gu = true;
    else if (v == "narrow") x->wide_gu = false;
    else return report(VFM_E_INVALID_ARG, "gate_up_tiles must be 'wide' or 'narrow'");
    return VFM_OK;
  }
  if (k == "o_tiles") {
    if (v == "auto") x->half_o = true;
    else if (v == "full") x->half_o = false;
    else return report(VFM_E_INVALID_ARG, "o_tiles must be 'auto' or 'full'");
    return VFM_OK;
  }
  if (k == "qkv_tiles") {
    if (v == "auto") x->half_qkv = true;
    else if (v == "full") x->half_qkv = false;
    else return report(VFM_E_INVALID_ARG, "qkv_tiles must be 'auto' or 'full'");
    return VFM_OK;
  }
  if (k == "down_tiles") {
    if (v == "wide") x->wide_down = true;
    else if (v == "narrow") x->wide_down = false;
    else return report(VFM_E_INVALID_ARG, "down_tiles must be 'wide' or 'narrow'");
    return VFM_OK;
  }
  return report(VFM_E_INVALID_ARG, "unknown option '%s'", key);
}

vfm_status vfm_prefix_destroy(vfm_prefix* x) {
  if (!x) return VFM_OK;
  (void)hipDeviceSynchronize();
  free_prefix(x);
  delete x;
  return VFM_OK;
}

}  // extern "C"
