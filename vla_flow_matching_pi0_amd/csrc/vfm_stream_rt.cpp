// vfm_stream_rt.cpp -- host side of the streaming batch-1 kernel (vfm_stream.h):
// work plans, workspace, create-time shift x W tables, launch.
#include "vfm_stream_rt.h"

#include <algorithm>
#include <cstring>

namespace vfm {
vfm_status report(vfm_status s, const char* fmt, ...);
hipError_t zero_words(unsigned* p, int n, hipStream_t st);
namespace sk {

namespace {

constexpr int LDS_MAX = 160 * 1024;

// K = 0: a tile plan without a contraction to split (the in projection)
bool plan_gemm(int T, int K, int S, int G, int per_xcd, int umax, GemmPlanH& out, std::string* why, const char* name) {
  out = GemmPlanH{};
  out.T = T;
  out.S = S;
  if (K > 0) {
    if (K % 32 || (K / 32) % S) { *why = std::string(name) + ": K not a multiple of 32 x splits"; return false; }
    out.nkb = K / 32;
    out.nkbs = out.nkb / S;
    if (out.nkbs % 2 || out.nkbs > 2 * MAXJ) {
      *why = std::string(name) + ": K slice must be an even number of 32-K blocks <= 1024";
      return false;
    }
  }
  if (S > SMAX || per_xcd < S) { *why = std::string(name) + ": too many K splits"; return false; }
  std::vector<std::vector<uint32_t>> lists(G);
  for (int x = 0; x < NXCD; ++x) {
    std::vector<int> tiles;
    for (int t = x; t < T; t += NXCD) tiles.push_back(t);
    for (int s = 0; s < S; ++s) {
      std::vector<int> slots;
      for (int j = s; j < per_xcd; j += S) slots.push_back(j);
      for (size_t i = 0; i < tiles.size(); ++i) {
        const int w = x * per_xcd + slots[i % slots.size()];
        lists[w].push_back(((uint32_t)tiles[i] << 8) | (uint32_t)s);
      }
    }
  }
  int U = 0;
  for (auto& l : lists) U = std::max(U, (int)l.size());
  if (U > umax) { *why = std::string(name) + ": more units per workgroup than the kernel holds"; return false; }
  out.U = std::max(U, 1);
  out.units.assign((size_t)G * out.U, 0xFFFFFFFFu);
  for (int w = 0; w < G; ++w)
    for (size_t i = 0; i < lists[w].size(); ++i) out.units[(size_t)w * out.U + i] = lists[w][i];
  return true;
}

}  // namespace

bool stream_plan(const StreamShape& s, int G, const int splits[4], StreamPlan* out, std::string* why) {
  StreamPlan P;
  if (G <= 0 || G % NXCD) { *why = "compute-unit count is not a multiple of 8"; return false; }
  P.G = G;
  P.per_xcd = G / NXCD;
  if (s.H < 1 || s.H > 64) { *why = "action horizon above 64"; return false; }
  if (s.d != 64 && s.d != 128 && s.d != 256) { *why = "head dim not 64, 128 or 256"; return false; }
  if (s.W % 256 || s.W > 2048) { *why = "width not a multiple of 256 up to 2048"; return false; }
  if (s.A % 4 || s.A > 64) { *why = "action dim"; return false; }
  if (s.L < 1 || s.L > MAX_LAYERS) { *why = "layer count"; return false; }
  if (s.Hq % s.Hkv) { *why = "query heads not a multiple of KV heads"; return false; }
  const int Nq = (s.Hq + 2 * s.Hkv) * s.d;
  const int umax[4] = {UMAX, UMAX, UMAX, UMAX};
  const int T[4] = {Nq / 16, s.W / 16, 2 * s.F / 16, s.W / 16};
  const int K[4] = {s.W, s.Hq * s.d, s.W, s.F};
  const char* names[4] = {"qkv", "o", "gate/up", "down"};
  for (int gi = 0; gi < 4; ++gi) {
    if (!plan_gemm(T[gi], K[gi], splits[gi], G, P.per_xcd, umax[gi], P.g[gi], why, names[gi])) return false;
    if ((gi == GQ || gi == GG) && splits[gi] != 1) { *why = "qkv and gate/up run unsplit"; return false; }
  }
  if (!plan_gemm(s.W / 16, 0, 1, G, P.per_xcd, IUMAX, P.in, why, "in")) return false;
  int off = 0, umx = 1;
  for (int gi = 0; gi < 4; ++gi) {
    P.regions[gi] = off;
    int bytes = P.g[gi].U * P.g[gi].nkbs * 1024;
    // attention stages one unit's keys and values (4 d / 32 fragments of 1 KiB) in the qkv region
    if (gi == GQ) bytes = std::max(bytes, 4 * (s.d / 32) * 1024);
    off += bytes;
    umx = std::max(umx, P.g[gi].U);
  }
  P.scratch = off;
  off += umx * 4 * 1024;
  P.ctl = off;
  off += CTL;
  P.lds = off;
  if (P.lds > LDS_MAX) { *why = "weight tiles of one layer exceed the LDS of a compute unit"; return false; }
  *out = std::move(P);
  return true;
}

bool stream_attn_plan(const StreamShape& s, int G, int per_xcd, int P, std::vector<uint32_t>* units, int* AU, int* KS,
                      int* KSp, std::string* why) {
  const int ksp = (P + 31) / 32, ksc = (s.H + 31) / 32;
  const int ks = ksp + ksc;
  if (ks > 64) { *why = "prefix too long for the attention merge (at most 64 splits of 32 keys)"; return false; }
  std::vector<std::vector<uint32_t>> lists(G);
  for (int x = 0; x < NXCD; ++x) {
    int i = 0;
    for (int j = x; j < s.Hq; j += NXCD)
      for (int c = 0; c < ks; ++c, ++i) lists[x * per_xcd + i % per_xcd].push_back(((uint32_t)j << 8) | (uint32_t)c);
  }
  int au = 0;
  for (auto& l : lists) au = std::max(au, (int)l.size());
  if (au > AUMAX) { *why = "too many attention units per workgroup"; return false; }
  au = std::max(au, 1);
  units->assign((size_t)G * au, 0xFFFFFFFFu);
  for (int w = 0; w < G; ++w)
    for (size_t i = 0; i < lists[w].size(); ++i) (*units)[(size_t)w * au + i] = lists[w][i];
  *AU = au;
  *KS = ks;
  *KSp = ksp;
  return true;
}

struct StreamState {
  StreamShape s{};
  StreamPlan plan;
  std::vector<void*> allocs;
  const uint8_t* w[4][MAX_LAYERS] = {};
  const float* mod = nullptr;
  uint32_t* d_units[4] = {};
  uint32_t* d_in = nullptr;
  uint32_t* d_attn = nullptr;       // [G][AUMAX]
  unsigned* counters = nullptr;     // cnt(o) [T], cnt(down) [T], hcnt [Hq]
  int n_counters = 0;
  float *part_o = nullptr, *part_d = nullptr;
  float *apart = nullptr, *aml = nullptr;
  bf16* vt = nullptr;
  int Ppad_max = 0, KS_max = 0;
  uint8_t* ring = nullptr;
  size_t slab = 0, o_ya = 0, o_ssa = 0, o_q = 0, o_k = 0, o_vt = 0, o_at = 0, o_ym = 0, o_ssm = 0, o_act = 0;
  float *shw_q = nullptr, *shw_g = nullptr;
  float *h = nullptr, *s_emb = nullptr;
  unsigned* bar = nullptr;
  unsigned* err = nullptr;
  unsigned* herr = nullptr;         // pinned, host-mapped
  unsigned* herr_dev = nullptr;
  int cur_P = -1, AU = 1, KS = 0, KSp = 0;

  void* dalloc(size_t bytes) {
    void* p = nullptr;
    if (hipMalloc(&p, bytes ? bytes : 16) != hipSuccess) return nullptr;
    allocs.push_back(p);
    return p;
  }
};

void stream_destroy(StreamState* s) {
  if (!s) return;
  (void)hipDeviceSynchronize();
  for (void* p : s->allocs) (void)hipFree(p);
  if (s->herr) (void)hipHostFree(s->herr);
  delete s;
}

vfm_status stream_create(const StreamShape& shape, const uint8_t* const* wq, const uint8_t* const* wo,
                         const uint8_t* const* wg, const uint8_t* const* wd, const float* mod, hipStream_t st,
                         StreamState** out, std::string* why) {
  *out = nullptr;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return report(VFM_E_HIP, "device query failed");
  // K splits: o and down until every K slice is at most 1024 (32 blocks of 32), at least 4
  auto split_for = [](int K) { int s = 4; while (K / s > 1024) s *= 2; return s; };
  const int splits[4] = {1, split_for(shape.Hq * shape.d), 1, split_for(shape.F)};
  StreamPlan plan;
  if (!stream_plan(shape, cus, splits, &plan, why)) return VFM_OK;   // not eligible: no state, no error
  StreamState* s = new StreamState();
  s->s = shape;
  s->plan = plan;
  s->mod = mod;
  auto bail = [&](vfm_status code, const char* msg) {
    stream_destroy(s);
    return report(code, "%s", msg);
  };
  for (int l = 0; l < shape.L; ++l) {
    s->w[GQ][l] = wq[l];
    s->w[GO][l] = wo[l];
    s->w[GG][l] = wg[l];
    s->w[GD][l] = wd[l];
  }
  const int L = shape.L, W = shape.W, Hq = shape.Hq, Hkv = shape.Hkv, d = shape.d, F = shape.F, N = shape.N;
  const int Nq = (Hq + 2 * Hkv) * d;
  for (int gi = 0; gi < 4; ++gi) {
    s->d_units[gi] = (uint32_t*)s->dalloc(plan.g[gi].units.size() * 4);
    if (!s->d_units[gi]) return bail(VFM_E_OOM, "stream plan allocation failed");
    if (hipMemcpy(s->d_units[gi], plan.g[gi].units.data(), plan.g[gi].units.size() * 4, hipMemcpyHostToDevice) != hipSuccess)
      return bail(VFM_E_HIP, "stream plan upload failed");
  }
  s->d_in = (uint32_t*)s->dalloc(plan.in.units.size() * 4);
  s->d_attn = (uint32_t*)s->dalloc((size_t)plan.G * AUMAX * 4);
  if (!s->d_in || !s->d_attn) return bail(VFM_E_OOM, "stream plan allocation failed");
  if (hipMemcpy(s->d_in, plan.in.units.data(), plan.in.units.size() * 4, hipMemcpyHostToDevice) != hipSuccess)
    return bail(VFM_E_HIP, "stream plan upload failed");
  s->n_counters = plan.g[GO].T + plan.g[GD].T + Hq;
  s->counters = (unsigned*)s->dalloc((size_t)s->n_counters * 4);
  s->part_o = (float*)s->dalloc((size_t)plan.g[GO].S * plan.g[GO].T * 64 * 16 * 4);
  s->part_d = (float*)s->dalloc((size_t)plan.g[GD].S * plan.g[GD].T * 64 * 16 * 4);
  s->Ppad_max = (shape.maxP + 31) / 32 * 32;
  s->KS_max = s->Ppad_max / 32 + (shape.H + 31) / 32;
  s->apart = (float*)s->dalloc((size_t)Hq * s->KS_max * 64 * d * 4);
  s->aml = (float*)s->dalloc((size_t)Hq * s->KS_max * 64 * 2 * 4);
  s->vt = (bf16*)s->dalloc((size_t)L * Hkv * d * s->Ppad_max * 2);
  {
    auto al = [](size_t b) { return (b + 255) / 256 * 256; };
    size_t off = 0;
    s->o_ya = off; off += al((size_t)W * 128);
    s->o_ssa = off; off += al((size_t)W * 16);
    s->o_q = off; off += al((size_t)Hq * d * 128);
    s->o_k = off; off += al((size_t)Hkv * d * 128);
    s->o_vt = off; off += al((size_t)Hkv * d * 128);
    s->o_at = off; off += al((size_t)Hq * d * 128);
    s->o_ym = off; off += al((size_t)W * 128);
    s->o_ssm = off; off += al((size_t)W * 16);
    s->o_act = off; off += al((size_t)F * 128);
    s->slab = off;
    s->ring = (uint8_t*)s->dalloc(s->slab * (size_t)N * L);
  }
  s->shw_q = (float*)s->dalloc((size_t)N * L * Nq * 4);
  s->shw_g = (float*)s->dalloc((size_t)N * L * 2 * F * 4);
  s->h = (float*)s->dalloc((size_t)64 * W * 4);
  s->s_emb = (float*)s->dalloc((size_t)64 * W * 4);
  s->bar = (unsigned*)s->dalloc((size_t)BAR_WORDS_S * 4);
  s->err = (unsigned*)s->dalloc(4);
  if (!s->counters || !s->part_o || !s->part_d || !s->apart || !s->aml || !s->vt || !s->ring || !s->shw_q || !s->shw_g ||
      !s->h || !s->s_emb || !s->bar || !s->err)
    return bail(VFM_E_OOM, "stream workspace allocation failed");
  if (hipHostMalloc((void**)&s->herr, 4, hipHostMallocMapped) != hipSuccess) return bail(VFM_E_OOM, "pinned allocation failed");
  *s->herr = 0u;
  if (hipHostGetDevicePointer((void**)&s->herr_dev, s->herr, 0) != hipSuccess) return bail(VFM_E_HIP, "host-mapped pointer");
  if (zero_words(s->counters, s->n_counters, st) != hipSuccess || zero_words(s->bar, BAR_WORDS_S, st) != hipSuccess ||
      zero_words(s->err, 1, st) != hipSuccess)
    return bail(VFM_E_HIP, "stream workspace clear failed");
  // shift x W tables (fp64 sums of the packed bf16 weights)
  const int n_norms = 2 * L + 1;
  if (shift_proj(s->shw_q, wq, L, W, Nq, mod, n_norms, 0, W, N, st) != hipSuccess ||
      shift_proj(s->shw_g, wg, L, W, 2 * F, mod, n_norms, 1, W, N, st) != hipSuccess)
    return bail(VFM_E_HIP, "shift projection tables failed");
  if (stream_prepare(d, plan.lds) != hipSuccess) return bail(VFM_E_HIP, "stream kernel attribute");
  int per_cu = 0;
  if (stream_occupancy(d, plan.lds, &per_cu) != hipSuccess || per_cu < 1) {
    stream_destroy(s);
    *why = "the streaming kernel does not fit on a compute unit";
    return VFM_OK;
  }
  if (hipStreamSynchronize(st) != hipSuccess) return bail(VFM_E_HIP, "stream create-time work failed");
  *out = s;
  return VFM_OK;
}

bool stream_accepts(const StreamState* s, int P, std::string* why) {
  if (P > s->s.maxP) { *why = "prefix longer than max_prefix_len"; return false; }
  std::vector<uint32_t> u;
  int au, ks, ksp;
  return stream_attn_plan(s->s, s->plan.G, s->plan.per_xcd, P, &u, &au, &ks, &ksp, why);
}

bool stream_failed(const StreamState* s) {
  return __atomic_load_n(s->herr, __ATOMIC_ACQUIRE) != 0u;
}

hipError_t stream_reset(StreamState* s, hipStream_t st) {
  hipError_t e;
  if ((e = zero_words(s->counters, s->n_counters, st)) != hipSuccess) return e;
  if ((e = zero_words(s->bar, BAR_WORDS_S, st)) != hipSuccess) return e;
  if ((e = zero_words(s->err, 1, st)) != hipSuccess) return e;
  if ((e = hipStreamSynchronize(st)) != hipSuccess) return e;
  __atomic_store_n(s->herr, 0u, __ATOMIC_RELEASE);
  return hipSuccess;
}

int stream_barriers(const StreamState* s) { return s->s.N * (5 * s->s.L + 2) - 1; }

vfm_status stream_debug_copy(const StreamState* s, const std::string& name, int index, void* dst, size_t bytes) {
  const void* src = nullptr;
  size_t n = 0;
  const StreamShape& sh = s->s;
  if (name == "slab") {
    if (index < 0 || index >= sh.N * sh.L) return report(VFM_E_INVALID_ARG, "slab index out of range");
    src = s->ring + (size_t)index * s->slab;
    n = s->slab;
  } else if (name == "h") { src = s->h; n = (size_t)64 * sh.W * 4; }
  else if (name == "s_emb") { src = s->s_emb; n = (size_t)64 * sh.W * 4; }
  else if (name == "vt") { src = s->vt; n = (size_t)sh.L * sh.Hkv * sh.d * s->Ppad_max * 2; }
  else if (name == "apart") { src = s->apart; n = (size_t)sh.Hq * s->KS_max * 64 * sh.d * 4; }
  else if (name == "aml") { src = s->aml; n = (size_t)sh.Hq * s->KS_max * 64 * 8; }
  else if (name == "shw_q") { src = s->shw_q; n = (size_t)sh.N * sh.L * (sh.Hq + 2 * sh.Hkv) * sh.d * 4; }
  else if (name == "shw_g") { src = s->shw_g; n = (size_t)sh.N * sh.L * 2 * sh.F * 4; }
  else return report(VFM_E_INVALID_ARG, "unknown stream buffer '%s'", name.c_str());
  if (bytes != n) return report(VFM_E_SHAPE, "stream buffer '%s' has %zu bytes", name.c_str(), n);
  if (hipDeviceSynchronize() != hipSuccess || hipMemcpy(dst, src, n, hipMemcpyDeviceToHost) != hipSuccess)
    return report(VFM_E_HIP, "stream buffer copy failed");
  return VFM_OK;
}

size_t stream_slab_layout(const StreamState* s, size_t* offs) {
  offs[0] = s->o_ya; offs[1] = s->o_ssa; offs[2] = s->o_q; offs[3] = s->o_k; offs[4] = s->o_vt;
  offs[5] = s->o_at; offs[6] = s->o_ym; offs[7] = s->o_ssm; offs[8] = s->o_act;
  return s->slab;
}
const StreamPlan& stream_plan_of(const StreamState* s) { return s->plan; }

vfm_status stream_run(StreamState* s, int P, const void* pk, const void* pv, const float* noise, const float* state,
                      float* x, const float* in_w, const float* in_b, const float* st_w, const float* st_b,
                      const float* out_w, const float* out_b, const float* rope, bool cooperative,
                      unsigned long long* trace, const StreamTune& tune, hipStream_t st) {
  const StreamShape& sh = s->s;
  const StreamPlan& pl = s->plan;
  if (P != s->cur_P) {
    std::vector<uint32_t> units;
    std::string why;
    if (!stream_attn_plan(sh, pl.G, pl.per_xcd, P, &units, &s->AU, &s->KS, &s->KSp, &why))
      return report(VFM_E_UNSUPPORTED, "streaming kernel: %s", why.c_str());
    // the previous launch may still read the old table: ordered on the same stream
    if (hipMemcpyAsync(s->d_attn, units.data(), units.size() * 4, hipMemcpyHostToDevice, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
      return report(VFM_E_HIP, "attention plan upload failed");
    s->cur_P = P;
  }
  SP p{};
  p.L = sh.L; p.W = sh.W; p.Hq = sh.Hq; p.Hkv = sh.Hkv; p.d = sh.d; p.F = sh.F; p.H = sh.H; p.A = sh.A; p.S = sh.S;
  p.N = sh.N; p.P = P; p.Ppad = (P + 31) / 32 * 32; p.KS = s->KS; p.KSp = s->KSp;
  p.G = pl.G; p.per_xcd = pl.per_xcd; p.AU = s->AU; p.IU = pl.in.U;
  p.eps = sh.eps;
  p.scratch = pl.scratch; p.ctl = pl.ctl;
  for (int gi = 0; gi < 4; ++gi) {
    for (int l = 0; l < sh.L; ++l) p.w[gi][l] = s->w[gi][l];
    const GemmPlanH& g = pl.g[gi];
    p.g[gi].T = g.T; p.g[gi].S = g.S; p.g[gi].nkb = g.nkb; p.g[gi].nkbs = g.nkbs; p.g[gi].U = g.U;
    p.g[gi].region = pl.regions[gi];
    p.g[gi].units = s->d_units[gi];
    p.g[gi].cnt = gi == GO ? s->counters : gi == GD ? s->counters + pl.g[GO].T : nullptr;
    p.g[gi].part = gi == GO ? s->part_o : gi == GD ? s->part_d : nullptr;
  }
  p.attn_units = s->d_attn;
  p.in_units = s->d_in;
  p.hcnt = s->counters + pl.g[GO].T + pl.g[GD].T;
  p.mod = s->mod;
  p.shw_q = s->shw_q;
  p.shw_g = s->shw_g;
  p.rope = rope;
  p.pk = (const bf16*)pk;
  p.pv = (const bf16*)pv;
  p.vt = s->vt;
  p.noise = noise; p.state = state; p.x = x;
  p.in_w = in_w; p.in_b = in_b; p.st_w = st_w; p.st_b = st_b; p.out_w = out_w; p.out_b = out_b;
  p.s_emb = s->s_emb; p.h = s->h;
  p.ring = s->ring; p.slab = s->slab;
  p.o_ya = s->o_ya; p.o_ssa = s->o_ssa; p.o_q = s->o_q; p.o_k = s->o_k; p.o_vt = s->o_vt; p.o_at = s->o_at;
  p.o_ym = s->o_ym; p.o_ssm = s->o_ssm; p.o_act = s->o_act;
  p.apart = s->apart; p.aml = s->aml;
  p.bar = s->bar; p.err = s->err; p.herr = s->herr_dev;
  p.trace = trace;
  p.stop_after = tune.stop_after;
  p.dma_cap = tune.dma_cap;
  p.fail_epoch = tune.fail_epoch;
  p.spin_limit = tune.spin_limit;
  const hipError_t e = stream_launch(p, (size_t)pl.lds, st, cooperative);
  if (e != hipSuccess) return report(VFM_E_HIP, "streaming kernel launch: %s", hipGetErrorString(e));
  return VFM_OK;
}

}  // namespace sk
}  // namespace vfm
