// vfm_stream.h -- the batch-1 denoise loop of a bf16 pi0.5-style expert as one
// persistent kernel whose GEMM weights stream into LDS ahead of their use.
//
// The pages' problem statement of this loop (PhyAI summary, profiling
// paragraph): at batch 1 the action expert is a small share of the FLOPs and a
// large share of the latency because every Euler step crosses many operator
// boundaries. On MI355X one operator boundary of this loop is a device-wide
// synchronisation (measured 1.7 us for a barrier of 256 workgroups) plus the
// broadcast of the next operator's input to every compute unit (about 65 GB/s
// per compute unit when all of them read the same bytes), so this kernel is
// built around making those boundaries few and cheap:
//
//  * Weights never sit on the dependency chain. Each workgroup (one per
//    compute unit) owns fixed tiles of every GEMM; a ninth wave, the loader,
//    copies the tiles of the next layer's GEMMs straight into LDS with
//    direct-to-LDS loads while the current layer runs, and the eight compute
//    waves read weight fragments from LDS only.
//  * The adaptive RMSNorms are folded into the GEMMs next to them
//    (FlashRT walk-through, component 8: residual + norm fused into the
//    neighbouring kernels). The phase that finishes a residual row block
//    writes y = h (1 + scale) as the next GEMM's bf16 operand plus the row
//    block's sums of squares; the consuming GEMM computes
//    xn W = r (y W) + shift W with r = 1 / sqrt(mean(h^2) + eps) from those
//    sums and shift W from a create-time table (the shift depends only on the
//    step and the layer).
//  * The o and down projections split K over several compute units; the last
//    unit of a tile to finish (an arrival counter) adds the partial sums and
//    applies the gated residual, the next norm's scale and the sums of
//    squares, so no separate residual/norm phase exists.
//  * Attention runs one head per XCD; the key splits of a head merge after a
//    barrier among the units of that head only.
//
// Per layer this leaves five device-wide barriers (before qkv, attention, o,
// gate/up and down) instead of eight, and per Euler step two more (out
// projection with the Euler update, in projection).
#pragma once
#include "vfm_device.h"
#include "vfm_stream_params.h"

namespace vfm {
namespace sk {

extern __shared__ __align__(16) char lds[];

// Loads of activations written earlier in the launch (by other XCDs) skip the
// compute unit's L1 and read L2 (the workgroup-scope policy sc0): a cold
// broadcast of 100 KB to every compute unit measured 2.0 us this way against
// 3.5 us with plain loads, while device-scope (sc1) loads lost L2 sharing.
constexpr int CPOL_SC0 = 1;
__device__ __forceinline__ u32x4 act_ld16_if(__amdgpu_buffer_rsrc_t r, uint32_t off, bool ok) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, ok ? off : OOB, 0, CPOL_SC0);
}

__device__ __forceinline__ void wg_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// wait for this wave's outstanding vector-memory operations (stores acknowledged)
__device__ __forceinline__ void vm_drain() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int N>
__device__ __forceinline__ void vmwait_c() { __builtin_amdgcn_s_waitcnt((N & 15) | 0x70 | 0xF00 | ((N >> 4) << 14)); }
template <int N>
__device__ __forceinline__ void vmwait_sel(int n) {
  if constexpr (N < 0) {
    (void)n;
  } else {
    if (n == N) vmwait_c<N>();
    else vmwait_sel<N - 1>(n);
  }
}
// s_waitcnt vmcnt(n) for a wave-uniform n in [0, 63]
__device__ __forceinline__ void vmwait(int n) { vmwait_sel<63>(n); }

// The launch parameters are read in place from the kernel-argument segment
// (constant address space): every field access is a scalar load, and the
// 2 KB block is never copied to private memory.
typedef __attribute__((address_space(4))) const SP KSP;
typedef __attribute__((address_space(4))) const SGemm KSG;

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }
__device__ __forceinline__ unsigned* ctl(KSP& p) { return reinterpret_cast<unsigned*>(lds + p.ctl); }

__device__ __forceinline__ void raise_err(KSP& p, unsigned code) {
  __hip_atomic_fetch_or(p.err, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (p.herr) __hip_atomic_store(p.herr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ unsigned ld_dev(const unsigned* a) { return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

__device__ __forceinline__ uint8_t* slab(KSP& p, int k, int l) { return p.ring + ((size_t)k * p.L + l) * p.slab; }
// GEMM operand order [K/32][64][32] bf16: element offset of (token m, feature c)
__device__ __forceinline__ uint32_t opo(int m, int c) { return (uint32_t)((((c >> 5) * 64 + m) << 5) + (c & 31)); }
// position of key k (0..31) of a 32-key block in the transposed value layout:
// the PV operand of lane group g holds keys 4g..4g+3 and 16+4g..16+4g+3
__device__ __forceinline__ int vperm(int k) { return 8 * ((k & 15) >> 2) + 4 * (k >> 4) + (k & 3); }

// ------------------------------------------------------------------ workgroup barrier
// The loader wave runs its own loop, so the eight compute waves meet at an
// LDS arrival counter instead of s_barrier (which would wait for the loader
// too). The counter only grows, NCW arrivals per use; a wave's target is the
// next multiple of NCW above the count it found, which stays right when a
// fast wave arrives at the next barrier before a slow one left this one.
typedef __attribute__((address_space(3))) unsigned lds_u32;
__device__ __forceinline__ lds_u32* ctl3(KSP& p) { return (lds_u32*)(lds + p.ctl); }
__device__ __forceinline__ unsigned lds_ld(lds_u32* a) { return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP); }
__device__ __forceinline__ void lds_st(lds_u32* a, unsigned v) { __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP); }

__device__ __forceinline__ void cw_sync(KSP& p) {
  lds_u32* c = ctl3(p) + C_CWB;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's LDS accesses are done
  unsigned old = 0;
  if (lane_id() == 0) old = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  const unsigned target = ((unsigned)__builtin_amdgcn_readfirstlane((int)old) / NCW + 1u) * NCW;
  while (lds_ld(c) < target) __builtin_amdgcn_s_sleep(1);
  asm volatile("" ::: "memory");
}

// ------------------------------------------------------------------ grid barrier
// Flat 64-counter barrier (the fastest of the variants measured on MI355X:
// 1.7 us for 256 workgroups; a two-level tree and a per-XCD tree measured
// 1.8 and 1.9 us), run by the compute waves. Wave 0 publishes the phase
// slots completed (`done`: the LDS regions they used may be refilled) and polls the
// counters; meanwhile wave 1 waits until the loader reports fill `need`
// (the next phase's weights) landed.
__device__ __forceinline__ bool gbar(KSP& p, unsigned& epoch, int done, int need) {
  ++epoch;
  const int wv = wave_id(), lane = lane_id();
  lds_u32* ct = ctl3(p);
  vm_drain();
  cw_sync(p);
  if (wv == 0) {
    if (lane == 0) {
      if (p.trace && blockIdx.x == 0) p.trace[3 * epoch] = __builtin_amdgcn_s_memrealtime();
      __hip_atomic_fetch_add(&p.bar[BW_CTR + 64 * (blockIdx.x % N_CTR)], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      lds_st(ct + C_FREE, (unsigned)done);
    }
    // barrier fail_epoch (diagnostics) waits for one arrival more than the grid holds
    const unsigned target = epoch * (unsigned)p.G + ((int)epoch == p.fail_epoch ? 1u : 0u);
    unsigned ok = 1;
    long spins = 0;
    for (;;) {
      unsigned v = ld_dev(&p.bar[BW_CTR + 64 * lane]);
#pragma unroll
      for (int sh = 1; sh < N_CTR; sh *= 2) v += __shfl_xor(v, sh);
      if (v >= target) break;
      if ((++spins & 255) == 0) {
        unsigned e = lane == 0 ? ld_dev(p.err) : 0u;
        e = __shfl(e, 0);
        if (e != 0u || spins > p.spin_limit) {
          if (lane == 0) raise_err(p, 1u);
          ok = 0;
          break;
        }
      }
    }
    if (lane == 0) {
      lds_st(ct + C_OK, ok);
      if (!ok) lds_st(ct + C_ABORT, 1u);
      if (p.trace && blockIdx.x == 0) p.trace[3 * epoch + 1] = __builtin_amdgcn_s_memrealtime();
    }
  } else if (wv == 1 && need >= 0) {
    long spins = 0;
    while (lds_ld(ct + C_LAND) <= (unsigned)need) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > SPIN_LIMIT) {
        if (lane == 0) {
          raise_err(p, 8u);
          lds_st(ct + C_LFAIL, 1u);
          lds_st(ct + C_ABORT, 1u);
        }
        break;
      }
    }
  }
  cw_sync(p);
  if (p.trace && blockIdx.x == 0 && threadIdx.x == 0) p.trace[3 * epoch + 2] = __builtin_amdgcn_s_memrealtime();
  return lds_ld(ct + C_OK) != 0u && lds_ld(ct + C_LFAIL) == 0u;
}

// ------------------------------------------------------------------ loader
// The weight stream of one workgroup is a sequence of fills, one per (layer
// instance lambda = k L + l, GEMM gi), f = 4 lambda + gi; fill f copies the
// workgroup's tiles of that GEMM (1 KiB blocks, one direct-to-LDS load of 16
// bytes per lane each) into the GEMM's LDS region. Fill f may start once
// the previous users of the region (the same GEMM one layer earlier, and for
// the qkv region the attention phase that follows it) have completed, so every
// region is refilled about a layer ahead of its next use. The loader wave
// runs this sequence on its own, issuing as far ahead as the regions allow
// and publishing in LDS how many fills have landed.
struct Loader {
  int nb0, nb1, nb2, nb3;    // blocks per fill of each GEMM
  int nbl;                   // blocks per layer
  int issued, landed;        // direct-to-LDS loads issued / known complete
  int pub;                   // fills published as landed
  int total;                 // fills in the launch
  __device__ __forceinline__ int nb(int gi) const { return gi == 0 ? nb0 : gi == 1 ? nb1 : gi == 2 ? nb2 : nb3; }
  __device__ __forceinline__ int pre(int gi) const {
    return (gi > 0 ? nb0 : 0) + (gi > 1 ? nb1 : 0) + (gi > 2 ? nb2 : 0);
  }
  // loads issued up to the end of fill f
  __device__ __forceinline__ int end(int f) const { return (f >> 2) * nbl + pre(f & 3) + nb(f & 3); }
};

// The loader's own LDS control accesses are written as inline asm: the
// compiler treats any LDS access after a direct-to-LDS load as possibly
// aliasing its destination and would wait for every copy in flight first
// (s_waitcnt vmcnt(0)), draining the stream at each publication.
__device__ __forceinline__ uint32_t lds_addr(lds_u32* a) { return (uint32_t)(uintptr_t)a; }
__device__ __forceinline__ void loader_st(lds_u32* a, unsigned v) {
  asm volatile("ds_write_b32 %0, %1" : : "v"(lds_addr(a)), "v"(v) : "memory");
}
__device__ __forceinline__ unsigned loader_ld(lds_u32* a) {
  unsigned v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(a)) : "memory");
  return (unsigned)__builtin_amdgcn_readfirstlane((int)v);
}

// units of GEMM gi this workgroup holds (entries copied to LDS at start)
__device__ __forceinline__ int units_of(KSP& p, int gi) {
  int n = 0;
  for (int i = 0; i < UMAX; ++i) n += loader_ld(ctl3(p) + C_UNITS + gi * UMAX + i) != 0xFFFFFFFFu;
  return n;
}

__device__ __forceinline__ void loader_init(KSP& p, Loader& ld) {
  ld.nb0 = units_of(p, 0) * p.g[0].nkbs;
  ld.nb1 = units_of(p, 1) * p.g[1].nkbs;
  ld.nb2 = units_of(p, 2) * p.g[2].nkbs;
  ld.nb3 = units_of(p, 3) * p.g[3].nkbs;
  ld.nbl = ld.nb0 + ld.nb1 + ld.nb2 + ld.nb3;
  ld.issued = ld.landed = ld.pub = 0;
  ld.total = p.N * p.L * 4;
}

// publish every fill whose loads are known complete (fills without blocks
// count as landed once the fills before them have)
__device__ __forceinline__ void loader_publish(KSP& p, Loader& ld) {
  const int old = ld.pub;
  while (ld.pub < ld.total && ld.end(ld.pub) <= ld.landed) ++ld.pub;
  if (ld.pub != old) loader_st(ctl3(p) + C_LAND, (unsigned)ld.pub);
}

__device__ void loader_run(KSP& p) {
  Loader ld;
  loader_init(p, ld);
  lds_u32* ct = ctl3(p);
  // everything the copy loop needs, read once: per GEMM the 32-K blocks
  // (all, per split), the LDS region and the unit entries; the loop itself
  // then issues copies with no scalar or LDS loads in between
  int nkb[4], nkbs[4], region[4];
  uint32_t ue[4][UMAX];
#pragma unroll
  for (int gi = 0; gi < 4; ++gi) {
    nkb[gi] = p.g[gi].nkb;
    nkbs[gi] = p.g[gi].nkbs;
    region[gi] = p.g[gi].region;
#pragma unroll
    for (int i = 0; i < UMAX; ++i) ue[gi][i] = loader_ld(ct + C_UNITS + gi * UMAX + i);
  }
  const int cap = p.dma_cap;
  const uint32_t lane16 = (uint32_t)lane_id() * 16u;
  for (int f = 0; f < ld.total; ++f) {
    const int gi = f & 3, nbf = __builtin_amdgcn_readfirstlane(ld.nb(gi));
    if (nbf == 0) continue;
    // the region's previous users must have completed: the same GEMM one
    // layer earlier, and for the qkv region the attention after it (which
    // stages its keys and values there); phase slots count 5 per layer
    // (qkv, attention, o, gate/up, down)
    const unsigned free_at = (unsigned)(5 * ((f >> 2) - 1) + 2 + gi);
    if (f >= 4 && loader_ld(ct + C_FREE) < free_at) {
      vmwait(0);
      ld.landed = ld.issued;
      loader_publish(p, ld);
      long spins = 0;
      while (loader_ld(ct + C_FREE) < free_at) {
        if (loader_ld(ct + C_ABORT) != 0u) return;   // nothing in flight: the wait above drained it
        __builtin_amdgcn_s_sleep(2);
        if (++spins > SPIN_LIMIT) {
          if (lane_id() == 0) raise_err(p, 8u);
          return;
        }
      }
    }
    // select this GEMM's constants (uniform, unrolled selects keep them in registers)
    int kb_all = 0, kbs = 0, reg = 0;
    uint32_t u[UMAX];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (q == gi) {
        kb_all = nkb[q];
        kbs = nkbs[q];
        reg = region[q];
#pragma unroll
        for (int i = 0; i < UMAX; ++i) u[i] = ue[q][i];
      }
    }
    kb_all = __builtin_amdgcn_readfirstlane(kb_all);
    kbs = __builtin_amdgcn_readfirstlane(kbs);
    reg = __builtin_amdgcn_readfirstlane(reg);
#pragma unroll
    for (int i = 0; i < UMAX; ++i) u[i] = (uint32_t)__builtin_amdgcn_readfirstlane((int)u[i]);
    const uint8_t* wsrc = p.w[gi][(f >> 2) % p.L];
    // the workgroup's units of one GEMM are its first nbf / kbs entries
#pragma unroll
    for (int i = 0; i < UMAX; ++i) {
      if (i * kbs >= nbf) break;
      const int tile = (int)(u[i] >> 8), split = (int)(u[i] & 0xFF);
      const uint8_t* src = wsrc + (((size_t)tile * kb_all + (size_t)split * kbs) << 10) + lane16;
      const uint32_t dst0 = (uint32_t)(reg + i * kbs * 1024);
      for (int j = 0; j < kbs; ++j) {
        // the loader's only vector-memory operations are its copies, so
        // vmcnt counts exactly them
        if (ld.issued - ld.landed >= cap) {
          vmwait(cap - 1);
          ld.landed = ld.issued - (cap - 1);
          loader_publish(p, ld);
        }
        auto* dst = (__attribute__((address_space(3))) void*)(lds + dst0 + j * 1024);
        __builtin_amdgcn_global_load_lds((const void*)(src + ((size_t)j << 10)), dst, 16, 0, 0);
        ++ld.issued;
      }
    }
  }
  vmwait(0);
  ld.landed = ld.issued;
  loader_publish(p, ld);
}

// ------------------------------------------------------------------ phase 0
// The prefix values transposed once per launch into the layout of the PV
// operand: vt[l][kvh][dim][key'], keys permuted within every 32 (vperm),
// zero beyond P. Eight keys of one dimension per thread, dims across lanes.
__device__ void ph_relayout(KSP& p, int w) {
  const int nkb = p.Ppad / 32;
  const size_t total = (size_t)p.L * p.Hkv * nkb * 4 * p.d;   // (l, kvh, key block, lane group, dim)
  const size_t stride = (size_t)p.G * NCW * 64;
  for (size_t idx = (size_t)w * NCW * 64 + threadIdx.x; idx < total; idx += stride) {
    const int dim = (int)(idx % p.d);
    size_t r = idx / p.d;
    const int g8 = (int)(r % 4); r /= 4;
    const int kb = (int)(r % nkb); r /= nkb;
    const int kvh = (int)(r % p.Hkv);
    const int l = (int)(r / p.Hkv);
    uint16_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = kb * 32 + (e < 4 ? 4 * g8 + e : 16 + 4 * g8 + (e - 4));
      v[e] = key < p.P ? __builtin_bit_cast(uint16_t, p.pv[(((size_t)l * p.P + key) * p.Hkv + kvh) * p.d + dim]) : (uint16_t)0;
    }
    const u32x4 o = {v[0] | ((uint32_t)v[1] << 16), v[2] | ((uint32_t)v[3] << 16), v[4] | ((uint32_t)v[5] << 16),
                     v[6] | ((uint32_t)v[7] << 16)};
    coh_st16(p.vt, (uint32_t)(((((size_t)l * p.Hkv + kvh) * p.d + dim) * p.Ppad + kb * 32 + 8 * g8) * 2), o);
  }
}

// ------------------------------------------------------------------ in projection
// h = x W_in + b_in + s (s = state W_s + b_s, computed at k = 0), then the
// first layer's y = h (1 + scale) and the tile's sums of squares. Unit = one
// 16-column tile; thread (m, c4) takes token m, columns 4 c4 .. 4 c4 + 3.
__device__ void ph_in(KSP& p, int k, int w) {
  const int tid = threadIdx.x;
  if (tid >= NCW * 64) return;
  const int m = tid >> 2, c4 = tid & 3;
  const bool act = m < p.H;
  const float* xin = k == 0 ? p.noise : p.x;
  uint8_t* sl = slab(p, k, 0);
  for (int i = 0; i < IUMAX; ++i) {
    const uint32_t ue = (uint32_t)__builtin_amdgcn_readfirstlane((int)ctl3(p)[C_IUNITS + i]);
    if (ue == 0xFFFFFFFFu) break;
    const int t = (int)(ue >> 8);   // table entries are (tile << 8) | split, split 0 here
    const int c = t * 16 + 4 * c4;
    floatx4 hv = {0, 0, 0, 0};
    if (act) {
      hv = as_f4(ro_ld16(p.in_b + c));
      const auto xr = rsrc(xin);
      for (int a = 0; a < p.A; a += 4) {
        const floatx4 xa = as_f4(coh_ld16(xin, (uint32_t)((m * p.A + a) * 4)));
#pragma unroll
        for (int e = 0; e < 4; ++e) hv += xa[e] * as_f4(ro_ld16(p.in_w + (size_t)(a + e) * p.W + c));
      }
      (void)xr;
      if (p.S > 0) {
        if (k == 0) {
          floatx4 sv = as_f4(ro_ld16(p.st_b + c));
          for (int j = 0; j < p.S; ++j) sv += p.state[j] * as_f4(ro_ld16(p.st_w + (size_t)j * p.W + c));
          coh_st16(p.s_emb, (uint32_t)((m * p.W + c) * 4), as_u4(sv));
          hv += sv;
        } else {
          hv += as_f4(coh_ld16(p.s_emb, (uint32_t)((m * p.W + c) * 4)));
        }
      }
      coh_st16(p.h, (uint32_t)((m * p.W + c) * 4), as_u4(hv));
      const floatx4 sc = as_f4(ro_ld16(p.mod + (size_t)k * (2 * p.L + 1) * 3 * p.W + c));
      const floatx4 y = hv * (1.0f + sc);
      coh_st8(sl + p.o_ya, opo(m, c) * 2, u32x2{pack_bf16x2(y.x, y.y), pack_bf16x2(y.z, y.w)});
    }
    float ss = hv.x * hv.x + hv.y * hv.y + hv.z * hv.z + hv.w * hv.w;
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    if (act && c4 == 0) coh_st4(sl + p.o_ssa, (uint32_t)((m * (p.W / 16) + t) * 4), __builtin_bit_cast(uint32_t, ss));
  }
}

// ------------------------------------------------------------------ out projection + Euler
// v = adaRMSNorm_final(h) W_out + b_out; x += dt v. One wave per (token m,
// group of 4 action columns); lane l sums features l W/64 .. (l+1) W/64 - 1.
__device__ void ph_out(KSP& p, int k, int w) {
  const int wv = wave_id(), lane = lane_id();
  if (wv >= NCW) return;
  const int nq = p.A / 4, units = p.H * nq, per = p.W / 64;
  const float dt = -1.0f / (float)p.N;
  const float* modf = p.mod + ((size_t)k * (2 * p.L + 1) + 2 * p.L) * 3 * p.W;
  for (int u = w * NCW + wv; u < units; u += p.G * NCW) {
    const int m = u / nq, q = u - m * nq;
    const int n0 = lane * per;
    float ss = 0.f;
    floatx4 hv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      hv[j] = j * 4 < per ? as_f4(coh_ld16(p.h, (uint32_t)((m * p.W + n0 + 4 * j) * 4))) : floatx4{0, 0, 0, 0};
      ss += hv[j].x * hv[j].x + hv[j].y * hv[j].y + hv[j].z * hv[j].z + hv[j].w * hv[j].w;
    }
    ss = warp_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)p.W + p.eps);
    floatx4 v = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j * 4 >= per) continue;
      const floatx4 sc = as_f4(ro_ld16(modf + n0 + 4 * j)), sh = as_f4(ro_ld16(modf + p.W + n0 + 4 * j));
      const floatx4 xn = hv[j] * r * (1.0f + sc) + sh;
#pragma unroll
      for (int e = 0; e < 4; ++e) v += xn[e] * as_f4(ro_ld16(p.out_w + (size_t)(n0 + 4 * j + e) * p.A + 4 * q));
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = warp_sum(v[e]);
    if (lane == 0) {
      const float* xin = k == 0 ? p.noise : p.x;
      const uint32_t off = (uint32_t)((m * p.A + 4 * q) * 4);
      const floatx4 xo = as_f4(coh_ld16(xin, off));
      const floatx4 xn = xo + dt * (v + as_f4(ro_ld16(p.out_b + 4 * q)));
      coh_st16(p.x, off, as_u4(xn));
    }
  }
}

// ------------------------------------------------------------------ GEMM phases
// Swap-AB skinny GEMM: the weight tile (16 output columns) is the MFMA A
// operand read from LDS, the 64 (padded) tokens the B operand from the
// operand-ordered activation. Wave (st, kp) takes token subtile st and the
// k-blocks of parity kp of the workgroup's K slice, so every activation
// fragment is fetched by exactly one wave; the two parities are added
// through LDS. A workgroup's units of one GEMM share their K split.
template <int GI>
__device__ __forceinline__ const uint8_t* gemm_input(KSP& p, const uint8_t* sl) {
  if constexpr (GI == GQ) return sl + p.o_ya;
  else if constexpr (GI == GO) return sl + p.o_at;
  else if constexpr (GI == GG) return sl + p.o_ym;
  else return sl + p.o_act;
}

// r = 1 / sqrt(mean(h^2) + eps) of token m from the per-tile sums of squares
// [64][W/16]; lane group g sums a quarter of the tiles.
__device__ __forceinline__ float row_rms_inv(KSP& p, const uint8_t* ss, int m) {
  const int nt = p.W / 16, per = nt / 4, g = lane_id() >> 4;
  const auto rs = rsrc(ss);
  float s = 0.f;
  for (int j = 0; j < per; j += 4) {
    const floatx4 v = as_f4(coh_ld16_if(rs, (uint32_t)((m * nt + g * per + j) * 4), m < p.H));
    s += v.x + v.y + v.z + v.w;
  }
  s += __shfl_xor(s, 16);
  s += __shfl_xor(s, 32);
  return 1.0f / sqrtf(s / (float)p.W + p.eps);
}

template <int GI>
__device__ __forceinline__ void ph_gemm(KSP& p, int k, int l, int w) {
  KSG& g = p.g[GI];
  int nu = 0;
  uint32_t ue[UMAX];
#pragma unroll
  for (int i = 0; i < UMAX; ++i) {
    ue[i] = (uint32_t)__builtin_amdgcn_readfirstlane((int)ctl3(p)[C_UNITS + GI * UMAX + i]);
    nu += ue[i] != 0xFFFFFFFFu;
  }
  if (nu == 0) return;
  const int wv = wave_id(), lane = lane_id(), c16 = lane & 15, gq = lane >> 4;
  const int st = wv & 3, kp = (wv >> 2) & 1;
  const bool ep = kp == 0;   // waves 0..3 finish the tiles
  const int split = (int)(ue[0] & 0xFF);
  const int kb0 = split * g.nkbs;
  uint8_t* sl = slab(p, k, l);
  const int m = 16 * st + c16;
  const bool mok = m < p.H;
  const int W = p.W;
  int tile[UMAX];
#pragma unroll
  for (int i = 0; i < UMAX; ++i) tile[i] = (int)(ue[i < nu ? i : 0] >> 8);
  // activation fragments of this wave's token subtile and k-block parity
  const auto ars = rsrc(gemm_input<GI>(p, sl));
  const int nj = g.nkbs >> 1;
  // the workgroups of an XCD all read the same activation; each starts at
  // a different k block (rotation by its slot)
  const int rot = (w % p.per_xcd) % nj;
  u32x4 a[MAXJ];
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    const int jr = j + rot < nj ? j + rot : j + rot - nj;
    const int kb = kb0 + kp + 2 * jr;
    a[j] = act_ld16_if(ars, (uint32_t)((((kb * 64 + m) << 5) + 8 * gq) * 2), mok && j < nj);
  }
  // everything the epilogue reads, issued now so that it lands during the
  // contraction: the shift tables (qkv, gate/up), the rotary table (qkv),
  // the residual, its gate and the next norm's scale (o, down)
  floatx4 e0[UMAX], e1[UMAX], e2[UMAX];
#pragma unroll
  for (int i = 0; i < UMAX; ++i) e0[i] = e1[i] = e2[i] = floatx4{0, 0, 0, 0};
  const int nrm_g = GI == GO ? 2 * l : 2 * l + 1;                 // norm whose gate scales this residual
  const bool next = GI == GO || l + 1 < p.L;                       // y of a following norm to write
  const int nrm_n = GI == GO ? 2 * l + 1 : 2 * l + 2;              // that norm
  if (ep && mok) {
#pragma unroll
    for (int i = 0; i < UMAX; ++i) {
      if (i >= nu) continue;
      const int col0 = tile[i] * 16;
      if constexpr (GI == GQ) {
        const int d = p.d, Nq = (p.Hq + 2 * p.Hkv) * d;
        e0[i] = as_f4(ro_ld16(p.shw_q + ((size_t)k * p.L + l) * Nq + col0 + 4 * gq));
        if (col0 / d < p.Hq + p.Hkv) {
          const int j0 = ((col0 % d) / 16) * 8 + 2 * gq;
          e1[i] = as_f4(ro_ld16(p.rope + ((size_t)m * (d / 2) + j0) * 2));
        }
      } else if constexpr (GI == GG) {
        e0[i] = as_f4(ro_ld16(p.shw_g + ((size_t)k * p.L + l) * 2 * p.F + col0 + 4 * gq));
      } else {
        const float* modk = p.mod + (size_t)k * (2 * p.L + 1) * 3 * W;
        const int c = col0 + 4 * gq;
        e0[i] = as_f4(coh_ld16(p.h, (uint32_t)((m * W + c) * 4)));
        e1[i] = as_f4(ro_ld16(modk + ((size_t)nrm_g * 3 + 2) * W + c));
        if (next) e2[i] = as_f4(ro_ld16(modk + (size_t)nrm_n * 3 * W + c));
      }
    }
  }
  float r = 1.0f;
  if constexpr (GI == GQ || GI == GG) r = row_rms_inv(p, sl + (GI == GQ ? p.o_ssa : p.o_ssm), m);
  // contraction: the weight fragments of step j + PF are read from LDS while
  // step j multiplies; the reads are unconditional (clamped to the unit's
  // last block), only the MFMAs depend on the slice length
  constexpr int PF = 2;
  const uint8_t* wr = reinterpret_cast<const uint8_t*>(lds) + g.region + lane * 16;
  const int njm1 = nj - 1;
  auto wblk = [&](int j, int i) -> u32x4 {
    const int jj = j < njm1 ? j : njm1;
    const int jr = jj + rot < nj ? jj + rot : jj + rot - nj;
    const int ii = i < nu ? i : nu - 1;
    return *reinterpret_cast<const u32x4*>(wr + (ii * g.nkbs + kp + 2 * jr) * 1024);
  };
  floatx4 acc[UMAX];
#pragma unroll
  for (int i = 0; i < UMAX; ++i) acc[i] = floatx4{0, 0, 0, 0};
  u32x4 wq[PF + 1][UMAX];
#pragma unroll
  for (int j = 0; j < PF; ++j)
#pragma unroll
    for (int i = 0; i < UMAX; ++i) wq[j][i] = wblk(j, i);
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    if (j + PF < MAXJ) {
#pragma unroll
      for (int i = 0; i < UMAX; ++i) wq[(j + PF) % (PF + 1)][i] = wblk(j + PF, i);
    }
    if (j < nj) {
#pragma unroll
      for (int i = 0; i < UMAX; ++i)
        if (i < nu) acc[i] = MT<bf16>::mma(wq[j % (PF + 1)][i], a[j], acc[i]);
    }
  }
  floatx4* scr = reinterpret_cast<floatx4*>(lds + p.scratch);
  if (kp == 1) {
#pragma unroll
    for (int i = 0; i < UMAX; ++i)
      if (i < nu) scr[(i * 4 + st) * 64 + lane] = acc[i];
  }
  cw_sync(p);
  if (ep) {
#pragma unroll
    for (int i = 0; i < UMAX; ++i)
      if (i < nu) acc[i] += scr[(i * 4 + st) * 64 + lane];
  }
  if constexpr (GI == GQ) {
    if (ep) {
      const int d = p.d;
#pragma unroll
      for (int i = 0; i < UMAX; ++i) {
        if (i >= nu) continue;
        const int col0 = tile[i] * 16;
        const floatx4 v = r * acc[i] + e0[i];
        const int head = col0 / d, tt = (col0 % d) / 16;
        if (head < p.Hq + p.Hkv) {
          if (!mok) continue;
          // packed lane order (x_j, x_j+1, x_j+d/2, x_j+1+d/2), j = 8 tt + 2 g
          const floatx4 rt = e1[i];
          const float y0 = v.x * rt[0] - v.z * rt[1], y0h = v.z * rt[0] + v.x * rt[1];
          const float y1 = v.y * rt[2] - v.w * rt[3], y1h = v.w * rt[2] + v.y * rt[3];
          const bool isq = head < p.Hq;
          uint8_t* dst = sl + (isq ? p.o_q : p.o_k);
          const int hb = isq ? head : head - p.Hq;
          const uint32_t o0 = (uint32_t)(((hb * (d / 16) + tt) * 64 + m) * 16 + 2 * gq);
          coh_st4(dst, o0 * 2, pack_bf16x2(y0, y1));
          coh_st4(dst, (o0 + 8) * 2, pack_bf16x2(y0h, y1h));
        } else {
          // values transposed: vt[kvh][dim][key'] with the key permutation of the PV operand
          const int kvh = head - p.Hq - p.Hkv;
          const int key = (m & ~31) + vperm(m & 31);
          uint8_t* dst = sl + p.o_vt;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int dim = tt * 16 + 4 * gq + e;
            coh_st2(dst, (uint32_t)(((kvh * d + dim) * 64 + key) * 2),
                    mok ? (uint32_t)__builtin_bit_cast(uint16_t, (bf16)v[e]) : 0u);
          }
        }
      }
    }
  } else if constexpr (GI == GG) {
    if (ep && mok) {
#pragma unroll
      for (int i = 0; i < UMAX; ++i) {
        if (i >= nu) continue;
        const floatx4 v = r * acc[i] + e0[i];
        // packed lane order (gate f, up f, gate f+1, up f+1), f = 8 tile + 2 g
        const int f0 = tile[i] * 8 + 2 * gq;
        const float a0 = gelu_tanh(v.x) * v.y, a1 = gelu_tanh(v.z) * v.w;
        coh_st4(sl + p.o_act, opo(m, f0) * 2, pack_bf16x2(a0, a1));
      }
    }
  } else {
    // split GEMM: partial sums, then the last unit of each tile finishes it
    const int S = g.S;
    if (ep && mok) {
#pragma unroll
      for (int i = 0; i < UMAX; ++i)
        if (i < nu)
          coh_st16(g.part, (uint32_t)((((split * g.T + tile[i]) * 64 + m) * 16 + 4 * gq) * 4), as_u4(acc[i]));
    }
    vm_drain();
    cw_sync(p);
    if ((int)threadIdx.x < nu) {
      const unsigned old = __hip_atomic_fetch_add(&g.cnt[tile[threadIdx.x]], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ctl3(p)[C_LAST + threadIdx.x] = (old + 1u) % (unsigned)S == 0u ? 1u : 0u;
    }
    cw_sync(p);
    if (ep) {
      const auto pr = rsrc(g.part);
      uint8_t* sln = GI == GO ? sl : (l + 1 < p.L ? slab(p, k, l + 1) : nullptr);
#pragma unroll
      for (int i = 0; i < UMAX; ++i) {
        if (i >= nu || ctl3(p)[C_LAST + i] == 0u) continue;
        const int c = tile[i] * 16 + 4 * gq;
        u32x4 pv[SMAX];
#pragma unroll
        for (int s = 0; s < SMAX; ++s)
          pv[s] = coh_ld16_if(pr, (uint32_t)((((s * g.T + tile[i]) * 64 + m) * 16 + 4 * gq) * 4), mok && s < S && s != split);
        // splits added in their fixed order 0 .. S-1 whichever one arrived
        // last, so the result does not depend on the arrival order
        floatx4 sum = {0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < SMAX; ++s)
          if (s < S) sum += s == split ? acc[i] : as_f4(pv[s]);
        const floatx4 hn = e0[i] + e1[i] * sum;
        float ss = hn.x * hn.x + hn.y * hn.y + hn.z * hn.z + hn.w * hn.w;
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
        if (mok) {
          coh_st16(p.h, (uint32_t)((m * W + c) * 4), as_u4(hn));
          if (next) {
            const floatx4 y = hn * (1.0f + e2[i]);
            coh_st8(sln + (GI == GO ? p.o_ym : p.o_ya), opo(m, c) * 2, u32x2{pack_bf16x2(y.x, y.y), pack_bf16x2(y.z, y.w)});
            if (gq == 0)
              coh_st4(sln + (GI == GO ? p.o_ssm : p.o_ssa), (uint32_t)((m * (W / 16) + tile[i]) * 4), __builtin_bit_cast(uint32_t, ss));
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------ attention
// Unit (head j, key split c): 32 keys, the prefix keys in splits first, then
// the chunk's own keys. Wave (qs, dh): query subtile qs (16 action tokens),
// half dh of the head dims for P V. Scores are computed transposed,
// S^T = K Q^T, so a lane holds 8 keys of one query (keys 4g..4g+3 and
// 16+4g..16+4g+3) and the probabilities feed the P V MFMA from registers (the
// transposed values are stored with the same key order). The unit's keys and
// values are fetched once per workgroup, one 1 KiB operand fragment per load
// spread over the eight waves, into LDS (the qkv weight region: its refill
// for the next layer waits for this phase); each wave then reads the
// fragments it needs from there, and only q comes from global memory per
// wave. After every split of a head is stored, the head's units (all on one
// XCD) meet at a counter and each merges a share of the query rows, loading
// the (max, sum) pairs and the partial outputs of all splits at once.
constexpr int MERGE_MAX = 32;   // splits merged per pass (more take further passes)

template <int D>
__device__ __forceinline__ bool ph_attn(KSP& p, int k, int l, int w) {
  constexpr int KB = D / 32, DT = D / 32;   // k-blocks of the scores, dim tiles per half
  constexpr int NKF = 2 * KB, NVF = 2 * DT; // 1 KiB fragments: keys (ks, kb), values (dh, dt)
  constexpr int PERW = (NKF + NVF + NCW - 1) / NCW;
  const int wv = wave_id(), lane = lane_id(), c16 = lane & 15, gq = lane >> 4;
  const int qs = wv & 3, dh = (wv >> 2) & 1;
  const uint8_t* sl = slab(p, k, l);
  const int group = p.Hq / p.Hkv;
  const float scale = 1.4426950408889634f / sqrtf((float)D);
  uint32_t au[AUMAX];
  int na = 0;
#pragma unroll
  for (int i = 0; i < AUMAX; ++i) {
    au[i] = (uint32_t)__builtin_amdgcn_readfirstlane((int)ctl3(p)[C_AUNITS + i]);
    na += au[i] != 0xFFFFFFFFu;
  }
  if (na == 0) return true;
  const int qrow = 16 * qs + c16;
  u32x4* stg = reinterpret_cast<u32x4*>(lds + p.g[GQ].region);
#pragma unroll
  for (int i = 0; i < AUMAX; ++i) {
    if (i >= na) continue;
    const int j = (int)(au[i] >> 8), c = (int)(au[i] & 0xFF), kvh = j / group;
    const bool pre = c < p.KSp;
    const int s0 = pre ? 32 * c : p.P + 32 * (c - p.KSp);
    const int s1 = pre ? min(p.P, s0 + 32) : min(p.P + p.H, s0 + 32);
    // this wave's queries (all dims) and its share of the unit's key / value fragments
    const auto qr = rsrc(sl + p.o_q);
    u32x4 qf[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int tt = 2 * kb + (gq >> 1);
      qf[kb] = act_ld16_if(qr, (uint32_t)((((j * (D / 16) + tt) * 64 + qrow) * 16 + (gq & 1) * 8) * 2), qrow < p.H);
    }
    u32x4 sf[PERW];
    {
      const auto kpr = rsrc(p.pk + (size_t)l * p.P * p.Hkv * D);
      const auto kcr = rsrc(sl + p.o_k);
      const uint8_t* vbase = pre ? reinterpret_cast<const uint8_t*>(p.vt + (size_t)(l * p.Hkv + kvh) * D * p.Ppad)
                                 : sl + p.o_vt + (size_t)kvh * D * 64 * 2;
      const int ld_keys = pre ? p.Ppad : 64;
      const int kofs = pre ? 32 * c : 32 * (c - p.KSp);
      const auto vr = rsrc(vbase);
#pragma unroll
      for (int r = 0; r < PERW; ++r) {
        const int fa = wv + NCW * r;
        if (fa < NKF) {
          const int ks = fa / KB, kb = fa % KB;
          const int key = s0 + 16 * ks + c16, tt = 2 * kb + (gq >> 1);
          const bool kok = key < s1;
          sf[r] = pre ? ld16_if(kpr, (uint32_t)(((key * p.Hkv + kvh) * D + 8 * tt + (gq & 1) * (D / 2)) * 2), kok)
                      : act_ld16_if(kcr, (uint32_t)((((kvh * (D / 16) + tt) * 64 + (key - p.P)) * 16 + (gq & 1) * 8) * 2), kok);
        } else if (fa < NKF + NVF) {
          const int dv = (fa - NKF) / DT, dt = (fa - NKF) % DT;
          const int dim = dv * (D / 2) + 16 * dt + c16;
          sf[r] = act_ld16_if(vr, (uint32_t)(((size_t)dim * ld_keys + kofs + 8 * gq) * 2), true);
        }
      }
    }
    if (i > 0) cw_sync(p);   // the previous unit's readers are done with the staging area
#pragma unroll
    for (int r = 0; r < PERW; ++r)
      if (wv + NCW * r < NKF + NVF) stg[(wv + NCW * r) * 64 + lane] = sf[r];
    cw_sync(p);
    floatx4 sacc[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) sacc[ks] = MT<bf16>::mma(stg[(ks * KB + kb) * 64 + lane], qf[kb], sacc[ks]);
    float pr[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pr[e] = s0 + 4 * gq + e < s1 ? sacc[0][e] * scale : -INFINITY;
      pr[4 + e] = s0 + 16 + 4 * gq + e < s1 ? sacc[1][e] * scale : -INFINITY;
    }
    float mx = pr[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, pr[e]);
    mx = am_max4(mx);
    float lsum = 0.f;
    bf16x8 pb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float pe = fast_exp2(pr[e] - mx);
      lsum += pe;
      pb[e] = (bf16)pe;
    }
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    const u32x4 pbu = __builtin_bit_cast(u32x4, pb);
    // the MFMAs run with every lane active (an MFMA reads its operands from
    // the whole wave); only the stores of rows beyond H are masked
    floatx4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = MT<bf16>::mma(stg[(NKF + dh * DT + dt) * 64 + lane], pbu, floatx4{0, 0, 0, 0});
    if (qrow < p.H) {
      const size_t row = ((size_t)j * p.KS + c) * 64 + qrow;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        coh_st16(p.apart, (uint32_t)((row * D + dh * (D / 2) + 16 * dt + 4 * gq) * 4), as_u4(o[dt]));
      if (dh == 0 && gq == 0)
        coh_st8(p.aml, (uint32_t)(row * 8), u32x2{__builtin_bit_cast(uint32_t, mx), __builtin_bit_cast(uint32_t, lsum)});
    }
  }
  // the head's units meet: every split output of the head is stored
  vm_drain();
  cw_sync(p);
  const unsigned inst = (unsigned)(k * p.L + l);
  if (threadIdx.x == 0) {
    unsigned ok = 1;
#pragma unroll
    for (int i = 0; i < AUMAX; ++i)
      if (i < na) __hip_atomic_fetch_add(&p.hcnt[au[i] >> 8], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int i = 0; i < AUMAX; ++i) {
      if (i >= na || !ok) continue;
      const unsigned target = (inst + 1u) * (unsigned)p.KS;
      long spins = 0;
      while (ld_dev(&p.hcnt[au[i] >> 8]) < target) {
        if ((++spins & 255) == 0 && (ld_dev(p.err) != 0u || spins > p.spin_limit)) {
          raise_err(p, 2u);
          ok = 0;
          break;
        }
      }
    }
    lds_st(ctl3(p) + C_OK, ok);
    if (!ok) lds_st(ctl3(p) + C_ABORT, 1u);
  }
  cw_sync(p);
  if (lds_ld(ctl3(p) + C_OK) == 0u) return false;
  // merge: unit (j, c) takes query rows c, c + KS, ...; one wave per row
  uint8_t* at = slab(p, k, l) + p.o_at;
  const auto apr = rsrc(p.apart);
  const auto amr = rsrc(p.aml);
#pragma unroll
  for (int i = 0; i < AUMAX; ++i) {
    if (i >= na) continue;
    const int j = (int)(au[i] >> 8), c = (int)(au[i] & 0xFF);
    for (int m = c + wv * p.KS; m < p.H; m += NCW * p.KS) {
      const size_t base = (size_t)j * p.KS * 64 + m;   // row m of split 0; split s at + s * 64
      floatx4 num = {0, 0, 0, 0};
      float den = 0.f, mrun = -INFINITY;
      for (int s0 = 0; s0 < p.KS; s0 += MERGE_MAX) {
        // (max, sum) of split s0 + lane and the partial rows of every split of this pass, issued together
        const u32x2 mlv = coh_ld8_if(amr, (uint32_t)((base + (size_t)(s0 + lane) * 64) * 8), lane < MERGE_MAX && s0 + lane < p.KS);
        u32x4 ov[MERGE_MAX];
#pragma unroll
        for (int e = 0; e < MERGE_MAX; ++e)
          ov[e] = coh_ld16_if(apr, (uint32_t)(((base + (size_t)(s0 + e) * 64) * D + 4 * lane) * 4), 4 * lane < D && s0 + e < p.KS);
        // whole-vector bit cast: casting single components of a loaded
        // vector reads component 0 for every one of them
        const floatx2 ml = __builtin_bit_cast(floatx2, mlv);
        const bool live = lane < MERGE_MAX && s0 + lane < p.KS;
        const float mi = live ? ml[0] : -INFINITY;
        float mx = mi;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        const float mnew = fmaxf(mrun, mx);
        const float resc = fast_exp2(mrun - mnew);   // 0 on the first pass
        const float wc = live ? fast_exp2(mi - mnew) : 0.f;
        den = den * resc + warp_sum(wc * (live ? ml[1] : 0.f));
        num *= resc;
#pragma unroll
        for (int e = 0; e < MERGE_MAX; ++e) num += __shfl(wc, e) * as_f4(ov[e]);
        mrun = mnew;
      }
      if (4 * lane < D) {
        const floatx4 o = num / den;
        const int col = j * D + 4 * lane;
        coh_st8(at, opo(m, col) * 2, u32x2{pack_bf16x2(o.x, o.y), pack_bf16x2(o.z, o.w)});
      }
    }
  }
  return true;
}

// ------------------------------------------------------------------ the kernel
template <int D>
__global__ __launch_bounds__(NT) void k_stream(SP) {
  KSP& p = *(KSP*)__builtin_amdgcn_kernarg_segment_ptr();
  const int wv = wave_id();
  lds_u32* ct = ctl3(p);
  // logical workgroup id: XCD-major, from the XCD this workgroup runs on
  if (threadIdx.x == 0) {
    unsigned x;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
    x &= 15u;
    int wid = -1;
    if (x < (unsigned)NXCD) {
      const unsigned slot = __hip_atomic_fetch_add(&p.bar[BW_SLOT + 64 * x], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (slot < (unsigned)p.per_xcd) wid = (int)(x * p.per_xcd + slot);
    }
    if (wid < 0) raise_err(p, 4u);
    ct[C_WID] = (unsigned)wid;
    ct[C_OK] = 1u;
    ct[C_CWB] = ct[C_FREE] = ct[C_LAND] = ct[C_ABORT] = ct[C_LFAIL] = 0u;
    if (p.trace && blockIdx.x == 0) p.trace[0] = p.trace[1] = p.trace[2] = __builtin_amdgcn_s_memrealtime();
  }
  wg_sync();
  const int w = __builtin_amdgcn_readfirstlane((int)ct[C_WID]);
  if (w < 0) return;
  // the workgroup's unit entries of every phase, read from LDS from here on
  {
    const int t = threadIdx.x;
    if (t < 4 * UMAX) {
      KSG& g = p.g[t / UMAX];
      const int i = t % UMAX;
      ct[C_UNITS + t] = i < g.U ? g.units[w * g.U + i] : 0xFFFFFFFFu;
    } else if (t < 4 * UMAX + AUMAX) {
      const int i = t - 4 * UMAX;
      ct[C_AUNITS + i] = i < p.AU ? p.attn_units[w * p.AU + i] : 0xFFFFFFFFu;
    } else if (t < 4 * UMAX + AUMAX + IUMAX) {
      const int i = t - 4 * UMAX - AUMAX;
      ct[C_IUNITS + i] = i < p.IU ? p.in_units[w * p.IU + i] : 0xFFFFFFFFu;
    }
  }
  wg_sync();   // the last s_barrier: from here on the loader runs on its own
  if (wv == LOADER) {
    loader_run(p);
    return;
  }
  unsigned epoch = 0;
  // stop_after > 0 (diagnostics): every workgroup leaves after that barrier,
  // so the intermediates of the phases before it stay in the workspace
#define VFM_GBAR(DONE, NEED)                                      \
  do {                                                            \
    if (!gbar(p, epoch, (DONE), (NEED))) return;                  \
    if (p.stop_after > 0 && (int)epoch >= p.stop_after) goto out; \
  } while (0)
  ph_relayout(p, w);
  ph_in(p, 0, w);
  for (int k = 0; k < p.N; ++k) {
    for (int l = 0; l < p.L; ++l) {
      const int q = 4 * (k * p.L + l);   // fill (GEMM phase) index of this layer's qkv
      const int z = 5 * (k * p.L + l);   // phase slots completed before this layer
      VFM_GBAR(z, q);
      ph_gemm<GQ>(p, k, l, w);
      VFM_GBAR(z + 1, -1);
      if (!ph_attn<D>(p, k, l, w)) return;
      VFM_GBAR(z + 2, q + 1);
      ph_gemm<GO>(p, k, l, w);
      VFM_GBAR(z + 3, q + 2);
      ph_gemm<GG>(p, k, l, w);
      VFM_GBAR(z + 4, q + 3);
      ph_gemm<GD>(p, k, l, w);
    }
    const int done = 5 * (k + 1) * p.L;
    VFM_GBAR(done, -1);
    ph_out(p, k, w);
    if (k + 1 < p.N) {
      VFM_GBAR(done, -1);
      ph_in(p, k + 1, w);
    }
  }
#undef VFM_GBAR
out:
  // the last workgroup out resets the barrier words for the next launch
  vm_drain();
  cw_sync(p);
  if (threadIdx.x == 0) {
    lds_st(ct + C_ABORT, 1u);   // a loader still waiting for a region stops
    const unsigned old = __hip_atomic_fetch_add(&p.bar[BW_EXIT], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1u == (unsigned)p.G) {
      for (int c = 0; c < N_CTR; ++c) __hip_atomic_store(&p.bar[BW_CTR + 64 * c], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int x = 0; x < NXCD; ++x) __hip_atomic_store(&p.bar[BW_SLOT + 64 * x], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int j = 0; j < p.Hq; ++j) __hip_atomic_store(&p.hcnt[j], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int t = 0; t < p.g[GO].T; ++t) __hip_atomic_store(&p.g[GO].cnt[t], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int t = 0; t < p.g[GD].T; ++t) __hip_atomic_store(&p.g[GD].cnt[t], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&p.bar[BW_EXIT], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace sk
}  // namespace vfm
