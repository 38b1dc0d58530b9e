// vfm_device.h -- device-side building blocks shared by every kernel of the
// action-expert denoise loop: vector types, the MFMA operand traits, coherent
// (device-scope) memory helpers and the grid barrier.
//
// Memory model used across workgroups inside one launch (measured on MI355X):
// the per-XCD L2 caches are not coherent with each other for ordinary
// stores, so every value one workgroup produces for another is written with
// device-scope (sc1) stores, which write through to the coherence point, and
// read with device-scope (sc1) loads. A phase boundary is then a wait for the
// wave's own outstanding memory operations plus a counter barrier made of
// relaxed device-scope atomics; no L2 writeback/invalidate is needed.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vfm_params.h"

namespace vfm {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef long long i64x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ MFMA traits
// Every operand fetch is 16 bytes per lane. For a 16-column tile, lane l
// (column / row l % 16, group g = l / 16) holds E consecutive k values
// k = kb * KB + E * g + e; the same mapping is used for both operands, so the
// hardware's pairing of operand slots always multiplies matching k.
// The 16x16 output tile: lane l holds rows 4 * g + r (r = 0..3) of column l % 16.
template <typename T> struct MT;
template <> struct MT<float> {
  static constexpr int E = 4;    // elements per 16-byte lane fetch
  static constexpr int KB = 16;  // k values per 16-byte block (4 MFMAs of K = 4)
  static __device__ __forceinline__ floatx4 mma(u32x4 a, u32x4 b, floatx4 c) {
    // whole-vector bit casts: casting single components of an ext_vector is
    // miscompiled (every component reads as component 0)
    const floatx4 af = __builtin_bit_cast(floatx4, a), bf = __builtin_bit_cast(floatx4, b);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(af[0], bf[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(af[1], bf[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(af[2], bf[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(af[3], bf[3], c, 0, 0, 0);
    return c;
  }
};
template <> struct MT<bf16> {
  static constexpr int E = 8;
  static constexpr int KB = 32;  // one 16x16x32 MFMA per block
  static __device__ __forceinline__ floatx4 mma(u32x4 a, u32x4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

// ------------------------------------------------------------------ conversions
__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }

// pack two values of T into the low bytes of a word (bf16: one u32; f32: u32x2)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16 x = (bf16)a, y = (bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// ------------------------------------------------------------------ coherent memory
// Buffer-resource based loads/stores with the device-scope (sc1) cache policy.
// Offsets are bytes from `base` and must stay below 2 GiB.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}
constexpr int CPOL_SC1 = 16;
__device__ __forceinline__ u32x4 coh_ld16(const void* base, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(rsrc(base), off, 0, CPOL_SC1);
}
__device__ __forceinline__ u32x2 coh_ld8(const void* base, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(rsrc(base), off, 0, CPOL_SC1);
}
__device__ __forceinline__ uint32_t coh_ld4(const void* base, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(rsrc(base), off, 0, CPOL_SC1);
}
__device__ __forceinline__ void coh_st16(void* base, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, rsrc(base), off, 0, CPOL_SC1);
}
__device__ __forceinline__ void coh_st8(void* base, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, rsrc(base), off, 0, CPOL_SC1);
}
__device__ __forceinline__ void coh_st4(void* base, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, rsrc(base), off, 0, CPOL_SC1);
}
__device__ __forceinline__ void coh_st2(void* base, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b16((unsigned short)v, rsrc(base), off, 0, CPOL_SC1);
}
// Ordinary write-back stores, for results read only by later launches (the
// kernel boundary makes them visible): partial lines merge in L2 instead of
// going through to memory one piece at a time as device-coherent stores do.
__device__ __forceinline__ void wb_st16(void* base, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, rsrc(base), off, 0, 0);
}
__device__ __forceinline__ void wb_st8(void* base, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, rsrc(base), off, 0, 0);
}
__device__ __forceinline__ void wb_st4(void* base, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, rsrc(base), off, 0, 0);
}
// read-only data (weights, prefix KV, tables): ordinary cached loads
__device__ __forceinline__ u32x4 ro_ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Predicated loads without branches: a lane whose `ok` is false gets an
// out-of-range offset, which the buffer unit answers with zeros and no
// memory access. Loads inside per-lane branches are serialised by the
// compiler's wait insertion; these are issued back to back.
constexpr uint32_t OOB = 0xFFFFFFF0u;
__device__ __forceinline__ u32x4 ld16_if(__amdgpu_buffer_rsrc_t r, uint32_t off, bool ok) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, ok ? off : OOB, 0, 0);
}
__device__ __forceinline__ u32x4 coh_ld16_if(__amdgpu_buffer_rsrc_t r, uint32_t off, bool ok) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, ok ? off : OOB, 0, CPOL_SC1);
}
__device__ __forceinline__ u32x2 coh_ld8_if(__amdgpu_buffer_rsrc_t r, uint32_t off, bool ok) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, ok ? off : OOB, 0, CPOL_SC1);
}
__device__ __forceinline__ u32x2 ld8_if(__amdgpu_buffer_rsrc_t r, uint32_t off, bool ok) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, ok ? off : OOB, 0, 0);
}
__device__ __forceinline__ uint32_t ld2_if(__amdgpu_buffer_rsrc_t r, uint32_t off, bool ok) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, ok ? off : OOB, 0, 0);
}

// Maximum over the four lanes c16 + 16 g (g = 0 .. 3) of a wave, in every
// one of them: two butterfly steps across the 16-lane rows. (The gfx950
// lane-swap instructions would do this without the LDS crossbar, but with
// both inputs the same value the compiler keeps one half of the swapped pair
// and drops the max between them, which returns lane group 0's value instead
// of the maximum.)
__device__ __forceinline__ float am_max4(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}

__device__ __forceinline__ floatx4 as_f4(u32x4 v) { return __builtin_bit_cast(floatx4, v); }
__device__ __forceinline__ u32x4 as_u4(floatx4 v) { return __builtin_bit_cast(u32x4, v); }

// ------------------------------------------------------------------ math
// exp2 via the hardware transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// GELU, tanh form: 0.5 u (1 + tanh(z)), z = sqrt(2/pi) (u + 0.044715 u^3).
// With e = exp(2z): 0.5 (1 + tanh z) = e / (e + 1), so the value is
// u - u / (e + 1), one exp2 and one hardware reciprocal (e = inf gives u,
// e = 0 gives 0); exp(2z) = exp2(2 log2(e) sqrt(2/pi) (u + 0.044715 u^3)).
__device__ __forceinline__ float gelu_tanh(float u) {
  const float t = __builtin_fmaf(0.044715f * u * u, u, u);
  const float e = fast_exp2(2.3022082f * t);
  return __builtin_fmaf(-u, __builtin_amdgcn_rcpf(e + 1.0f), u);
}

__device__ __forceinline__ float warp_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
// Sum over a 256-thread block; `red` is >= 4 floats of LDS.
__device__ __forceinline__ float block_sum256(float v, float* red) {
  v = warp_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// ------------------------------------------------------------------ grid barrier
// Layout of the barrier words (uint32): [0] global count of finished groups,
// [1] error flag, [64 + 64 * g] arrival count of group g (g = block % 8).
// Counts are monotonic within one launch (zeroed before it). Spins are
// bounded; on timeout the error flag is raised and every block returns.
constexpr long BARRIER_SPIN_LIMIT = BARRIER_SPIN_LIMIT_HOST;

__device__ __forceinline__ unsigned ld_agent(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct NoHook {
  __device__ __forceinline__ void operator()() const {}
};

// Device-wide barrier of a persistent grid. Arrival: after its stores have
// completed, each workgroup adds 1 to one of BAR_COUNTERS counters
// (blockIdx % BAR_COUNTERS, one 256-byte line each) without waiting for the
// old value; spreading the arrivals over many lines keeps the atomics from
// queueing on one address (64 counters measured fastest: 8.38 ms per pi0.5
// chunk against 8.88 with 8, 8.52 with 128). Wait: wave 0 reads the counters
// (lane c reads counters c, c + 64, ...) until their sum reaches
// epoch * gridDim.
// The sum of values read at slightly different times never exceeds the true
// count, so reaching the target proves every workgroup arrived. `hook` runs
// in every thread between arrival and wait: work that does not depend on the
// other workgroups (issuing loads of read-only data) overlaps the wait.
// bar[1] is a sticky error word: a wait that exceeds `spin_limit` polls sets
// it (and the host-mapped word `herr`), and every waiter gives up once it is
// set (returns false). Barrier
// `fail_epoch` (diagnostics, 0: none) waits for one arrival more than the grid
// holds, so its bounded wait gives up and every workgroup exits normally.
template <typename HOOK = NoHook>
__device__ __forceinline__ bool grid_barrier(unsigned* bar, unsigned& epoch, unsigned long long* trace, long spin_limit,
                                             int fail_epoch, unsigned* herr, const HOOK& hook = HOOK()) {
  __shared__ unsigned s_ok;
  ++epoch;
  __builtin_amdgcn_s_waitcnt(0);   // this wave's stores (and loads) have completed
  __syncthreads();
  // optional timeline: workgroup 0 stamps (arrive, release) of every barrier
  if (trace && blockIdx.x == 0 && threadIdx.x == 0) trace[2 * epoch] = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(&bar[64 + 64 * (blockIdx.x % BAR_COUNTERS)], 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  hook();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const unsigned target = epoch * gridDim.x + ((int)epoch == fail_epoch ? 1u : 0u);
    unsigned ok = 1;
    long spins = 0;
    for (;;) {
      unsigned v = 0;
#pragma unroll
      for (int c = lane; c < 64 * ((BAR_COUNTERS + 63) / 64); c += 64)
        if (c < BAR_COUNTERS) v += ld_agent(&bar[64 + 64 * c]);
#pragma unroll
      for (int sh = 1; sh < BAR_COUNTERS && sh < 64; sh *= 2) v += __shfl_xor(v, sh);
      v = __shfl(v, 0);
      if (v >= target) break;
      if ((++spins & 1023) == 0) {
        unsigned err = lane == 0 ? ld_agent(&bar[1]) : 0u;
        err = __shfl(err, 0);
        if (err != 0u || spins > spin_limit) {
          if (lane == 0) {
            __hip_atomic_fetch_or(&bar[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (herr) __hip_atomic_store(herr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
          }
          ok = 0;
          break;
        }
      }
    }
    if (lane == 0) {
      s_ok = ok;
      if (trace && blockIdx.x == 0) trace[2 * epoch + 1] = __builtin_amdgcn_s_memrealtime();
    }
  }
  __syncthreads();
  return s_ok != 0;
}

// Wait until the arrival counter *cnt reaches `target` (thread 0 polls, the
// workgroup then proceeds together), with grid_barrier's bounded spin and
// sticky error word: returns false, in every thread, when the wait gave up or
// another wait already had. Every thread of the workgroup must call it.
__device__ __forceinline__ bool counter_wait(const unsigned* cnt, unsigned target, unsigned* bar, long spin_limit,
                                             unsigned* herr) {
  __shared__ unsigned s_cok;
  if (threadIdx.x == 0) {
    unsigned ok = 1;
    long spins = 0;
    while (ld_agent(cnt) < target) {
      if ((++spins & 1023) == 0 && (ld_agent(&bar[1]) != 0u || spins > spin_limit)) {
        __hip_atomic_fetch_or(&bar[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (herr) __hip_atomic_store(herr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        ok = 0;
        break;
      }
    }
    s_cok = ok;
  }
  __syncthreads();
  return s_cok != 0;
}

}  // namespace vfm
