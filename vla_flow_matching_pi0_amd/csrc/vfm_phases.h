// vfm_phases.h -- HIP kernels (gfx950) of the flow-matching action expert.
// Included by one translation unit per weight format (vfm_k_*.hip), each of
// which instantiates the kernels of its format.
//
// The denoise loop (PhyAI summary, "Real-Time Physical AI at the Edge,
// Scalable Rollouts in the Cloud": pi0.5's ten Euler steps of the action
// expert) is written as a fixed sequence of phases. Every phase is a device
// function that a workgroup calls with (its index, the number of workgroups)
// and that covers its work units in a grid-stride loop, so the same code runs
//   * inside one persistent cooperative kernel, phases separated by a
//     device-wide barrier (no launch gaps), or
//   * as one kernel launch per phase (eager, or captured into a hipGraph).
//
// Phases of one Euler step t_k (dt = -1/N), per layer l:
//   qkv       [q|k|v] = xn W_qkv, rotary on q, k at P..P+H-1   (fused GEMM)
//   attn      split-K flash attention of q over prefix KV + chunk KV (GQA)
//   combine   merge the key splits (log-sum-exp)
//   o         partial_s = attn[:, K_s] W_o[K_s, :]            (K-split GEMM)
//   rn_mlp    h += gate * sum_s partial_s; xn = adaRMSNorm(h)  (fused)
//   gateup    a = gelu_tanh(xn W_gate) * (xn W_up)             (fused GEMM)
//   down      partial_s = a[:, K_s] W_down[K_s, :]             (K-split GEMM)
//   rn_attn   h += gate * sum_s partial_s; xn = adaRMSNorm(h)  (next layer)
// and at a step boundary (one phase, row-owned):
//   final     h += gate * sum_s partial_s; x += dt (adaRMSNorm_f(h) W_out + b_out)
//   in_proj   h = x W_in + b_in + s; xn = adaRMSNorm(h) (layer 0)
// The fusions (QKV as one GEMM, gate/up as one GEMM, residual+norm, RoPE in
// the projection epilogue) follow the PhyAI optimisation paragraph and the
// hand-written memory-bound kernels listed in the FlashRT walk-through
// (component 8, kernel library). The K-split of the residual GEMMs, whose
// partial sums the following row-parallel norm phase reduces, is ours: it
// lets every GEMM phase use all compute units without atomics.
#pragma once
#include <type_traits>

#include "vfm_device.h"
#include "vfm_gemm_wide.h"
#include "vfm_params.h"

namespace vfm {

extern __shared__ __align__(16) char smem[];

constexpr int NTH = NTHREADS;          // threads per workgroup (8 waves)
constexpr int NWAVES = NTH / 64;

// The thread index as an opaque value: every phase derives its lane
// constants from this, so the compiler cannot hoist them out of the
// persistent kernel's step/layer loops and keep every phase's constants live
// at once (which made the fused kernel spill).
__device__ __forceinline__ int tid_opaque() {
  int t;
  asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"((int)threadIdx.x));
  return t;
}

// The launch parameters as a fresh reference into the kernel-argument
// segment (every kernel here takes the VP block as its first argument). Each
// phase starts from one, so it re-reads the fields it uses with scalar loads
// (scalar-cache hits) instead of the compiler hoisting values derived from
// them out of the step and layer loops and keeping them live across the whole
// persistent kernel, which overflowed the scalar registers into vector
// registers (hundreds of lane spills and reloads).
typedef __attribute__((address_space(4))) const VP KVP;
__device__ __forceinline__ const VP& vp_fresh() {
  KVP* q = (KVP*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(q));
  return *(const VP*)q;
}

// Sum over the workgroup; `red` is >= NWAVES floats of LDS.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = warp_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NWAVES; ++i) s += red[i];
  return s;
}

__device__ __forceinline__ float ldf_coh(const void* base, size_t idx) {
  return __builtin_bit_cast(float, coh_ld4(base, (uint32_t)(idx * 4)));
}
__device__ __forceinline__ void stf_coh(void* base, size_t idx, float v) {
  coh_st4(base, (uint32_t)(idx * 4), __builtin_bit_cast(uint32_t, v));
}

// Activations that many workgroups read (xn, q/k/v, attn, act) live in a
// ring of per-(step, layer) slabs that are written exactly once per launch,
// each 128-byte line by one workgroup, and only read after a phase barrier.
// No L2 of any XCD can then hold a stale copy (the caches start clean at
// every launch), so readers use ordinary cached loads and an XCD fetches
// each line from memory once instead of every workgroup going to the
// coherence point.
__device__ __forceinline__ uint8_t* slab(const VP& p, int k, int l) { return p.ring + ((size_t)k * p.L + l) * p.slab; }

// GEMM inputs (xn_attn, attn, xn_mlp, act) are stored in MFMA operand order,
// [K / KB][Mpad][KB] with KB = MT<T>::KB k values per block (32 bf16, 16
// fp32): the 16 tokens x KB values one wave fetches for one MFMA block form
// one contiguous 1 KiB run. Element offset of (token m, feature k):
template <typename T>
__device__ __forceinline__ size_t act_off(const VP& p, int m, int k) {
  constexpr int KB = MT<T>::KB;
  const int Mpad = ((p.M + 63) / 64) * 64;
  return ((size_t)(k / KB) * Mpad + m) * KB + k % KB;
}

// FP8 experts store their GEMM inputs as e4m3 codes, quantised once by the
// producing phase with the input's calibrated 1/act_scale (the residual +
// norm + quantise fusion the FlashRT walk-through lists among its
// hand-written kernels, component 8). Layout: 64-k blocks, [K/64][Mpad][4
// lane groups g][16 bytes]; the 16 bytes of group g are k = 8g..8g+7 and
// 32+8g..32+8g+7 of the block, the operands of the two 16x16x32 fp8 MFMAs of
// one weight block, fetched with one load. Byte offset of (token m, feature k):
__device__ __forceinline__ size_t act_off8(const VP& p, int m, int k) {
  const int Mpad = ((p.M + 63) / 64) * 64;
  const int kk = k % 64, r = kk / 32, g = (kk % 32) / 8, e = kk % 8;
  return (((size_t)(k / 64) * Mpad + m) * 4 + g) * 16 + r * 8 + e;
}

// e4m3 codes of x * inv, saturated to +-448 (the conversion rounds to nearest
// even and would give NaN beyond 448), two values per call.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2(float a, float b, float inv, uint32_t old) {
  a = fminf(fmaxf(a * inv, -448.0f), 448.0f);
  b = fminf(fmaxf(b * inv, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

// 1/act_scale of GEMM input `which` of layer l (FP8 experts)
__device__ __forceinline__ float act_inv(const VP& p, int l, int which) { return p.qs[(l * 4 + which) * 2 + 1]; }

// Four consecutive features k..k+3 (k % 4 == 0) of token m of a GEMM input,
// in the consumer's operand layout: the activation type, or e4m3 codes.
template <typename T, bool Q8>
__device__ __forceinline__ void store_gemm_in4(const VP& p, void* base, int m, int k, floatx4 y, float inv) {
  if constexpr (Q8) {
    const uint32_t w = fp8x2<true>(y.z, y.w, inv, fp8x2<false>(y.x, y.y, inv, 0u));
    coh_st4(base, (uint32_t)act_off8(p, m, k), w);
  } else if constexpr (sizeof(T) == 4) {
    coh_st16(base, (uint32_t)(act_off<T>(p, m, k) * 4), as_u4(y));
  } else {
    coh_st8(base, (uint32_t)(act_off<T>(p, m, k) * 2), u32x2{pack_bf16x2(y.x, y.y), pack_bf16x2(y.z, y.w)});
  }
}

// q/k/v are stored tile-major, [sample][head][d/16 tiles][64 tokens][16];
// within a q/k tile the 16 slots hold dims 8t..8t+7, then their rotary
// partners 8t+d/2..8t+7+d/2. Element offset of (token i, canonical dim e)
// for a chunk of up to 8 consecutive dims that stays inside one half.
__device__ __forceinline__ size_t qk_off(int d, size_t head_block, int i, int e) {
  const int hd = d / 2;
  const int tt = e < hd ? e / 8 : (e - hd) / 8;
  const int pos = e < hd ? e % 8 : 8 + (e - hd) % 8;
  return ((head_block * (d / 16) + tt) * 64 + i) * 16 + pos;
}
__device__ __forceinline__ size_t v_off(int d, size_t head_block, int i, int e) {
  return ((head_block * (d / 16) + e / 16) * 64 + i) * 16 + e % 16;
}

// ============================================================ row phases
// Row m of the residual stream is always handled by workgroup m % nwg, in
// every row phase, so a row of h and x is only ever touched by one workgroup.

// Sum over the waves of one half of the workgroup (threads [0, NTH/2) or
// [NTH/2, NTH)); every thread of the workgroup must call it.
__device__ __forceinline__ float half_block_sum(float v, float* red, int half) {
  v = warp_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NWAVES / 2; ++i) s += red[half * (NWAVES / 2) + i];
  return s;
}

// h[m] += gate * sum_s part[s][m]; xn[m] = adaRMSNorm(h[m]) with norm `ni`
// (ni < 0: no norm). Four columns per thread. RPP rows per pass: 1 (W <=
// 4 * NTH), or 2 (W <= 2 * NTH; threads [0, NTH/2) take row m of the pair,
// the others row m + 1, each half with its own reduction; a row m >= M is
// a no-op for its half).
template <typename T, bool Q8, int RPP = 1>
__device__ __forceinline__ void row_residual_norm(const VP& p, int step, int m, const float* part, int S, int gate_ni,
                                                  int ni, void* xn, float* red, float inv) {
  const int tid = tid_opaque();
  const int W4 = p.W / 4;
  const int half = RPP == 2 ? tid / (NTH / 2) : 0;
  const int c = RPP == 2 ? tid - half * (NTH / 2) : tid;
  if (RPP == 2) m += half;
  const bool act = c < W4 && m < p.M;
  const auto mr = rsrc(p.mod);
  const size_t mrow = ((size_t)step * p.n_norms + (ni >= 0 ? ni : 0)) * 3 * p.W + c * 4;
  const floatx4 sc = as_f4(ld16_if(mr, (uint32_t)(mrow * 4), act && ni >= 0));
  const floatx4 sh = as_f4(ld16_if(mr, (uint32_t)((mrow + p.W) * 4), act && ni >= 0));
  floatx4 hv = as_f4(coh_ld16_if(rsrc(p.h), (uint32_t)(((size_t)m * p.W + c * 4) * 4), act));
  if (S > 0) {
    const auto pr = rsrc(part);
    u32x4 pv[MAX_KSPLIT];
#pragma unroll
    for (int s = 0; s < MAX_KSPLIT; ++s)
      pv[s] = coh_ld16_if(pr, (uint32_t)((((size_t)s * p.M + m) * p.W + c * 4) * 4), act && s < S);
    // gate_ni < 0: the partial sums of pi0's time-MLP output, ungated
    const floatx4 gate = gate_ni < 0 ? floatx4{1.f, 1.f, 1.f, 1.f}
        : as_f4(ld16_if(mr, (uint32_t)(((((size_t)step * p.n_norms + gate_ni) * 3 + 2) * p.W + c * 4) * 4), act));
    floatx4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < MAX_KSPLIT; ++s) acc += as_f4(pv[s]);
    hv += gate * acc;
    if (act) coh_st16(p.h, (uint32_t)(((size_t)m * p.W + c * 4) * 4), as_u4(hv));
  }
  if (ni < 0) return;
  float ss = hv.x * hv.x + hv.y * hv.y + hv.z * hv.z + hv.w * hv.w;
  ss = RPP == 2 ? half_block_sum(ss, red, half) : block_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)p.W + p.eps);
  if (act) {
    const floatx4 y = hv * r * (1.0f + sc) + sh;
    store_gemm_in4<T, Q8>(p, xn, m, c * 4, y, inv);
  }
}

// Storage format of the per-layer GEMM weights. A lane's 16-byte weight load
// ("weight block") feeds R MFMA k blocks of K = MT<T>::KB each:
//   WF_NATIVE  weights in the activation type (fp32 or bf16), R = 1;
//   WF_FP8     OCP e4m3 codes with a per-tensor scale, R = 2: bytes 8r..8r+7
//              are the fp8 operand of block r, the activations are quantised
//              to e4m3 with the calibrated activation scale as they are
//              loaded, and alpha = act_scale * weight_scale scales the
//              accumulator (FlashRT walk-through, component 6, calibration);
//   WF_W4      symmetric int4 with an fp16 scale per (column, 128-K group),
//              R = 4: word r holds the 8 nibbles of block r, dequantised to
//              bf16 in registers before the MFMA (the W4A16 variant of the
//              PhyAI optimisation paragraph);
//   WF_I8      symmetric int8 with an fp32 scale per output column (W8A16),
//              R = 2: bytes 8r..8r+7 are the codes of block r, turned into
//              bf16 in registers (exact: |q| <= 127) before the MFMA; the
//              column scale multiplies the accumulated sum in the epilogue;
//   WF_W4A8    the int4 codes and group scales of WF_W4 with the e4m3
//              activations of WF_FP8 (W4A8): the codes become e4m3 in
//              registers (exact: |q| <= 8), one group's four fp8 MFMAs
//              accumulate apart and are added to the sum times the group
//              scales of the output columns; alpha = act_scale.
enum { WF_NATIVE = 0, WF_FP8 = 1, WF_W4 = 2, WF_I8 = 3, WF_W4A8 = 4 };
template <int WF> struct WFmt { static constexpr int R = WF == WF_NATIVE ? 1 : (WF == WF_W4 || WF == WF_W4A8) ? 4 : 2; };
// GEMM inputs stored as e4m3 with the calibrated activation scale.
template <int WF> constexpr bool act_fp8() { return WF == WF_FP8 || WF == WF_W4A8; }
// Kernel sets with a folded-norm persistent kernel: bf16 activations, and
// bf16, int4-with-group-scales or int8-with-column-scales weights.
template <typename T, int WF> constexpr bool fusable() {
  return sizeof(T) == 2 && (WF == WF_NATIVE || WF == WF_W4 || WF == WF_I8);
}

// Residual + adaRMSNorm between sublayers: gate_ni is the norm whose gate
// scales the partial sums, ni the norm applied.
template <typename T, int WF = 0>
__device__ __forceinline__ void ph_rn(const VP&, int step, int layer, bool mlp, int wg, int nwg) {
  const VP& p = vp_fresh();
  constexpr bool Q8 = act_fp8<WF>();
  const int tid = tid_opaque();
  float* red = reinterpret_cast<float*>(smem);
  const float* part = mlp ? p.part_o : p.part_d;
  const int S = mlp ? p.S_o : layer == 0 ? p.gp_s[4] : p.S_down;   // layer 0 (pi0 only): the time-MLP output
  const int gate_ni = mlp ? 2 * layer : 2 * layer - 1, ni = mlp ? 2 * layer + 1 : 2 * layer;
  void* xn = slab(p, step, layer) + (mlp ? p.off_xnm : p.off_xna);
  const float inv = Q8 ? act_inv(p, layer, mlp ? 2 : 0) : 1.0f;
  if (p.bigm && p.W <= 2 * NTH) {
    // per-phase launch with many rows: two rows per workgroup pass (at W = 1024 one row occupies half the threads)
    for (int m = 2 * wg; m < p.M; m += 2 * nwg) {
      row_residual_norm<T, Q8, 2>(p, step, m, part, S, gate_ni, ni, xn, red, inv);
      __syncthreads();
    }
    return;
  }
  for (int m = wg; m < p.M; m += nwg) {
    row_residual_norm<T, Q8>(p, step, m, part, S, gate_ni, ni, xn, red, inv);
    __syncthreads();
  }
}

// Step boundary for row m: finish step `kp` (if kp >= 0): add the last
// layer's partials, x += dt * (adaRMSNorm_final(h) W_out + b_out); then
// start step `kn` (if kn < N): h = x W_in + b_in + s, xn = adaRMSNorm(h).
// kp = -1 also initialises x from the noise and the state embedding s.
// Thread c owns columns 4c..4c+3 of the row; every weight load is issued
// before it is used.
constexpr int MAX_A = MAX_A_HOST;
template <typename T, int WF = 0, bool FUSE = false>
__device__ __forceinline__ void ph_boundary(const VP&, int kp, int kn, int wg, int nwg) {
  const VP& p = vp_fresh();
  constexpr bool Q8 = act_fp8<WF>();
  const int tid = tid_opaque();
  float* red = reinterpret_cast<float*>(smem);                       // [NWAVES]
  float* xs = red + NWAVES;                                          // [W]
  floatx4* part = reinterpret_cast<floatx4*>(xs + p.W);              // [NTH]
  float* xrow = reinterpret_cast<float*>(part + NTH);                // [MAX_A]
  const int A = p.A, W = p.W, W4 = W / 4, c = tid;
  const float dt = -1.0f / (float)p.N;
  const auto wout = rsrc(p.out_w), win = rsrc(p.in_w), wst = rsrc(p.st_w);
  for (int m = wg; m < p.M; m += nwg) {
    const int b = m / p.H, i = m - b * p.H;
    const bool srow = p.pi0 && i == 0;                     // pi0's state token: no action of its own
    const int xm = p.pi0 ? b * (p.H - 1) + i - 1 : m;     // row of x / noise
    if (kp < 0) {
      if (c < A && !srow) {
        const float v = p.noise[(size_t)xm * A + c];
        xrow[c] = v;
        if (p.noise != p.x) stf_coh(p.x, (size_t)xm * A + c, v);
      }
    } else if (!srow) {
      // h += gate * sum_s partial_s of the last layer, then the final adaRMSNorm into LDS
      floatx4 hv = {0, 0, 0, 0};
      if (c < W4) {
        hv = as_f4(coh_ld16(p.h, (uint32_t)(((size_t)m * W + c * 4) * 4)));
        if (p.L > 0) {
          const auto pr = rsrc(p.part_d);
          u32x4 pv[MAX_KSPLIT];
#pragma unroll
          for (int s = 0; s < MAX_KSPLIT; ++s)
            pv[s] = coh_ld16_if(pr, (uint32_t)((((size_t)s * p.M + m) * W + c * 4) * 4), s < p.S_down);
          floatx4 acc = {0, 0, 0, 0};
#pragma unroll
          for (int s = 0; s < MAX_KSPLIT; ++s) acc += as_f4(pv[s]);
          const floatx4 gate = as_f4(ro_ld16(p.mod + (((size_t)kp * p.n_norms + 2 * p.L - 1) * 3 + 2) * W + c * 4));
          hv += gate * acc;
        }
      }
      const float ss = block_sum(hv.x * hv.x + hv.y * hv.y + hv.z * hv.z + hv.w * hv.w, red);
      const float r = 1.0f / sqrtf(ss / (float)W + p.eps);
      if (c < W4) {
        const float* mod = p.mod + ((size_t)kp * p.n_norms + (p.n_norms - 1)) * 3 * W;
        const floatx4 y = hv * r * (1.0f + as_f4(ro_ld16(mod + c * 4))) + as_f4(ro_ld16(mod + W + c * 4));
        *reinterpret_cast<floatx4*>(xs + c * 4) = y;
      }
      __syncthreads();
      // v[4q..4q+3] = sum_n xs[n] W_out[n][4q..4q+3]: thread (q, sub) sums n = sub + nsub * j
      const int nq = A / 4, nsub = NTH / nq, q = c % nq, sub = c / nq;
      floatx4 acc = {0, 0, 0, 0};
      for (int j0 = 0; j0 * nsub < W; j0 += 16) {
        u32x4 wv[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int n = sub + (j0 + j) * nsub;
          wv[j] = ld16_if(wout, (uint32_t)(((size_t)n * A + 4 * q) * 4), n < W);
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int n = sub + (j0 + j) * nsub;
          acc += (n < W ? xs[n] : 0.f) * as_f4(wv[j]);
        }
      }
      part[c] = acc;
      __syncthreads();
      if (c < nq) {
        floatx4 v = as_f4(ro_ld16(p.out_b + 4 * c));
        for (int j = 0; j < nsub; ++j) v += part[c + j * nq];
        const uint32_t off = (uint32_t)(((size_t)xm * A + 4 * c) * 4);
        const floatx4 x = as_f4(coh_ld16(p.x, off)) + dt * v;
        coh_st16(p.x, off, as_u4(x));
        *reinterpret_cast<floatx4*>(xrow + 4 * c) = x;
      }
    }
    __syncthreads();
    if (kn < p.N && p.pi0) {
      // pi0: the state token starts from s = state W_s + b_s; an action token
      // from the time-MLP output bias, its hidden u = SiLU(x (W_in W_mi) +
      // tbias[t]) going to the time-MLP output GEMM (the state row's u is 0)
      floatx4 hv = {0, 0, 0, 0}, u = {0, 0, 0, 0};
      if (c < W4) {
        if (srow) {
          if (kp < 0) {
            floatx4 sv = as_f4(ro_ld16(p.st_b + c * 4));
            for (int j0 = 0; j0 < p.S; j0 += 16) {
              u32x4 wv[16];
#pragma unroll
              for (int j = 0; j < 16; ++j)
                wv[j] = ld16_if(wst, (uint32_t)(((size_t)(j0 + j) * W + c * 4) * 4), j0 + j < p.S);
#pragma unroll
              for (int j = 0; j < 16; ++j)
                if (j0 + j < p.S) sv += p.state[(size_t)b * p.S + j0 + j] * as_f4(wv[j]);
            }
            coh_st16(p.s_emb, (uint32_t)(((size_t)m * W + c * 4) * 4), as_u4(sv));
            hv = sv;
          } else {
            hv = as_f4(coh_ld16(p.s_emb, (uint32_t)(((size_t)m * W + c * 4) * 4)));
          }
        } else {
          floatx4 pre = as_f4(ro_ld16(p.tbias + (size_t)kn * W + c * 4));
          for (int a0 = 0; a0 < A; a0 += 16) {
            u32x4 wv[16];
#pragma unroll
            for (int j = 0; j < 16; ++j)
              wv[j] = ld16_if(win, (uint32_t)(((size_t)(a0 + j) * W + c * 4) * 4), a0 + j < A);
#pragma unroll
            for (int j = 0; j < 16; ++j) pre += (a0 + j < A ? xrow[a0 + j] : 0.f) * as_f4(wv[j]);
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) u[q] = pre[q] / (1.0f + expf(-pre[q]));
          hv = as_f4(ro_ld16(p.tmlp_b + c * 4));
        }
        coh_st16(p.h, (uint32_t)(((size_t)m * W + c * 4) * 4), as_u4(hv));
        store_gemm_in4<T, false>(p, slab(p, kn, 0) + p.off_u, m, c * 4, u, 1.0f);
      }
    } else if (kn < p.N) {
      // h = x W_in + b_in + s, four columns per thread
      floatx4 hv = {0, 0, 0, 0};
      if (c < W4) {
        hv = as_f4(ro_ld16(p.in_b + c * 4));
        if (p.S > 0) {
          if (kp < 0) {   // state embedding, computed once per denoise call
            floatx4 sv = as_f4(ro_ld16(p.st_b + c * 4));
            for (int j0 = 0; j0 < p.S; j0 += 16) {
              u32x4 wv[16];
#pragma unroll
              for (int j = 0; j < 16; ++j)
                wv[j] = ld16_if(wst, (uint32_t)(((size_t)(j0 + j) * W + c * 4) * 4), j0 + j < p.S);
#pragma unroll
              for (int j = 0; j < 16; ++j)
                if (j0 + j < p.S) sv += p.state[(size_t)b * p.S + j0 + j] * as_f4(wv[j]);
            }
            coh_st16(p.s_emb, (uint32_t)(((size_t)m * W + c * 4) * 4), as_u4(sv));
            hv += sv;
          } else {
            hv += as_f4(coh_ld16(p.s_emb, (uint32_t)(((size_t)m * W + c * 4) * 4)));
          }
        }
        for (int a0 = 0; a0 < A; a0 += 16) {
          u32x4 wv[16];
#pragma unroll
          for (int j = 0; j < 16; ++j)
            wv[j] = ld16_if(win, (uint32_t)(((size_t)(a0 + j) * W + c * 4) * 4), a0 + j < A);
#pragma unroll
          for (int j = 0; j < 16; ++j) hv += (a0 + j < A ? xrow[a0 + j] : 0.f) * as_f4(wv[j]);
        }
        coh_st16(p.h, (uint32_t)(((size_t)m * W + c * 4) * 4), as_u4(hv));
      }
      if (FUSE && p.L > 0) {
        // norms folded into the GEMMs: layer 0's qkv applies r and the shift;
        // here y = h (1 + scale) and the sums of squares of h per 16 columns
        // (threads 4t .. 4t + 3 of a wave hold tile t)
        float ss = hv.x * hv.x + hv.y * hv.y + hv.z * hv.z + hv.w * hv.w;
        ss += __shfl_xor(ss, 1);
        ss += __shfl_xor(ss, 2);
        if (c < W4) {
          const float* mod = p.mod + ((size_t)kn * p.n_norms) * 3 * W;
          const floatx4 y = hv * (1.0f + as_f4(ro_ld16(mod + c * 4)));
          store_gemm_in4<T, false>(p, slab(p, kn, 0) + p.off_xna, m, c * 4, y, 1.0f);
          if ((c & 3) == 0)
            coh_st4(slab(p, kn, 0) + p.off_ssa, (uint32_t)(((size_t)m * (W / 16) + c / 4) * 4), __builtin_bit_cast(uint32_t, ss));
        }
      } else if (p.L > 0) {
        const float ss = block_sum(hv.x * hv.x + hv.y * hv.y + hv.z * hv.z + hv.w * hv.w, red);
        const float r = 1.0f / sqrtf(ss / (float)W + p.eps);
        if (c < W4) {
          const float* mod = p.mod + ((size_t)kn * p.n_norms) * 3 * W;
          const floatx4 y = hv * r * (1.0f + as_f4(ro_ld16(mod + c * 4))) + as_f4(ro_ld16(mod + W + c * 4));
          uint8_t* xn = slab(p, kn, 0) + p.off_xna;
          store_gemm_in4<T, Q8>(p, xn, m, c * 4, y, Q8 ? act_inv(p, 0, 0) : 1.0f);
        }
      }
    }
    __syncthreads();
  }
}

// ============================================================ skinny GEMM on MFMA
// C[M x N] = A[M x K] (act type T in MFMA operand order, see act_off,
// produced by an earlier phase) times a packed weight. Swap-AB: the weight supplies the 16 MFMA rows
// (output features) and the tokens the 16 MFMA columns, so the 50 tokens of
// a chunk pad to 64 = 4 column tiles and a lane ends with 4 consecutive
// output features of one token. Packed weight layout:
// [N/16 tiles][K/KB blocks][64 lanes][16 bytes], one contiguous 1 KiB block
// per MFMA step.
// Work unit = nt (1 or 2) 16-column tiles x a K range K/S x 64 tokens. The 8
// waves of the workgroup split the K range; every wave issues all its weight
// and activation loads of a pass before its MFMAs, and the 8 partial tiles
// are summed through LDS. Nonlinear epilogues (RoPE, GeGLU) need S = 1; the
// linear residual GEMMs (o, down) write S partial sums that the next row
// phase adds.
enum { G_QKV = 0, G_O = 1, G_GU = 2, G_DOWN = 3, G_TMLP = 4 };
constexpr int GEMM_PASS = 4;     // MFMA k blocks per wave per pass



// Weight fragments of one pass of one unit, held in registers. The
// persistent kernel loads a workgroup's first pass of the next GEMM while it
// waits at the barrier before that GEMM.
struct WPre {
  u32x4 w[2][GEMM_PASS];
  uint32_t sc[2];          // WF_W4: the fp16 group scale of each tile's column
  u32x2 sc4[2];            // WF_W4A8: the group scales of the 4 output columns a lane accumulates
};

struct GemmShape {
  const uint8_t* Wp;
  const uint8_t* Ws;       // after the codes: WF_W4(A8) scales [N/16][K/128][16] fp16, WF_I8 scales [N] fp32
  int K, N, nt, S, ngroups, units, nkb, KR, nkbw;
};

template <typename T, int WHICH, int WF>
__device__ __forceinline__ GemmShape gemm_shape(const VP& p, int layer) {
  constexpr int KW = MT<T>::KB * WFmt<WF>::R;   // K per weight block
  GemmShape g;
  if (WHICH == G_QKV) { g.K = p.W; g.N = (p.Hq + 2 * p.Hkv) * p.d; g.Wp = p.w_qkv[layer]; }
  else if (WHICH == G_O) { g.K = p.Hq * p.d; g.N = p.W; g.Wp = p.w_o[layer]; }
  else if (WHICH == G_GU) { g.K = p.W; g.N = 2 * p.F; g.Wp = p.w_gu[layer]; }
  else if (WHICH == G_DOWN) { g.K = p.F; g.N = p.W; g.Wp = p.w_down[layer]; }
  else { g.K = p.W; g.N = p.W; g.Wp = p.w_tmlp; }
  g.Ws = g.Wp + (WF == WF_I8 ? (size_t)g.N * g.K : (size_t)g.N * g.K / 2);
  g.nt = p.gp_nt[WHICH];
  g.S = p.gp_s[WHICH];
  g.ngroups = g.N / (16 * g.nt);
  g.units = g.ngroups * g.S * ((p.M + 63) / 64);
  g.nkb = g.K / KW;
  g.KR = g.K / g.S;
  g.nkbw = g.KR / KW / NWAVES;
  return g;
}

// Weight fragments of pass pb (in weight blocks) of unit u for this lane
// (zeros where the pass or the tile does not exist).
template <typename T, int WHICH, int WF>
__device__ __forceinline__ void gemm_load_weights(const GemmShape& gs, int u, int pb, int tid, WPre& out) {
  constexpr int R = WFmt<WF>::R, KW = MT<T>::KB * R, PW = GEMM_PASS / R;
  const int lane = tid & 63, wv = tid >> 6;
  const int ng = u % gs.ngroups, s = (u / gs.ngroups) % gs.S;
  const int t0 = ng * gs.nt;
  const int kb0 = (s * gs.KR) / KW + wv * gs.nkbw;
  const auto wrs = rsrc(gs.Wp);
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const bool ok = pb + i < gs.nkbw;
    const int kb = kb0 + pb + i;
#pragma unroll
    for (int t = 0; t < 2; ++t)
      out.w[t][i] = ld16_if(wrs, (uint32_t)((((size_t)(t0 + t) * gs.nkb + kb) * 64 + lane) * 16), ok && t < gs.nt);
  }
  if constexpr (WF == WF_W4) {
    const auto srs = rsrc(gs.Ws);
    const bool ok = pb < gs.nkbw;
#pragma unroll
    for (int t = 0; t < 2; ++t)
      out.sc[t] = ld2_if(srs, (uint32_t)((((size_t)(t0 + t) * gs.nkb + kb0 + pb) * 16 + (lane & 15)) * 2),
                         ok && t < gs.nt);
  }
  if constexpr (WF == WF_W4A8) {
    // the lane's output rows are columns 4 g .. 4 g + 3 of the tile: their 4 fp16 scales are adjacent
    const auto srs = rsrc(gs.Ws);
    const bool ok = pb < gs.nkbw;
#pragma unroll
    for (int t = 0; t < 2; ++t)
      out.sc4[t] = ld8_if(srs, (uint32_t)((((size_t)(t0 + t) * gs.nkb + kb0 + pb) * 16 + 4 * (lane >> 4)) * 2),
                          ok && t < gs.nt);
  }
}

template <typename T, int WHICH, int WF>
__device__ __forceinline__ void gemm_prefetch(const VP&, int layer, int wg, WPre& out) {
  const VP& p = vp_fresh();
  const GemmShape gs = gemm_shape<T, WHICH, WF>(p, layer);
  const int tid = tid_opaque();
  out = WPre{};   // a full write, so the previous prefetch is dead from here on
  if (wg < gs.units) gemm_load_weights<T, WHICH, WF>(gs, wg, 0, tid, out);
}

template <typename T, int WHICH, int WF>
struct PrefetchHook {
  const VP& p;
  int layer, wg;
  WPre& out;
  __device__ __forceinline__ void operator()() const { gemm_prefetch<T, WHICH, WF>(p, layer, wg, out); }
};

// 8 signed nibbles (element e in bits 4e..4e+3) times an fp16 scale -> 8 bf16.
__device__ __forceinline__ u32x4 w4_to_bf16(uint32_t wd, uint32_t scale_bits) {
  const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)scale_bits);
  float f[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = (float)(((int)(wd << (28 - 4 * e))) >> 28) * s;
  return u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])};
}

// 8 signed nibbles (element e in bits 4e..4e+3) -> 8 e4m3 codes (byte e),
// exact: every integer in [-8, 7] is an e4m3 value.
__device__ __forceinline__ long w4_to_fp8(uint32_t wd) {
  uint32_t o[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float f[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = (float)(((int)(wd << (28 - 4 * (4 * h + e)))) >> 28);
    o[h] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false), true);
  }
  return (long)(((unsigned long long)o[1] << 32) | o[0]);
}

// 4 fp16 values (2 words) -> floatx4.
__device__ __forceinline__ floatx4 half4_to_f4(u32x2 h) {
  return floatx4{(float)__builtin_bit_cast(_Float16, (uint16_t)(h[0] & 0xffffu)),
                 (float)__builtin_bit_cast(_Float16, (uint16_t)(h[0] >> 16)),
                 (float)__builtin_bit_cast(_Float16, (uint16_t)(h[1] & 0xffffu)),
                 (float)__builtin_bit_cast(_Float16, (uint16_t)(h[1] >> 16))};
}

// 8 int8 codes (byte e of the pair of words is element e) -> 8 bf16, exact
// since |q| <= 127 needs 7 significand bits: the upper half of the float32.
__device__ __forceinline__ u32x4 i8_to_bf16(uint32_t lo, uint32_t hi) {
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t wd = q < 2 ? lo : hi;
    const int b = 2 * (q & 1);
    const float f0 = (float)((int)(wd << (24 - 8 * b)) >> 24);
    const float f1 = (float)((int)(wd << (16 - 8 * b)) >> 24);
    o[q] = (__builtin_bit_cast(uint32_t, f0) >> 16) | (__builtin_bit_cast(uint32_t, f1) & 0xffff0000u);
  }
  return o;
}

// Largest |x| of a lane's 16-byte activation fragment (calibration).
template <typename T>
__device__ __forceinline__ float frag_amax(u32x4 a) {
  float m = 0.f;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t wd = a[q];
      m = fmaxf(m, fmaxf(fabsf(__builtin_bit_cast(float, wd << 16)), fabsf(__builtin_bit_cast(float, wd & 0xffff0000u))));
    }
  } else {
    const floatx4 f = as_f4(a);
    m = fmaxf(fmaxf(fabsf(f[0]), fabsf(f[1])), fmaxf(fabsf(f[2]), fabsf(f[3])));
  }
  return m;
}

// FUSE (bf16 weights and activations): the norms next to the GEMM are folded
// into it. qkv and gate/up read y = h (1 + scale) and finish
// xn W = r (y W) + shift W with r = 1 / sqrt(mean(h^2) + eps) from the per-16-
// column sums of squares and shift W from the step's table. o and down (not
// the last layer's down, which the step boundary finishes) store their K-split
// partial sums; the last unit of a column group to arrive (an arrival counter
// per group and 64-row tile) adds the splits in the fixed order 0 .. S-1,
// applies the gated residual h += gate * sum, and writes h, the next norm's
// y = h (1 + scale) and the group's sums of squares.
//
// xl (set by the persistent kernel once every workgroup is known to run on
// XCD blockIdx % 8): the S split units of a column group are units
// ng + ngroups (s + S mt) with ngroups and the grid multiples of 8, so they
// all run on XCD ng % 8 and exchange their partial sums through that XCD's
// L2 alone: write-back stores, an arrival atomic performed in the L2 (a
// counter per 128-byte line, never cleared by the kernel: S is a power of
// two, every complete launch adds a multiple of S, and the host clears them
// when the split plan changes or a launch fails), and, in the last unit, an
// L1 invalidation before ordinary loads that the L2 serves.
template <typename T, int WHICH, bool PRE, int WF = WF_NATIVE, bool CAL = false, bool FUSE = false>
__device__ __forceinline__ void ph_gemm(const VP&, int step, int layer, int wg, int nwg, const WPre& pre,
                                        bool xl = false, bool arrive = false) {
  const VP& p = vp_fresh();
  const int tid = tid_opaque();
  constexpr int E = MT<T>::E, KM = MT<T>::KB, R = WFmt<WF>::R, KW = KM * R, PW = GEMM_PASS / R;
  static_assert(WF == WF_NATIVE || sizeof(T) == 2, "quantised weights run with bf16 activations");
  static_assert(!FUSE || (fusable<T, WF>() && !CAL), "folded norms: bf16 activations, bf16 / W4 / W8 weights");
  constexpr bool FIN = FUSE && (WHICH == G_QKV || WHICH == G_GU);    // applies r and the shift
  constexpr bool FOUT = FUSE && (WHICH == G_O || WHICH == G_DOWN);   // finishes the residual
  const bool fout = FOUT && (WHICH == G_O || layer + 1 < p.L);
  __shared__ unsigned s_last;
  uint8_t* sl = slab(p, step, layer);
  const T* A;
  if (WHICH == G_QKV) A = (const T*)(sl + p.off_xna);
  else if (WHICH == G_O) A = (const T*)(sl + p.off_attn);
  else if (WHICH == G_GU) A = (const T*)(sl + p.off_xnm);
  else if (WHICH == G_DOWN) A = (const T*)(sl + p.off_act);
  else A = (const T*)(sl + p.off_u);
  const GemmShape gs = gemm_shape<T, WHICH, WF>(p, layer);
  const int K = gs.K, nt = gs.nt, S = gs.S, ngroups = gs.ngroups, units = gs.units, KR = gs.KR, nkbw = gs.nkbw;
  const int Mpad = ((p.M + 63) / 64) * 64;
  const int lane = tid & 63, wv = tid >> 6, g = lane >> 4, c16 = lane & 15;
  float alpha = 1.0f;
  if constexpr (act_fp8<WF>()) alpha = p.qs[(layer * 4 + WHICH) * 2];
  float amax = 0.f;
  floatx4* red = reinterpret_cast<floatx4*>(smem);  // [NWAVES][2][4][64]
  for (int u = wg; u < units; u += nwg) {
    const int ng = u % ngroups, rest = u / ngroups, s = rest % S, mt = rest / S;
    const int t0 = ng * nt, m0 = mt * 64;
    const int kb0 = (s * KR) / KW + wv * nkbw;
    floatx4 acc[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int st = 0; st < 4; ++st) acc[t][st] = floatx4{0, 0, 0, 0};
    floatx4 tmp[2][4];   // WF_W4A8: one group's sum before its scales
    bool rowok[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) rowok[st] = m0 + st * 16 + c16 < p.M;
    // rotary (cos, sin) pairs of the epilogue item this wave finalises, fetched
    // with the operands rather than after the products
    floatx4 rot = {0, 0, 0, 0};
    if constexpr (WHICH == G_QKV) {
      const int t = wv / 4, st = wv % 4;
      const int gm = m0 + st * 16 + c16, col0 = (t0 + t) * 16;
      const int head = col0 / p.d, tt = (col0 % p.d) / 16;
      const bool ok = wv < nt * 4 && gm < p.M && head < p.Hq + p.Hkv;
      const int i = gm % p.H, j0 = tt * 8 + 2 * g;
      rot = as_f4(ld16_if(rsrc(p.rope), (uint32_t)((((size_t)i * (p.d / 2) + j0) * 2) * 4), ok));
    }
    // folded norm: shift W of the item's columns and this lane's quarter of the
    // row's per-tile sums of squares (W <= 1024: at most 4 loads; write-once
    // slab data, read through L2), fetched up front too
    floatx4 shv = {0, 0, 0, 0};
    u32x4 ssv[4];
    if constexpr (FIN) {
      const int t = wv / 4, st = wv % 4;
      const int gm = m0 + st * 16 + c16;
      const bool ok = wv < nt * 4 && gm < p.M;
      const float* shw = (WHICH == G_QKV ? p.shw_q : p.shw_g) + ((size_t)step * p.L + layer) * gs.N;
      shv = as_f4(ld16_if(rsrc(shw), (uint32_t)(((t0 + t) * 16 + 4 * g) * 4), ok));
      const int per = p.W / 64;
      const auto sr = rsrc(sl + (WHICH == G_QKV ? p.off_ssa : p.off_ssm));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        ssv[j] = ld16_if(sr, (uint32_t)(((size_t)gm * (p.W / 16) + g * per + 4 * j) * 4), ok && 4 * j < per);
    }
    // W8A16: the column scales of that epilogue item, fetched up front too
    floatx4 csc = {1.f, 1.f, 1.f, 1.f};
    if constexpr (WF == WF_I8) csc = as_f4(ld16_if(rsrc(gs.Ws), (uint32_t)(((t0 + wv / 4) * 16 + 4 * g) * 4), wv < nt * 4));
    const auto ars = rsrc(A);
    for (int pb = 0; pb < nkbw; pb += PW) {
      WPre wl;
      u32x4 ar[4][GEMM_PASS];
      if (PRE && u == wg && pb == 0) wl = pre;
      else gemm_load_weights<T, WHICH, WF>(gs, u, pb, tid, wl);
      if constexpr (WF == WF_W4A8) {
        // e4m3 inputs (act_off8): a 128-K weight block spans two 64-K activation blocks
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bool ok = pb < nkbw;
          const int kblk = (kb0 + pb) * 2 + h;
#pragma unroll
          for (int st = 0; st < 4; ++st) {
            const size_t row = (size_t)(m0 + st * 16 + c16);
            ar[st][h] = ld16_if(ars, (uint32_t)((((size_t)kblk * Mpad + row) * 4 + g) * 16), ok && rowok[st]);
          }
        }
      } else if constexpr (WF == WF_FP8) {
        // e4m3 inputs (act_off8): one 16-byte fetch per weight block and token subtile
#pragma unroll
        for (int i = 0; i < PW; ++i) {
          const bool ok = pb + i < nkbw;
          const int kblk = kb0 + pb + i;
#pragma unroll
          for (int st = 0; st < 4; ++st) {
            const size_t row = (size_t)(m0 + st * 16 + c16);
            ar[st][i] = ld16_if(ars, (uint32_t)((((size_t)kblk * Mpad + row) * 4 + g) * 16), ok && rowok[st]);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < GEMM_PASS; ++j) {
          const int i = j / R, r = j % R;
          const bool ok = pb + i < nkbw;
          const int k = (kb0 + pb + i) * KW + r * KM + g * E;
#pragma unroll
          for (int st = 0; st < 4; ++st) {
            const size_t row = (size_t)(m0 + st * 16 + c16);
            const size_t off = ((size_t)(k / KM) * Mpad + row) * KM + k % KM;   // operand order, see act_off
            ar[st][j] = ld16_if(ars, (uint32_t)(off * sizeof(T)), ok && rowok[st]);
          }
        }
      }
      if constexpr (CAL) {
#pragma unroll
        for (int j = 0; j < GEMM_PASS; ++j)
#pragma unroll
          for (int st = 0; st < 4; ++st) amax = fmaxf(amax, frag_amax<T>(ar[st][j]));
      }
#pragma unroll
      for (int j = 0; j < GEMM_PASS; ++j) {
        const int i = j / R, r = j % R;
        if constexpr (WF == WF_NATIVE) {
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int st = 0; st < 4; ++st)
              if (t < nt) acc[t][st] = MT<T>::mma(wl.w[t][i], ar[st][j], acc[t][st]);
        } else if constexpr (WF == WF_FP8) {
          long a8[4];
#pragma unroll
          for (int st = 0; st < 4; ++st) a8[st] = (long)__builtin_bit_cast(i64x2, ar[st][i])[r];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const i64x2 w2 = __builtin_bit_cast(i64x2, wl.w[t][i]);
            const long w8 = (long)w2[r];
#pragma unroll
            for (int st = 0; st < 4; ++st)
              if (t < nt) acc[t][st] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(w8, a8[st], acc[t][st], 0, 0, 0);
          }
        } else if constexpr (WF == WF_W4A8) {
          // one weight block = one 128-K group: its four MFMAs go to tmp, then acc += tmp x group scales
          if (r == 0) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
              for (int st = 0; st < 4; ++st) tmp[t][st] = floatx4{0, 0, 0, 0};
          }
          long a8[4];
#pragma unroll
          for (int st = 0; st < 4; ++st) a8[st] = (long)__builtin_bit_cast(i64x2, ar[st][r / 2])[r % 2];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const long w8 = w4_to_fp8(wl.w[t][i][r]);
#pragma unroll
            for (int st = 0; st < 4; ++st)
              if (t < nt) tmp[t][st] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(w8, a8[st], tmp[t][st], 0, 0, 0);
          }
          if (r == R - 1) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              const floatx4 gsc = half4_to_f4(wl.sc4[t]);
#pragma unroll
              for (int st = 0; st < 4; ++st) acc[t][st] += tmp[t][st] * gsc;
            }
          }
        } else if constexpr (WF == WF_I8) {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const u32x4 wb = i8_to_bf16(wl.w[t][i][2 * r], wl.w[t][i][2 * r + 1]);
#pragma unroll
            for (int st = 0; st < 4; ++st)
              if (t < nt) acc[t][st] = MT<T>::mma(wb, ar[st][j], acc[t][st]);
          }
        } else {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const u32x4 wb = w4_to_bf16(wl.w[t][i][r], wl.sc[t]);
#pragma unroll
            for (int st = 0; st < 4; ++st)
              if (t < nt) acc[t][st] = MT<T>::mma(wb, ar[st][j], acc[t][st]);
          }
        }
      }
    }
    // sum the 8 waves' partial tiles through LDS
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int st = 0; st < 4; ++st)
        if (t < nt) red[((wv * 2 + t) * 4 + st) * 64 + lane] = acc[t][st];
    __syncthreads();
    // epilogue: wave w finalises item w = (tile t, token subtile st)
    floatx4 v = {0, 0, 0, 0};
    if (wv < nt * 4) {
      const int t = wv / 4, st = wv % 4;
#pragma unroll
      for (int w2 = 0; w2 < NWAVES; ++w2) v += red[((w2 * 2 + t) * 4 + st) * 64 + lane];
      if constexpr (act_fp8<WF>()) v *= alpha;
      const int gm = m0 + st * 16 + c16;
      const int tile = t0 + t;
      if constexpr (WF == WF_I8) v *= csc;
      if constexpr (FIN) {
        float sq = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const floatx4 q = as_f4(ssv[j]);
          sq += (q.x + q.y) + (q.z + q.w);
        }
        sq += __shfl_xor(sq, 16);
        sq += __shfl_xor(sq, 32);
        v = (1.0f / sqrtf(sq / (float)p.W + p.eps)) * v + shv;
      }
      if (gm < p.M) {
        if (WHICH == G_QKV) {
          const int d = p.d, hd = d / 2;
          const int col0 = tile * 16;
          const int head = col0 / d, tt = (col0 % d) / 16;
          const int b = gm / p.H, i = gm % p.H;
          if (head < p.Hq + p.Hkv) {
            // packed lane order (x_j, x_j+1, x_j+d/2, x_j+1+d/2), j = 8 tt + 2 g
            const int j0 = tt * 8 + 2 * g;
            const float c0 = rot[0], s0 = rot[1], c1 = rot[2], s1 = rot[3];
            const float y0 = v.x * c0 - v.z * s0, y0h = v.z * c0 + v.x * s0;
            const float y1 = v.y * c1 - v.w * s1, y1h = v.w * c1 + v.y * s1;
            const bool isq = head < p.Hq;
            uint8_t* dst = sl + (isq ? p.off_q : p.off_k);
            const size_t hb = isq ? (size_t)b * p.Hq + head : (size_t)b * p.Hkv + (head - p.Hq);
            const size_t e0 = ((hb * (d / 16) + tt) * 64 + i) * 16 + 2 * g;   // slots 2g, 2g+1 and 8+2g, 9+2g
            if constexpr (sizeof(T) == 4) {
              coh_st8(dst, (uint32_t)(e0 * 4), u32x2{__builtin_bit_cast(uint32_t, y0), __builtin_bit_cast(uint32_t, y1)});
              coh_st8(dst, (uint32_t)((e0 + 8) * 4), u32x2{__builtin_bit_cast(uint32_t, y0h), __builtin_bit_cast(uint32_t, y1h)});
            } else {
              coh_st4(dst, (uint32_t)(e0 * 2), pack_bf16x2(y0, y1));
              coh_st4(dst, (uint32_t)((e0 + 8) * 2), pack_bf16x2(y0h, y1h));
            }
          } else {
            const int kvh = head - p.Hq - p.Hkv;
            const size_t e0 = ((((size_t)b * p.Hkv + kvh) * (d / 16) + tt) * 64 + i) * 16 + 4 * g;
            uint8_t* dst = sl + p.off_v;
            if constexpr (sizeof(T) == 4) coh_st16(dst, (uint32_t)(e0 * 4), as_u4(v));
            else coh_st8(dst, (uint32_t)(e0 * 2), u32x2{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)});
          }
        } else if (WHICH == G_GU) {
          // packed lane order (gate f, up f, gate f+1, up f+1), f = 8 tile + 2 g
          const int f0 = tile * 8 + 2 * g;
          const float a0 = gelu_tanh(v.x) * v.y, a1 = gelu_tanh(v.z) * v.w;
          uint8_t* dst = sl + p.off_act;
          if constexpr (act_fp8<WF>()) {
            const uint32_t w = fp8x2<false>(a0, a1, act_inv(p, layer, G_DOWN), 0u);
            coh_st2(dst, (uint32_t)act_off8(p, gm, f0), w & 0xffffu);
          } else {
            const size_t e0 = act_off<T>(p, gm, f0);
            if constexpr (sizeof(T) == 4)
              coh_st8(dst, (uint32_t)(e0 * 4), u32x2{__builtin_bit_cast(uint32_t, a0), __builtin_bit_cast(uint32_t, a1)});
            else coh_st4(dst, (uint32_t)(e0 * 2), pack_bf16x2(a0, a1));
          }
        } else if (!fout || S > 1) {
          float* part = WHICH == G_O ? p.part_o : p.part_d;
          const int n0 = tile * 16 + 4 * g;
          const uint32_t off = (uint32_t)((((size_t)s * p.M + gm) * p.W + n0) * 4);
          if (FOUT && fout && xl) wb_st16(part, off, as_u4(v));
          else coh_st16(part, off, as_u4(v));
        }
      }
    }
    if (FOUT && fout) {
      const int t = wv / 4, st = wv % 4;
      const int gm = m0 + st * 16 + c16, c = (t0 + t) * 16 + 4 * g, W = p.W;
      const bool mine = wv < nt * 4 && gm < p.M;
      const int gate_ni = WHICH == G_O ? 2 * layer : 2 * layer + 1, next_ni = gate_ni + 1;
      const auto mr = rsrc(p.mod);
      // the residual, its gate and the next norm's scale, issued before the
      // wait for the partial sums' stores
      const floatx4 h0 = as_f4(coh_ld16_if(rsrc(p.h), (uint32_t)(((size_t)gm * W + c) * 4), mine));
      const floatx4 gt = as_f4(ld16_if(mr, (uint32_t)(((((size_t)step * p.n_norms + gate_ni) * 3 + 2) * W + c) * 4), mine));
      const floatx4 sc = as_f4(ld16_if(mr, (uint32_t)(((((size_t)step * p.n_norms + next_ni) * 3) * W + c) * 4), mine));
      bool last = true;
      if (S > 1) {
        __builtin_amdgcn_s_waitcnt(0);   // this wave's partial sums are stored
        __syncthreads();
        if (tid == 0) {
          const int ci = (WHICH == G_O ? 0 : FCNT_MAX) + mt * ngroups + ng;
          const unsigned old =
              xl ? __hip_atomic_fetch_add(&p.xcnt[ci * XCNT_STRIDE], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)
                 : __hip_atomic_fetch_add(&p.fcnt[ci], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          s_last = (old + 1u) % (unsigned)S == 0u ? 1u : 0u;
        }
        __syncthreads();
        last = s_last != 0u;
      }
      if (last && wv < nt * 4) {
        const float* part = WHICH == G_O ? p.part_o : p.part_d;
        const auto pr = rsrc(part);
        // the other splits' sums sit in this XCD's L2; lines this compute
        // unit's L1 kept from earlier reads of the buffer are dropped first
        if (xl && S > 1) asm volatile("buffer_inv sc0" ::: "memory");
        floatx4 sum = {0, 0, 0, 0};
        for (int s0 = 0; s0 < S; s0 += 8) {
          u32x4 pv[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint32_t off = (uint32_t)((((size_t)(s0 + j) * p.M + gm) * W + c) * 4);
            const bool ok = mine && s0 + j < S && s0 + j != s;
            pv[j] = xl ? ld16_if(pr, off, ok) : coh_ld16_if(pr, off, ok);
          }
          // splits added in their fixed order whichever arrived last
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (s0 + j < S) sum += s0 + j == s ? v : as_f4(pv[j]);
        }
        const floatx4 hn = h0 + gt * sum;
        float sq = hn.x * hn.x + hn.y * hn.y + hn.z * hn.z + hn.w * hn.w;
        sq += __shfl_xor(sq, 16);
        sq += __shfl_xor(sq, 32);
        if (mine) {
          coh_st16(p.h, (uint32_t)(((size_t)gm * W + c) * 4), as_u4(hn));
          uint8_t* dsl = WHICH == G_O ? sl : slab(p, step, layer + 1);
          store_gemm_in4<T, false>(p, dsl + (WHICH == G_O ? p.off_xnm : p.off_xna), gm, c, hn * (1.0f + sc), 1.0f);
          if (g == 0)
            coh_st4(dsl + (WHICH == G_O ? p.off_ssm : p.off_ssa), (uint32_t)(((size_t)gm * (W / 16) + c / 16) * 4),
                    __builtin_bit_cast(uint32_t, sq));
        }
      }
    }
    if (WHICH == G_QKV && (FUSE || arrive)) {
      // no barrier between qkv and attention (the persistent kernel's merged
      // attention): once its outputs are stored, the unit adds its tiles to
      // the counter of their head (q), or of their key / value head (k and v
      // share one)
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) {
        const int head = (t0 * 16) / p.d;   // the nt tiles of a unit lie in one head
        const int ci = head < p.Hq ? head : QCNT_KV + (head - p.Hq) % p.Hkv;
        __hip_atomic_fetch_add(&p.qcnt[ci * HCNT_STRIDE], (unsigned)nt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if constexpr (CAL) {
    // calibration: the largest |activation| this workgroup loaded, per GEMM input
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    if (lane == 0 && amax > 0.f)
      __hip_atomic_fetch_max(reinterpret_cast<unsigned*>(p.amax) + layer * 4 + WHICH, __builtin_bit_cast(unsigned, amax),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ============================================================ attention
// Flash-style attention of one query head over keys [s0, s1) of
// [prefix (P) ; chunk (H)], at most 64 keys. Work unit = (sample b, query
// head j, key split c), one per workgroup. Each wave owns 16 query rows,
// kept in registers as MFMA operands; the split's K (row-major) and V
// (transposed) are staged in LDS with every load issued up front. The two
// groups of 4 waves both compute the scores (cheap) and each applies P to
// half of the head dims, so a workgroup reads K and V once.
// Scores are computed transposed, S^T = K Q^T, so a lane holds 8 keys of one
// query and the row max / sum need only two cross-lane exchanges; the
// probabilities then feed the PV MFMA directly from registers.
constexpr int ATT_KEYS = ATT_KEYS_HOST;   // keys per split

template <typename T, int D, int MODE>   // MODE 0: prefix keys, 1: the chunk's own keys
__device__ __forceinline__ void attn_load_kv(const VP& p, int tid, int b, int kvh, int s0, int s1,
                                             __amdgpu_buffer_rsrc_t pkr, __amdgpu_buffer_rsrc_t pvr,
                                             __amdgpu_buffer_rsrc_t kgr, __amdgpu_buffer_rsrc_t vgr,
                                             u32x4* kreg, u32x4* vreg) {
  constexpr int EPC = 16 / (int)sizeof(T), CPR = D / EPC;
  constexpr int LOADS = ATT_KEYS * CPR / NTH;
  const int P = p.P;
  const int hbase = (b * p.Hkv + kvh) * D * 64;                 // chunk k/v block of this head
  const int pstride = p.Hkv * D;                                // elements between prefix keys
  const int pbase = ((b * P + s0) * p.Hkv + kvh) * D;           // prefix key s0
  // K: a wave covers whole key rows; V: a wave covers one dim chunk of 64 keys
  const int kk0 = tid / CPR, ke0 = (tid % CPR) * EPC;
  const int ktt = ke0 < D / 2 ? ke0 / 8 : (ke0 - D / 2) / 8;
  const int kpos = ke0 < D / 2 ? ke0 % 8 : 8 + (ke0 - D / 2) % 8;
  const int vkk = tid % ATT_KEYS, ve00 = (tid / ATT_KEYS) * EPC;
#pragma unroll
  for (int j = 0; j < LOADS; ++j) {
    const int kk = kk0 + j * (NTH / CPR), s = s0 + kk;
    const int ve0 = ve00 + j * (NTH / ATT_KEYS) * EPC, vs = s0 + vkk;
    const uint32_t kpo = (uint32_t)((pbase + kk * pstride + ke0) * (int)sizeof(T));
    const uint32_t vpo = (uint32_t)((pbase + vkk * pstride + ve0) * (int)sizeof(T));
    const uint32_t kco = (uint32_t)((hbase + (ktt * 64 + (s - P)) * 16 + kpos) * (int)sizeof(T));
    const uint32_t vco = (uint32_t)((hbase + ((ve0 / 16) * 64 + (vs - P)) * 16 + ve0 % 16) * (int)sizeof(T));
    if constexpr (MODE == 0) {
      kreg[j] = ld16_if(pkr, kpo, s < s1);
      vreg[j] = ld16_if(pvr, vpo, vs < s1);
    } else {
      kreg[j] = ld16_if(kgr, kco, s < s1);
      vreg[j] = ld16_if(vgr, vco, vs < s1);
    }
  }
}

// K/V fragments of a workgroup's first attention unit when its keys all lie
// in the prefix: they depend on nothing computed in this call, so the
// persistent kernel loads them while the workgroup waits at the barrier
// before the attention phase.
template <typename T, int D>
struct APre {
  static constexpr int LOADS = ATT_KEYS * (D / (16 / (int)sizeof(T))) / NTH;
  u32x4 k[LOADS], v[LOADS];
};

// Key range [s0, s1) of split c: the prefix keys in splits of ATT_KEYS, then
// the chunk's own keys in splits of their own, so that only the chunk
// splits depend on the projection phase just before attention.
__device__ __forceinline__ void attn_split(const VP& p, int c, int& s0, int& s1) {
  const int KSp = (p.P + ATT_KEYS - 1) / ATT_KEYS;
  if (c < KSp) {
    s0 = c * ATT_KEYS;
    s1 = min(p.P, s0 + ATT_KEYS);
  } else {
    s0 = p.P + (c - KSp) * ATT_KEYS;
    s1 = min(p.P + p.H, s0 + ATT_KEYS);
  }
}

// Attention unit of grid slot v: (sample x head bh, split c); false past
// the last unit. Plain order v = bh KS + c. XCD order (xl: the grid a
// multiple of 8, workgroup w on XCD w % 8): head bh's splits run on XCD
// bh % 8, v = bh % 8 + 8 ((bh / 8) KS + c), so that the merge of its splits
// (ph_combine, same placement) reads them from that XCD's L2.
__device__ __forceinline__ bool attn_unit(const VP& p, int v, bool xl, int& bh, int& c) {
  const int KS = p.KS, nbh = p.B * p.Hq;
  if (!xl) {
    bh = v / KS;
    c = v % KS;
    return bh < nbh;
  }
  const int r = v >> 3;
  bh = (r / KS) * 8 + (v & 7);
  c = r % KS;
  return bh < nbh;
}
__device__ __forceinline__ int attn_slots(const VP& p, bool xl) {
  const int nbh = p.B * p.Hq;
  return (xl ? (nbh + 7) / 8 * 8 : nbh) * p.KS;
}

template <typename T, int D>
__device__ __forceinline__ bool attn_prefix_unit(const VP& p, int v, bool xl, int& b, int& kvh, int& s0, int& s1) {
  int bh, c;
  if (v >= attn_slots(p, xl) || !attn_unit(p, v, xl, bh, c)) return false;
  const int jh = bh % p.Hq;
  b = bh / p.Hq;
  kvh = jh / (p.Hq / p.Hkv);
  attn_split(p, c, s0, s1);
  return s1 <= p.P;
}

template <typename T, int D>
struct AttnPrefetchHook {
  const VP& p;
  int layer, wg;
  APre<T, D>& out;
  bool xl;
  __device__ __forceinline__ void operator()() const {
    const VP& p = vp_fresh();
    int b, kvh, s0, s1;
    if (!attn_prefix_unit<T, D>(p, wg, xl, b, kvh, s0, s1)) return;
    const size_t layer_elems = (size_t)p.B * p.P * p.Hkv * D;
    const auto pkr = rsrc(reinterpret_cast<const T*>(p.prefix_k) + (size_t)layer * layer_elems);
    const auto pvr = rsrc(reinterpret_cast<const T*>(p.prefix_v) + (size_t)layer * layer_elems);
    attn_load_kv<T, D, 0>(p, tid_opaque(), b, kvh, s0, s1, pkr, pvr, pkr, pvr, out.k, out.v);
  }
};

template <typename T, bool Q8>
__device__ __forceinline__ void combine_row(const VP& p, int layer, uint8_t* attn, int b, int jh, int i, int lane,
                                            bool xl);

// xl: XCD-ordered units (attn_unit) whose split outputs stay in the XCD's
// L2 (write-back stores) for the XCD-local merge.
// MERGE (the persistent kernel): the key splits of a head are merged in
// this phase instead of a combine phase behind a device-wide barrier, and
// each unit starts once its head's qkv tiles are stored (counters instead of
// the barrier after qkv). Each unit, once its split output is stored, adds 1 to its head's
// arrival counter (one 128-byte line per head, so that a head's arrivals and
// polls do not queue behind other heads'); after its last unit, a workgroup
// waits for each of its units' heads to have all KS splits and merges that
// unit's share of the head's query rows (rows c, c + KS, ...). Every arrival
// comes before any wait, so the waits cannot form a cycle. Returns false when
// a wait gave up.
template <typename T, int D, bool PRE = false, int WF = WF_NATIVE, bool MERGE = false>
__device__ __forceinline__ bool ph_attn(const VP&, int step, int layer, int wg, int nwg,
                                        const APre<T, D>& pre = APre<T, D>{}, bool xl = false) {
  const VP& p = vp_fresh();
  const int tid = tid_opaque();
  constexpr int E = MT<T>::E, KB = MT<T>::KB;
  constexpr int EPC = 16 / (int)sizeof(T);          // elements per 16-byte chunk
  constexpr int LDK = D + EPC;                       // padded K row (elements)
  constexpr int LDV = ATT_KEYS + EPC;                // padded V^T row (elements)
  constexpr int CPR = D / EPC;                       // 16-byte chunks per key row
  constexpr int LOADS = ATT_KEYS * CPR / NTH;        // K (and V) chunks per thread
  constexpr int DT = D / 32;                         // dim tiles per group
  T* Ks = reinterpret_cast<T*>(smem);                // [64][LDK]
  T* Vt = Ks + ATT_KEYS * LDK;                       // [D][LDV]
  const int grp = tid >> 8, gtid = tid & 255;
  const int lane = tid & 63, wv = gtid >> 6, g = lane >> 4, c16 = lane & 15;
  const int H = p.H, P = p.P, KS = p.KS;
  const int group = p.Hq / p.Hkv;
  const int slots = attn_slots(p, xl);
  const float scale = 1.4426950408889634f / sqrtf((float)D);   // log2(e) / sqrt(d)
  const size_t layer_elems = (size_t)p.B * P * p.Hkv * D;
  const auto pkr = rsrc(reinterpret_cast<const T*>(p.prefix_k) + (size_t)layer * layer_elems);
  const auto pvr = rsrc(reinterpret_cast<const T*>(p.prefix_v) + (size_t)layer * layer_elems);
  const uint8_t* sl = slab(p, step, layer);
  const auto qrs = rsrc(sl + p.off_q), kgr = rsrc(sl + p.off_k), vgr = rsrc(sl + p.off_v);
  for (int u = wg; u < slots; u += nwg) {
    int bh, c;
    if (!attn_unit(p, u, xl, bh, c)) continue;   // the same for the whole workgroup
    const int jh = bh % p.Hq, b = bh / p.Hq;
    const int kvh = jh / group;
    int s0, s1;
    attn_split(p, c, s0, s1);
    if constexpr (MERGE) {
      // no barrier after qkv: wait for this head's query tiles (every
      // 64-row tile), and for a split of the chunk's own keys also for its
      // key / value head's tiles
      const unsigned inst = (unsigned)(step * p.L + layer + 1), mtl = (unsigned)((p.M + 63) / 64);
      if (!counter_wait(&p.qcnt[jh * HCNT_STRIDE], inst * (unsigned)(D / 16) * mtl, p.bar, p.spin_limit, p.herr))
        return false;
      if (s1 > P && !counter_wait(&p.qcnt[(QCNT_KV + kvh) * HCNT_STRIDE], inst * (unsigned)(2 * D / 16) * mtl, p.bar,
                                  p.spin_limit, p.herr))
        return false;
    }
    const int qrow = wv * 16 + c16;
    const bool active = wv * 16 < H;
    // query fragments (B operand of S^T): Q[qrow][kb*KB + g*E .. +E]; the
    // permuted q/k tile layout keeps each 16-byte chunk contiguous
    u32x4 qf[D / KB];
    {
      const int qbase = (b * p.Hq + jh) * D * 64;
      const bool ok = active && qrow < H;
#pragma unroll
      for (int kb = 0; kb < D / KB; ++kb) {
        const int e = kb * KB + g * E;
        const int tt = e < D / 2 ? e / 8 : (e - D / 2) / 8, pos = e < D / 2 ? e % 8 : 8 + (e - D / 2) % 8;
        qf[kb] = ld16_if(qrs, (uint32_t)((qbase + (tt * 64 + qrow) * 16 + pos) * (int)sizeof(T)), ok);
      }
    }
    u32x4 kreg[LOADS], vreg[LOADS];
    if (PRE && u == wg && s1 <= P) {
#pragma unroll
      for (int j = 0; j < LOADS; ++j) { kreg[j] = pre.k[j]; vreg[j] = pre.v[j]; }
    } else if (s1 <= P) attn_load_kv<T, D, 0>(p, tid, b, kvh, s0, s1, pkr, pvr, kgr, vgr, kreg, vreg);
    else attn_load_kv<T, D, 1>(p, tid, b, kvh, s0, s1, pkr, pvr, kgr, vgr, kreg, vreg);
    __syncthreads();   // the previous unit's LDS reads are done
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int idx = tid + j * NTH;
      *reinterpret_cast<u32x4*>(Ks + (idx / CPR) * LDK + (idx % CPR) * EPC) = kreg[j];
      const int kk = idx % ATT_KEYS, e0 = (idx / ATT_KEYS) * EPC;
      const T* ve = reinterpret_cast<const T*>(&vreg[j]);
#pragma unroll
      for (int e = 0; e < EPC; ++e) Vt[(e0 + e) * LDV + kk] = ve[e];
    }
    __syncthreads();
    if (active) {
    float m_run = -INFINITY, l_run = 0.f;
    floatx4 O[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) O[dt] = floatx4{0, 0, 0, 0};
    const int dbase = grp * (D / 2);
#pragma unroll
    for (int ci = 0; ci < ATT_KEYS / 32; ++ci) {
      const int sc = s0 + ci * 32;
      if (sc >= s1) break;
      floatx4 slo = {0, 0, 0, 0}, shi = {0, 0, 0, 0};
      constexpr int KH = D / KB < 4 ? D / KB : 4;     // K fragments read ahead per batch
#pragma unroll
      for (int k0 = 0; k0 < D / KB; k0 += KH) {
        u32x4 alo[KH], ahi[KH];
#pragma unroll
        for (int kb = 0; kb < KH; ++kb) {
          alo[kb] = *reinterpret_cast<const u32x4*>(Ks + (ci * 32 + c16) * LDK + (k0 + kb) * KB + g * E);
          ahi[kb] = *reinterpret_cast<const u32x4*>(Ks + (ci * 32 + 16 + c16) * LDK + (k0 + kb) * KB + g * E);
        }
#pragma unroll
        for (int kb = 0; kb < KH; ++kb) {
          slo = MT<T>::mma(alo[kb], qf[k0 + kb], slo);
          shi = MT<T>::mma(ahi[kb], qf[k0 + kb], shi);
        }
      }
      float pr[8];
      // pi0: the state token (query row 0) sees the prefix and its own key only
      const int lim = (p.pi0 && qrow == 0) ? min(s1, P + 1) : s1;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pr[r] = (sc + 4 * g + r < lim) ? slo[r] * scale : -INFINITY;
        pr[4 + r] = (sc + 16 + 4 * g + r < lim) ? shi[r] * scale : -INFINITY;
      }
      float cmax = pr[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) cmax = fmaxf(cmax, pr[e]);
      cmax = am_max4(cmax);
      const float m_new = fmaxf(m_run, cmax);
      const float alpha = fast_exp2(m_run - m_new);
      // l_run: this lane's share of the row sum, reduced after the last chunk
      l_run *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) { pr[e] = fast_exp2(pr[e] - m_new); l_run += pr[e]; }
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) O[dt] *= alpha;
      // PV on this group's dims: key order of the k slots is
      // (4g..4g+3, 16+4g..16+4g+3) for both operands
      if constexpr (sizeof(T) == 2) {
        bf16x8 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = (bf16)pr[e];
        const u32x4 pbu = __builtin_bit_cast(u32x4, pb);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const T* vr = Vt + (dbase + dt * 16 + c16) * LDV + ci * 32;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vr + 4 * g);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vr + 16 + 4 * g);
          O[dt] = MT<T>::mma(u32x4{lo.x, lo.y, hi.x, hi.y}, pbu, O[dt]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int key = ci * 32 + (e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4));
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
            O[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(to_f(Vt[(dbase + dt * 16 + c16) * LDV + key]), pr[e], O[dt], 0, 0, 0);
        }
      }
    }
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    if (qrow < H) {
      const size_t base = ((size_t)(b * p.Hq + jh) * KS + c) * 64 + qrow;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const size_t e0 = base * D + dbase + dt * 16 + 4 * g;
        if constexpr (sizeof(T) == 4) {
          if (xl) wb_st16(p.opart, (uint32_t)(e0 * 4), as_u4(O[dt]));
          else coh_st16(p.opart, (uint32_t)(e0 * 4), as_u4(O[dt]));
        } else {
          const u32x2 ov = {pack_bf16x2(O[dt][0], O[dt][1]), pack_bf16x2(O[dt][2], O[dt][3])};
          if (xl) wb_st8(p.opart, (uint32_t)(e0 * 2), ov);
          else coh_st8(p.opart, (uint32_t)(e0 * 2), ov);
        }
      }
      if (g == 0 && grp == 0) {
        const u32x2 mlv = {__builtin_bit_cast(uint32_t, m_run), __builtin_bit_cast(uint32_t, l_run)};
        if (xl) wb_st8(p.ml, (uint32_t)(base * 8), mlv);
        else coh_st8(p.ml, (uint32_t)(base * 8), mlv);
      }
    }
    }   // active
    if constexpr (MERGE) {
      __builtin_amdgcn_s_waitcnt(0);   // this wave's split output is stored
      __syncthreads();
      if (tid == 0)
        __hip_atomic_fetch_add(&p.hcnt[bh * HCNT_STRIDE], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if constexpr (MERGE) {
    // the counters count every arrival of the launch: this layer's target is
    // KS times the number of (step, layer) instances so far
    const unsigned target = (unsigned)((step * p.L + layer + 1) * KS);
    uint8_t* attn = slab(p, step, layer) + p.off_attn;
    const int wv8 = tid >> 6;
    for (int u = wg; u < slots; u += nwg) {
      int bh, c;
      if (!attn_unit(p, u, xl, bh, c)) continue;
      if (!counter_wait(&p.hcnt[bh * HCNT_STRIDE], target, p.bar, p.spin_limit, p.herr)) return false;
      if (xl) asm volatile("buffer_inv sc0" ::: "memory");
      for (int i = c + wv8 * KS; i < H; i += NWAVES * KS)
        combine_row<T, act_fp8<WF>()>(p, layer, attn, bh / p.Hq, bh % p.Hq, i, lane, xl);
    }
  }
  return true;
}

// Merge the key splits of query row i of head jh (sample b), one wave:
// attn[b*H+i][jh*d + dd] = sum_c w_c O_c / sum_c w_c l_c, w_c = 2^(m_c - max m).
// Lane c first fetches split c's (max, sum), then every lane merges four
// head dims over all splits. xl: the splits were stored on this XCD and are
// read from its L2 with ordinary loads (the caller has invalidated its L1);
// else from the coherence point.
template <typename T, bool Q8>
__device__ __forceinline__ void combine_row(const VP& p, int layer, uint8_t* attn, int b, int jh, int i, int lane,
                                            bool xl) {
  const int D = p.d, KS = p.KS;
  const int gm = b * p.H + i;
  const size_t base0 = ((size_t)(b * p.Hq + jh) * KS) * 64 + i;
  if constexpr (sizeof(T) == 2) {
    if (D <= 256 && KS <= 16) {
      // one round trip: each lane's four dims of every split are requested
      // together with the splits' (max, sum) pairs
      const auto opr = rsrc(p.opart);
      const int d4 = lane;
      u32x2 ov[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t oo = (uint32_t)(((base0 + (size_t)j * 64) * D + d4 * 4) * 2);
        const bool ok = j < KS && d4 < D / 4;
        ov[j] = xl ? ld8_if(opr, oo, ok) : coh_ld8_if(opr, oo, ok);
      }
      const uint32_t mo = (uint32_t)((base0 + (size_t)lane * 64) * 8);
      const floatx2 ml = __builtin_bit_cast(floatx2, xl ? ld8_if(rsrc(p.ml), mo, lane < KS) : coh_ld8_if(rsrc(p.ml), mo, lane < KS));
      const float mc = lane < KS ? ml[0] : -INFINITY, lc = lane < KS ? ml[1] : 0.f;
      float mx = mc;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      const float wc = lane < KS ? fast_exp2(mc - mx) : 0.f;
      const float den = warp_sum(wc * lc);
      floatx4 num = {0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const floatx4 f = {__builtin_bit_cast(float, ov[j][0] << 16), __builtin_bit_cast(float, ov[j][0] & 0xffff0000u),
                           __builtin_bit_cast(float, ov[j][1] << 16), __builtin_bit_cast(float, ov[j][1] & 0xffff0000u)};
        num += __shfl(wc, j) * f;
      }
      if (d4 < D / 4) store_gemm_in4<T, Q8>(p, attn, gm, jh * D + d4 * 4, num / den, Q8 ? act_inv(p, layer, 1) : 1.0f);
      return;
    }
  }
  float mc = -INFINITY, lc = 0.f;
  if (lane < KS) {
    const uint32_t mo = (uint32_t)((base0 + (size_t)lane * 64) * 8);
    const floatx2 ml = __builtin_bit_cast(floatx2, xl ? ld8_if(rsrc(p.ml), mo, true) : coh_ld8(p.ml, mo));
    mc = ml[0];
    lc = ml[1];
  }
  float mx = mc;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  const float wc = lane < KS ? fast_exp2(mc - mx) : 0.f;
  const float den = warp_sum(wc * lc);
  const auto opr = rsrc(p.opart);
  for (int d4 = lane; d4 < D / 4; d4 += 64) {
    floatx4 num = {0, 0, 0, 0};
    for (int c0 = 0; c0 < KS; c0 += 16) {
      if constexpr (sizeof(T) == 4) {
        u32x4 ov[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const uint32_t oo = (uint32_t)(((base0 + (size_t)(c0 + j) * 64) * D + d4 * 4) * 4);
          ov[j] = xl ? ld16_if(opr, oo, c0 + j < KS) : coh_ld16_if(opr, oo, c0 + j < KS);
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) num += __shfl(wc, (c0 + j) & 63) * as_f4(ov[j]);
      } else {
        u32x2 ov[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const uint32_t oo = (uint32_t)(((base0 + (size_t)(c0 + j) * 64) * D + d4 * 4) * 2);
          ov[j] = xl ? ld8_if(opr, oo, c0 + j < KS) : coh_ld8_if(opr, oo, c0 + j < KS);
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const floatx4 f = {__builtin_bit_cast(float, ov[j][0] << 16), __builtin_bit_cast(float, ov[j][0] & 0xffff0000u),
                             __builtin_bit_cast(float, ov[j][1] << 16), __builtin_bit_cast(float, ov[j][1] & 0xffff0000u)};
          num += __shfl(wc, (c0 + j) & 63) * f;
        }
      }
    }
    const floatx4 o = num / den;
    store_gemm_in4<T, Q8>(p, attn, gm, jh * D + d4 * 4, o, Q8 ? act_inv(p, layer, 1) : 1.0f);
  }
}

// Merge phase: one wave per (row, head) item.
// xl: the rows of head bh are merged on XCD bh % 8, where attn_unit placed
// its splits: their outputs are read from that XCD's L2 (ordinary loads
// after this compute unit's L1 is invalidated) instead of from memory.
template <typename T, int WF = 0>
__device__ __forceinline__ void ph_combine(const VP&, int step, int layer, int wg, int nwg, bool xl = false) {
  const VP& p = vp_fresh();
  constexpr bool Q8 = act_fp8<WF>();
  const int tid = tid_opaque();
  const int lane = tid & 63, wv = tid >> 6;
  // item order: plain (row gm, head jh) = it / Hq, it % Hq over every wave of
  // the grid; XCD-local: the waves of XCD x take (head 8 q + x, row i) = it / H, it % H
  const int nbh = p.B * p.Hq, x = wg & 7;
  const int items = xl ? (nbh > x ? (nbh - x + 7) / 8 : 0) * p.H : p.M * p.Hq;
  const int it0 = xl ? (wg >> 3) * NWAVES + wv : wg * NWAVES + wv;
  const int its = xl ? (nwg >> 3) * NWAVES : nwg * NWAVES;
  if (xl) asm volatile("buffer_inv sc0" ::: "memory");
  uint8_t* attn = slab(p, step, layer) + p.off_attn;
  for (int it = it0; it < items; it += its) {
    int jh, b, i;
    if (xl) {
      const int bh = (it / p.H) * 8 + x;
      jh = bh % p.Hq;
      b = bh / p.Hq;
      i = it % p.H;
    } else {
      jh = it % p.Hq;
      b = (it / p.Hq) / p.H;
      i = (it / p.Hq) % p.H;
    }
    combine_row<T, Q8>(p, layer, attn, b, jh, i, lane, xl);
  }
}

// ============================================================ large-M GEMM
// For many tokens (a batch of samples) the skinny GEMM above re-reads every
// weight slice once per 64-token tile. In the graph and eager launch modes a
// bf16 expert with M >= 256 rows runs its GEMM phases with this kernel
// instead: 128 output columns x 128 tokens per workgroup (4 waves of 64 x 64,
// 16x16x32 bf16 MFMA), both operand tiles staged through LDS in the packed
// lane order, double-buffered with the next stage's global loads in flight,
// and the same epilogues (RoPE into the q/k/v tiles, GeGLU into the
// activation operand, K-split partial sums) as the skinny GEMM. The
// activation tile comes from the operand order [K/32][Mpad][32], whose
// 16-token x 32-K block is 1 KiB with lane (c, g) at c * 64 + g * 16 bytes;
// the LDS store moves it to lane order (g * 16 + c) so that every LDS read
// is one contiguous 1 KiB.
constexpr int GM_THREADS = 256;
constexpr int GM_LDS = 2 * 32768;   // two stages of (A tile + B tile)

// One 16 x 16 accumulator tile of a large-M GEMM: this lane's four columns
// 16 tile + 4g .. +3 of token gm (the MFMA output layout), through the
// GEMM's epilogue: RoPE into the q / k tiles (v as is), GeGLU into the
// down projection's operand, or the K split's partial sums. These GEMMs
// run as launches of their own, so their results take write-back stores.
template <typename T, int WHICH>
__device__ __forceinline__ void gemm_m_store(const VP& p, uint8_t* sl, int tile, int gm, int s, int g, floatx4 vv) {
  if (WHICH == G_QKV) {
    const int d = p.d;
    const int col0 = tile * 16;
    const int head = col0 / d, tt = (col0 % d) / 16;
    const int b = gm / p.H, ti = gm % p.H;
    if (head < p.Hq + p.Hkv) {
      const int j0 = tt * 8 + 2 * g;
      const floatx4 rot = as_f4(ro_ld16(p.rope + ((size_t)ti * (d / 2) + j0) * 2));
      const float y0 = vv.x * rot[0] - vv.z * rot[1], y0h = vv.z * rot[0] + vv.x * rot[1];
      const float y1 = vv.y * rot[2] - vv.w * rot[3], y1h = vv.w * rot[2] + vv.y * rot[3];
      const bool isq = head < p.Hq;
      uint8_t* dst = sl + (isq ? p.off_q : p.off_k);
      const size_t hb = isq ? (size_t)b * p.Hq + head : (size_t)b * p.Hkv + (head - p.Hq);
      const size_t e0 = ((hb * (d / 16) + tt) * 64 + ti) * 16 + 2 * g;
      wb_st4(dst, (uint32_t)(e0 * 2), pack_bf16x2(y0, y1));
      wb_st4(dst, (uint32_t)((e0 + 8) * 2), pack_bf16x2(y0h, y1h));
    } else {
      const int kvh = head - p.Hq - p.Hkv;
      const size_t e0 = ((((size_t)b * p.Hkv + kvh) * (d / 16) + tt) * 64 + ti) * 16 + 4 * g;
      wb_st8(sl + p.off_v, (uint32_t)(e0 * 2), u32x2{pack_bf16x2(vv.x, vv.y), pack_bf16x2(vv.z, vv.w)});
    }
  } else if (WHICH == G_GU) {
    const int f0 = tile * 8 + 2 * g;
    const float a0 = gelu_tanh(vv.x) * vv.y, a1 = gelu_tanh(vv.z) * vv.w;
    wb_st4(sl + p.off_act, (uint32_t)(act_off<T>(p, gm, f0) * 2), pack_bf16x2(a0, a1));
  } else {
    float* part = WHICH == G_O ? p.part_o : p.part_d;
    const int n0 = tile * 16 + 4 * g;
    wb_st16(part, (uint32_t)((((size_t)s * p.M + gm) * p.W + n0) * 4), as_u4(vv));
  }
}

// BM: tokens per tile, 128 or 64 (a 64-token tile where 128-token tiles
// would leave a few compute units with a second tile: waves then take 64
// columns x 32 tokens).
template <typename T, int WHICH, int BM>
__global__ __launch_bounds__(GM_THREADS, 2) void k_gemm_m(VP p, int step, int layer) {
  static_assert(sizeof(T) == 2, "the large-M GEMM runs bf16 operands");
  static_assert(BM == 128 || BM == 64, "token tile of 128 or 64");
  constexpr int NJ = BM / 32;   // 16-token blocks per wave; also B chunks per thread
  uint8_t* lds = reinterpret_cast<uint8_t*>(smem);
  const GemmShape gs = gemm_shape<T, WHICH, WF_NATIVE>(p, layer);
  const int K = gs.K, N = gs.N, S = gs.S;
  const int Mpad = ((p.M + 63) / 64) * 64;
  const int MTL = (p.M + BM - 1) / BM, NTL = N / 128, total = MTL * NTL * S;
  const int per = (total + 7) >> 3;
  const int v = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (v >= total) return;
  const int mt = v % MTL, nt = (v / MTL) % NTL, s = v / (MTL * NTL);
  const int KB32 = K >> 5, Ks = K / S, nk = Ks / 64, kb0 = (s * Ks) >> 5;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wn = w >> 1, wm = w & 1;
  uint8_t* sl = slab(p, step, layer);
  const uint8_t* act;
  if (WHICH == G_QKV) act = sl + p.off_xna;
  else if (WHICH == G_O) act = sl + p.off_attn;
  else if (WHICH == G_GU) act = sl + p.off_xnm;
  else if (WHICH == G_DOWN) act = sl + p.off_act;
  else act = sl + p.off_u;
  const __amdgpu_buffer_rsrc_t ra = rsrc(gs.Wp), rb = rsrc(act);
  uint32_t aoff[4], boff[4];
  int bdst[4];
  bool bok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i, blk = c >> 7, rest = c & 127;
    aoff[i] = (uint32_t)(((nt * 8 + blk) * KB32 + kb0) * 1024 + rest * 16);
    const int kk = rest >> 6, u = rest & 63;
    const int m = mt * BM + blk * 16 + (u >> 2);
    bok[i] = m < Mpad && i < NJ;
    boff[i] = (uint32_t)((((kb0 + kk) * Mpad + m) * 32 + (u & 3) * 8) * 2);
    bdst[i] = (blk * 2 + kk) * 64 + (u & 3) * 16 + (u >> 2);
  }
  const uint32_t bstep = (uint32_t)(2 * Mpad * 64);   // two 32-K blocks of activations
  u32x4 ga[4], gb[4];
  auto gload = [&](int it) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ga[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, aoff[i] + (uint32_t)it * 2048u, 0, 0);
      if (i < NJ) gb[i] = ld16_if(rb, boff[i] + (uint32_t)it * bstep, bok[i]);
    }
  };
  auto lstore = [&](int buf) {
    u32x4* A = reinterpret_cast<u32x4*>(lds + buf * (GM_LDS / 2));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      A[tid + 256 * i] = ga[i];
      if (i < NJ) A[1024 + bdst[i]] = gb[i];
    }
  };
  floatx4 acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  gload(0);
  lstore(0);
  __syncthreads();
  for (int it = 0; it < nk; ++it) {
    if (it + 1 < nk) gload(it + 1);
    const u32x4* A = reinterpret_cast<const u32x4*>(lds + (it & 1) * (GM_LDS / 2));
    const u32x4* B = A + 1024;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      u32x4 a[4], b[NJ];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = A[(wn * 4 + i) * 128 + kb * 64 + lane];
#pragma unroll
      for (int j = 0; j < NJ; ++j) b[j] = B[(wm * NJ + j) * 128 + kb * 64 + lane];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = MT<T>::mma(a[i], b[j], acc[i][j]);
    }
    if (it + 1 < nk) lstore((it + 1) & 1);
    __syncthreads();
  }
  // epilogue: lane holds rows 4g..4g+3 of 16-column tile `tile` for token gm
  const int g = lane >> 4, c16 = lane & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tile = nt * 8 + wn * 4 + i;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int gm = mt * BM + wm * (BM / 2) + j * 16 + c16;
      if (gm < p.M) gemm_m_store<T, WHICH>(p, sl, tile, gm, s, g, acc[i][j]);
    }
  }
}

// ============================================================ wide large-M GEMM
// The tiles above stage 32 KB of operands through registers into LDS per
// 64-K step and read 16 KB of it back per wave for 32 MFMAs, so the vector
// memory, LDS and MFMA pipes each need about the same cycles and the single
// stage in flight leaves the load latency exposed. The 256-column tiles of
// vfm_gemm_wide.h (one workgroup per compute unit, a 5-stage direct-to-LDS
// ring) run gate/up by default; the activation operand's token blocks come
// from [K/32][Mpad][32] and are permuted to the MFMA lane order by the
// copies' per-lane addresses.
static_assert(GW<7>::NS == GW_RING_224 && GW<8>::NS == GW_RING_256, "ring depths known to the planner");

// One wave per SIMD (the LDS ring takes the compute unit): the scheduler is
// told so, or it trades latency hiding for registers it cannot use.
template <typename T, int WHICH, int MB>
__global__ __launch_bounds__(GW_THREADS, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_w(VP p, int step,
                                                                                                     int layer) {
  static_assert(sizeof(T) == 2, "the wide large-M GEMM runs bf16 operands");
  using C = GW<MB>;
  const GemmShape gs = gemm_shape<T, WHICH, WF_NATIVE>(p, layer);
  const int K = gs.K, N = gs.N, S = gs.S;
  const int Mpad = ((p.M + 63) / 64) * 64;
  const int MTL = (p.M + C::BMT - 1) / C::BMT, NTL = N / 256, total = MTL * NTL * S;
  const int per = (total + 7) >> 3;
  const int v = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (v >= total) return;
  const int mt = v % MTL, nt = (v / MTL) % NTL, s = v / (MTL * NTL);
  const int KB32 = K >> 5, nst = (K / S) >> 5, kb0 = s * nst;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), wn = w & 1, wm = w >> 1;
  uint8_t* sl = slab(p, step, layer);
  const uint8_t* act;
  if (WHICH == G_QKV) act = sl + p.off_xna;
  else if (WHICH == G_O) act = sl + p.off_attn;
  else if (WHICH == G_GU) act = sl + p.off_xnm;
  else if (WHICH == G_DOWN) act = sl + p.off_act;
  else act = sl + p.off_u;
  // this wave's copies per stage: blocks w + 4i; i < 4 are weight column tiles
  // nt * 16 + w + 4i, the rest token blocks j = w + 4 (i - 4) (16 tokens, rows
  // past the padded count read its last row; their outputs are dropped). The
  // LDS block of copy i is w + 4i either way. A token block goes to LDS in
  // lane order: lane (c, g) (c = lane & 15) takes token c's K-group g.
  uint32_t voff[C::CW];
#pragma unroll
  for (int i = 0; i < C::CW; ++i) {
    if (i < 4) {
      voff[i] = (uint32_t)(((nt * 16 + w + 4 * i) * KB32 + kb0) * 1024 + lane * 16);
    } else {
      const int j = w + 4 * (i - 4);
      int m = mt * C::BMT + j * 16 + (lane & 15);
      m = m < Mpad ? m : Mpad - 1;
      voff[i] = (uint32_t)((((size_t)kb0 * Mpad + m) * 32 + (lane >> 4) * 8) * 2);
    }
  }
  floatx4 acc[8][MB];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  gw_mainloop<MB>(acc, reinterpret_cast<uint8_t*>(smem), gs.Wp, act, voff, (uint32_t)(Mpad * 64), nst, w, lane);

  const int g = lane >> 4, c16 = lane & 15;
  if constexpr (WHICH == G_GU || WHICH == G_QKV) {
    // Epilogues that compute on the sums (GeGLU, RoPE) take them back from
    // LDS, half a wave tile at a time: computing on them in place leads the
    // register allocator to keep the accumulators in ordinary registers (the
    // loop's operands then spill), and GeGLU reads them back transposed for
    // whole-row stores. The ring is free once every wave is past this
    // barrier (all copies have landed: each wave waited for its own).
    gw_barrier();
    floatx4* E = reinterpret_cast<floatx4*>(smem + w * (4 * MB * 1024));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < MB; ++j) E[(i * MB + j) * 64 + lane] = acc[4 * h + i][j];
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if constexpr (WHICH == G_GU) {
        // Read back transposed: lane (token c, tile il of the four) takes
        // all 16 sums of its token in that tile (the four 16-byte pieces of
        // lanes (c, 0..3)), i.e. gate and up of 8 consecutive features, and
        // stores their 8 GeGLU values as one 16-byte piece; the four tiles
        // of a token are one 64-byte row of the down projection's operand,
        // so each store writes 16 whole rows.
        // Rows past the batch get an offset beyond the buffer range, which
        // drops the store: the code stays one block, so the reads are all
        // issued before the first GeGLU.
        const int c = lane & 15, il = lane >> 4;
        const int f0 = (nt * 16 + wn * 8 + 4 * h + il) * 8;
        floatx4 q[MB][4];
#pragma unroll
        for (int j = 0; j < MB; ++j)
#pragma unroll
          for (int gg = 0; gg < 4; ++gg) q[j][gg] = E[(il * MB + j) * 64 + gg * 16 + c];
#pragma unroll
        for (int j = 0; j < MB; ++j) {
          u32x4 y;
#pragma unroll
          for (int gg = 0; gg < 4; ++gg)
            y[gg] = pack_bf16x2(gelu_tanh(q[j][gg].x) * q[j][gg].y, gelu_tanh(q[j][gg].z) * q[j][gg].w);
          const int gm = mt * C::BMT + (wm * MB + j) * 16 + c;
          const uint32_t off = gm < p.M ? (uint32_t)(act_off<T>(p, gm, f0) * 2) : 0x80000000u;
          wb_st16(sl + p.off_act, off, y);
        }
      } else {
        floatx4 vq[4 * MB];
#pragma unroll
        for (int q = 0; q < 4 * MB; ++q) vq[q] = E[q * 64 + lane];
#pragma unroll
        for (int q = 0; q < 4 * MB; ++q) {
          const int i = q / MB, j = q % MB;
          const int tile = nt * 16 + wn * 8 + 4 * h + i;
          const int gm = mt * C::BMT + (wm * MB + j) * 16 + c16;
          if (gm < p.M) gemm_m_store<T, WHICH>(p, sl, tile, gm, s, g, vq[q]);
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int tile = nt * 16 + wn * 8 + i;
#pragma unroll
      for (int j = 0; j < MB; ++j) {
        const int gm = mt * C::BMT + (wm * MB + j) * 16 + c16;
        if (gm < p.M) gemm_m_store<T, WHICH>(p, sl, tile, gm, s, g, acc[i][j]);
      }
    }
  }
}

// ============================================================ large-batch attention
// With the large-M GEMMs (graph / eager launch, bf16, M >= 256 rows), the
// attention of a batch runs in one pass instead of key splits plus a combine
// phase: one workgroup per (sample, query head) takes the head's H queries
// (wave w: rows 16w .. 16w + 15) over all P + H keys with an online softmax
// (the flash-attention recurrence, R8's result) and writes the o
// projection's input itself. The chunk's own H keys and values are staged
// into LDS once; the prefix streams through two LDS stages of 32 keys, the
// next tile's global loads in flight during the current tile's MFMAs. K is
// kept in natural dim order, [key][D]; V as [key / 4][D][4 keys], so that a
// lane's operand of the P.V product (4 keys of one dim, twice) is two 8-byte
// LDS reads. The workgroups of one sample share an XCD (blockIdx % 8), so
// its keys and values come from HBM once and from that XCD's L2 for the
// other heads.
constexpr int AM_KEYS = 32;
constexpr int AM_GT = 256;              // threads of one tile group (4 waves, 16 query rows each)
constexpr int AM_THREADS = 2 * AM_GT;   // two groups take alternate prefix tiles
constexpr int AM_CHUNK = 64;   // chunk keys staged once (H <= 64)

template <int D>
struct AttnMLds {
  static constexpr int K_LD = D + 8;                  // elements per K row (16-byte pad)
  static constexpr int V_LD = D * 8 + 128;            // bytes per 4-key group: [D][4] bf16, shifts, pad
  static constexpr int K_TILE = AM_KEYS * K_LD * 2;
  static constexpr int STAGE = K_TILE + (AM_KEYS / 4) * V_LD;
  static constexpr int CK = 2 * STAGE;                // chunk K: [AM_CHUNK][K_LD]
  static constexpr int CV = CK + AM_CHUNK * K_LD * 2; // chunk V: [AM_CHUNK / 4][V_LD]
  static constexpr int TOTAL = CV + (AM_CHUNK / 4) * V_LD;
  static_assert((D - 1) * 8 + ((D - 1) / 32) * 8 + 8 <= V_LD, "V key group row too short for its shifts");
};

// Byte offset of dim e in a V key group ([D][4 keys] bf16): every 32 dims
// shift by 8 bytes, so that the 32 lanes storing dims 8c .. 8c + 7 of one
// group (c = 0 .. 31) hit distinct bank pairs instead of four.
__device__ __forceinline__ int am_v_off(int e) { return e * 8 + (e >> 5) * 8; }

// Transpose 4 keys x 8 dims (rows of natural-order bf16) into LDS as
// [key group][dim][4 keys]: dims 8c .. 8c + 7 of one key group.
__device__ __forceinline__ void am_store_v(uint8_t* grp, int c, const u32x4 (&row)[4]) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint32_t w0 = row[0][m], w1 = row[1][m], w2 = row[2][m], w3 = row[3][m];
    const u32x2 lo = {(w0 & 0xffffu) | (w1 << 16), (w2 & 0xffffu) | (w3 << 16)};
    const u32x2 hi = {(w0 >> 16) | (w1 & 0xffff0000u), (w2 >> 16) | (w3 & 0xffff0000u)};
    uint8_t* dst = grp + am_v_off(8 * c + 2 * m);   // dims 8c + 2m and 8c + 2m + 1 share the shift
    *reinterpret_cast<u32x2*>(dst) = lo;
    *reinterpret_cast<u32x2*>(dst + 8) = hi;
  }
}

template <typename T, int D>
__global__ __launch_bounds__(AM_THREADS, 1) void k_attn_m(VP p, int step, int layer) {
  static_assert(sizeof(T) == 2, "the large-batch attention runs bf16 operands");
  using L = AttnMLds<D>;
  constexpr int KCH = D / 8;                          // 16-byte chunks per key row
  constexpr int KL = AM_KEYS * KCH / AM_GT;           // prefix K chunks per group thread per tile
  constexpr int VI = (D + AM_GT - 1) / AM_GT;         // (4 keys x 8 dims) V items per group thread per tile
  static_assert(KL >= 1 && AM_KEYS * KCH % AM_GT == 0, "K tile must split evenly over a group's threads");
  static_assert(AttnMLds<D>::CK >= (4 * (D / 16) * 64 * 16 + 4 * 64 * 8), "the merge reuses the two stages");
  uint8_t* lds = reinterpret_cast<uint8_t*>(smem);
  // sample b on XCD b % 8: blockIdx = 8 * (Hq * (b / 8) + head) + b % 8
  const int xcd = (int)(blockIdx.x & 7), loc = (int)(blockIdx.x >> 3);
  const int jh = loc % p.Hq, b = (loc / p.Hq) * 8 + xcd;
  if (b >= p.B) return;
  const int H = p.H, P = p.P;
  const int kvh = jh / (p.Hq / p.Hkv);
  const int tid = threadIdx.x, grp = tid / AM_GT, gtid = tid % AM_GT;
  const int lane = tid & 63, w = gtid >> 6, g = lane >> 4, c16 = lane & 15;
  const size_t layer_elems = (size_t)p.B * P * p.Hkv * D;
  const auto pkr = rsrc(reinterpret_cast<const T*>(p.prefix_k) + (size_t)layer * layer_elems);
  const auto pvr = rsrc(reinterpret_cast<const T*>(p.prefix_v) + (size_t)layer * layer_elems);
  uint8_t* sl = slab(p, step, layer);
  const auto qrs = rsrc(sl + p.off_q), kgr = rsrc(sl + p.off_k), vgr = rsrc(sl + p.off_v);
  const size_t kvb = (size_t)b * p.Hkv + kvh;
  const int qrow = w * 16 + c16;
  const bool active = w * 16 < H;

  // -- prologue: query fragments, the chunk's keys and values into LDS
  u32x4 qf[D / 32];
  {
    const size_t hb = (size_t)b * p.Hq + jh;
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb)
      qf[kb] = ld16_if(qrs, (uint32_t)(qk_off(D, hb, qrow < H ? qrow : 0, kb * 32 + 8 * g) * 2), qrow < H);
    // rows i fastest, so a wave reads whole 32-byte rows of the tiles
    constexpr int CKL = AM_CHUNK * KCH / AM_THREADS;
#pragma unroll
    for (int j = 0; j < CKL; ++j) {
      const int idx = tid + j * AM_THREADS, i = idx % AM_CHUNK, c = idx / AM_CHUNK;
      const u32x4 v = ld16_if(kgr, (uint32_t)(qk_off(D, kvb, i < H ? i : 0, 8 * c) * 2), i < H);
      *reinterpret_cast<u32x4*>(lds + L::CK + (i * L::K_LD + 8 * c) * 2) = v;
    }
    constexpr int CVI = (AM_CHUNK / 4) * KCH / AM_THREADS;
#pragma unroll
    for (int j = 0; j < (CVI > 0 ? CVI : 1); ++j) {
      const int idx = tid + j * AM_THREADS, kq = idx % (AM_CHUNK / 4), c = idx / (AM_CHUNK / 4);
      if (idx >= (AM_CHUNK / 4) * KCH) break;
      u32x4 row[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * kq + r;
        row[r] = ld16_if(vgr, (uint32_t)(v_off(D, kvb, i < H ? i : 0, 8 * c) * 2), i < H);
      }
      am_store_v(lds + L::CV + kq * L::V_LD, c, row);
    }
    // complete every prologue load here: left in flight into the loop, the
    // in-order load counter would make each tile's MFMAs wait for the next
    // tile's loads as well
    __builtin_amdgcn_s_waitcnt(0);
  }

  // -- prefix tiles: per-thread byte offsets of tile 0, plus t * tile stride
  const uint32_t tstride = (uint32_t)(AM_KEYS * p.Hkv * D * 2);
  uint32_t kofs[KL], vofs[VI][4];
  int kkey[KL], vkey[VI];
#pragma unroll
  for (int j = 0; j < KL; ++j) {
    const int idx = gtid + j * AM_GT;
    kkey[j] = idx / KCH;
    kofs[j] = (uint32_t)(((((size_t)b * P + kkey[j]) * p.Hkv + kvh) * D + 8 * (idx % KCH)) * 2);
  }
#pragma unroll
  for (int j = 0; j < VI; ++j) {
    const int idx = gtid + j * AM_GT, kq = idx / KCH, c = idx % KCH;
    vkey[j] = idx < D ? 4 * kq : 1 << 30;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      vofs[j][r] = (uint32_t)(((((size_t)b * P + 4 * kq + r) * p.Hkv + kvh) * D + 8 * c) * 2);
  }
  // a group's next tile (t + 2) is loaded during its tile t's MFMAs
  u32x4 kr[KL], vr[VI][4];
  auto gload = [&](int t) {
    const int s0 = t * AM_KEYS;
#pragma unroll
    for (int j = 0; j < KL; ++j) kr[j] = ld16_if(pkr, kofs[j] + (uint32_t)t * tstride, s0 + kkey[j] < P);
#pragma unroll
    for (int j = 0; j < VI; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) vr[j][r] = ld16_if(pvr, vofs[j][r] + (uint32_t)t * tstride, s0 + vkey[j] + r < P);
  };
  auto lstore = [&](int buf) {
    uint8_t* kb = lds + buf * L::STAGE;
#pragma unroll
    for (int j = 0; j < KL; ++j) {
      const int idx = gtid + j * AM_GT;
      *reinterpret_cast<u32x4*>(kb + ((idx / KCH) * L::K_LD + (idx % KCH) * 8) * 2) = kr[j];
    }
#pragma unroll
    for (int j = 0; j < VI; ++j) {
      const int idx = gtid + j * AM_GT;
      if (idx < D) am_store_v(kb + L::K_TILE + (idx / KCH) * L::V_LD, idx % KCH, vr[j]);
    }
  };

  floatx4 O[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) O[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float scale = 1.4426950408889634f / sqrtf((float)D);   // log2(e) / sqrt(d)
  // One 32-key tile: keys s0 + kk (kk = 0..31) valid while below `limit`.
  auto tile = [&](const T* Ks, const uint8_t* Vq, int s0, int limit) {
    floatx4 slo = {0.f, 0.f, 0.f, 0.f}, shi = {0.f, 0.f, 0.f, 0.f};
    constexpr int KH = D / 32 < 4 ? D / 32 : 4;   // K fragments read ahead per batch
#pragma unroll
    for (int k0 = 0; k0 < D / 32; k0 += KH) {
      u32x4 alo[KH], ahi[KH];
#pragma unroll
      for (int kb = 0; kb < KH; ++kb) {
        alo[kb] = *reinterpret_cast<const u32x4*>(Ks + c16 * L::K_LD + (k0 + kb) * 32 + 8 * g);
        ahi[kb] = *reinterpret_cast<const u32x4*>(Ks + (16 + c16) * L::K_LD + (k0 + kb) * 32 + 8 * g);
      }
#pragma unroll
      for (int kb = 0; kb < KH; ++kb) {
        slo = MT<T>::mma(alo[kb], qf[k0 + kb], slo);
        shi = MT<T>::mma(ahi[kb], qf[k0 + kb], shi);
      }
    }
    // lane (c16, g): keys 4g .. 4g + 3 and 16 + 4g .. 16 + 4g + 3 of query c16
    float pr[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pr[r] = (s0 + 4 * g + r < limit) ? slo[r] * scale : -INFINITY;
      pr[4 + r] = (s0 + 16 + 4 * g + r < limit) ? shi[r] * scale : -INFINITY;
    }
    float cmax = pr[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) cmax = fmaxf(cmax, pr[e]);
    cmax = am_max4(cmax);
    // Lazy rescaling: the reference point m_run of the exponentials moves
    // only when a row's maximum exceeds it by more than 8 (log2 units), so
    // every weight stays <= 2^8 and the running sums are rescaled on few
    // tiles; O / l is the same for any reference point.
    const bool grow = cmax > m_run + 8.f;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_set = grow ? cmax : m_run;
      // 0 on the first tile (m_run = -inf), 1 for rows that did not grow
      const float alpha = m_set == m_run ? 1.f : fast_exp2(m_run - m_set);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) O[dt] *= alpha;
      m_run = m_set;
    }
    // (before any valid key m_run is -inf and every weight is 0)
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    // l_run is this lane's share (its 8 keys per tile); the four lanes of a
    // row are summed once, after the last tile
#pragma unroll
    for (int e = 0; e < 8; ++e) { pr[e] = fast_exp2(pr[e] - m_use); l_run += pr[e]; }
    bf16x8 pb;
#pragma unroll
    for (int e = 0; e < 8; ++e) pb[e] = (bf16)pr[e];
    const u32x4 pbu = __builtin_bit_cast(u32x4, pb);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const u32x2 lo = *reinterpret_cast<const u32x2*>(Vq + g * L::V_LD + am_v_off(dt * 16 + c16));
      const u32x2 hi = *reinterpret_cast<const u32x2*>(Vq + (4 + g) * L::V_LD + am_v_off(dt * 16 + c16));
      O[dt] = MT<T>::mma(u32x4{lo.x, lo.y, hi.x, hi.y}, pbu, O[dt]);
    }
  };

  // Group grp takes prefix tiles grp, grp + 2, ... through its own LDS
  // stage (one wave of each group per SIMD, so one group's latency chain
  // overlaps the other's work), then chunk keys 32 grp .. 32 grp + 31.
  const int ptiles = (P + AM_KEYS - 1) / AM_KEYS;
  const uint8_t* st = lds + grp * L::STAGE;
  gload(grp);   // past the last tile: predicated off, fetches nothing
  lstore(grp);
  __syncthreads();
  for (int t = grp; t - grp < ptiles; t += 2) {
    gload(t + 2);
    if (active && t < ptiles) tile(reinterpret_cast<const T*>(st), st + L::K_TILE, t * AM_KEYS, P);
    __syncthreads();   // both groups' LDS reads of this pass are done
    if (t + 2 < ptiles) lstore(grp);
    __syncthreads();
  }
  // the chunk's keys: P + i for i < H (pi0: the state token, query row 0,
  // sees only the first of them, its own)
  const int lim = (p.pi0 && qrow == 0) ? P + 1 : P + H;
  const int j0 = grp * AM_KEYS;
  if (active && j0 < H)
    tile(reinterpret_cast<const T*>(lds + L::CK) + j0 * L::K_LD, lds + L::CV + (j0 / 4) * L::V_LD, P + j0, lim);
  // merge: group 1 leaves its running output, reference maximum and sum
  // shares in the (now free) stages; group 0 combines them with its own
  floatx4* mo = reinterpret_cast<floatx4*>(lds);                       // [4 waves][D / 16][64]
  float* mm = reinterpret_cast<float*>(lds + 4 * (D / 16) * 64 * 16);  // [4 waves][64][2]
  if (grp == 1 && active) {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) mo[(w * (D / 16) + dt) * 64 + lane] = O[dt];
    mm[(w * 64 + lane) * 2] = m_run;
    mm[(w * 64 + lane) * 2 + 1] = l_run;
  }
  __syncthreads();
  if (grp == 0 && active) {
    const float m1 = mm[(w * 64 + lane) * 2], l1 = mm[(w * 64 + lane) * 2 + 1];
    const float mx = fmaxf(m_run, m1);
    // (a group that saw no key keeps m = -inf, O = 0, l = 0: weight 0)
    const float a0 = m_run == -INFINITY ? 0.f : fast_exp2(m_run - mx);
    const float a1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - mx);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) O[dt] = O[dt] * a0 + mo[(w * (D / 16) + dt) * 64 + lane] * a1;
    float l = l_run * a0 + l1 * a1;
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (qrow < H) {
      const float inv = 1.f / l;
      uint8_t* attn = sl + p.off_attn;
      const int gm = b * H + qrow;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
        store_gemm_in4<T, false>(p, attn, gm, jh * D + dt * 16 + 4 * g, O[dt] * inv, 1.0f);
    }
  }
}

// Instantiated in vfm_k_attn.hip only (built with MFMA accumulators in
// VGPRs, which keeps the running output out of AGPR copies around its
// rescaling); other translation units refer to those instantiations.
#ifndef VFM_ATTN_M_INSTANTIATE
extern template __global__ void k_attn_m<bf16, 64>(VP, int, int);
extern template __global__ void k_attn_m<bf16, 128>(VP, int, int);
extern template __global__ void k_attn_m<bf16, 256>(VP, int, int);
#endif

// ============================================================ kernels
// Persistent: the whole loop in one cooperative launch.
// FUSE: the norms are folded into the GEMMs (ph_gemm), the key-split merge
// into the attention phase (ph_attn), and attention waits for its heads'
// qkv tiles through counters, so a layer runs qkv + attention | o |
// gate/up | down with four device-wide barriers instead of eight (bf16
// pi0.5 experts).
template <typename T, int D, int WF, bool FUSE = false>
__global__ __launch_bounds__(NTH) void k_persistent(VP p) {
  unsigned epoch = 0;
  const int wg = blockIdx.x, nwg = gridDim.x;
  if (p.trace && wg == 0 && threadIdx.x == 0) p.trace[0] = p.trace[1] = __builtin_amdgcn_s_memrealtime();
#define VFM_BAR() do { if (!grid_barrier(p.bar, epoch, p.trace, p.spin_limit, p.fail_epoch, p.herr)) return; } while (0)
  // The next GEMM's first weight pass is loaded while the workgroup waits at
  // the barrier before it: weights do not depend on the other workgroups.
#define VFM_BAR_PF(WHICH, LAYER) \
  do { if (!grid_barrier(p.bar, epoch, p.trace, p.spin_limit, p.fail_epoch, p.herr, PrefetchHook<T, WHICH, WF>{p, LAYER, wg, pre})) return; } while (0)
  WPre pre;
  // XCD-local split sums (ph_gemm): only while every workgroup runs on XCD
  // blockIdx % 8; one that does not raises a word that every workgroup reads
  // after the first barrier, and the launch takes the device-scope path
  if ((FUSE ? p.xl : (p.xl & 2)) && threadIdx.x == 0) {
    unsigned xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    if ((xcc & 15u) != (blockIdx.x & 7u))
      __hip_atomic_fetch_or(&p.bar[BAR_XL_BAD], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  ph_boundary<T, WF, FUSE>(p, -1, 0, wg, nwg);
  if (p.pi0) VFM_BAR_PF(G_TMLP, 0);
  else if (p.L > 0) VFM_BAR_PF(G_QKV, 0);
  else VFM_BAR();
  // o / down split sums (folded norms only), attention splits and their merge
  const bool xl = FUSE && p.xl && ld_agent(&p.bar[BAR_XL_BAD]) == 0u;
  const bool xla = FUSE ? xl && (p.xl & 2) : (p.xl & 2) && ld_agent(&p.bar[BAR_XL_BAD]) == 0u;
  // merged attention, counters instead of two barriers (always with folded norms)
  const bool mg = FUSE || (p.xl & XL_MERGE);
  for (int k = 0; k < p.N; ++k) {
    if (p.pi0) {
      // the action tokens' time-MLP output, then layer 0's norm
      ph_gemm<T, G_TMLP, true, WF>(p, k, 0, wg, nwg, pre);
      VFM_BAR();
      ph_rn<T, WF>(p, k, 0, false, wg, nwg);
      VFM_BAR_PF(G_QKV, 0);
    }
    for (int l = 0; l < p.L; ++l) {
      if (!FUSE && l > 0) {
        ph_rn<T, WF>(p, k, l, false, wg, nwg);
        VFM_BAR_PF(G_QKV, l);
      }
      ph_gemm<T, G_QKV, true, WF, false, FUSE>(p, k, l, wg, nwg, pre, false, mg);
      {
        APre<T, D> apre;
        if (mg) {
          // dependency-scoped: attention units wait for their heads' qkv
          // tiles, and merge the key splits in place
          AttnPrefetchHook<T, D>{p, l, wg, apre, xla}();
          if (!ph_attn<T, D, true, WF, true>(p, k, l, wg, nwg, apre, xla)) return;
        } else {
          if (!grid_barrier(p.bar, epoch, p.trace, p.spin_limit, p.fail_epoch, p.herr, AttnPrefetchHook<T, D>{p, l, wg, apre, xla})) return;
          ph_attn<T, D, true, WF, false>(p, k, l, wg, nwg, apre, xla);
          VFM_BAR();
          ph_combine<T, WF>(p, k, l, wg, nwg, xla);
        }
      }
      VFM_BAR_PF(G_O, l);
      ph_gemm<T, G_O, true, WF, false, FUSE>(p, k, l, wg, nwg, pre, xl);
      if (!FUSE) {
        VFM_BAR();
        ph_rn<T, WF>(p, k, l, true, wg, nwg);
      }
      VFM_BAR_PF(G_GU, l);
      ph_gemm<T, G_GU, true, WF, false, FUSE>(p, k, l, wg, nwg, pre);
      VFM_BAR_PF(G_DOWN, l);
      ph_gemm<T, G_DOWN, true, WF, false, FUSE>(p, k, l, wg, nwg, pre, xl);
      if (FUSE && l + 1 < p.L) VFM_BAR_PF(G_QKV, l + 1);
      else VFM_BAR();
    }
    ph_boundary<T, WF, FUSE>(p, k, k + 1, wg, nwg);
    if (p.pi0 && k + 1 < p.N) VFM_BAR_PF(G_TMLP, 0);
    else if (p.L > 0 && k + 1 < p.N) VFM_BAR_PF(G_QKV, 0);
    else VFM_BAR();
  }
#undef VFM_BAR_PF
#undef VFM_BAR
  // Every workgroup has passed the last barrier; the last one to leave (an
  // exit count) clears the arrival counters for the next launch, so no
  // workgroup can still be polling them. A launch that gave up leaves them
  // behind and the host clears them when it reports the failure.
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add(&p.bar[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1u == gridDim.x) {
      for (int c = 0; c < BAR_COUNTERS; ++c)
        __hip_atomic_store(&p.bar[64 + 64 * c], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if constexpr (FUSE) {
        // the split GEMMs' arrival counters (multiples of their split counts
        // here), so that the next launch may split differently
        const int mt = (p.M + 63) / 64;
        const int no = p.W / (16 * p.gp_nt[1]) * mt, nd = p.W / (16 * p.gp_nt[3]) * mt;
        for (int c = 0; c < no; ++c) __hip_atomic_store(&p.fcnt[c], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int c = 0; c < nd; ++c) __hip_atomic_store(&p.fcnt[FCNT_MAX + c], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (FUSE || (p.xl & 2)) __hip_atomic_store(&p.bar[BAR_XL_BAD], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (FUSE || (p.xl & XL_MERGE)) {
        for (int c = 0; c < p.B * p.Hq; ++c)
          __hip_atomic_store(&p.hcnt[c * HCNT_STRIDE], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int c = 0; c < 2 * QCNT_KV; ++c)
          __hip_atomic_store(&p.qcnt[c * HCNT_STRIDE], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __hip_atomic_store(&p.bar[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// One phase per launch (eager / graph modes, and the calibration pass); one
// kernel symbol per phase so a kernel trace attributes time to phases.
template <typename T, int D, int PH, int WF, bool CAL>
__global__ __launch_bounds__(NTH) void k_phase(VP p, int k, int l) {
  const int wg = blockIdx.x, nwg = gridDim.x;
  if constexpr (PH == PH_BOUNDARY) ph_boundary<T, WF>(p, k - 1, k, wg, nwg);
  else if constexpr (PH == PH_RN_ATTN) ph_rn<T, WF>(p, k, l, false, wg, nwg);
  else if constexpr (PH == PH_QKV) ph_gemm<T, G_QKV, false, WF, CAL>(p, k, l, wg, nwg, WPre{});
  else if constexpr (PH == PH_ATTN) ph_attn<T, D>(p, k, l, wg, nwg);
  else if constexpr (PH == PH_COMBINE) ph_combine<T, WF>(p, k, l, wg, nwg);
  else if constexpr (PH == PH_O) ph_gemm<T, G_O, false, WF, CAL>(p, k, l, wg, nwg, WPre{});
  else if constexpr (PH == PH_RN_MLP) ph_rn<T, WF>(p, k, l, true, wg, nwg);
  else if constexpr (PH == PH_GU) ph_gemm<T, G_GU, false, WF, CAL>(p, k, l, wg, nwg, WPre{});
  else if constexpr (PH == PH_DOWN) ph_gemm<T, G_DOWN, false, WF, CAL>(p, k, l, wg, nwg, WPre{});
  else if constexpr (PH == PH_TMLP) ph_gemm<T, G_TMLP, false, WF, CAL>(p, k, l, wg, nwg, WPre{});
}

template <typename T, int D, int WF, bool CAL>
__host__ const void* phase_kernel(int ph, bool bigm = false, int bm = 128) {
  if constexpr (sizeof(T) == 2 && WF == WF_NATIVE && !CAL) {
    if (bigm && (bm == 224 || bm == 256)) {
      // the wide tiles: 256 columns x bm tokens
      if (bm == 224) {
        switch (ph) {
          case PH_QKV: return (const void*)&k_gemm_w<T, G_QKV, 7>;
          case PH_O: return (const void*)&k_gemm_w<T, G_O, 7>;
          case PH_GU: return (const void*)&k_gemm_w<T, G_GU, 7>;
          case PH_DOWN: return (const void*)&k_gemm_w<T, G_DOWN, 7>;
          case PH_TMLP: return (const void*)&k_gemm_w<T, G_TMLP, 7>;
          default: break;
        }
      } else {
        switch (ph) {
          case PH_QKV: return (const void*)&k_gemm_w<T, G_QKV, 8>;
          case PH_O: return (const void*)&k_gemm_w<T, G_O, 8>;
          case PH_GU: return (const void*)&k_gemm_w<T, G_GU, 8>;
          case PH_DOWN: return (const void*)&k_gemm_w<T, G_DOWN, 8>;
          case PH_TMLP: return (const void*)&k_gemm_w<T, G_TMLP, 8>;
          default: break;
        }
      }
    }
    if (bigm && bm == 64) {
      switch (ph) {
        case PH_QKV: return (const void*)&k_gemm_m<T, G_QKV, 64>;
        case PH_O: return (const void*)&k_gemm_m<T, G_O, 64>;
        case PH_GU: return (const void*)&k_gemm_m<T, G_GU, 64>;
        case PH_DOWN: return (const void*)&k_gemm_m<T, G_DOWN, 64>;
        case PH_TMLP: return (const void*)&k_gemm_m<T, G_TMLP, 64>;
        default: break;
      }
    }
    if (bigm) {
      switch (ph) {
        case PH_ATTN: return (const void*)&k_attn_m<T, D>;
        case PH_QKV: return (const void*)&k_gemm_m<T, G_QKV, 128>;
        case PH_O: return (const void*)&k_gemm_m<T, G_O, 128>;
        case PH_GU: return (const void*)&k_gemm_m<T, G_GU, 128>;
        case PH_DOWN: return (const void*)&k_gemm_m<T, G_DOWN, 128>;
        case PH_TMLP: return (const void*)&k_gemm_m<T, G_TMLP, 128>;
        default: break;
      }
    }
  }
  switch (ph) {
    case PH_BOUNDARY: return (const void*)&k_phase<T, D, PH_BOUNDARY, WF, CAL>;
    case PH_RN_ATTN: return (const void*)&k_phase<T, D, PH_RN_ATTN, WF, CAL>;
    case PH_QKV: return (const void*)&k_phase<T, D, PH_QKV, WF, CAL>;
    case PH_ATTN: return (const void*)&k_phase<T, D, PH_ATTN, WF, CAL>;
    case PH_COMBINE: return (const void*)&k_phase<T, D, PH_COMBINE, WF, CAL>;
    case PH_O: return (const void*)&k_phase<T, D, PH_O, WF, CAL>;
    case PH_RN_MLP: return (const void*)&k_phase<T, D, PH_RN_MLP, WF, CAL>;
    case PH_GU: return (const void*)&k_phase<T, D, PH_GU, WF, CAL>;
    case PH_DOWN: return (const void*)&k_phase<T, D, PH_DOWN, WF, CAL>;
    default: return (const void*)&k_phase<T, D, PH_TMLP, WF, CAL>;
  }
}

// ============================================================ host-side launch helpers
// mode 0: persistent kernel, cooperative launch; 3: persistent kernel,
// ordinary launch of the same grid; otherwise one phase. The calibration
// variant (CAL) has phase kernels only.
template <typename T, int D, int WF, bool CAL>
hipError_t launch_one(const VP& p, int mode, int phase, int k, int l, int grid, size_t lds, hipStream_t st) {
  if (mode == 0 || mode == 3) {
    if constexpr (CAL) {
      return hipErrorInvalidValue;
    } else {
      void* args[] = {const_cast<VP*>(&p)};
      const void* f = reinterpret_cast<const void*>(&k_persistent<T, D, WF>);
      if (p.fuse) {
        if constexpr (fusable<T, WF>()) f = reinterpret_cast<const void*>(&k_persistent<T, D, WF, true>);
        else return hipErrorInvalidValue;
      }
      if (mode == 0) return hipLaunchCooperativeKernel(f, dim3(grid), dim3(NTH), args, (unsigned)lds, st);
      return hipLaunchKernel(f, dim3(grid), dim3(NTH), args, lds, st);
    }
  }
  void* args[] = {const_cast<VP*>(&p), &k, &l};
  const bool gemm = phase == PH_QKV || phase == PH_O || phase == PH_GU || phase == PH_DOWN || phase == PH_TMLP;
  const bool bigm = p.bigm && (gemm || phase == PH_ATTN);
  if (bigm && phase == PH_ATTN) {
    if constexpr (sizeof(T) == 2 && WF == WF_NATIVE && !CAL) {
      // the single-pass attention keeps every query row of a head in one
      // workgroup (H <= 64) and needs its two LDS stages
      if (p.H > AM_CHUNK || D % 32) return hipErrorInvalidValue;
      return hipLaunchKernel(phase_kernel<T, D, WF, CAL>(phase, true), dim3(grid), dim3(AM_THREADS), args,
                             (size_t)AttnMLds<D>::TOTAL, st);
    } else {
      return hipErrorInvalidValue;
    }
  }
  int bm = 128;
  if (bigm) {
    const int gi = phase == PH_QKV ? 0 : phase == PH_O ? 1 : phase == PH_GU ? 2 : phase == PH_DOWN ? 3 : 4;
    bm = p.gp_bm[gi];
    if constexpr (sizeof(T) == 2 && WF == WF_NATIVE && !CAL) {
      if (bm == 224 || bm == 256)   // the wide tiles' LDS ring
        return hipLaunchKernel(phase_kernel<T, D, WF, CAL>(phase, true, bm), dim3(grid), dim3(GW_THREADS), args,
                               (size_t)(bm == 224 ? GW<7>::LDS : GW<8>::LDS), st);
    }
  }
  return hipLaunchKernel(phase_kernel<T, D, WF, CAL>(phase, bigm, bm), dim3(grid), dim3(bigm ? GM_THREADS : NTH),
                         args, lds, st);
}

template <typename T, int D, int WF, bool CAL>
hipError_t set_lds_limit(int bytes) {
  hipError_t e = hipSuccess;
  if constexpr (!CAL)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_persistent<T, D, WF>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if constexpr (!CAL && fusable<T, WF>())
    if (e == hipSuccess)
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_persistent<T, D, WF, true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  for (int ph = 0; ph < PH_COUNT && e == hipSuccess; ++ph) {
    e = hipFuncSetAttribute(phase_kernel<T, D, WF, CAL>(ph), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    for (int bm : {128, 64, 224, 256}) {
      const void* big = phase_kernel<T, D, WF, CAL>(ph, true, bm);
      if (e == hipSuccess && big != phase_kernel<T, D, WF, CAL>(ph)) {
        const int need = ph == PH_ATTN ? AttnMLds<D>::TOTAL : bm == 224 ? GW<7>::LDS : bm == 256 ? GW<8>::LDS : GM_LDS;
        e = hipFuncSetAttribute(big, hipFuncAttributeMaxDynamicSharedMemorySize, bytes > need ? bytes : need);
      }
    }
  }
  return e;
}

template <typename T, int D, int WF, bool CAL>
hipError_t occupancy(size_t lds, int* per_cu) {
  if constexpr (CAL) {
    *per_cu = 0;
    return hipErrorInvalidValue;
  } else {
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        per_cu, reinterpret_cast<const void*>(&k_persistent<T, D, WF>), NTH, lds);
    if constexpr (fusable<T, WF>()) {
      // the grid must fit with either kernel resident
      int fused = 0;
      if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &fused, reinterpret_cast<const void*>(&k_persistent<T, D, WF, true>), NTH, lds);
      if (e == hipSuccess && fused < *per_cu) *per_cu = fused;
    }
    return e;
  }
}

// The entry points of one kernel set (activation type T, weight format WF,
// calibration flag CAL) over the head dimensions Ds it is built for.
template <typename T, int WF, bool CAL, int... Ds>
struct KernelSet {
  static hipError_t launch(const VP& p, int mode, int phase, int k, int l, int grid, size_t lds, hipStream_t st) {
    hipError_t e = hipErrorInvalidValue;
    ((p.d == Ds ? (void)(e = launch_one<T, Ds, WF, CAL>(p, mode, phase, k, l, grid, lds, st)) : (void)0), ...);
    return e;
  }
  static hipError_t prepare(int d, int lds) {
    hipError_t e = hipErrorInvalidValue;
    ((d == Ds ? (void)(e = set_lds_limit<T, Ds, WF, CAL>(lds)) : (void)0), ...);
    return e;
  }
  static hipError_t occupancy_of(int d, size_t lds, int* per_cu) {
    hipError_t e = hipErrorInvalidValue;
    ((d == Ds ? (void)(e = occupancy<T, Ds, WF, CAL>(lds, per_cu)) : (void)0), ...);
    return e;
  }
};

#define VFM_DEFINE_KERNEL_SET(NAME, ...)                                                                             \
  hipError_t NAME##_launch(const VP& p, int mode, int phase, int k, int l, int grid, size_t lds, hipStream_t st) { \
    return KernelSet<__VA_ARGS__>::launch(p, mode, phase, k, l, grid, lds, st);                                    \
  }                                                                                                                \
  hipError_t NAME##_prepare(int d, int lds) { return KernelSet<__VA_ARGS__>::prepare(d, lds); }                    \
  hipError_t NAME##_occupancy(int d, size_t lds, int* per_cu) {                                                    \
    return KernelSet<__VA_ARGS__>::occupancy_of(d, lds, per_cu);                                                   \
  }

}  // namespace vfm
