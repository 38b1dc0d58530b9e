// vfm_kernels.hip -- HIP kernels (gfx950) of the flow-matching action expert.
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
//   in_proj   h = x W_in + b_in + s                      (s = state W_s + b_s)
//   norm      xn = rms(h) * (1 + scale) + shift           (adaRMSNorm, attn)
//   qkv       [q|k|v] = xn W_qkv, rotary on q, k at P..P+H-1   (fused GEMM)
//   attn      split-K flash attention of q over prefix KV + chunk KV (GQA)
//   combine   merge the key splits (log-sum-exp)
//   o         h += gate * (attn W_o)                      (gated residual)
//   norm      xn = adaRMSNorm(h) (mlp)
//   gateup    a = gelu_tanh(xn W_gate) * (xn W_up)         (fused GEMM)
//   down      h += gate * (a W_down)
//   final     x += dt * (adaRMSNorm_final(h) W_out + b_out)
// The fusions (QKV as one GEMM, gate/up as one GEMM, residual+norm, RoPE in
// the projection epilogue) follow the PhyAI optimisation paragraph and the
// hand-written memory-bound kernels listed in the FlashRT walk-through
// (component 8, kernel library).
#include "vfm_device.h"
#include "vfm_params.h"

namespace vfm {

extern __shared__ __align__(16) char smem[];

// =============================================================== elementwise phases
// x = noise (skipped when the two alias) and s = state W_s + b_s.
__device__ void ph_init(const VP& p, int wg, int nwg) {
  const int nx = p.B * p.H * p.A;
  if (p.noise != p.x) {
    for (int i = wg * 256 + threadIdx.x; i < nx; i += nwg * 256)
      coh_st4(p.x, i * 4, __builtin_bit_cast(uint32_t, p.noise[i]));
  }
  if (p.S > 0) {
    const int ns = p.B * p.W;
    for (int i = wg * 256 + threadIdx.x; i < ns; i += nwg * 256) {
      const int b = i / p.W, n = i % p.W;
      float acc = p.st_b[n];
      for (int j = 0; j < p.S; ++j) acc += p.state[b * p.S + j] * p.st_w[j * p.W + n];
      coh_st4(p.s, i * 4, __builtin_bit_cast(uint32_t, acc));
    }
  }
}

// h[m][n] = sum_a x[m][a] W_in[a][n] + b_in[n] + s[b][n]; 4 columns per thread.
__device__ void ph_in_proj(const VP& p, int wg, int nwg) {
  const int W4 = p.W / 4, total = p.M * W4;
  for (int it = wg * 256 + threadIdx.x; it < total; it += nwg * 256) {
    const int m = it / W4, n = (it % W4) * 4;
    const int b = m / p.H;
    floatx4 acc = as_f4(ro_ld16(p.in_b + n));
    if (p.S > 0) acc += as_f4(coh_ld16(p.s, (b * p.W + n) * 4));
    for (int a = 0; a < p.A; ++a) {
      const float xv = __builtin_bit_cast(float, coh_ld4(p.x, (m * p.A + a) * 4));
      acc += xv * as_f4(ro_ld16(p.in_w + a * p.W + n));
    }
    coh_st16(p.h, (m * p.W + n) * 4, as_u4(acc));
  }
}

// adaRMSNorm of rows of h into xn (act type T); one row per workgroup unit.
template <typename T>
__device__ void ph_norm(const VP& p, int step, int ni, int wg, int nwg) {
  float* red = reinterpret_cast<float*>(smem);
  const float* mod = p.mod + ((size_t)step * p.n_norms + ni) * 3 * p.W;
  const int W4 = p.W / 4;
  for (int m = wg; m < p.M; m += nwg) {
    floatx4 hv[4];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = threadIdx.x + j * 256;
      hv[j] = c < W4 ? as_f4(coh_ld16(p.h, (m * p.W + c * 4) * 4)) : floatx4{0, 0, 0, 0};
      ss += hv[j].x * hv[j].x + hv[j].y * hv[j].y + hv[j].z * hv[j].z + hv[j].w * hv[j].w;
    }
    ss = block_sum256(ss, red);
    const float r = 1.0f / sqrtf(ss / (float)p.W + p.eps);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = threadIdx.x + j * 256;
      if (c >= W4) continue;
      const floatx4 sc = as_f4(ro_ld16(mod + c * 4));
      const floatx4 sh = as_f4(ro_ld16(mod + p.W + c * 4));
      const floatx4 y = hv[j] * r * (1.0f + sc) + sh;
      if constexpr (sizeof(T) == 4) {
        coh_st16(p.xn, (m * p.W + c * 4) * 4, as_u4(y));
      } else {
        coh_st8(p.xn, (m * p.W + c * 4) * 2, u32x2{pack_bf16x2(y.x, y.y), pack_bf16x2(y.z, y.w)});
      }
    }
  }
}

// =============================================================== skinny GEMM on MFMA
// C[M x N] = A[M x K] (act type T, row-major, produced by an earlier phase)
// times a packed weight. Swap-AB: the weight supplies the 16 MFMA rows
// (output features) and the tokens the 16 MFMA columns, so the 50 tokens of
// a chunk pad to 64 = 4 column tiles and a lane ends with 4 consecutive
// output features of one token. Packed weight layout:
// [N/16 tiles][K/KB blocks][64 lanes][16 bytes], one contiguous 1 KiB block
// per MFMA step, so a wave streams its tile's weights sequentially.
// Work unit = 64 output columns (4 waves x 16) x 64 tokens.
enum { G_QKV = 0, G_O = 1, G_GU = 2, G_DOWN = 3 };

template <typename T, int WHICH>
__device__ void ph_gemm(const VP& p, int step, int layer, int wg, int nwg) {
  constexpr int E = MT<T>::E, KB = MT<T>::KB;
  constexpr int KC = 512 / (int)sizeof(T);        // k per staged chunk (512 bytes of a row)
  constexpr int LDA = KC + 16 / (int)sizeof(T);   // padded LDS row (elements)
  constexpr int NBLK = KC / KB;                   // MFMA blocks per chunk (= 8)
  const void* A;
  const uint8_t* Wp;
  int K, N;
  if (WHICH == G_QKV) { A = p.xn; K = p.W; N = (p.Hq + 2 * p.Hkv) * p.d; Wp = p.w_qkv[layer]; }
  else if (WHICH == G_O) { A = p.attn; K = p.Hq * p.d; N = p.W; Wp = p.w_o[layer]; }
  else if (WHICH == G_GU) { A = p.xn; K = p.W; N = 2 * p.F; Wp = p.w_gu[layer]; }
  else { A = p.act; K = p.F; N = p.W; Wp = p.w_down[layer]; }

  T* As = reinterpret_cast<T*>(smem);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 4, c16 = lane & 15;
  const int ngroups = N / 64, mtiles = (p.M + 63) / 64, units = ngroups * mtiles;
  const int nkb = K / KB;
  for (int u = wg; u < units; u += nwg) {
    const int ng = u % ngroups, mt = u / ngroups;
    const int t = ng * 4 + wv;                     // this wave's 16-column tile
    const int m0 = mt * 64;
    floatx4 acc[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) acc[s] = floatx4{0, 0, 0, 0};
    const uint8_t* wt = Wp + ((size_t)t * nkb * 64 + lane) * 16;
    for (int k0 = 0; k0 < K; k0 += KC) {
      u32x4 wreg[NBLK];
#pragma unroll
      for (int i = 0; i < NBLK; ++i) wreg[i] = ro_ld16(wt + ((size_t)(k0 / KB + i) * 64) * 16);
      __syncthreads();
      // stage A[m0 .. m0+64)[k0 .. k0+KC) : 64 rows x 32 chunks of 16 bytes
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int idx = threadIdx.x + i * 256;
        const int row = idx >> 5, cc = idx & 31;
        const int gm = m0 + row;
        u32x4 v = {0, 0, 0, 0};
        if (gm < p.M) v = coh_ld16(A, (uint32_t)(((size_t)gm * K + k0) * sizeof(T) + cc * 16));
        *reinterpret_cast<u32x4*>(As + row * LDA + cc * (16 / (int)sizeof(T))) = v;
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < NBLK; ++i) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const u32x4 b = *reinterpret_cast<const u32x4*>(As + (s * 16 + c16) * LDA + i * KB + g * E);
          acc[s] = MT<T>::mma(wreg[i], b, acc[s]);
        }
      }
    }
    // ---------------- epilogues
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int gm = m0 + s * 16 + c16;
      if (gm >= p.M) continue;
      const floatx4 v = acc[s];
      if (WHICH == G_QKV) {
        const int d = p.d, hd = d / 2;
        const int col0 = t * 16;
        const int head = col0 / d, tt = (col0 % d) / 16;
        const int b = gm / p.H, i = gm % p.H;
        if (head < p.Hq + p.Hkv) {
          // packed lane order (x_j, x_j+1, x_j+d/2, x_j+1+d/2), j = 8 tt + 2 g
          const int j0 = tt * 8 + 2 * g;
          const float* rp = p.rope + ((size_t)i * hd + j0) * 2;
          const float c0 = rp[0], s0 = rp[1], c1 = rp[2], s1 = rp[3];
          const float y0 = v.x * c0 - v.z * s0, y0h = v.z * c0 + v.x * s0;
          const float y1 = v.y * c1 - v.w * s1, y1h = v.w * c1 + v.y * s1;
          void* dst;
          size_t row;
          if (head < p.Hq) { dst = p.q; row = ((size_t)b * p.Hq + head) * p.H + i; }
          else { dst = p.ks; row = ((size_t)b * p.Hkv + (head - p.Hq)) * p.H + i; }
          const size_t e0 = row * d + j0;
          if constexpr (sizeof(T) == 4) {
            coh_st8(dst, (uint32_t)(e0 * 4), u32x2{__builtin_bit_cast(uint32_t, y0), __builtin_bit_cast(uint32_t, y1)});
            coh_st8(dst, (uint32_t)((e0 + hd) * 4), u32x2{__builtin_bit_cast(uint32_t, y0h), __builtin_bit_cast(uint32_t, y1h)});
          } else {
            coh_st4(dst, (uint32_t)(e0 * 2), pack_bf16x2(y0, y1));
            coh_st4(dst, (uint32_t)((e0 + hd) * 2), pack_bf16x2(y0h, y1h));
          }
        } else {
          const int kvh = head - p.Hq - p.Hkv;
          const size_t e0 = (((size_t)b * p.Hkv + kvh) * p.H + i) * d + tt * 16 + 4 * g;
          if constexpr (sizeof(T) == 4) coh_st16(p.vs, (uint32_t)(e0 * 4), as_u4(v));
          else coh_st8(p.vs, (uint32_t)(e0 * 2), u32x2{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)});
        }
      } else if (WHICH == G_GU) {
        // packed lane order (gate f, up f, gate f+1, up f+1), f = 8 t + 2 g
        const int f0 = t * 8 + 2 * g;
        const float a0 = gelu_tanh(v.x) * v.y, a1 = gelu_tanh(v.z) * v.w;
        const size_t e0 = (size_t)gm * p.F + f0;
        if constexpr (sizeof(T) == 4) coh_st8(p.act, (uint32_t)(e0 * 4), u32x2{__builtin_bit_cast(uint32_t, a0), __builtin_bit_cast(uint32_t, a1)});
        else coh_st4(p.act, (uint32_t)(e0 * 2), pack_bf16x2(a0, a1));
      } else {
        // gated residual: h += gate * v (this lane owns h[gm][n0 .. n0+4))
        const int ni = WHICH == G_O ? 2 * layer : 2 * layer + 1;
        const int n0 = t * 16 + 4 * g;
        const floatx4 gate = as_f4(ro_ld16(p.mod + (((size_t)step * p.n_norms + ni) * 3 + 2) * p.W + n0));
        const uint32_t off = (uint32_t)(((size_t)gm * p.W + n0) * 4);
        const floatx4 h = as_f4(coh_ld16(p.h, off));
        coh_st16(p.h, off, as_u4(h + gate * v));
      }
    }
  }
}

// =============================================================== attention
// Flash-style attention of one query head over keys [s0, s1) of
// [prefix (P) ; chunk (H)]. Work unit = (sample b, query head j, key split c).
// Each wave owns 16 query rows; a 32-key chunk of K (row-major) and V
// (transposed) is staged in LDS and shared by the 4 waves. Scores are
// computed transposed, S^T = K Q^T, so a lane holds 8 keys of one query and
// the row max / sum need only two cross-lane exchanges; the probabilities
// then feed the PV MFMA directly from registers.
template <typename T, int D>
__device__ void ph_attn(const VP& p, int layer, int wg, int nwg) {
  constexpr int E = MT<T>::E, KB = MT<T>::KB;
  constexpr int LDQ = D + 16 / (int)sizeof(T);
  constexpr int LDV = 32 + 16 / (int)sizeof(T);
  constexpr int CPR = D * (int)sizeof(T) / 16;    // 16-byte chunks per row
  T* Qs = reinterpret_cast<T*>(smem);             // [64][LDQ]
  T* Ks = Qs + 64 * LDQ;                          // [32][LDQ]
  T* Vt = Ks + 32 * LDQ;                          // [D][LDV]
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 4, c16 = lane & 15;
  const int H = p.H, P = p.P, S_tot = P + H, KS = p.KS, KPS = p.kps;
  const int group = p.Hq / p.Hkv;
  const int units = p.B * p.Hq * KS;
  const float scale = 1.4426950408889634f / sqrtf((float)D);   // log2(e) / sqrt(d)
  const T* pk_base = reinterpret_cast<const T*>(p.prefix_k);
  const T* pv_base = reinterpret_cast<const T*>(p.prefix_v);
  for (int u = wg; u < units; u += nwg) {
    const int c = u % KS, bh = u / KS, jh = bh % p.Hq, b = bh / p.Hq;
    const int kvh = jh / group;
    const int s0 = c * KPS, s1 = min(S_tot, s0 + KPS);
    __syncthreads();
    for (int idx = threadIdx.x; idx < 64 * CPR; idx += 256) {
      const int row = idx / CPR, cc = idx % CPR;
      u32x4 v = {0, 0, 0, 0};
      if (row < H) v = coh_ld16(p.q, (uint32_t)((((size_t)(b * p.Hq + jh) * H + row) * D) * sizeof(T) + cc * 16));
      *reinterpret_cast<u32x4*>(Qs + row * LDQ + cc * (16 / (int)sizeof(T))) = v;
    }
    float m_run = -INFINITY, l_run = 0.f;
    floatx4 O[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) O[dt] = floatx4{0, 0, 0, 0};
    const bool active = wv * 16 < H;
    for (int sc = s0; sc < s1; sc += 32) {
      __syncthreads();
      for (int idx = threadIdx.x; idx < 32 * CPR; idx += 256) {
        const int kk = idx / CPR, cc = idx % CPR;
        const int s = sc + kk;
        u32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
        if (s < s1) {
          if (s < P) {
            const size_t e = ((((size_t)layer * p.B + b) * P + s) * p.Hkv + kvh) * D;
            kv = ro_ld16(pk_base + e + cc * (16 / (int)sizeof(T)));
            vv = ro_ld16(pv_base + e + cc * (16 / (int)sizeof(T)));
          } else {
            const uint32_t off = (uint32_t)(((((size_t)b * p.Hkv + kvh) * H + (s - P)) * D) * sizeof(T) + cc * 16);
            kv = coh_ld16(p.ks, off);
            vv = coh_ld16(p.vs, off);
          }
        }
        *reinterpret_cast<u32x4*>(Ks + kk * LDQ + cc * (16 / (int)sizeof(T))) = kv;
        const T* ve = reinterpret_cast<const T*>(&vv);
        const int d0 = cc * (16 / (int)sizeof(T));
#pragma unroll
        for (int e = 0; e < 16 / (int)sizeof(T); ++e) Vt[(d0 + e) * LDV + kk] = ve[e];
      }
      __syncthreads();
      if (!active) continue;
      floatx4 slo = {0, 0, 0, 0}, shi = {0, 0, 0, 0};
#pragma unroll
      for (int kb = 0; kb < D / KB; ++kb) {
        const u32x4 bq = *reinterpret_cast<const u32x4*>(Qs + (wv * 16 + c16) * LDQ + kb * KB + g * E);
        const u32x4 alo = *reinterpret_cast<const u32x4*>(Ks + c16 * LDQ + kb * KB + g * E);
        const u32x4 ahi = *reinterpret_cast<const u32x4*>(Ks + (16 + c16) * LDQ + kb * KB + g * E);
        slo = MT<T>::mma(alo, bq, slo);
        shi = MT<T>::mma(ahi, bq, shi);
      }
      float pr[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pr[r] = (sc + 4 * g + r < s1) ? slo[r] * scale : -INFINITY;
        pr[4 + r] = (sc + 16 + 4 * g + r < s1) ? shi[r] * scale : -INFINITY;
      }
      float cmax = pr[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) cmax = fmaxf(cmax, pr[e]);
      cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
      cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
      const float m_new = fmaxf(m_run, cmax);
      const float alpha = fast_exp2(m_run - m_new);
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) { pr[e] = fast_exp2(pr[e] - m_new); psum += pr[e]; }
      psum += __shfl_xor(psum, 16);
      psum += __shfl_xor(psum, 32);
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) O[dt] *= alpha;
      // PV: key order of the k slots is (4g..4g+3, 16+4g..16+4g+3) for both operands
      if constexpr (sizeof(T) == 2) {
        bf16x8 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = (bf16)pr[e];
        const u32x4 pbu = __builtin_bit_cast(u32x4, pb);
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          const T* vr = Vt + (dt * 16 + c16) * LDV;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vr + 4 * g);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vr + 16 + 4 * g);
          O[dt] = MT<T>::mma(u32x4{lo.x, lo.y, hi.x, hi.y}, pbu, O[dt]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int key = e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4);
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt)
            O[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(to_f(Vt[(dt * 16 + c16) * LDV + key]), pr[e], O[dt], 0, 0, 0);
        }
      }
    }
    if (active) {
      const int qrow = wv * 16 + c16;
      if (qrow < H) {
        const size_t base = ((size_t)(b * p.Hq + jh) * KS + c) * 64 + qrow;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
          coh_st16(p.opart, (uint32_t)((base * D + dt * 16 + 4 * g) * 4), as_u4(O[dt]));
        if (g == 0) coh_st8(p.ml, (uint32_t)(base * 8), u32x2{__builtin_bit_cast(uint32_t, m_run), __builtin_bit_cast(uint32_t, l_run)});
      }
    }
  }
}

// Merge the key splits: attn[b*H+i][j*d + dd] = sum_c w_c O_c / sum_c w_c l_c,
// w_c = 2^(m_c - max m). Four head dims per thread.
template <typename T>
__device__ void ph_combine(const VP& p, int wg, int nwg) {
  const int D = p.d, D4 = D / 4, KS = p.KS;
  const int total = p.M * p.Hq * D4;
  for (int it = wg * 256 + threadIdx.x; it < total; it += nwg * 256) {
    const int d4 = it % D4, r = it / D4, jh = r % p.Hq, gm = r / p.Hq;
    const int b = gm / p.H, i = gm % p.H;
    const size_t base0 = ((size_t)(b * p.Hq + jh) * KS) * 64 + i;
    float mx = -INFINITY;
    for (int c = 0; c < KS; ++c) mx = fmaxf(mx, __builtin_bit_cast(float, coh_ld4(p.ml, (uint32_t)((base0 + c * 64) * 8))));
    floatx4 num = {0, 0, 0, 0};
    float den = 0.f;
    for (int c = 0; c < KS; ++c) {
      const size_t base = base0 + (size_t)c * 64;
      const floatx2 ml = __builtin_bit_cast(floatx2, coh_ld8(p.ml, (uint32_t)(base * 8)));
      const float w = fast_exp2(ml[0] - mx);
      den += w * ml[1];
      num += w * as_f4(coh_ld16(p.opart, (uint32_t)((base * D + d4 * 4) * 4)));
    }
    const floatx4 o = num / den;
    const size_t e0 = (size_t)gm * p.Hq * D + jh * D + d4 * 4;
    if constexpr (sizeof(T) == 4) coh_st16(p.attn, (uint32_t)(e0 * 4), as_u4(o));
    else coh_st8(p.attn, (uint32_t)(e0 * 2), u32x2{pack_bf16x2(o.x, o.y), pack_bf16x2(o.z, o.w)});
  }
}

// =============================================================== final norm + out proj + Euler
// One row per unit: v = adaRMSNorm_final(h[m]) W_out + b_out; x[m] += dt * v.
__device__ void ph_final(const VP& p, int step, int wg, int nwg) {
  float* red = reinterpret_cast<float*>(smem);          // [4]
  float* xs = red + 4;                                   // [W]
  float* part = xs + p.W;                                // [256]
  const float* mod = p.mod + ((size_t)step * p.n_norms + (p.n_norms - 1)) * 3 * p.W;
  const int A = p.A, nsub = 256 / A;
  const float dt = -1.0f / (float)p.N;
  for (int m = wg; m < p.M; m += nwg) {
    float ss = 0.f;
    for (int n = threadIdx.x; n < p.W; n += 256) {
      const float v = __builtin_bit_cast(float, coh_ld4(p.h, (m * p.W + n) * 4));
      xs[n] = v;
      ss += v * v;
    }
    ss = block_sum256(ss, red);
    const float r = 1.0f / sqrtf(ss / (float)p.W + p.eps);
    for (int n = threadIdx.x; n < p.W; n += 256) xs[n] = xs[n] * r * (1.0f + mod[n]) + mod[p.W + n];
    __syncthreads();
    float acc = 0.f;
    const int a = threadIdx.x % A, sub = threadIdx.x / A;
    if (sub < nsub)
      for (int n = sub; n < p.W; n += nsub) acc += xs[n] * p.out_w[n * A + a];
    part[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x < A) {
      float v = p.out_b[threadIdx.x];
      for (int j = 0; j < nsub; ++j) v += part[threadIdx.x + j * A];
      const uint32_t off = (uint32_t)((m * A + threadIdx.x) * 4);
      const float x = __builtin_bit_cast(float, coh_ld4(p.x, off));
      coh_st4(p.x, off, __builtin_bit_cast(uint32_t, x + dt * v));
    }
    __syncthreads();
  }
}

// =============================================================== kernels
// Persistent: the whole loop in one cooperative launch.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_persistent(VP p) {
  unsigned epoch = 0;
  const int wg = blockIdx.x, nwg = gridDim.x;
#define VFM_BAR() do { if (!grid_barrier(p.bar, epoch)) return; } while (0)
  ph_init(p, wg, nwg);
  VFM_BAR();
  for (int k = 0; k < p.N; ++k) {
    ph_in_proj(p, wg, nwg);
    VFM_BAR();
    for (int l = 0; l < p.L; ++l) {
      ph_norm<T>(p, k, 2 * l, wg, nwg);
      VFM_BAR();
      ph_gemm<T, G_QKV>(p, k, l, wg, nwg);
      VFM_BAR();
      ph_attn<T, D>(p, l, wg, nwg);
      VFM_BAR();
      ph_combine<T>(p, wg, nwg);
      VFM_BAR();
      ph_gemm<T, G_O>(p, k, l, wg, nwg);
      VFM_BAR();
      ph_norm<T>(p, k, 2 * l + 1, wg, nwg);
      VFM_BAR();
      ph_gemm<T, G_GU>(p, k, l, wg, nwg);
      VFM_BAR();
      ph_gemm<T, G_DOWN>(p, k, l, wg, nwg);
      VFM_BAR();
    }
    ph_final(p, k, wg, nwg);
    VFM_BAR();
  }
#undef VFM_BAR
}

// One phase per launch (eager / graph modes).
template <typename T, int D>
__global__ __launch_bounds__(256) void k_phase(VP p, int phase, int k, int l) {
  const int wg = blockIdx.x, nwg = gridDim.x;
  switch (phase) {
    case PH_INIT: ph_init(p, wg, nwg); break;
    case PH_IN_PROJ: ph_in_proj(p, wg, nwg); break;
    case PH_NORM_ATTN: ph_norm<T>(p, k, 2 * l, wg, nwg); break;
    case PH_QKV: ph_gemm<T, G_QKV>(p, k, l, wg, nwg); break;
    case PH_ATTN: ph_attn<T, D>(p, l, wg, nwg); break;
    case PH_COMBINE: ph_combine<T>(p, wg, nwg); break;
    case PH_O: ph_gemm<T, G_O>(p, k, l, wg, nwg); break;
    case PH_NORM_MLP: ph_norm<T>(p, k, 2 * l + 1, wg, nwg); break;
    case PH_GU: ph_gemm<T, G_GU>(p, k, l, wg, nwg); break;
    case PH_DOWN: ph_gemm<T, G_DOWN>(p, k, l, wg, nwg); break;
    case PH_FINAL: ph_final(p, k, wg, nwg); break;
    default: break;
  }
}

}  // namespace vfm

// =============================================================== host-side launch table
namespace vfm {

size_t lds_bytes(const VP& p, int act_bytes) {
  const size_t gemm = 64 * (512 + 16);
  const size_t ldq = p.d + 16 / act_bytes, ldv = 32 + 16 / act_bytes;
  const size_t attn = (96 * ldq + (size_t)p.d * ldv) * act_bytes;
  const size_t fin = (4 + (size_t)p.W + 256) * 4;
  size_t m = gemm > attn ? gemm : attn;
  return m > fin ? m : fin;
}

template <typename T, int D>
static hipError_t launch_one(const VP& p, int mode, int phase, int k, int l, int grid, size_t lds, hipStream_t st) {
  if (mode == 0) {
    void* args[] = {const_cast<VP*>(&p)};
    return hipLaunchCooperativeKernel(reinterpret_cast<void*>(&k_persistent<T, D>), dim3(grid), dim3(256), args,
                                      (unsigned)lds, st);
  }
  hipLaunchKernelGGL((k_phase<T, D>), dim3(grid), dim3(256), lds, st, p, phase, k, l);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t set_lds_limit(int bytes) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_persistent<T, D>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&k_phase<T, D>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

hipError_t prepare_kernels(int act_bf16, int d, int lds) {
  if (act_bf16) {
    if (d == 64) return set_lds_limit<bf16, 64>(lds);
    if (d == 128) return set_lds_limit<bf16, 128>(lds);
    return set_lds_limit<bf16, 256>(lds);
  }
  if (d == 64) return set_lds_limit<float, 64>(lds);
  if (d == 128) return set_lds_limit<float, 128>(lds);
  return set_lds_limit<float, 256>(lds);
}

// mode 0 = persistent (phase ignored), 1 = one phase.
hipError_t launch_phase(const VP& p, int act_bf16, int mode, int phase, int k, int l, int grid, size_t lds,
                        hipStream_t st) {
  if (act_bf16) {
    if (p.d == 64) return launch_one<bf16, 64>(p, mode, phase, k, l, grid, lds, st);
    if (p.d == 128) return launch_one<bf16, 128>(p, mode, phase, k, l, grid, lds, st);
    return launch_one<bf16, 256>(p, mode, phase, k, l, grid, lds, st);
  }
  if (p.d == 64) return launch_one<float, 64>(p, mode, phase, k, l, grid, lds, st);
  if (p.d == 128) return launch_one<float, 128>(p, mode, phase, k, l, grid, lds, st);
  return launch_one<float, 256>(p, mode, phase, k, l, grid, lds, st);
}

hipError_t max_cooperative_grid(int act_bf16, int d, size_t lds, int* grid) {
  const void* f;
  if (act_bf16) f = d == 64 ? (const void*)&k_persistent<bf16, 64> : d == 128 ? (const void*)&k_persistent<bf16, 128> : (const void*)&k_persistent<bf16, 256>;
  else f = d == 64 ? (const void*)&k_persistent<float, 64> : d == 128 ? (const void*)&k_persistent<float, 128> : (const void*)&k_persistent<float, 256>;
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, f, 256, lds);
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
