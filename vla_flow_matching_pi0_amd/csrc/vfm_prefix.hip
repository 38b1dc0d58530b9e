// vfm_prefix.hip -- kernels of the prefix producer: one decoder pass over the
// P prefix tokens of every sample (Gemma-shaped: pre-norm blocks with a
// (1 + w) RMSNorm gain, grouped-query bidirectional attention with rotary
// encoding, GeGLU MLP), writing each layer's rotary-encoded keys and values
// in the layout the action expert binds: [L][B][P][Hkv][d] bf16.
//
// Unlike the action expert (50 tokens, bandwidth- and latency-bound), the
// prefill GEMMs have M = B * P tokens (560 at batch 1) and are dense
// contractions: they run on bf16 MFMA (16x16x32) with 128 x 128 tiles staged
// through LDS, two workgroups per compute unit.
#include "vfm_device.h"
#include "vfm_gemm_wide.h"
#include "vfm_prefix.h"

namespace vfm {
namespace pfx {

// Byte offset of element (row r, k) in a packed operand [R/16][K/32][64][8 x bf16]:
// lane (r % 16) + 16 ((k % 32) / 8) of block (r / 16, k / 32), element k % 8.
__device__ __forceinline__ uint32_t pk_off(int r, int k, int K) {
  return ((uint32_t)(((r >> 4) * (K >> 5) + (k >> 5)) * 64 + ((k & 31) >> 3) * 16 + (r & 15)) << 4) +
         (uint32_t)((k & 7) << 1);
}

__device__ __forceinline__ uint32_t bf16_bits(float v) { return (uint32_t)__builtin_bit_cast(uint16_t, (bf16)v); }

// ------------------------------------------------------------------ GEMM
// Tile: TN output columns (weights, MFMA rows) x TM tokens (MFMA columns);
// 4 waves as 2 x 2, each 64 x 64 (4 x 4 MFMA blocks). Per stage one TK = 64
// slice of both operand tiles (8 blocks x 2 k-blocks x 1 KB each) goes
// global -> registers -> LDS, double-buffered, one barrier per stage; the
// next stage's global loads are in flight while the current one computes.
// Block b runs on XCD b % 8; each XCD takes a contiguous range of tiles,
// tokens fastest, so the token tiles that share a weight tile share an L2.
// TNC = 64 (half-width tiles, twice as many: a GEMM with few 128 x 128
// tiles, such as the fused QKV projection) keeps the stage layout, the A
// half of the stage half filled, and gives each wave 32 x 64.
constexpr int STAGE = 2 * 16384;   // A tile + B tile bytes

template <int EPI, int TNC = TN>
__global__ __launch_bounds__(256, 2) void k_gemm(const GemmArgs g) {
  extern __shared__ __align__(16) uint8_t lds[];
  constexpr int NB = TNC / 32;          // 16-column blocks per wave
  constexpr int AL = TNC / 32;          // A chunks per thread and stage (16 bytes each)
  const int MTL = g.Mpad / TM, NTL = g.N / TNC, total = MTL * NTL * g.S;
  const int per = (total + 7) >> 3;
  const int v = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (v >= total) return;
  const int mt = v % MTL, nt = (v / MTL) % NTL, s = v / (MTL * NTL);
  const int KB32 = g.K >> 5, Ks = g.K / g.S, nk = Ks / TK;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wn = w >> 1, wm = w & 1;
  const __amdgpu_buffer_rsrc_t ra = rsrc(g.A), rb = rsrc(g.B);
  uint32_t aoff[4], boff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i, blk = c >> 7, rest = c & 127;
    aoff[i] = (uint32_t)(((nt * (TNC / 16) + blk) * KB32 + (s * Ks >> 5)) * 1024 + rest * 16);
    boff[i] = (uint32_t)(((mt * 8 + blk) * KB32 + (s * Ks >> 5)) * 1024 + rest * 16);
  }
  u32x4 ga[4], gb[4];
  auto gload = [&](int it) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < AL) ga[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, aoff[i] + (uint32_t)it * 2048u, 0, 0);
      gb[i] = __builtin_amdgcn_raw_buffer_load_b128(rb, boff[i] + (uint32_t)it * 2048u, 0, 0);
    }
  };
  auto lstore = [&](int buf) {
    u32x4* A = reinterpret_cast<u32x4*>(lds + buf * STAGE);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < AL) A[tid + 256 * i] = ga[i];
      A[1024 + tid + 256 * i] = gb[i];
    }
  };
  floatx4 acc[NB][4];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  gload(0);
  lstore(0);
  __syncthreads();
  for (int it = 0; it < nk; ++it) {
    if (it + 1 < nk) gload(it + 1);
    const u32x4* A = reinterpret_cast<const u32x4*>(lds + (it & 1) * STAGE);
    const u32x4* B = A + 1024;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      u32x4 a[NB], b[4];
#pragma unroll
      for (int i = 0; i < NB; ++i) a[i] = A[(wn * NB + i) * 128 + kb * 64 + lane];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = B[(wm * 4 + j) * 128 + kb * 64 + lane];
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = MT<bf16>::mma(a[i], b[j], acc[i][j]);
    }
    if (it + 1 < nk) lstore((it + 1) & 1);
    __syncthreads();
  }

  // epilogue: lane holds D[n0 + r][token], r = 0..3
  const int g4 = 4 * (lane >> 4);
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int n0 = nt * TNC + wn * (TNC / 2) + i * 16 + g4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int token = mt * TM + wm * 64 + j * 16 + (lane & 15);
      const floatx4 c = acc[i][j];
      if constexpr (EPI == EPI_PART) {
        *reinterpret_cast<floatx4*>(g.part + ((size_t)s * g.Mpad + token) * g.N + n0) = c;
      } else if constexpr (EPI == EPI_GU) {
        // columns (gate j, up j, gate j+1, up j+1), j = n0 / 2
        const float a0 = gelu_tanh(c[0]) * c[1], a1 = gelu_tanh(c[2]) * c[3];
        *reinterpret_cast<uint32_t*>(g.act + pk_off(token, n0 >> 1, g.N >> 1)) = bf16_bits(a0) | (bf16_bits(a1) << 16);
      } else {
        if (token >= g.M) continue;
        const int d = g.d, kd = g.Hkv * d, half = d >> 1;
        const int b = token / g.P, pp = token - b * g.P;
        if (n0 >= kd && n0 < 2 * kd) {
          const int hv = (n0 - kd) / d, dim = (n0 - kd) - hv * d;
          u32x2 vv;
          vv[0] = bf16_bits(c[0]) | (bf16_bits(c[1]) << 16);
          vv[1] = bf16_bits(c[2]) | (bf16_bits(c[3]) << 16);
          *reinterpret_cast<u32x2*>(g.v_out + ((size_t)token * g.Hkv + hv) * d + dim) = vv;
          uint16_t* vt = g.vt + (((size_t)b * g.Hkv + hv) * d + dim) * g.Ppad + pp;
#pragma unroll
          for (int r = 0; r < 4; ++r) vt[(size_t)r * g.Ppad] = (uint16_t)bf16_bits(c[r]);
        } else {
          // rotary pairs (i0, i0 + d/2) and (i0 + 1, i0 + 1 + d/2) at position pp
          const bool isk = n0 < kd;
          const int base = isk ? n0 : n0 - 2 * kd;
          const int head = base / d, p4 = base - head * d, i0 = p4 >> 1;
          const float* rp = g.rope + ((size_t)pp * half + i0) * 2;
          const float c0 = rp[0], s0 = rp[1], c1 = rp[2], s1 = rp[3];
          const float y0 = c[0] * c0 - c[2] * s0, y2 = c[2] * c0 + c[0] * s0;
          const float y1 = c[1] * c1 - c[3] * s1, y3 = c[3] * c1 + c[1] * s1;
          uint16_t* dst = isk ? g.k_out + ((size_t)token * g.Hkv + head) * d : g.q + ((size_t)token * g.Hq + head) * d;
          *reinterpret_cast<uint32_t*>(dst + i0) = bf16_bits(y0) | (bf16_bits(y1) << 16);
          *reinterpret_cast<uint32_t*>(dst + i0 + half) = bf16_bits(y2) | (bf16_bits(y3) << 16);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ wide GEMMs
// The gate/up GEMM (the largest of the pass) and the down projection on the
// 256-column tiles of vfm_gemm_wide.h: one workgroup per compute unit, four
// waves of 128 columns x 16 MB tokens, both operands through a 5-stage
// direct-to-LDS ring. The token blocks are stored in the MFMA lane order
// already, so the copies are linear.
// EPI_GU: the sums go through LDS half a wave tile at a time and come back
// transposed, lane (token c, tile il) taking the 16 sums of its token in one
// 16-column tile (gate and up of 8 features): their 8 GeGLU values are one
// 16-byte piece of the packed operand, and the 64 lanes of a store fill whole
// 1 KiB blocks.
// EPI_PART: split s of g.S takes K range [s K / S, (s + 1) K / S) and stores
// its sums straight from the accumulators into part[s] (the next norm adds
// the splits); the tiles cover every padded token row (part_plan).
template <int MB, int EPI>
__global__ __launch_bounds__(GW_THREADS, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_w(const GemmArgs g) {
  extern __shared__ __align__(16) uint8_t lds[];
  using C = GW<MB>;
  const int S = EPI == EPI_PART ? g.S : 1;
  const int MTL = (g.M + C::BMT - 1) / C::BMT, NTL = g.N / 256, total = MTL * NTL * S;
  const int per = (total + 7) >> 3;
  const int v = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (v >= total) return;
  const int mt = v % MTL, nt = (v / MTL) % NTL, s = v / (MTL * NTL);
  const int KB32 = g.K >> 5, nblk = g.Mpad >> 4, nst = KB32 / S, kb0 = s * nst;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), wn = w & 1, wm = w >> 1;
  // copy i: weight tile nt * 16 + w + 4i (i < 4), else token block
  // 2 MB mt + w + 4 (i - 4) (clamped to the last padded block; its outputs
  // are not stored)
  uint32_t voff[C::CW];
#pragma unroll
  for (int i = 0; i < C::CW; ++i) {
    int blk;
    if (i < 4) {
      blk = nt * 16 + w + 4 * i;
    } else {
      blk = 2 * MB * mt + w + 4 * (i - 4);
      blk = blk < nblk ? blk : nblk - 1;
    }
    voff[i] = (uint32_t)(blk * KB32 + kb0) * 1024u + (uint32_t)lane * 16u;
  }
  floatx4 acc[8][MB];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  gw_mainloop<MB>(acc, lds, g.A, g.B, voff, 1024u, nst, w, lane);

  if constexpr (EPI == EPI_PART) {
    // lane (c, g) of block (i, j): columns n0 .. n0 + 3 of token c
    const int g4 = 4 * (lane >> 4), c = lane & 15;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int n0 = nt * 256 + (wn * 8 + i) * 16 + g4;
#pragma unroll
      for (int j = 0; j < MB; ++j) {
        const int token = mt * C::BMT + (wm * MB + j) * 16 + c;
        if (token < g.Mpad) *reinterpret_cast<floatx4*>(g.part + ((size_t)s * g.Mpad + token) * g.N + n0) = acc[i][j];
      }
    }
    return;
  }
  gw_barrier();   // every wave is done with the ring (and every copy has landed)
  floatx4* E = reinterpret_cast<floatx4*>(lds + w * (4 * MB * 1024));
  const int c = lane & 15, il = lane >> 4;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < MB; ++j) E[(i * MB + j) * 64 + lane] = acc[4 * h + i][j];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    floatx4 q[MB][4];
#pragma unroll
    for (int j = 0; j < MB; ++j)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) q[j][gg] = E[(il * MB + j) * 64 + gg * 16 + c];
    const int f0 = (nt * 16 + wn * 8 + 4 * h + il) * 8;
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      u32x4 y;
#pragma unroll
      for (int gg = 0; gg < 4; ++gg)
        y[gg] = bf16_bits(gelu_tanh(q[j][gg].x) * q[j][gg].y) | (bf16_bits(gelu_tanh(q[j][gg].z) * q[j][gg].w) << 16);
      // tokens past the padded count: an offset beyond the buffer range drops the store
      const int token = mt * C::BMT + (wm * MB + j) * 16 + c;
      const uint32_t off = token < g.Mpad ? pk_off(token, f0, g.N >> 1) : 0x80000000u;
      __builtin_amdgcn_raw_buffer_store_b128(y, rsrc(g.act), off, 0, 0);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
}

// Tokens per tile of the wide gate/up GEMM for M tokens (0: the shape does
// not fit it): the choice with the least work per compute unit, counting a
// second round of tiles and a fixed cost per 32-K stage.
static int gu_wide_tokens(const GemmArgs& g) {
  if (g.N % 256 != 0 || g.S != 1 || g.K % 64 != 0 || g.K / 32 < GW<5>::NS - 1) return 0;
  int best = 0;
  long best_cost = -1;
  for (int mb : {5, 6, 7}) {
    const long tiles = (long)(g.N / 256) * ((g.M + 32 * mb - 1) / (32 * mb));
    const long cost = (tiles + 255) / 256 * (mb * 8 * 17 + 350);
    if (best_cost < 0 || cost < best_cost) best_cost = cost, best = 32 * mb;
  }
  return best;
}

// ------------------------------------------------------------------ attention
// Workgroup (query block of AQ = 32, head h, sample b), two groups of two
// waves: group q takes the key tiles kt = q, q + 2, ..., each through its own
// LDS stage, and wave w of a group owns queries 16 (w % 2) .. + 15; the two
// groups' running outputs are merged through LDS at the end (one wave per
// SIMD: one group's LDS -> MFMA -> softmax chain overlaps the other's).
// Per 32-key tile: K [32][d] and V^T [d][32] staged in LDS (padded rows);
// S^T = K Q^T on MFMA (lane: keys 4g..4g+3 of each 16-key half, query l % 16),
// online softmax in the log2 domain per query column, then O^T += V^T P^T
// where the 32 keys of the MFMA's k index are ordered (4g..4g+3, 16+4g..16+4g+3)
// on both operands, so P^T comes straight from the S^T registers.
template <int D>
__global__ __launch_bounds__(2 * AQ / 16 * 64, 2) void k_attn(const AttnArgs a) {
  constexpr int GT = AQ / 16 * 64;     // threads of one group (one wave per 16 queries)
  constexpr int KROW = 2 * D + 16;     // bytes per K row in LDS
  constexpr int VROW = 2 * AK + 16;    // bytes per V^T row in LDS
  constexpr int CPT = AK * D / 8 / GT; // 16-byte chunks per thread per operand tile
  constexpr int GLDS = AK * KROW + D * VROW;   // one group's stage
  static_assert(AK * D / 8 % GT == 0, "tiles must split evenly over a group's threads");
  static_assert((D / 16) * 4 * 4 * GT + 2 * 4 * GT <= GLDS, "the merge fits in one group's stage");
  __shared__ __align__(16) uint8_t lds[2 * GLDS];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c16 = lane & 15;
  const int grp = tid / GT, gtid = tid % GT, wq = w % (AQ / 16);
  uint8_t* sk = lds + grp * GLDS;
  uint8_t* sv = sk + AK * KROW;
  const int h = blockIdx.y, b = blockIdx.z, kvh = h / (a.Hq / a.Hkv);
  const int P = a.P;
  const int qi = blockIdx.x * AQ + wq * 16 + c16;
  const bool qok = qi < P;
  const __amdgpu_buffer_rsrc_t rq = rsrc(a.q), rk = rsrc(a.k), rv = rsrc(a.vt);

  u32x4 qf[D / 32];
#pragma unroll
  for (int kb = 0; kb < D / 32; ++kb)
    qf[kb] = ld16_if(rq, (uint32_t)((((size_t)b * P + qi) * a.Hq + h) * D + 32 * kb + 8 * g) * 2, qok);

  floatx4 o[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) o[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  u32x4 pkk[CPT], pvv[CPT];
  const int ntile = (P + AK - 1) / AK;
  auto fetch = [&](int kt) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = gtid + GT * i;
      const int key = c / (D / 8), part = c % (D / 8);
      const int kk = kt * AK + key;
      pkk[i] = ld16_if(rk, (uint32_t)((((size_t)b * P + kk) * a.Hkv + kvh) * D + part * 8) * 2, kk < P);
      const int dim = c >> 2, vp = c & 3;
      pvv[i] = __builtin_amdgcn_raw_buffer_load_b128(
          rv, (uint32_t)((((size_t)b * a.Hkv + kvh) * D + dim) * a.Ppad + kt * AK + vp * 8) * 2, 0, 0);
    }
  };
  if (grp < ntile) fetch(grp);
  // both groups take the same number of steps (barriers are workgroup-wide);
  // a group past the last tile idles through its final step
  for (int it = 0; it < (ntile + 1) / 2; ++it) {
    const int kt = 2 * it + grp;
    const bool live = kt < ntile;
    __syncthreads();
    if (live) {
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int c = gtid + GT * i;
        *reinterpret_cast<u32x4*>(sk + (c / (D / 8)) * KROW + (c % (D / 8)) * 16) = pkk[i];
        *reinterpret_cast<u32x4*>(sv + (c >> 2) * VROW + (c & 3) * 16) = pvv[i];
      }
    }
    __syncthreads();
    if (kt + 2 < ntile) fetch(kt + 2);
    if (!live) continue;

    floatx4 s[2];
#pragma unroll
    for (int h16 = 0; h16 < 2; ++h16) {
      s[h16] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb) {
        const u32x4 kf = *reinterpret_cast<const u32x4*>(sk + (h16 * 16 + c16) * KROW + (32 * kb + 8 * g) * 2);
        s[h16] = MT<bf16>::mma(kf, qf[kb], s[h16]);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int h16 = 0; h16 < 2; ++h16)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kt * AK + h16 * 16 + 4 * g + r;
        const float x = key < P ? s[h16][r] * a.scale_log2 : -INFINITY;
        s[h16][r] = x;
        mx = fmaxf(mx, x);
      }
    mx = am_max4(mx);
    // Lazy rescaling: the reference point m moves only when a row's maximum
    // exceeds it by more than 8 (log2 units), so every weight stays <= 2^8
    // and the output is rescaled on few tiles (O / l does not depend on m).
    // l is this lane's share of the row sum, reduced after the last tile.
    const bool grow = mx > m + 8.f;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float mset = grow ? mx : m;
      const float alpha = mset == m ? 1.f : fast_exp2(m - mset);   // 0 on the first tile (m = -inf)
      l *= alpha;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) o[db] *= alpha;
      m = mset;
    }
    const float muse = m == -INFINITY ? 0.f : m;
#pragma unroll
    for (int h16 = 0; h16 < 2; ++h16)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2(s[h16][r] - muse);
        s[h16][r] = p;
        l += p;
      }
    u32x4 pb;
    pb[0] = bf16_bits(s[0][0]) | (bf16_bits(s[0][1]) << 16);
    pb[1] = bf16_bits(s[0][2]) | (bf16_bits(s[0][3]) << 16);
    pb[2] = bf16_bits(s[1][0]) | (bf16_bits(s[1][1]) << 16);
    pb[3] = bf16_bits(s[1][2]) | (bf16_bits(s[1][3]) << 16);
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const uint8_t* row = sv + (db * 16 + c16) * VROW;
      const u32x2 lo = *reinterpret_cast<const u32x2*>(row + 8 * g);
      const u32x2 hi = *reinterpret_cast<const u32x2*>(row + 32 + 8 * g);
      u32x4 vf;
      vf[0] = lo[0]; vf[1] = lo[1]; vf[2] = hi[0]; vf[3] = hi[1];
      o[db] = MT<bf16>::mma(vf, pb, o[db]);
    }
  }
  // merge: group 1 leaves (m, l, o) in its stage; group 0 rescales both to
  // the larger reference point (a group that saw no key has m = -inf and
  // weight 0) and stores
  __syncthreads();
  float* xo = reinterpret_cast<float*>(lds + GLDS);
  if (grp == 1) {
#pragma unroll
    for (int db = 0; db < D / 16; ++db) *reinterpret_cast<floatx4*>(xo + (db * GT + gtid) * 4) = o[db];
    xo[(D / 16) * GT * 4 + gtid] = m;
    xo[(D / 16) * GT * 4 + GT + gtid] = l;
  }
  __syncthreads();
  if (grp == 1) return;
  {
    const float m1 = xo[(D / 16) * GT * 4 + gtid], l1 = xo[(D / 16) * GT * 4 + GT + gtid];
    const float mm = fmaxf(m, m1);
    const float a0 = m == -INFINITY ? 0.f : fast_exp2(m - mm), a1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - mm);
    l = l * a0 + l1 * a1;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) o[db] = o[db] * a0 + *reinterpret_cast<const floatx4*>(xo + (db * GT + gtid) * 4) * a1;
  }
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (!qok) return;
  const float inv = 1.0f / l;
  const int token = b * P + qi, K = a.Hq * D;
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    const int k = h * D + db * 16 + 4 * g;
    u32x2 ov;
    ov[0] = bf16_bits(o[db][0] * inv) | (bf16_bits(o[db][1] * inv) << 16);
    ov[1] = bf16_bits(o[db][2] * inv) | (bf16_bits(o[db][3] * inv) << 16);
    *reinterpret_cast<u32x2*>(a.out + pk_off(token, k, K)) = ov;
  }
}

// ------------------------------------------------------------------ norm
// One workgroup per token row: x (+ the K-split partial sums of the previous
// projection, or the bf16 embeddings for the first layer), then
// xn = x / sqrt(mean(x^2) + eps) * (1 + w) packed for the next GEMM. Rows
// M..Mpad-1 get zeros.
template <bool FIRST>
__global__ __launch_bounds__(256) void k_norm(const NormArgs n) {
  __shared__ float red[4];
  const int token = blockIdx.x, tid = threadIdx.x, nch = n.W >> 3;
  if (token >= n.M) {
    for (int c = tid; c < nch; c += 256)
      *reinterpret_cast<u32x4*>(n.xn + pk_off(token, c * 8, n.W)) = u32x4{0u, 0u, 0u, 0u};
    return;
  }
  float v[2][8];
  float ss = 0.f;
#pragma unroll
  for (int ci = 0; ci < 2; ++ci) {
    const int c = tid + 256 * ci;
    if (c >= nch) continue;
    float* xr = n.x + (size_t)token * n.W + c * 8;
    if constexpr (FIRST) {
      const u32x4 e = *reinterpret_cast<const u32x4*>(n.embeds + (size_t)token * n.W + c * 8);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[ci][2 * q] = __builtin_bit_cast(float, e[q] << 16);
        v[ci][2 * q + 1] = __builtin_bit_cast(float, e[q] & 0xffff0000u);
      }
    } else {
      const floatx4 a0 = *reinterpret_cast<const floatx4*>(xr), a1 = *reinterpret_cast<const floatx4*>(xr + 4);
#pragma unroll
      for (int q = 0; q < 4; ++q) { v[ci][q] = a0[q]; v[ci][4 + q] = a1[q]; }
      for (int s = 0; s < n.S; ++s) {
        const float* pr = n.part + ((size_t)s * n.Mpad + token) * n.W + c * 8;
        const floatx4 p0 = *reinterpret_cast<const floatx4*>(pr), p1 = *reinterpret_cast<const floatx4*>(pr + 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) { v[ci][q] += p0[q]; v[ci][4 + q] += p1[q]; }
      }
    }
    floatx4 o0, o1;
#pragma unroll
    for (int q = 0; q < 4; ++q) { o0[q] = v[ci][q]; o1[q] = v[ci][4 + q]; }
    *reinterpret_cast<floatx4*>(xr) = o0;
    *reinterpret_cast<floatx4*>(xr + 4) = o1;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += v[ci][e] * v[ci][e];
  }
  const float tot = block_sum256(ss, red);
  const float r = 1.0f / sqrtf(tot / (float)n.W + n.eps);
#pragma unroll
  for (int ci = 0; ci < 2; ++ci) {
    const int c = tid + 256 * ci;
    if (c >= nch) continue;
    const floatx4 g0 = *reinterpret_cast<const floatx4*>(n.gain + c * 8);
    const floatx4 g1 = *reinterpret_cast<const floatx4*>(n.gain + c * 8 + 4);
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      o[q] = bf16_bits(v[ci][2 * q] * r * (1.0f + g0[2 * q])) | (bf16_bits(v[ci][2 * q + 1] * r * (1.0f + g0[2 * q + 1])) << 16);
      o[2 + q] = bf16_bits(v[ci][4 + 2 * q] * r * (1.0f + g1[2 * q])) |
                 (bf16_bits(v[ci][4 + 2 * q + 1] * r * (1.0f + g1[2 * q + 1])) << 16);
    }
    *reinterpret_cast<u32x4*>(n.xn + pk_off(token, c * 8, n.W)) = o;
  }
}

// ------------------------------------------------------------------ host side
hipError_t prepare() {
  hipError_t e;
  if ((e = hipFuncSetAttribute((const void*)k_gemm<EPI_PART>, hipFuncAttributeMaxDynamicSharedMemorySize, 2 * STAGE)) != hipSuccess)
    return e;
  if ((e = hipFuncSetAttribute((const void*)k_gemm<EPI_GU>, hipFuncAttributeMaxDynamicSharedMemorySize, 2 * STAGE)) != hipSuccess)
    return e;
  const void* wide[6] = {(const void*)k_gemm_w<5, EPI_GU>, (const void*)k_gemm_w<6, EPI_GU>, (const void*)k_gemm_w<7, EPI_GU>,
                         (const void*)k_gemm_w<5, EPI_PART>, (const void*)k_gemm_w<6, EPI_PART>,
                         (const void*)k_gemm_w<7, EPI_PART>};
  const int wlds[3] = {GW<5>::LDS, GW<6>::LDS, GW<7>::LDS};
  for (int i = 0; i < 6; ++i)
    if ((e = hipFuncSetAttribute(wide[i], hipFuncAttributeMaxDynamicSharedMemorySize, wlds[i % 3])) != hipSuccess) return e;
  if ((e = hipFuncSetAttribute((const void*)k_gemm<EPI_QKV, 64>, hipFuncAttributeMaxDynamicSharedMemorySize, 2 * STAGE)) !=
      hipSuccess)
    return e;
  if ((e = hipFuncSetAttribute((const void*)k_gemm<EPI_PART, 64>, hipFuncAttributeMaxDynamicSharedMemorySize, 2 * STAGE)) !=
      hipSuccess)
    return e;
  return hipFuncSetAttribute((const void*)k_gemm<EPI_QKV>, hipFuncAttributeMaxDynamicSharedMemorySize, 2 * STAGE);
}

PartPlan part_plan(int M, int Mpad, int N, int K, int narrow_split, bool wide) {
  PartPlan best{0, narrow_split};
  if (!wide || N % 256 != 0 || K % 64 != 0) return best;
  long best_fill = 0;
  for (int mb : {5, 6, 7}) {
    const int bmt = 32 * mb, mtl = (M + bmt - 1) / bmt;
    if ((long)mtl * bmt < Mpad) continue;   // every padded row gets its partial sums
    const int ring = mb == 5 ? GW<5>::NS : mb == 6 ? GW<6>::NS : GW<7>::NS;
    const long tiles = (long)mtl * (N / 256);
    for (int sp = 1; sp <= MAX_SPLIT; sp *= 2) {
      const int nst = K / 32 / sp;
      if (K % (64 * sp) != 0 || nst < ring - 1 || nst * 32 < 1024 || tiles * sp > 256) continue;
      if (tiles * sp > best_fill) best_fill = tiles * sp, best = PartPlan{bmt, sp};
    }
  }
  // one round of tiles on at least three quarters of the compute units
  return best_fill >= 192 ? best : PartPlan{0, narrow_split};
}

hipError_t gemm(int epi, const GemmArgs& g, hipStream_t st, bool wide_gu) {
  if (epi == EPI_GU && wide_gu) {
    const int bm = gu_wide_tokens(g);
    if (bm > 0) {
      const int tiles = (g.N / 256) * ((g.M + bm - 1) / bm), grid = (tiles + 7) / 8 * 8;
      if (bm == 160) hipLaunchKernelGGL((k_gemm_w<5, EPI_GU>), dim3(grid), dim3(GW_THREADS), GW<5>::LDS, st, g);
      else if (bm == 192) hipLaunchKernelGGL((k_gemm_w<6, EPI_GU>), dim3(grid), dim3(GW_THREADS), GW<6>::LDS, st, g);
      else hipLaunchKernelGGL((k_gemm_w<7, EPI_GU>), dim3(grid), dim3(GW_THREADS), GW<7>::LDS, st, g);
      return hipGetLastError();
    }
  }
  if (epi == EPI_PART && g.bm > 0) {
    const int tiles = (g.N / 256) * ((g.M + g.bm - 1) / g.bm) * g.S, grid = (tiles + 7) / 8 * 8;
    if (g.bm == 160) hipLaunchKernelGGL((k_gemm_w<5, EPI_PART>), dim3(grid), dim3(GW_THREADS), GW<5>::LDS, st, g);
    else if (g.bm == 192) hipLaunchKernelGGL((k_gemm_w<6, EPI_PART>), dim3(grid), dim3(GW_THREADS), GW<6>::LDS, st, g);
    else if (g.bm == 224) hipLaunchKernelGGL((k_gemm_w<7, EPI_PART>), dim3(grid), dim3(GW_THREADS), GW<7>::LDS, st, g);
    else return hipErrorInvalidValue;
    return hipGetLastError();
  }
  const int total = (g.Mpad / TM) * (g.N / TN) * g.S;
  const int grid = (total + 7) / 8 * 8;
  if (epi == EPI_QKV && g.qkv_half && total <= 128 && g.N % 64 == 0) {
    // fewer 128 x 128 tiles than half the compute units: 128 x 64 tiles
    const int grid64 = (2 * total + 7) / 8 * 8;
    hipLaunchKernelGGL((k_gemm<EPI_QKV, 64>), dim3(grid64), dim3(256), 2 * STAGE, st, g);
    return hipGetLastError();
  }
  if (epi == EPI_PART && g.part_half && g.N % 64 == 0) {
    const int grid64 = (2 * total + 7) / 8 * 8;
    hipLaunchKernelGGL((k_gemm<EPI_PART, 64>), dim3(grid64), dim3(256), 2 * STAGE, st, g);
    return hipGetLastError();
  }
  switch (epi) {
    case EPI_PART: hipLaunchKernelGGL(k_gemm<EPI_PART>, dim3(grid), dim3(256), 2 * STAGE, st, g); break;
    case EPI_GU: hipLaunchKernelGGL(k_gemm<EPI_GU>, dim3(grid), dim3(256), 2 * STAGE, st, g); break;
    default: hipLaunchKernelGGL(k_gemm<EPI_QKV>, dim3(grid), dim3(256), 2 * STAGE, st, g); break;
  }
  return hipGetLastError();
}

hipError_t attention(int d, const AttnArgs& a, int B, hipStream_t st) {
  const dim3 grid((a.P + AQ - 1) / AQ, a.Hq, B);
  switch (d) {
    case 64: hipLaunchKernelGGL(k_attn<64>, grid, dim3(2 * AQ / 16 * 64), 0, st, a); break;
    case 128: hipLaunchKernelGGL(k_attn<128>, grid, dim3(2 * AQ / 16 * 64), 0, st, a); break;
    case 256: hipLaunchKernelGGL(k_attn<256>, grid, dim3(2 * AQ / 16 * 64), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t norm(bool first, const NormArgs& n, hipStream_t st) {
  if (first) hipLaunchKernelGGL(k_norm<true>, dim3(n.Mpad), dim3(256), 0, st, n);
  else hipLaunchKernelGGL(k_norm<false>, dim3(n.Mpad), dim3(256), 0, st, n);
  return hipGetLastError();
}

}  // namespace pfx
}  // namespace vfm
