// vfm_params.h -- the launch-parameter block shared by the host runtime and
// the kernels, and the host entry points of the kernel translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace vfm {

constexpr int MAX_LAYERS = 48;
constexpr int NTHREADS = 512;      // threads per workgroup
constexpr int MAX_KSPLIT = 16;     // K splits of the residual GEMMs
// Grid-barrier words: [0] exit count, [1] sticky error flag, then BAR_COUNTERS
// arrival counters, each on its own 256-byte line (word 64 + 64 c).
constexpr int BAR_COUNTERS = 64;
constexpr int BAR_WORDS = 64 + 64 * BAR_COUNTERS;
constexpr long BARRIER_SPIN_LIMIT_HOST = 1L << 22;   // default polls before a device-wide wait gives up
// large-M GEMM, 256-column tiles of 224 / 256 tokens: stages of 32 K in the
// LDS ring (a pass takes an even stage count of at least the ring less one)
constexpr int GW_RING_224 = 5;
constexpr int GW_RING_256 = 4;

enum Phase {
  PH_BOUNDARY = 0, PH_RN_ATTN, PH_QKV, PH_ATTN, PH_COMBINE, PH_O, PH_RN_MLP, PH_GU, PH_DOWN, PH_TMLP, PH_COUNT
};

// Everything a phase needs; passed by value as the kernel argument.
struct VP {
  // H: suffix tokens per sample (the action horizon; pi0: one state token
  // more, token 0); M = B H rows
  int L, W, Hq, Hkv, d, F, H, A, S, N, B, P, M, n_norms, KS, kps;
  int pi0;                 // variant: 0 pi0.5 (adaptive norms), 1 pi0 (state token, action-time MLP)
  int bigm;                // graph / eager launch of a bf16 expert with many rows: large-tile GEMM kernels
  int gp_bm[5];            // large-M GEMMs: tokens per tile (128 or 64; 224 or 256: 256-column tiles), same order as gp_nt
  int gp_nt[5], gp_s[5];   // GEMM plan (qkv, o, gateup, down, time MLP out): tiles per unit, K splits
  int S_o, S_down;         // = gp_s[1], gp_s[3]
  float eps;
  const uint8_t* w_qkv[MAX_LAYERS];   // packed [N/16][K/KB][64][16 B]
  const uint8_t* w_o[MAX_LAYERS];
  const uint8_t* w_gu[MAX_LAYERS];
  const uint8_t* w_down[MAX_LAYERS];
  const float *in_w, *in_b, *st_w, *st_b, *out_w, *out_b;   // f32 copies (pi0: in_w = W_in W_mi[:W], in_b unused)
  const uint8_t* w_tmlp;   // pi0: packed time-MLP output weight [W][W]
  const float* tbias;      // pi0: [N][W] b_in W_mi[:W] + sincos(t_k) W_mi[W:] + b_mi
  const float* tmlp_b;     // pi0: [W] time-MLP output bias
  const float* mod;        // [N][2L+1][3][W]  (scale, shift, gate) per step and norm
  const float* rope;       // [H][d/2][2]      (cos, sin) at positions P..P+H-1
  const void* prefix_k;    // [L][B][P][Hkv][d] act type
  const void* prefix_v;
  const float* noise;      // [B][H][A]
  const float* state;      // [B][S]
  float* x;                // [B][H][A]  actions, updated in place
  float* s_emb;            // [M][W]     state embedding, per action token
  float* h;                // [M][W]     residual stream
  // write-once activation ring: one slab per (step, layer) holding, at the
  // offsets below, q [B][Hq][d/16][64][16], k and v [B][Hkv][d/16][64][16]
  // and the GEMM inputs in MFMA operand order [K/KB][Mpad][KB]: xn_attn
  // (K = W), attn (K = Hq*d), xn_mlp (K = W), act (K = F)
  uint8_t* ring;
  size_t slab;
  size_t off_xna, off_q, off_k, off_v, off_attn, off_xnm, off_act, off_u;   // off_u: pi0 time-MLP hidden (slab of layer 0)
  void* opart;             // [B*Hq*KS*64][d]  unnormalised split outputs (activation type)
  float* ml;               // [B*Hq*KS*64][2]  (max, sum) per split row, log2 domain
  float* part_o;           // [S_o][M][W]  K-split partial sums of the o projection
  float* part_d;           // [S_down][M][W] ... of the down projection
  const float* qs;         // FP8 weights: [L][4 GEMMs][alpha, 1/act_scale]
  float* amax;             // calibration: [L][4 GEMMs] largest |input| (null: off)
  unsigned* bar;           // grid-barrier words
  unsigned long long* trace;  // optional phase timeline of the persistent kernel (null: off)
  long spin_limit;         // polls before a barrier wait gives up
  unsigned* herr;          // host-mapped error word (set with a system-scope store when a wait gives up)
  int fail_epoch;          // diagnostics: barrier whose target is never reached (0: none)
  // Norms folded into the GEMMs (persistent kernel, bf16 pi0.5 experts). The
  // o and down projections finish the residual in the epilogue of the last
  // K split of a tile to arrive and write y = h (1 + scale) of the next norm
  // plus per-16-column sums of squares of h; qkv and gate/up compute
  // r (y W) + shift W, r = 1 / sqrt(mean(h^2) + eps).
  int fuse;                // 1: the fused kernel runs
  const float* shw_q;      // [N][L][Nqkv] shift W of each attention norm (packed column order)
  const float* shw_g;      // [N][L][2F]   ... of each MLP norm
  size_t off_ssa;          // slab offset of [Mpad][W/16] f32: sums of squares of h over each 16 columns, before qkv
  size_t off_ssm;          // ... before gate/up
  unsigned* fcnt;          // arrival counters: [2 (o, down)][FCNT_MAX]; zero between launches
  int xl;                  // bit 0: the o / down split units of a column group share an XCD (see ph_gemm);
                           // bit 1: the attention splits of a head share one (attn_unit);
                           // XL_MERGE: the separate-norm persistent kernel merges the attention splits in
                           // place (see ph_attn; the folded-norm kernel always does)
  unsigned* xcnt;          // their XCD-local arrival counters, [2][FCNT_MAX] at XCNT_STRIDE words
  unsigned* hcnt;          // attention heads' arrival counters, [HCNT_MAX] at HCNT_STRIDE words; zero between launches
  unsigned* qcnt;          // qkv tiles stored per query head [QCNT_KV] and per key / value head [QCNT_KV], same stride
};
constexpr int XL_MERGE = 4;
constexpr int HCNT_MAX = 1024;   // samples x query heads the folded attention merge takes
constexpr int HCNT_STRIDE = 32;
constexpr int QCNT_KV = 64;      // query heads the folded kernel takes (the kv counters follow)
constexpr int FCNT_MAX = 4096;   // counters per split GEMM: 16-column tile groups x 64-row tiles
constexpr int XCNT_STRIDE = 32;  // one 128-byte line per XCD-local counter
constexpr int XCNT_WORDS = 2 * FCNT_MAX * XCNT_STRIDE;
constexpr int BAR_XL_BAD = 32;   // grid-barrier word: set when a workgroup runs off its XCD (blockIdx % 8)

// Kernel sets: activation type x weight format (x calibration).
enum KernelSetId { KS_F32 = 0, KS_BF16 = 1, KS_FP8 = 2, KS_W4 = 3, KS_CAL = 4, KS_I8 = 5, KS_W4A8 = 6 };
constexpr int ATT_KEYS_HOST = 64;   // keys per attention split (the kernels' ATT_KEYS)
constexpr int MAX_A_HOST = 64;      // largest action dim (the kernels' MAX_A)

size_t lds_bytes(const VP& p, int act_bytes);
hipError_t prepare_kernels(int kset, int d, int lds);
// mode 0: persistent kernel (cooperative launch), 3: persistent kernel
// (ordinary launch), otherwise the single phase `phase` at step k, layer l.
hipError_t launch_phase(const VP& p, int kset, int mode, int phase, int k, int l, int grid, size_t lds,
                        hipStream_t st);
hipError_t max_cooperative_grid(int kset, int d, size_t lds, int* grid);

// create-time preparation (vfm_prep.hip)
hipError_t pack_weight(uint8_t* dst, int K, int Npk, const int* d_col_src, const int* d_col_idx,
                       const void* s0, int n0, const void* s1, int n1, const void* s2, int n2,
                       int src_bf16, int dst_bf16, hipStream_t st);
hipError_t to_f32(float* dst, const void* src, size_t n, int src_bf16, hipStream_t st);
// quantised packing (bf16 masters): fmt 0 = FP8 e4m3 per tensor (scale from
// *amax), 1 = int4 with fp16 scales per (column, 128-K group), 2 = int8 with
// fp32 scales per output column
hipError_t amax_into(unsigned* out, const void* src, size_t n, int src_bf16, hipStream_t st);
hipError_t pack_weight_q(uint8_t* dst, int fmt, int K, int Npk, const int* d_col_src, const int* d_col_idx,
                         const void* s0, int n0, const void* s1, int n1, const void* s2, int n2, const unsigned* amax,
                         hipStream_t st);
hipError_t fp8_to_bf16_packed(uint8_t* dst, const uint8_t* src, int K, int Npk, const unsigned* amax, hipStream_t st);
hipError_t w4_to_bf16_packed(uint8_t* dst, const uint8_t* src, int K, int Npk, hipStream_t st);
hipError_t build_mod_table(float* tab, const void* const* mod_w, const void* const* mod_b, int n_norms,
                           const void* t1w, const void* t1b, const void* t2w, const void* t2b,
                           int N, int E, int W, int src_bf16, double* scratch, hipStream_t st);
// pi0: plain-norm modulation rows (w, 0, 1), the folded action projection
// fold = W_in W_mi[:W] ([A][W]) and the per-step bias tbias ([N][W]); scratch >= N W doubles
hipError_t build_pi0_tables(float* mod, const void* const* norm_w, int n_norms, float* fold, float* tbias,
                            const void* in_w, const void* in_b, const void* wmi, const void* bmi, int A, int W, int N,
                            int src_bf16, double* scratch, hipStream_t st);
hipError_t build_rope(float* rope, int H, int d, int P, float base, hipStream_t st);
hipError_t zero_words(unsigned* p, int n, hipStream_t st);
hipError_t copy_probe(const void* src, void* dst, size_t bytes, int policy, hipStream_t st);

}  // namespace vfm
