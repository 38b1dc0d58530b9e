// vfm_stream_params.h -- launch parameters of the streaming batch-1 kernel
// (vfm_stream.h), shared by the host runtime and the kernel.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "vfm_params.h"

namespace vfm {
typedef __bf16 bf16;
namespace sk {

constexpr int NCW = 8;                 // compute waves per workgroup
constexpr int NT = (NCW + 1) * 64;     // + the loader wave
constexpr int LOADER = NCW;
constexpr int NXCD = 8;
constexpr int MAXJ = 16;               // act fragments per wave per GEMM (K slice <= 1024)
constexpr int UMAX = 2;                // GEMM units per workgroup
constexpr int AUMAX = 2;               // attention units per workgroup
constexpr int SMAX = 8;                // K splits of the o and down projections
constexpr int CTL = 256;               // bytes of LDS control words (64 words)
constexpr int DMA_CAP = 56;            // loader: default of the most direct-to-LDS loads in flight
constexpr long SPIN_LIMIT = 1L << 21;

enum { GQ = 0, GO = 1, GG = 2, GD = 3 };
// barrier words: [0] exit count, [64 + 64 x] slot count of XCD x, [1024 + 64 c] arrival counter c
constexpr int BW_EXIT = 0, BW_SLOT = 64, BW_CTR = 1024, N_CTR = 64;
constexpr int BAR_WORDS_S = BW_CTR + 64 * N_CTR;
// control words in LDS: workgroup id, barrier outcome, last-arriver flags
// (UMAX), compute-wave barrier counter, GEMM phases completed (regions the
// loader may refill), fills landed, stop request to the loader, failed
// weight wait, the workgroup's unit entries: GEMMs (4 x UMAX), attention
// (AUMAX), in projection (IUMAX)
constexpr int IUMAX = 4;
enum { C_WID = 0, C_OK = 1, C_LAST = 4, C_CWB = 8, C_FREE = 9, C_LAND = 10, C_ABORT = 11, C_LFAIL = 12, C_UNITS = 16,
       C_AUNITS = 32, C_IUNITS = 36 };
static_assert(C_IUNITS + IUMAX <= CTL / 4, "control words exceed their LDS block");
static_assert(C_UNITS + 4 * UMAX <= C_AUNITS && C_AUNITS + AUMAX <= C_IUNITS, "control word overlap");

struct SGemm {
  int T, S, nkb, nkbs, U;    // 16-column tiles, K splits, 32-K blocks (all, per split), units per workgroup
  int region;                // LDS byte offset of the weight region
  const uint32_t* units;     // [G][U]: (tile << 8) | split, 0xFFFFFFFF = none
  unsigned* cnt;             // [T] arrival counters (split GEMMs)
  float* part;               // [S][T][64][16] partial sums (split GEMMs)
};

// Launch parameters (kernel argument).
struct SP {
  int L, W, Hq, Hkv, d, F, H, A, S, N, P, Ppad, KS, KSp;
  int G, per_xcd, AU, IU;
  float eps;
  int scratch, ctl;          // LDS byte offsets
  const uint8_t* w[4][MAX_LAYERS];
  SGemm g[4];
  const uint32_t* attn_units;   // [G][AU] (head << 8) | split
  const uint32_t* in_units;     // [G][IU] (tile << 8), 0xFFFFFFFF = none
  unsigned* hcnt;               // [Hq] attention-merge counters
  const float* mod;             // [N][2L+1][3][W]
  const float* shw_q;           // [N][L][(Hq+2Hkv)d] shift x W_qkv, packed column order
  const float* shw_g;           // [N][L][2F] shift x W_gateup, packed column order
  const float* rope;            // [H][d/2][2]
  const bf16* pk;               // prefix keys [L][1][P][Hkv][d]
  const bf16* pv;               // prefix values
  bf16* vt;                     // prefix values transposed [L][Hkv][d][Ppad], keys permuted per 32
  const float* noise;
  const float* state;
  float* x;                     // actions [H][A]
  const float *in_w, *in_b, *st_w, *st_b, *out_w, *out_b;
  float* s_emb;                 // [64][W]
  float* h;                     // [64][W] residual stream
  uint8_t* ring;                // one slab per (step, layer), written once per launch
  size_t slab, o_ya, o_ssa, o_q, o_k, o_vt, o_at, o_ym, o_ssm, o_act;
  float* apart;                 // [Hq][KS][64][d] attention split outputs (unnormalised)
  float* aml;                   // [Hq][KS][64][2] (max, sum), log2 domain
  unsigned* bar;
  unsigned* err;                // sticky error word: kernels OR into it, the host clears it
  unsigned* herr;               // host-mapped copy of the error word (may be null)
  unsigned long long* trace;    // optional timeline of workgroup 0's barriers
  int stop_after;               // diagnostics: leave after this barrier (0: run the whole loop)
  int dma_cap;                  // loader: most direct-to-LDS loads in flight (1 .. 63)
  int fail_epoch;               // diagnostics: barrier whose target is never reached (0: none)
  long spin_limit;              // polls before a device-wide or head wait gives up
};

hipError_t stream_launch(const SP& p, size_t lds, hipStream_t st, bool cooperative);
hipError_t stream_prepare(int d, int lds);
hipError_t stream_occupancy(int d, size_t lds, int* per_cu);
// out[k][l][pc] = sum_n shift(k, norm of l)[n] W_l[n][pc] over the packed bf16
// weight W_l (K x Npk), for every step k; norm = 2 l + which (0: attention, 1: MLP)
hipError_t shift_proj(float* out, const uint8_t* const* packed, int L, int K, int Npk, const float* mod, int n_norms,
                      int which, int W, int N, hipStream_t st);
// ... over quantised weights: fmt 1 W4A16, 2 W8A16 (vfm_k_stream.hip)
hipError_t shift_proj_q(float* out, const uint8_t* const* packed, int L, int K, int Npk, const float* mod, int n_norms,
                        int which, int W, int N, int fmt, hipStream_t st);

}  // namespace sk
}  // namespace vfm
