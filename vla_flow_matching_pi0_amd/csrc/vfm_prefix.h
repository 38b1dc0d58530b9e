// vfm_prefix.h -- launch parameters and host entry points of the prefix
// producer's kernels (vfm_prefix.hip), used by its runtime (vfm_prefix_rt.cpp).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "vfm.h"

namespace vfm {

// Error text for vfm_last_error() (defined with the expert's runtime).
vfm_status report(vfm_status s, const char* fmt, ...);

namespace pfx {

constexpr int TM = 128;   // tokens per GEMM tile
constexpr int TN = 128;   // output columns per GEMM tile
constexpr int TK = 64;    // K per pipeline stage
constexpr int AQ = 32;    // queries per attention workgroup (2 waves x 16)
constexpr int AK = 32;    // keys per attention tile
constexpr int MAX_SPLIT = 8;

enum Epi { EPI_PART = 0, EPI_GU = 1, EPI_QKV = 2 };

// One GEMM D[n][token] = sum_k A[n][k] B[token][k] over tiles of TN x TM.
// A: weights packed [N/16][K/32][64][16 B]; B: activations packed
// [Mpad/16][K/32][64][16 B] (lane (c, g) of a 16-row block holds row c,
// k = 32 kb + 8 g .. + 7).
struct GemmArgs {
  const uint8_t* A;
  const uint8_t* B;
  int N, K, M, Mpad, S;     // S: K splits (EPI_PART only)
  int bm;                   // EPI_PART: tokens per 256-column tile (part_plan), 0: 128 x 128 tiles
  int qkv_half;             // EPI_QKV: 128 x 64 tiles where 128 x 128 tiles would fill at most half the units
  int part_half;            // EPI_PART with bm = 0: 128 x 64 tiles (the caller halves S)
  // EPI_PART: part[s][Mpad][N] fp32
  float* part;
  // EPI_GU: act packed [Mpad/16][N/2/32][64][16 B] (gate/up interleaved columns)
  uint8_t* act;
  // EPI_QKV: packed columns [k heads | v heads | q heads], rotary pairs arranged
  // so that 4 consecutive columns hold dims (2j, 2j+1, 2j+d/2, 2j+1+d/2)
  uint16_t* k_out;          // [B][P][Hkv][d] of this layer
  uint16_t* v_out;
  uint16_t* q;              // [B*P][Hq][d]
  uint16_t* vt;             // [B][Hkv][d][Ppad]
  const float* rope;        // [P][d/2][2] (cos, sin) at positions 0..P-1
  int P, Ppad, Hq, Hkv, d;
};

struct AttnArgs {
  const uint16_t* q;        // [B*P][Hq][d]
  const uint16_t* k;        // [B][P][Hkv][d] (this layer's prefix keys)
  const uint16_t* vt;       // [B][Hkv][d][Ppad]
  uint8_t* out;             // packed [Mpad/16][Hq*d/32][64][16 B]
  int P, Ppad, Hq, Hkv;
  float scale_log2;         // log2(e) / sqrt(d)
};

struct NormArgs {
  const uint16_t* embeds;   // first layer: [M][W] bf16 token embeddings
  float* x;                 // [Mpad][W] residual stream
  const float* part;        // [S][Mpad][W] partial sums to add (S = 0: none)
  int S;
  const float* gain;        // [W] w of the (1 + w) gain
  uint8_t* xn;              // packed [Mpad/16][W/32][64][16 B]
  int M, Mpad, W;
  float eps;
};

// Tile plan of a K-split GEMM (EPI_PART): bm tokens per 256-column tile
// with S splits when that fills one round of at least 192 compute units with
// at least 1024 K per split and the tiles cover all Mpad rows; else bm = 0
// (128 x 128 tiles) with narrow_split splits.
struct PartPlan {
  int bm, S;
};
PartPlan part_plan(int M, int Mpad, int N, int K, int narrow_split, bool wide);

hipError_t prepare();
// wide_gu: the gate/up GEMM (epi EPI_GU) on the 256-column tiles where the shape takes them
hipError_t gemm(int epi, const GemmArgs& g, hipStream_t st, bool wide_gu = true);
hipError_t attention(int d, const AttnArgs& a, int B, hipStream_t st);
hipError_t norm(bool first, const NormArgs& n, hipStream_t st);

}  // namespace pfx
}  // namespace vfm
