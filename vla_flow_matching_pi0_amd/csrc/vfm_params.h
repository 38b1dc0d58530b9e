// vfm_params.h -- the launch-parameter block shared by the host runtime and
// the kernels, and the host entry points of the kernel translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace vfm {

constexpr int MAX_LAYERS = 48;

enum Phase {
  PH_INIT = 0, PH_IN_PROJ, PH_NORM_ATTN, PH_QKV, PH_ATTN, PH_COMBINE,
  PH_O, PH_NORM_MLP, PH_GU, PH_DOWN, PH_FINAL, PH_COUNT
};

// Everything a phase needs; passed by value as the kernel argument.
struct VP {
  int L, W, Hq, Hkv, d, F, H, A, S, N, B, P, M, n_norms, KS, kps;
  float eps;
  const uint8_t* w_qkv[MAX_LAYERS];   // packed [N/16][K/KB][64][16 B]
  const uint8_t* w_o[MAX_LAYERS];
  const uint8_t* w_gu[MAX_LAYERS];
  const uint8_t* w_down[MAX_LAYERS];
  const float *in_w, *in_b, *st_w, *st_b, *out_w, *out_b;   // f32 copies
  const float* mod;        // [N][2L+1][3][W]  (scale, shift, gate) per step and norm
  const float* rope;       // [H][d/2][2]      (cos, sin) at positions P..P+H-1
  const void* prefix_k;    // [L][B][P][Hkv][d] act type
  const void* prefix_v;
  const float* noise;      // [B][H][A]
  const float* state;      // [B][S]
  float* x;                // [B][H][A]  actions, updated in place
  float* s;                // [B][W]     state embedding
  float* h;                // [M][W]     residual stream
  void* xn;                // [M][W]     normalised activations (act type)
  void* q;                 // [B][Hq][H][d]
  void* ks;                // [B][Hkv][H][d]
  void* vs;
  float* opart;            // [B*Hq*KS*64][d]  unnormalised split outputs
  float* ml;               // [B*Hq*KS*64][2]  (max, sum) per split row, log2 domain
  void* attn;              // [M][Hq*d]
  void* act;               // [M][F]      GeGLU output
  unsigned* bar;           // grid-barrier words
};

size_t lds_bytes(const VP& p, int act_bytes);
hipError_t prepare_kernels(int act_bf16, int d, int lds);
hipError_t launch_phase(const VP& p, int act_bf16, int mode, int phase, int k, int l, int grid, size_t lds,
                        hipStream_t st);
hipError_t max_cooperative_grid(int act_bf16, int d, size_t lds, int* grid);

// create-time preparation (vfm_prep.hip)
hipError_t pack_weight(uint8_t* dst, int K, int Npk, const int* d_col_src, const int* d_col_idx,
                       const void* s0, int n0, const void* s1, int n1, const void* s2, int n2,
                       int src_bf16, int dst_bf16, hipStream_t st);
hipError_t to_f32(float* dst, const void* src, size_t n, int src_bf16, hipStream_t st);
hipError_t build_mod_table(float* tab, const void* const* mod_w, const void* const* mod_b, int n_norms,
                           const void* t1w, const void* t1b, const void* t2w, const void* t2b,
                           int N, int E, int W, int src_bf16, double* scratch, hipStream_t st);
hipError_t build_rope(float* rope, int H, int d, int P, float base, hipStream_t st);
hipError_t zero_words(unsigned* p, int n, hipStream_t st);

}  // namespace vfm
