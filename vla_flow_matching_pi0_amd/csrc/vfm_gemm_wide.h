// vfm_gemm_wide.h -- the pipeline of the 256-column large-M GEMM tiles,
// shared by the action expert's many-row launches (vfm_phases.h) and the
// prefix producer (vfm_prefix.hip).
//
// A workgroup (one per compute unit, four waves) computes 256 output
// columns x 32 MB tokens: wave w takes columns 128 (w & 1) .. + 127 and
// tokens 16 MB (w >> 1) .. + 16 MB - 1, so that a 32-K step reads 8 + MB
// operand fragments per wave for 8 MB MFMAs (16x16x32 bf16), with the
// accumulators (32 MB registers) in the accumulation half of the unified
// register file. Both operand tiles go from global memory straight into an
// LDS ring of NS stages of 32 K (direct-to-LDS loads of 16 bytes per lane,
// no registers), issued NS - 1 stages ahead of their use. The copies are
// inline asm: the compiler would otherwise treat each later LDS read as
// possibly aliasing a copy in flight and wait for all of them; each wave
// waits for its own copies by count instead. One barrier per stage: after
// it the stage has landed everywhere and every wave is done with the
// previous stage, whose slot the copies issued during this stage refill.
// Within the stage the weight fragments are read two MFMA groups ahead of
// their use and the copies are spread over the groups, so that the MFMAs
// cover both.
//
// LDS of one stage: blocks 0..15 hold the 16 weight column tiles (1 KiB:
// 16 columns x 32 K in the MFMA lane order), blocks 16 .. 16 + 2 MB - 1 the
// token blocks (16 tokens x 32 K, same order).
#pragma once
#include <stdint.h>

#include "vfm_device.h"

namespace vfm {

constexpr int GW_THREADS = 256;
constexpr int GW_LDS_MAX = 160 * 1024;

template <int MB>
struct GW {
  static constexpr int NB = 16 + 2 * MB;   // 1 KiB blocks per 32-K stage: 16 of weights, 2 MB of tokens
  static constexpr int SLOT = NB * 1024;
  // copies per wave and stage, the same for every wave (so that every wait
  // is one immediate): blocks w, w + 4, ...; a wave with a slot left over
  // copies its first block once more into a spare KiB past the ring
  static constexpr int CW = (NB + 3) / 4;
  static constexpr int SPARE = (4 * CW - NB) * 1024;
  static constexpr int NS = (GW_LDS_MAX - 4096) / SLOT >= 5 ? 5 : (GW_LDS_MAX - 4096) / SLOT;
  static constexpr int LDS = NS * SLOT + SPARE;
  static constexpr int BMT = 32 * MB;                          // tokens per tile
  static_assert(NS >= 4, "the ring needs four stages");
  static_assert((NS - 2) * CW <= 63, "vmcnt range");
  static_assert(CW <= 8, "one copy per MFMA group");
  static_assert(16 * MB * 1024 <= NS * SLOT, "the epilogue's staging fits in the ring");
};

template <int N>
__device__ __forceinline__ void gw_vmcnt() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
__device__ __forceinline__ void gw_barrier() { asm volatile("s_barrier" ::: "memory"); }
// one direct-to-LDS copy of 16 bytes per lane: global base + voff -> LDS m0 + 16 lane
__device__ __forceinline__ void gw_copy(const void* base, uint32_t voff, uint32_t lds_dst) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_dst), "v"(voff), "s"(base)
               : "memory", "m0");
}


// acc[i][j] += the product of weight column tile 8 (w & 1) + i and token
// block MB (w >> 1) + j over nst stages. voff[i]: this wave's copy i of
// stage 0 (the block w + 4 i of a stage: weight tiles for i < 4, token
// blocks after), as a byte offset from wsrc (i < 4) or act; a stage further
// is 1024 bytes further for the weights and astep for the tokens. Requires
// nst even and nst >= NS - 1; every copy has landed when it returns.
template <int MB>
__device__ __forceinline__ void gw_mainloop(floatx4 (&acc)[8][MB], uint8_t* lds, const uint8_t* wsrc,
                                            const uint8_t* act, const uint32_t (&voff)[GW<MB>::CW], uint32_t astep,
                                            int nst, int w, int lane) {
  using C = GW<MB>;
  const int wn = w & 1, wm = w >> 1;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds;
  const u32x4* L = reinterpret_cast<const u32x4*>(lds);
  auto frag_a = [&](int st, int i) { return L[(st % C::NS) * (C::SLOT / 16) + (wn * 8 + i) * 64 + lane]; };
  auto frag_b = [&](int st, int j) { return L[(st % C::NS) * (C::SLOT / 16) + (16 + wm * MB + j) * 64 + lane]; };

  // Every stage issues the same copies (CW per wave: the stages past the
  // last one copy the last one again, into the slot that is free anyway), so
  // every wait is the same immediate and the loop body is straight-line code
  // but for the wait's branch: the copies' and reads' issue can hide behind
  // the MFMAs.
  constexpr int CW = C::CW;
  const int nreal = (C::NB - w + 3) / 4;   // this wave's real copies; the rest repeat copy 0 into a spare KiB
  const uint32_t spare = lds0 + (uint32_t)(C::NS * C::SLOT + (w & 1) * 1024);
  // copy i of stage cst into slot `slot`
  auto copy = [&](int i, int cst, int slot) {
    const uint32_t dst = lds0 + (uint32_t)(slot * C::SLOT + w * 1024 + 4096 * i);
    if (i < 4) {
      gw_copy(wsrc, voff[i] + (uint32_t)cst * 1024u, dst);
    } else {
      const bool real = i < nreal;
      gw_copy(real ? act : wsrc, real ? voff[i] + (uint32_t)cst * astep : voff[0] + (uint32_t)cst * 1024u,
              real ? dst : spare);
    }
  };
  // prologue: stages 0 .. NS - 2 in flight (nst >= NS - 1)
#pragma unroll
  for (int st = 0; st < C::NS - 1; ++st)
#pragma unroll
    for (int i = 0; i < CW; ++i) copy(i, st, st);
  for (int st = 0; st < nst; ++st) {
    // this wave's copies of stage st have landed (the NS - 2 stages after it
    // may still be in flight), then the barrier: every wave's copies of stage
    // st have landed and every wave is done with stage st - 1, whose slot
    // this stage's copies refill (with stage st + NS - 1, or the last again)
    // (the last NS - 2 stages wait for every copy: the same for the stages
    // that count, and the branch keeps the register allocator from turning
    // the accumulation into copy-and-accumulate pairs, as it does when the
    // whole loop body is one basic block)
    if (st + C::NS - 2 < nst) gw_vmcnt<(C::NS - 2) * CW>();
    else gw_vmcnt<0>();
    gw_barrier();
    const int cst = st + C::NS - 1 < nst ? st + C::NS - 1 : nst - 1;
    const int cslot = (st + C::NS - 1) % C::NS;
    u32x4 fa[8], fb[MB];
    fa[0] = frag_a(st, 0);
#pragma unroll
    for (int j = 0; j < MB; ++j) fb[j] = frag_b(st, j);
    fa[1] = frag_a(st, 1);
    // Program order is kept (scheduling barriers): weight fragment i + 2 is
    // requested during MFMA group i, and copy i issued in its middle, so
    // that the MFMAs cover both the reads' latency and the copies' issue.
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < MB; ++j) {
        acc[i][j] = MT<bf16>::mma(fa[i], fb[j], acc[i][j]);
        if (j == 0 && i + 2 < 8) fa[i + 2] = frag_a(st, i + 2);
        if (j == 2 && i < CW) copy(i, cst, cslot);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  gw_vmcnt<0>();   // the repeated copies of the last stages land before the ring is reused or released
}

}  // namespace vfm
