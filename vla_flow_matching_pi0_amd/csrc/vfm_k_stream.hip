// vfm_k_stream.hip -- instantiates the streaming batch-1 kernel (vfm_stream.h)
// for head dims 64, 128 and 256, and the create-time shift x W tables.
#include "vfm_stream.h"

namespace vfm {
namespace sk {

template <int D>
static hipError_t launch_d(const SP& p, size_t lds, hipStream_t st, bool coop) {
  void* args[] = {const_cast<SP*>(&p)};
  const void* f = reinterpret_cast<const void*>(&k_stream<D>);
  if (coop) return hipLaunchCooperativeKernel(f, dim3(p.G), dim3(NT), args, (unsigned)lds, st);
  return hipLaunchKernel(f, dim3(p.G), dim3(NT), args, lds, st);
}

hipError_t stream_launch(const SP& p, size_t lds, hipStream_t st, bool cooperative) {
  switch (p.d) {
    case 64: return launch_d<64>(p, lds, st, cooperative);
    case 128: return launch_d<128>(p, lds, st, cooperative);
    case 256: return launch_d<256>(p, lds, st, cooperative);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
static const void* kernel_of() { return reinterpret_cast<const void*>(&k_stream<D>); }
static const void* kernel_for(int d) {
  return d == 64 ? kernel_of<64>() : d == 128 ? kernel_of<128>() : d == 256 ? kernel_of<256>() : nullptr;
}

hipError_t stream_prepare(int d, int lds) {
  const void* f = kernel_for(d);
  if (!f) return hipErrorInvalidValue;
  return hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
}

hipError_t stream_occupancy(int d, size_t lds, int* per_cu) {
  const void* f = kernel_for(d);
  if (!f) return hipErrorInvalidValue;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, f, NT, lds);
}

// One thread per (step k, packed column pc) of one layer: fp64 sum over the
// K rows of the packed bf16 weight (lane order of the MFMA stream layout).
__global__ void k_shift_proj(float* out, size_t out_k_stride, const uint8_t* packed, int K, int Npk,
                             const float* mod, int n_norms, int ni, int W, int N) {
  const int nkb = K / 32;
  const size_t total = (size_t)N * Npk;
  for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < total; idx += (size_t)gridDim.x * blockDim.x) {
    const int pc = (int)(idx % Npk), k = (int)(idx / Npk);
    const int t = pc / 16, c16 = pc % 16;
    const float* shift = mod + (((size_t)k * n_norms + ni) * 3 + 1) * W;
    double s = 0.0;
    for (int n = 0; n < K; ++n) {
      const int kb = n / 32, g = (n % 32) / 8, e = n % 8;
      const uint16_t bits = *reinterpret_cast<const uint16_t*>(packed + (((size_t)t * nkb + kb) * 64 + c16 + 16 * g) * 16 + e * 2);
      const float wv = __builtin_bit_cast(float, (uint32_t)bits << 16);
      s += (double)shift[n] * (double)wv;
    }
    out[(size_t)k * out_k_stride + pc] = (float)s;
  }
}

// The same table for quantised weights, over the weights the GEMMs multiply
// by: fmt 1 (W4A16), bf16(q s) from the int4 codes q ([Npk/16][K/128][64
// lanes][4 words], word r the 8 nibbles of MFMA block r) and their fp16
// group scales s ([Npk/16][K/128][16], after the codes), each product
// rounded to bf16 as the GEMM's dequantisation does; fmt 2 (W8A16), the int8
// codes ([Npk/16][K/64][64 lanes][2 x 8 bytes]) times the fp32 column scales
// (after the codes), which the GEMM applies to its sums.
__global__ void k_shift_proj_q(float* out, size_t out_k_stride, const uint8_t* packed, int K, int Npk,
                               const float* mod, int n_norms, int ni, int W, int N, int fmt) {
  const size_t total = (size_t)N * Npk;
  for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < total; idx += (size_t)gridDim.x * blockDim.x) {
    const int pc = (int)(idx % Npk), k = (int)(idx / Npk);
    const int t = pc / 16, c16 = pc % 16;
    const float* shift = mod + (((size_t)k * n_norms + ni) * 3 + 1) * W;
    double s = 0.0;
    if (fmt == 1) {
      const int nkb = K / 128;
      const uint16_t* sc = reinterpret_cast<const uint16_t*>(packed + (size_t)Npk * K / 2);
      for (int n = 0; n < K; ++n) {
        const int kb = n / 128, r = (n % 128) / 32, g = (n % 32) / 8, e = n % 8;
        const uint32_t wd = *reinterpret_cast<const uint32_t*>(packed + (((size_t)t * nkb + kb) * 64 + c16 + 16 * g) * 16 + 4 * r);
        const int q = ((int)(wd << (28 - 4 * e))) >> 28;
        const float gs = (float)__builtin_bit_cast(_Float16, sc[((size_t)t * nkb + kb) * 16 + c16]);
        const float wv = (float)(bf16)((float)q * gs);
        s += (double)shift[n] * (double)wv;
      }
    } else {
      const int nkb = K / 64;
      const float csc = reinterpret_cast<const float*>(packed + (size_t)Npk * K)[pc];
      for (int n = 0; n < K; ++n) {
        const int kb = n / 64, r = (n % 64) / 32, g = (n % 32) / 8, e = n % 8;
        const int8_t q = *reinterpret_cast<const int8_t*>(packed + (((size_t)t * nkb + kb) * 64 + c16 + 16 * g) * 16 + 8 * r + e);
        s += (double)shift[n] * (double)q;
      }
      s *= (double)csc;
    }
    out[(size_t)k * out_k_stride + pc] = (float)s;
  }
}

hipError_t shift_proj_q(float* out, const uint8_t* const* packed, int L, int K, int Npk, const float* mod, int n_norms,
                        int which, int W, int N, int fmt, hipStream_t st) {
  for (int l = 0; l < L; ++l) {
    const size_t total = (size_t)N * Npk;
    const int blocks = (int)((total + 255) / 256);
    hipLaunchKernelGGL(k_shift_proj_q, dim3(blocks), dim3(256), 0, st, out + (size_t)l * Npk, (size_t)L * Npk, packed[l],
                       K, Npk, mod, n_norms, 2 * l + which, W, N, fmt);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t shift_proj(float* out, const uint8_t* const* packed, int L, int K, int Npk, const float* mod, int n_norms,
                      int which, int W, int N, hipStream_t st) {
  for (int l = 0; l < L; ++l) {
    const size_t total = (size_t)N * Npk;
    const int blocks = (int)((total + 255) / 256);
    hipLaunchKernelGGL(k_shift_proj, dim3(blocks), dim3(256), 0, st, out + (size_t)l * Npk, (size_t)L * Npk, packed[l], K,
                       Npk, mod, n_norms, 2 * l + which, W, N);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace sk
}  // namespace vfm
