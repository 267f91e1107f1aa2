// Code packing and output un-permutation.
//
// "El balance de errores de la inferencia de pocos bits", sections 1 and 6:
// a low-bit format has to state its packing layout, which decides what the
// runtime must unpack. Layout used here (gptq.h): per row, code k (original
// column order) at bits [k*b, k*b+b) of an LSB-first stream of uint32 words,
// straddling into the next word when needed (3-bit: 32 codes per 3 words).
#include "common.h"

#include <algorithm>

namespace gq {

// One thread per output word (grid: words of a row in x, rows in y, so no
// 64-bit division); codes gathered through invperm (processing order ->
// original order) when given. Without invperm and with b = 2 or 4 the
// word's codes are one aligned 16- or 8-byte read.
__global__ void __launch_bounds__(256)
k_pack(const uint8_t* __restrict__ codes, int64_t ldc, const int32_t* __restrict__ invperm,
       int64_t d_out, int64_t nq, int bits, int64_t wpr, uint32_t* __restrict__ qw) {
  const int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (w >= wpr) return;
  const uint32_t mask = (1u << bits) - 1u;
  const int64_t bit0 = 32 * w;
  const int64_t k0 = bit0 / bits;
  const int64_t k1 = min(nq - 1, (bit0 + 31) / bits);
  for (int64_t r = blockIdx.y; r < d_out; r += gridDim.y) {
    const uint8_t* row = codes + r * ldc;
    uint32_t word = 0;
    const bool direct = invperm == nullptr && (bits == 2 || bits == 4) &&
                        (((uintptr_t)row & 15) == 0) && k0 + 32 / bits <= nq;
    if (direct && bits == 4) {
      const uint2 v = *reinterpret_cast<const uint2*>(row + k0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        word |= ((v.x >> (8 * i)) & 15u) << (4 * i);
        word |= ((v.y >> (8 * i)) & 15u) << (4 * i + 16);
      }
    } else if (direct && bits == 2) {
      const uint4 v = *reinterpret_cast<const uint4*>(row + k0);
      const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) word |= ((q[j] >> (8 * i)) & 3u) << (2 * (4 * j + i));
    } else {
      for (int64_t k = k0; k <= k1; ++k) {
        const int64_t src = invperm ? invperm[k] : k;
        const uint32_t c = row[src] & mask;
        const int64_t o = k * bits - bit0;
        word |= (o < 0) ? (c >> (-o)) : (c << o);
      }
    }
    qw[r * wpr + w] = word;
  }
}

hipError_t launch_pack(hipStream_t s, const uint8_t* codes, int64_t ldc, const int32_t* invperm,
                       int64_t d_out, int64_t n_quant, int bits, uint32_t* qweight) {
  const int64_t wpr = ceil_div(n_quant * bits, 32);
  const int64_t total = d_out * wpr;
  if (total == 0) return hipSuccess;
  // rows run along the grid's y dimension (at most 65535, looped beyond)
  hipLaunchKernelGGL(k_pack, dim3((unsigned)ceil_div(wpr, 256), (unsigned)std::min<int64_t>(d_out, 65535)),
                     dim3(256), 0, s, codes, ldc,
                     invperm, d_out, n_quant, bits, wpr, qweight);
  return hipGetLastError();
}

__global__ void __launch_bounds__(256)
k_unpack(const uint32_t* __restrict__ qw, int64_t d_out, int64_t nq, int bits, int64_t wpr,
         uint8_t* __restrict__ codes) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= d_out * nq) return;
  const int64_t r = id / nq, k = id % nq;
  const int64_t o = k * bits;
  const int64_t w = o >> 5;
  const int sh = (int)(o & 31);
  uint32_t v = qw[r * wpr + w] >> sh;
  if (sh + bits > 32) v |= qw[r * wpr + w + 1] << (32 - sh);
  codes[id] = (uint8_t)(v & ((1u << bits) - 1u));
}

hipError_t launch_unpack(hipStream_t s, const uint32_t* qweight, int64_t d_out, int64_t n_quant,
                         int bits, uint8_t* codes) {
  const int64_t total = d_out * n_quant;
  if (total == 0) return hipSuccess;
  const int64_t wpr = ceil_div(n_quant * bits, 32);
  hipLaunchKernelGGL(k_unpack, dim3((unsigned)ceil_div(total, 256)), dim3(256), 0, s, qweight,
                     d_out, n_quant, bits, wpr, codes);
  return hipGetLastError();
}

// w_hat[r][k] = Wf[r][invperm[k]], codes_out[r][k] = codes_p[r][invperm[k]]
__global__ void __launch_bounds__(256)
k_finish(const float* __restrict__ Wf, const uint8_t* __restrict__ codes_p,
         const int32_t* __restrict__ invperm, int64_t n, int64_t nq, float* __restrict__ w_hat,
         uint8_t* __restrict__ codes_out) {
  const int64_t r = blockIdx.x;
  for (int64_t k = threadIdx.x; k < n; k += 256) {
    const int64_t p = invperm[k];
    if (w_hat) w_hat[r * n + k] = Wf[r * n + p];
    if (codes_out && k < nq) codes_out[r * nq + k] = codes_p[r * nq + p];
  }
}

__global__ void k_gidx(const int32_t* __restrict__ invperm, int64_t nq, int group,
                       int32_t* __restrict__ g_idx) {
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (k < nq) g_idx[k] = invperm[k] / group;
}

hipError_t launch_finish(hipStream_t s, const float* Wf, const uint8_t* codes_p,
                         const int32_t* invperm, int64_t d_out, int64_t n, int64_t n_quant,
                         int group, float* w_hat, uint8_t* codes_out, int32_t* g_idx) {
  if (d_out > 0 && (w_hat || codes_out))
    hipLaunchKernelGGL(k_finish, dim3((unsigned)d_out), dim3(256), 0, s, Wf, codes_p, invperm, n,
                       n_quant, w_hat, codes_out);
  if (g_idx)
    hipLaunchKernelGGL(k_gidx, dim3((unsigned)ceil_div(n_quant, 256)), dim3(256), 0, s, invperm,
                       n_quant, group, g_idx);
  return hipGetLastError();
}

}  // namespace gq
