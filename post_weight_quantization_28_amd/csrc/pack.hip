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

// One workgroup per row with the row's codes staged in LDS (16-byte reads):
// the permuted or 3-bit straddling gathers then read LDS, not scattered
// bytes of memory. Rows of up to 64 KiB of codes.
__global__ void __launch_bounds__(256)
k_pack_lds(const uint8_t* __restrict__ codes, int64_t ldc, const int32_t* __restrict__ invperm, int64_t nq,
           int bits, int64_t wpr, uint32_t* __restrict__ qw) {
  extern __shared__ __align__(16) uint8_t crow[];
  const int64_t r = blockIdx.x;
  const uint8_t* row = codes + r * ldc;
  const bool vec = ((ldc & 15) == 0) && (((uintptr_t)codes & 15) == 0);
  const int64_t n16 = vec ? nq / 16 : 0;
  for (int64_t v = threadIdx.x; v < n16; v += 256)
    *reinterpret_cast<uint4*>(crow + 16 * v) = *reinterpret_cast<const uint4*>(row + 16 * v);
  for (int64_t k = 16 * n16 + threadIdx.x; k < nq; k += 256) crow[k] = row[k];
  __syncthreads();
  const uint32_t mask = (1u << bits) - 1u;
  for (int64_t w = threadIdx.x; w < wpr; w += 256) {
    const int64_t bit0 = 32 * w;
    const int64_t k0 = bit0 / bits;
    const int64_t k1 = min(nq - 1, (bit0 + 31) / bits);
    uint32_t word = 0;
    for (int64_t k = k0; k <= k1; ++k) {
      const uint32_t c = crow[invperm ? invperm[k] : k] & mask;
      const int64_t o = k * bits - bit0;
      word |= (o < 0) ? (c >> (-o)) : (c << o);
    }
    qw[r * wpr + w] = word;
  }
}

hipError_t launch_pack(hipStream_t s, const uint8_t* codes, int64_t ldc, const int32_t* invperm,
                       int64_t d_out, int64_t n_quant, int bits, uint32_t* qweight) {
  const int64_t wpr = ceil_div(n_quant * bits, 32);
  const int64_t total = d_out * wpr;
  if (total == 0) return hipSuccess;
  if ((invperm || bits == 3) && n_quant <= 65536) {
    hipLaunchKernelGGL(k_pack_lds, dim3((unsigned)std::min<int64_t>(d_out, 1ll << 31)), dim3(256), (size_t)n_quant, s,
                       codes, ldc, invperm, n_quant, bits, wpr, qweight);
    return hipGetLastError();
  }
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

// The same with the row of Wf and of the codes staged in LDS (coalesced
// reads, the permuted gather in LDS, coalesced writes).
__global__ void __launch_bounds__(256)
k_finish_lds(const float* __restrict__ Wf, const uint8_t* __restrict__ codes_p,
             const int32_t* __restrict__ invperm, int64_t n, int64_t nq, float* __restrict__ w_hat,
             uint8_t* __restrict__ codes_out, int vec) {
  extern __shared__ __align__(16) float frow[];
  uint8_t* crow = reinterpret_cast<uint8_t*>(frow + n);
  const int64_t r = blockIdx.x;
  if (vec) {
    // n % 4 == 0, nq % 16 == 0 and 16-byte aligned rows: 16-byte loads, four
    // gathered values per store
    if (w_hat)
      for (int64_t k = threadIdx.x; k < n / 4; k += 256)
        reinterpret_cast<float4*>(frow)[k] = reinterpret_cast<const float4*>(Wf + r * n)[k];
    if (codes_out)
      for (int64_t k = threadIdx.x; k < nq / 16; k += 256)
        reinterpret_cast<uint4*>(crow)[k] = reinterpret_cast<const uint4*>(codes_p + r * nq)[k];
    __syncthreads();
    for (int64_t k0 = 4 * (int64_t)threadIdx.x; k0 < n; k0 += 1024) {
      const int4 pv = *reinterpret_cast<const int4*>(invperm + k0);
      if (w_hat)
        *reinterpret_cast<float4*>(w_hat + r * n + k0) = make_float4(frow[pv.x], frow[pv.y], frow[pv.z], frow[pv.w]);
      if (codes_out && k0 < nq)
        *reinterpret_cast<uchar4*>(codes_out + r * nq + k0) = make_uchar4(crow[pv.x], crow[pv.y], crow[pv.z], crow[pv.w]);
    }
    return;
  }
  if (w_hat)
    for (int64_t k = threadIdx.x; k < n; k += 256) frow[k] = Wf[r * n + k];
  if (codes_out)
    for (int64_t k = threadIdx.x; k < nq; k += 256) crow[k] = codes_p[r * nq + k];
  __syncthreads();
  for (int64_t k = threadIdx.x; k < n; k += 256) {
    const int64_t p = invperm[k];
    if (w_hat) w_hat[r * n + k] = frow[p];
    if (codes_out && k < nq) codes_out[r * nq + k] = crow[p];
  }
}

hipError_t launch_finish(hipStream_t s, const float* Wf, const uint8_t* codes_p,
                         const int32_t* invperm, int64_t d_out, int64_t n, int64_t n_quant,
                         int group, float* w_hat, uint8_t* codes_out, int32_t* g_idx) {
  const size_t lds = (size_t)n * sizeof(float) + (size_t)n_quant;
  const int vec = n % 4 == 0 && n_quant % 16 == 0 && ((uintptr_t)Wf & 15) == 0 && ((uintptr_t)codes_p & 15) == 0 &&
                  ((uintptr_t)invperm & 15) == 0 && ((uintptr_t)w_hat & 15) == 0 && ((uintptr_t)codes_out & 3) == 0;
  if (d_out > 0 && (w_hat || codes_out) && lds <= 65536)
    hipLaunchKernelGGL(k_finish_lds, dim3((unsigned)d_out), dim3(256), lds, s, Wf, codes_p, invperm, n,
                       n_quant, w_hat, codes_out, vec);
  else if (d_out > 0 && (w_hat || codes_out))
    hipLaunchKernelGGL(k_finish, dim3((unsigned)d_out), dim3(256), 0, s, Wf, codes_p, invperm, n,
                       n_quant, w_hat, codes_out);
  if (g_idx)
    hipLaunchKernelGGL(k_gidx, dim3((unsigned)ceil_div(n_quant, 256)), dim3(256), 0, s, invperm,
                       n_quant, group, g_idx);
  return hipGetLastError();
}

}  // namespace gq

namespace gq {

// Round-to-nearest of a matrix on the affine grid of the quantizer (range
// widened to 0, (-1, 1) when degenerate, s = (xmax - xmin) / maxq,
// z = rint(-xmin / s), q = clamp(rint(x / s) + z, 0, maxq), x_hat = s (q - z)),
// groups of `group` consecutive columns of a row; one wave per (row, group).
// "Resumen Técnico: GPTQ-intrinsic LoRA", "Resultados Clave": the low-rank
// factors themselves quantized to 4 and 8 bits.
__global__ void __launch_bounds__(64)
k_rtn(const float* __restrict__ X, int64_t ldx, int64_t cols, int group, float maxq, uint8_t* __restrict__ codes,
      float* __restrict__ scales, uint8_t* __restrict__ zeros, float* __restrict__ xh) {
  const int64_t r = blockIdx.y, g = blockIdx.x, ng = cols / group;
  const int lane = threadIdx.x;
  const float* x = X + r * ldx + g * group;
  float mn = INFINITY, mx = -INFINITY;
  for (int c = lane; c < group; c += 64) {
    mn = fminf(mn, x[c]);
    mx = fmaxf(mx, x[c]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, o));
    mx = fmaxf(mx, __shfl_xor(mx, o));
  }
  float xmin = fminf(mn, 0.f), xmax = fmaxf(mx, 0.f);
  if (xmin == xmax) {
    xmin = -1.f;
    xmax = 1.f;
  }
  const float s = (xmax - xmin) / maxq;
  const float z = rintf(-xmin / s);
  if (lane == 0) {
    scales[r * ng + g] = s;
    zeros[r * ng + g] = (uint8_t)z;
  }
  for (int c = lane; c < group; c += 64) {
    const float q = fminf(fmaxf(rintf(x[c] / s) + z, 0.f), maxq);
    codes[r * cols + g * group + c] = (uint8_t)q;
    if (xh) xh[r * cols + g * group + c] = s * (q - z);
  }
}

hipError_t launch_rtn(hipStream_t s, const float* X, int64_t ldx, int64_t rows, int64_t cols, int bits, int group,
                      uint8_t* codes, float* scales, uint8_t* zeros, float* xh) {
  if (rows == 0 || cols == 0) return hipSuccess;
  hipLaunchKernelGGL(k_rtn, dim3((unsigned)(cols / group), (unsigned)rows), dim3(64), 0, s, X, ldx, cols, group,
                     (float)((1 << bits) - 1), codes, scales, zeros, xh);
  return hipGetLastError();
}

}  // namespace gq
