// Preparation of the damped, ordered Hessian and the fp32 working weights.
//
// "Resumen Técnico: GPTQ-intrinsic LoRA", "Detalles de Implementación":
// standard GPTQ regularises the Hessian with lambda before its Cholesky
// factorisation (here lambda = damp * mean(diag H)).
// "GPTQ" (wikiprompt.org), "Enfoque Técnico": the weights to quantize are
// picked greedily (here: act-order, descending diag H, stable).
//
// The factorisation works on the index-reversed matrix A = J H_d J (J the
// reversal permutation): the lower Cholesky factor L of A gives the upper
// factor of H_d^{-1} as U = J L^{-1} J, so building A flipped here lets every
// later kernel work with lower-triangular storage.
#include "common.h"

#include <algorithm>

namespace gq {

__global__ void k_status_init(DevStatus* st) {
  st->flags = 0;
  st->pad = 0;
  st->col = ~0ull;
}

hipError_t launch_status_init(hipStream_t s, DevStatus* st) {
  hipLaunchKernelGGL(k_status_init, dim3(1), dim3(1), 0, s, st);
  return hipGetLastError();
}

__global__ void k_fill_f32(float* __restrict__ p, size_t count, float v) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) p[i] = v;
}

hipError_t launch_fill_f32(hipStream_t s, float* p, size_t count, float v) {
  if (count == 0) return hipSuccess;
  size_t blocks = (count + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(k_fill_f32, dim3((unsigned)blocks), dim3(256), 0, s, p, count, v);
  return hipGetLastError();
}

// diag[i] = H_ii (zero -> 1), lam = damp * mean(diag); one workgroup, fixed
// reduction order (per-thread strided partial sums in double, then a tree).
__global__ void __launch_bounds__(1024)
k_prep_diag(const float* __restrict__ H, int64_t n, float* __restrict__ diag,
            double* __restrict__ lam_out, float damp, DevStatus* st) {
  __shared__ double red[1024];
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += 1024) {
    float v = H[i * n + i];
    if (!isfinite(v)) raise_status(st, kNonFinite, i);
    if (v == 0.f) v = 1.f;
    diag[i] = v;
    acc += (double)v;
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) lam_out[0] = (double)damp * (red[0] / (double)n);
}

hipError_t launch_prep_diag(hipStream_t s, const float* H, int64_t n, float* diag,
                            double* lam_out, float damp, DevStatus* st) {
  hipLaunchKernelGGL(k_prep_diag, dim3(1), dim3(1024), 0, s, H, n, diag, lam_out, damp, st);
  return hipGetLastError();
}

// Stable descending rank over the first nq diagonal entries: NaN sorts
// last, equal keys keep index order, so the ranks are always a permutation.
__device__ inline float order_key(float d) { return isnan(d) ? -INFINITY : d; }

__global__ void __launch_bounds__(256)
k_order(const float* __restrict__ diag, int64_t n, int64_t nq, int act_order,
        int32_t* __restrict__ perm, int32_t* __restrict__ invperm) {
  __shared__ float keys[1024];
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool mine = i < nq;
  const float ki = mine ? order_key(diag[i]) : 0.f;
  int64_t rank = 0;
  if (act_order) {
    for (int64_t base = 0; base < nq; base += 1024) {
      __syncthreads();
      for (int t = threadIdx.x; t < 1024; t += 256)
        keys[t] = (base + t < nq) ? order_key(diag[base + t]) : 0.f;
      __syncthreads();
      if (mine) {
        const int64_t lim = min((int64_t)1024, nq - base);
        for (int64_t t = 0; t < lim; ++t) {
          const float kj = keys[t];
          const int64_t j = base + t;
          rank += (kj > ki) || (kj == ki && j < i);
        }
      }
    }
  } else {
    rank = i;
  }
  if (i < n) {
    const int64_t r = mine ? rank : i;
    perm[r] = (int32_t)i;
    invperm[i] = (int32_t)r;
  }
}

// The same ranks with the comparisons spread over a second grid dimension:
// workgroup (x, y) counts, for its 256 entries i, the keys of the y-th chunk
// of j that precede i, and adds the count to rank[i] (integer atomics: the
// sums do not depend on the order). rank must start at zero.
__global__ void __launch_bounds__(256)
k_rank_part(const float* __restrict__ diag, int64_t nq, int64_t jchunk, int32_t* __restrict__ rank) {
  __shared__ float keys[1024];
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool mine = i < nq;
  const float ki = mine ? order_key(diag[i]) : 0.f;
  const int64_t jlo = (int64_t)blockIdx.y * jchunk, jhi = min(nq, jlo + jchunk);
  int cnt = 0;
  for (int64_t base = jlo; base < jhi; base += 1024) {
    __syncthreads();
    for (int t = threadIdx.x; t < 1024; t += 256) keys[t] = (base + t < jhi) ? order_key(diag[base + t]) : 0.f;
    __syncthreads();
    if (mine) {
      const int lim = (int)min((int64_t)1024, jhi - base);
      for (int t = 0; t < lim; ++t) {
        const float kj = keys[t];
        const int64_t j = base + t;
        cnt += (kj > ki) || (kj == ki && j < i);
      }
    }
  }
  if (mine && cnt) atomicAdd(&rank[i], cnt);
}

// invperm holds the ranks of the first nq entries; the rest keep their place
__global__ void k_rank_write(int64_t n, int64_t nq, int32_t* __restrict__ perm, int32_t* __restrict__ invperm) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int32_t r = i < nq ? invperm[i] : (int32_t)i;
  invperm[i] = r;
  perm[r] = (int32_t)i;
}

hipError_t launch_order(hipStream_t s, const float* diag, int64_t n, int64_t n_quant,
                        int act_order, int32_t* perm, int32_t* invperm) {
  if (!act_order || n_quant <= 1024) {
    hipLaunchKernelGGL(k_order, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, diag, n,
                       n_quant, act_order, perm, invperm);
    return hipGetLastError();
  }
  // about 1024 workgroups in all
  const int64_t ib = ceil_div(n_quant, 256);
  const int64_t nj = std::min<int64_t>(std::max<int64_t>(1, ceil_div(1024, ib)), ceil_div(n_quant, 256));
  const int64_t jchunk = ceil_div(n_quant, nj);
  hipError_t e = launch_fill_f32(s, reinterpret_cast<float*>(invperm), (size_t)n_quant, 0.f);   // int zero
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_rank_part, dim3((unsigned)ib, (unsigned)nj), dim3(256), 0, s, diag, n_quant, jchunk, invperm);
  hipLaunchKernelGGL(k_rank_write, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, n, n_quant, perm, invperm);
  return hipGetLastError();
}

// A[a][b] = H_d[p][q], p = perm[n-1-a], q = perm[n-1-b]; lower part only
// (b <= a). The diagonal uses the dead-fixed value plus lambda. perm ==
// nullptr: the identity order, where a row of A is a row of H read
// backwards (16-byte loads when n % 4 == 0). Four outputs per thread and
// pass, all loads of a pass issued before its stores.
__global__ void __launch_bounds__(256)
k_build_flipped(const float* __restrict__ H, int64_t n, const int32_t* __restrict__ perm,
                const float* __restrict__ diag, const double* __restrict__ lam,
                float* __restrict__ A, DevStatus* st) {
  const int64_t a = blockIdx.x;
  const int64_t p = perm ? perm[n - 1 - a] : n - 1 - a;
  const float lamf = (float)lam[0];
  const bool vec = perm == nullptr && (n & 3) == 0 && (((uintptr_t)H & 15) == 0) && (((uintptr_t)A & 15) == 0);
  for (int64_t b0 = 4 * threadIdx.x; b0 <= a; b0 += 4 * 256) {
    float v[4];
    int64_t q[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t b = min(b0 + e, a);
      q[e] = perm ? perm[n - 1 - b] : n - 1 - b;
    }
    if (vec) {
      // H[p][n-4-b0 .. n-1-b0] holds q[3], q[2], q[1], q[0] (b0 + 3 may pass a:
      // those entries are not stored)
      const float4 h = *reinterpret_cast<const float4*>(H + p * n + (n - 4 - b0));
      v[0] = h.w; v[1] = h.z; v[2] = h.y; v[3] = h.x;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = H[p * n + q[e]];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t b = b0 + e;
      if (b > a) break;
      if (b == a) {
        v[e] = diag[p] + lamf;
      } else if (!isfinite(v[e])) {
        raise_status(st, kNonFinite, min(p, q[e]));
      }
      A[a * n + b] = v[e];
    }
  }
}

// The permuted build with row p of H staged in LDS: the row is read once,
// coalesced, and the permuted gather happens in LDS (read straight from
// memory, each 4-byte element at a permuted column costs a whole sector).
// Rows of up to 16384 floats (64 KiB of LDS).
constexpr int64_t kRowLdsMax = 16384;

__global__ void __launch_bounds__(256)
k_build_flipped_lds(const float* __restrict__ H, int64_t n, const int32_t* __restrict__ perm,
                    const float* __restrict__ diag, const double* __restrict__ lam,
                    float* __restrict__ A, DevStatus* st, int vec) {
  extern __shared__ __align__(16) float hrow[];
  const int64_t a = blockIdx.x;
  const int64_t p = perm[n - 1 - a];
  const float lamf = (float)lam[0];
  if (vec) {
    // n % 4 == 0 and 16-byte aligned rows: 16-byte loads and stores
    const float4* src = reinterpret_cast<const float4*>(H + p * n);
    for (int64_t c = threadIdx.x; c < n / 4; c += 256) reinterpret_cast<float4*>(hrow)[c] = src[c];
  } else {
    for (int64_t c = threadIdx.x; c < n; c += 256) hrow[c] = H[p * n + c];
  }
  __syncthreads();
  if (vec) {
    // four consecutive b per thread; the group that holds the diagonal (and
    // the columns past it, which are not stored) goes element by element
    for (int64_t b0 = 4 * (int64_t)threadIdx.x; b0 <= a; b0 += 1024) {
      // perm[n-4-b0 .. n-1-b0] holds q for b0+3, b0+2, b0+1, b0
      const int4 qv = *reinterpret_cast<const int4*>(perm + (n - 4 - b0));
      const int64_t q[4] = {qv.w, qv.z, qv.y, qv.x};
      if (b0 + 3 < a) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = hrow[q[e]];
          if (!isfinite(v[e])) raise_status(st, kNonFinite, min(p, q[e]));
        }
        *reinterpret_cast<float4*>(A + a * n + b0) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t b = b0 + e;
          if (b > a) break;
          float v;
          if (b == a) {
            v = diag[p] + lamf;
          } else {
            v = hrow[q[e]];
            if (!isfinite(v)) raise_status(st, kNonFinite, min(p, q[e]));
          }
          A[a * n + b] = v;
        }
      }
    }
    return;
  }
  for (int64_t b = threadIdx.x; b <= a; b += 256) {
    const int64_t q = perm[n - 1 - b];
    float v;
    if (b == a) {
      v = diag[p] + lamf;
    } else {
      v = hrow[q];
      if (!isfinite(v)) raise_status(st, kNonFinite, min(p, q));
    }
    A[a * n + b] = v;
  }
}

hipError_t launch_build_flipped(hipStream_t s, const float* H, int64_t n, const int32_t* perm,
                                const float* diag, const double* lam, float* A, DevStatus* st) {
  if (perm && n <= kRowLdsMax) {
    const int vec = n % 4 == 0 && ((uintptr_t)H & 15) == 0 && ((uintptr_t)A & 15) == 0 && ((uintptr_t)perm & 15) == 0;
    hipLaunchKernelGGL(k_build_flipped_lds, dim3((unsigned)n), dim3(256), (size_t)n * sizeof(float), s, H, n,
                       perm, diag, lam, A, st, vec);
  }
  else
    hipLaunchKernelGGL(k_build_flipped, dim3((unsigned)n), dim3(256), 0, s, H, n, perm, diag, lam, A, st);
  return hipGetLastError();
}

// Wf[r][p] = float(W[r][perm[p]])
template <bool kBF16>
__global__ void __launch_bounds__(256)
k_w_prep(const void* __restrict__ Wv, int64_t n, int64_t ldw, const int32_t* __restrict__ perm,
         float* __restrict__ Wf, DevStatus* st) {
  // four consecutive outputs per thread and pass; all loads of a pass are
  // issued before its stores. perm == nullptr: the identity order, read and
  // written as 8/16-byte vectors when the rows allow.
  const int64_t r = blockIdx.x;
  const bool vec = perm == nullptr && (n & 3) == 0 && (ldw & 3) == 0 && (((uintptr_t)Wv & 15) == 0) &&
                   (((uintptr_t)Wf & 15) == 0);
  for (int64_t p0 = 4 * threadIdx.x; p0 < n; p0 += 4 * 256) {
    int64_t c[4];
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) c[e] = perm ? perm[min(p0 + e, n - 1)] : min(p0 + e, n - 1);
    if (vec) {
      if (kBF16) {
        const uint2 u = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(Wv) + r * ldw + p0);
        v[0] = __uint_as_float(u.x << 16);
        v[1] = __uint_as_float(u.x & 0xFFFF0000u);
        v[2] = __uint_as_float(u.y << 16);
        v[3] = __uint_as_float(u.y & 0xFFFF0000u);
      } else {
        const float4 f = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(Wv) + r * ldw + p0);
        v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (kBF16) {
          const uint16_t u = reinterpret_cast<const uint16_t*>(Wv)[r * ldw + c[e]];
          v[e] = __uint_as_float((uint32_t)u << 16);
        } else {
          v[e] = reinterpret_cast<const float*>(Wv)[r * ldw + c[e]];
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (p0 + e < n && !isfinite(v[e])) raise_status(st, kNonFinite, c[e]);
    if (vec) {
      *reinterpret_cast<float4*>(Wf + r * n + p0) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (p0 + e < n) Wf[r * n + p0 + e] = v[e];
    }
  }
}

// The permuted W preparation with the row staged in LDS as fp32 (coalesced
// read, gather in LDS, coalesced write).
template <bool kBF16>
__global__ void __launch_bounds__(256)
k_w_prep_lds(const void* __restrict__ Wv, int64_t n, int64_t ldw, const int32_t* __restrict__ perm,
             float* __restrict__ Wf, DevStatus* st, int vec) {
  extern __shared__ __align__(16) float wrow[];
  const int64_t r = blockIdx.x;
  if (vec) {
    // n % 8 == 0, ldw % 8 == 0 and 16-byte aligned rows: 16-byte loads of
    // the row, four gathered values per 16-byte store
    if (kBF16) {
      const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(Wv) + r * ldw);
      for (int64_t c = threadIdx.x; c < n / 8; c += 256) {
        const uint4 u = src[c];
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
        float4* d = reinterpret_cast<float4*>(wrow + 8 * c);
        d[0] = make_float4(__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xFFFF0000u),
                           __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xFFFF0000u));
        d[1] = make_float4(__uint_as_float(w[2] << 16), __uint_as_float(w[2] & 0xFFFF0000u),
                           __uint_as_float(w[3] << 16), __uint_as_float(w[3] & 0xFFFF0000u));
      }
    } else {
      const float4* src = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(Wv) + r * ldw);
      for (int64_t c = threadIdx.x; c < n / 4; c += 256) reinterpret_cast<float4*>(wrow)[c] = src[c];
    }
    __syncthreads();
    for (int64_t q0 = 4 * (int64_t)threadIdx.x; q0 < n; q0 += 1024) {
      const int4 cv = *reinterpret_cast<const int4*>(perm + q0);
      const int64_t c[4] = {cv.x, cv.y, cv.z, cv.w};
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = wrow[c[e]];
        if (!isfinite(v[e])) raise_status(st, kNonFinite, c[e]);
      }
      *reinterpret_cast<float4*>(Wf + r * n + q0) = make_float4(v[0], v[1], v[2], v[3]);
    }
    return;
  }
  for (int64_t c = threadIdx.x; c < n; c += 256) {
    if (kBF16) {
      const uint16_t u = reinterpret_cast<const uint16_t*>(Wv)[r * ldw + c];
      wrow[c] = __uint_as_float((uint32_t)u << 16);
    } else {
      wrow[c] = reinterpret_cast<const float*>(Wv)[r * ldw + c];
    }
  }
  __syncthreads();
  for (int64_t q = threadIdx.x; q < n; q += 256) {
    const int64_t c = perm[q];
    const float v = wrow[c];
    if (!isfinite(v)) raise_status(st, kNonFinite, c);
    Wf[r * n + q] = v;
  }
}

hipError_t launch_w_prep(hipStream_t s, const void* W, int wdt_bf16, int64_t d_out, int64_t n,
                         int64_t ldw, const int32_t* perm, float* Wf, DevStatus* st) {
  if (d_out == 0) return hipSuccess;
  dim3 grid((unsigned)d_out);
  if (perm && n <= kRowLdsMax) {
    const size_t lds = (size_t)n * sizeof(float);
    const int vec = n % 8 == 0 && ldw % 8 == 0 && ((uintptr_t)W & 15) == 0 && ((uintptr_t)Wf & 15) == 0 &&
                    ((uintptr_t)perm & 15) == 0;
    if (wdt_bf16)
      hipLaunchKernelGGL(k_w_prep_lds<true>, grid, dim3(256), lds, s, W, n, ldw, perm, Wf, st, vec);
    else
      hipLaunchKernelGGL(k_w_prep_lds<false>, grid, dim3(256), lds, s, W, n, ldw, perm, Wf, st, vec);
    return hipGetLastError();
  }
  if (wdt_bf16)
    hipLaunchKernelGGL(k_w_prep<true>, grid, dim3(256), 0, s, W, n, ldw, perm, Wf, st);
  else
    hipLaunchKernelGGL(k_w_prep<false>, grid, dim3(256), 0, s, W, n, ldw, perm, Wf, st);
  return hipGetLastError();
}

}  // namespace gq
