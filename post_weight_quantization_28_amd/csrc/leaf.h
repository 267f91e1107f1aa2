// Leaf of the factorisation: Cholesky and inverse of one <= 64 x 64
// diagonal block in one wavefront, and the workgroup task that updates the
// next diagonal block and factors it beside a trailing update. Included by
// the kernels that run it (device code, inline).
#pragma once
#include "common.h"

#include <utility>

namespace gq {

// ---------------------------------------------------------------- leaf
// Cholesky and inverse of the m <= 64 diagonal block A[k0:k0+m, k0:k0+m]
// (lower part read), in ONE wavefront: lane i holds row i in 64 registers,
// so the 64 pivot steps need no workgroup barrier. Step k: the pivot comes
// from lane k (v_readlane), every lane scales its entry of column k, the
// column goes through LDS and is read back by all lanes as broadcasts
// (same address in every lane) for the rank-1 update of their own row.
// The inverse X = L^{-1} is then formed column-per-lane: lane c holds
// column c of X and, for row i, subtracts L[i][k] x_k (row i of L read from
// LDS as broadcasts) before scaling by 1/L[i][i]. All loops are unrolled so
// every register index is a constant. Writes the lower triangle of
// X[k0:k0+m, k0:k0+m]; a non-positive or non-finite pivot raises kNotPD
// with the original column perm[n-1-(k0+k)].
template <int K>
__device__ __forceinline__ void leaf_chol_step(float (&a)[64], float (*sCol)[64], float* sInv, int lane,
                                               int& bad) {
  const float d2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a[K]), K));
  const bool ok = d2 > 0.f && isfinite(d2);
  bad = (!ok && bad == 64) ? K : bad;
  const float inv = ok ? __builtin_amdgcn_rsqf(d2) : 1.f;   // 1 / sqrt(d2)
  const float d = ok ? d2 * inv : 1.f;
  float l = (lane > K) ? a[K] * inv : 0.f;
  l = (lane == K) ? d : l;
  a[K] = l;
  sCol[K][lane] = l;
  if (lane == K) sInv[K] = inv;
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int q = (K + 1) / 4; q < 16; ++q) {
    const float4 c = *reinterpret_cast<const float4*>(&sCol[K][4 * q]);
    if (4 * q + 0 > K) a[4 * q + 0] = fmaf(-l, c.x, a[4 * q + 0]);
    if (4 * q + 1 > K) a[4 * q + 1] = fmaf(-l, c.y, a[4 * q + 1]);
    if (4 * q + 2 > K) a[4 * q + 2] = fmaf(-l, c.z, a[4 * q + 2]);
    if (4 * q + 3 > K) a[4 * q + 3] = fmaf(-l, c.w, a[4 * q + 3]);
  }
  // materialise this step's updates here (otherwise the compiler sinks them
  // to their next use and keeps every broadcast value alive)
#pragma unroll
  for (int j = K + 1; j < 64; ++j) asm volatile("" : "+v"(a[j]));
}

template <int... Ks>
__device__ __forceinline__ void leaf_chol(float (&a)[64], float (*sCol)[64], float* sInv, int lane,
                                          int& bad, std::integer_sequence<int, Ks...>) {
  (leaf_chol_step<Ks>(a, sCol, sInv, lane, bad), ...);
}

template <int I>
__device__ __forceinline__ void leaf_inv_step(float (&x)[64], const float (*sRow)[68], const float* sInv,
                                              int lane) {
  // four independent partial sums keep the dependent FMA chain short
  float acc[4] = {(lane == I) ? 1.f : 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; 4 * q < I; ++q) {
    const float4 r = *reinterpret_cast<const float4*>(&sRow[I][4 * q]);
    if (4 * q + 0 < I) acc[0] = fmaf(-r.x, x[4 * q + 0], acc[0]);
    if (4 * q + 1 < I) acc[1] = fmaf(-r.y, x[4 * q + 1], acc[1]);
    if (4 * q + 2 < I) acc[2] = fmaf(-r.z, x[4 * q + 2], acc[2]);
    if (4 * q + 3 < I) acc[3] = fmaf(-r.w, x[4 * q + 3], acc[3]);
  }
  x[I] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) * sInv[I];
  asm volatile("" : "+v"(x[I]));
}

template <int... Is>
__device__ __forceinline__ void leaf_inv(float (&x)[64], const float (*sRow)[68], const float* sInv,
                                         int lane, std::integer_sequence<int, Is...>) {
  (leaf_inv_step<Is>(x, sRow, sInv, lane), ...);
}

// One full wavefront (lane = threadIdx.x % 64) factors the m x m block whose
// lower part is at src (row pitch lds; src may point to LDS) and writes the
// lower triangle of D = L11^{-1} to X[k0:k0+m, k0:k0+m].
__device__ __forceinline__ void leaf_run(const float* src, int64_t lds, float* __restrict__ X, int64_t n,
                                         int64_t k0, int m, const int32_t* __restrict__ perm,
                                         DevStatus* st, LeafSmem& sm) {
  const int lane = threadIdx.x & 63;
  const int li = min(lane, m - 1);
  const float* arow = src + li * lds;
  float a[64];
#pragma unroll
  for (int j = 0; j < 64; ++j) {
    const float v = arow[min(j, m - 1)];                  // always in bounds
    a[j] = (lane < m && j < m) ? ((j <= lane) ? v : 0.f) : ((lane == j) ? 1.f : 0.f);
  }
  int bad = 64;   // first pivot that failed (uniform across the wave)
  leaf_chol(a, sm.sCol, sm.sInv, lane, bad, std::make_integer_sequence<int, 64>{});
  if (lane == 0 && bad < m) raise_status(st, kNotPD, perm[n - 1 - (k0 + bad)]);
  // publish the rows of L for the inverse
#pragma unroll
  for (int j = 0; j < 64; j += 4)
    *reinterpret_cast<float4*>(&sm.sRow[lane][j]) =
        make_float4(lane >= j ? a[j] : 0.f, lane >= j + 1 ? a[j + 1] : 0.f,
                    lane >= j + 2 ? a[j + 2] : 0.f, lane >= j + 3 ? a[j + 3] : 0.f);
  __builtin_amdgcn_wave_barrier();
  // x[i] = column `lane` of L^{-1}, row i
  float x[64];
  leaf_inv(x, sm.sRow, sm.sInv, lane, std::make_integer_sequence<int, 64>{});
  float* xrow = X + k0 * n + k0 + lane;
#pragma unroll
  for (int i = 0; i < 64; ++i)
    if (i < m && lane <= i) xrow[i * n] = x[i];
}

// Step k's Schur update of the next diagonal block followed by its leaf, for
// the workgroup that runs beside step k's trailing update:
//   Ad = A[k1:k1+m2, k1:k1+m2] - L21[0:m2] L21[0:m2]^T   (lower part)
//   D' = chol(Ad)^{-1} -> X[k1:k1+m2, k1:k1+m2]
// 256 threads stage L21's first m2 rows and Ad in LDS and apply the update
// (thread t: row t/4, 16 columns); wave 0 then runs the leaf from LDS.
__device__ inline void leaf_task_run(const LeafTask& t, LeafTaskSmem& sm) {
  const int tid = threadIdx.x;
  const int64_t n = t.n;
  for (int e = tid; e < 64 * 64; e += 256) {
    const int i = e >> 6, j = e & 63;
    sm.lrows[i][j] = (i < t.m2 && j < t.mk) ? t.L21[i * n + j] : 0.f;
    sm.blk[i][j] = (i < t.m2 && j <= i) ? t.A[(t.k1 + i) * n + t.k1 + j] : 0.f;
  }
  __syncthreads();
  {
    const int i = tid >> 2, j0 = 16 * (tid & 3);
    float acc[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) acc[c] = 0.f;
    for (int k = 0; k < t.mk; ++k) {
      const float li = sm.lrows[i][k];
#pragma unroll
      for (int c = 0; c < 16; ++c) acc[c] = fmaf(li, sm.lrows[j0 + c][k], acc[c]);
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 16; ++c)
      if (j0 + c <= i) sm.blk[i][j0 + c] -= acc[c];
  }
  __syncthreads();
  if (tid < 64) leaf_run(&sm.blk[0][0], 65, t.X, n, t.k1, t.m2, t.perm, t.st, sm.leaf);
}

}  // namespace gq
