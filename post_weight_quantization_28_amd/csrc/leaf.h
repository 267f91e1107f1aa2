// Leaf of the factorisation: Cholesky and inverse of one <= 64 x 64
// diagonal block by one workgroup of 4 wavefronts, and the task that first
// applies the preceding panel's update to that block. Included by the
// kernels that run it (device code, inline).
//
// "Resumen Técnico: GPTQ-intrinsic LoRA", "Detalles de Implementación":
// the standard method factorises the regularised Hessian by Cholesky.
//
// Work split (wave w = 0..3, lane = threadIdx.x % 64):
//  * Cholesky, right-looking: lane i holds row i; wave w holds the columns
//    j = 4q + w (q = 0..15) in registers a[q]. Step K: the owner wave of
//    column K (K % 4) takes the pivot from lane K (v_readlane), scales the
//    column and publishes it in LDS; after one barrier every wave applies
//    the rank-1 update to its own columns j > K (at most 16 FMAs per lane).
//  * Inverse X = L^{-1}, column-oriented forward substitution, one step
//    behind: lane c holds column c of X; wave w holds the rows i = 4q + w.
//    In step K the owner of row K-1 divides it by L[K-1][K-1] and publishes
//    it; after the same barrier every wave subtracts L[i][K-1] X[K-1][c]
//    from its rows i > K-1.
//  Both chains share one barrier per step. L's columns are stored
//  wave-interleaved (colw[k][16 w + q] = L[4q + w][k]) so that each wave
//  reads the 16 values it needs as four 16-byte broadcasts.
// A non-positive or non-finite pivot raises kNotPD with the original column
// perm[n-1-(k0+k)] (the matrix is the index-reversed Hessian).
#pragma once
#include "common.h"

#include <utility>

namespace gq {

struct LeafSmem {
  float colw[64][64];   // colw[k][16 w + q] = L[4q + w][k]
  float xrow[64][64];   // xrow[k][c] = X[k][c], final rows of L^{-1}
  float inv[64];        // 1 / L[k][k]
  int bad;              // first failed pivot (64: none)
};

struct LeafState {
  float a[16];          // A[lane][4q + w] -> Schur complement, lower part used
  float x[16];          // X[4q + w][lane]
  float lj[16];         // colw[K-1][16 w .. 16 w + 15] from the previous step
};

__device__ __forceinline__ void leaf_read16(const float* p, float (&v)[16]) {
#pragma unroll
  for (int q = 0; q < 16; q += 4) {
    const float4 t = *reinterpret_cast<const float4*>(p + q);
    v[q] = t.x; v[q + 1] = t.y; v[q + 2] = t.z; v[q + 3] = t.w;
  }
}

template <int K>
__device__ __forceinline__ void leaf_step(LeafState& S, LeafSmem& sm, int w, int lane) {
  constexpr int qK = K / 4, oK = K % 4;
  // ---- before the barrier: pivot column K, and row K-1 of X
  if (w == oK) {
    const float d2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(S.a[qK]), K));
    const bool ok = d2 > 0.f && isfinite(d2);
    if (!ok && lane == 0) atomicMin(&sm.bad, K);
    const float inv = ok ? __builtin_amdgcn_rsqf(d2) : 1.f;   // 1 / sqrt(d2)
    const float d = ok ? d2 * inv : 1.f;
    float l = (lane > K) ? S.a[qK] * inv : 0.f;
    l = (lane == K) ? d : l;
    sm.colw[K][16 * (lane & 3) + (lane >> 2)] = l;
    if (lane == K) sm.inv[K] = inv;
  }
  if constexpr (K >= 1) {
    constexpr int qP = (K - 1) / 4, oP = (K - 1) % 4;
    if (w == oP) {
      S.x[qP] *= sm.inv[K - 1];
      sm.xrow[K - 1][lane] = S.x[qP];
    }
  }
  __syncthreads();
  // ---- after the barrier: rank-1 update with column K, substitution with row K-1
  const float li = sm.colw[K][16 * (lane & 3) + (lane >> 2)];
  float lk[16];
  leaf_read16(&sm.colw[K][16 * w], lk);
#pragma unroll
  for (int q = qK; q < 16; ++q) {
    if (q == qK) {
      if (w > oK) S.a[q] = fmaf(-li, lk[q], S.a[q]);
    } else {
      S.a[q] = fmaf(-li, lk[q], S.a[q]);
    }
  }
  if constexpr (K >= 1) {
    constexpr int qP = (K - 1) / 4, oP = (K - 1) % 4;
    const float xk = sm.xrow[K - 1][lane];
#pragma unroll
    for (int q = qP; q < 16; ++q) {
      if (q == qP) {
        if (w > oP) S.x[q] = fmaf(-S.lj[q], xk, S.x[q]);
      } else {
        S.x[q] = fmaf(-S.lj[q], xk, S.x[q]);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < 16; ++q) S.lj[q] = lk[q];
}

template <int... Ks>
__device__ __forceinline__ void leaf_steps(LeafState& S, LeafSmem& sm, int w, int lane,
                                           std::integer_sequence<int, Ks...>) {
  (leaf_step<Ks>(S, sm, w, lane), ...);
}

// All 256 threads of the workgroup: factors the m x m block whose lower part
// is at src (row pitch lds; src may point to LDS) and writes the lower
// triangle of D = L11^{-1} to X[k0:k0+m, k0:k0+m].
__device__ __forceinline__ void leaf_run(const float* src, int64_t lds, float* __restrict__ X, int64_t n,
                                         int64_t k0, int m, const int32_t* __restrict__ perm,
                                         DevStatus* st, LeafSmem& sm) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  LeafState S;
  if (threadIdx.x == 0) sm.bad = 64;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int j = 4 * q + w;
    const float v = src[min(lane, m - 1) * lds + min(j, m - 1)];   // always in bounds
    S.a[q] = (lane < m && j < m) ? ((j <= lane) ? v : 0.f) : ((lane == j) ? 1.f : 0.f);
    S.x[q] = (j == lane) ? 1.f : 0.f;
    S.lj[q] = 0.f;
  }
  __syncthreads();   // sm.bad initialised before any pivot can fail
  leaf_steps(S, sm, w, lane, std::make_integer_sequence<int, 64>{});
  // last row of X: divide by L[63][63]
  if (w == 3) S.x[15] *= sm.inv[63];
  if (threadIdx.x == 0 && sm.bad < m) raise_status(st, kNotPD, perm[n - 1 - (k0 + sm.bad)]);
  float* xcol = X + k0 * n + k0 + lane;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int i = 4 * q + w;
    if (i < m && lane < m && lane <= i) xcol[(int64_t)i * n] = S.x[q];
  }
}

// Step k's Schur update of the next diagonal block followed by its leaf, for
// the workgroup that runs beside step k's trailing update:
//   Ad = A[k1:k1+m2, k1:k1+m2] - L21[0:m2] L21[0:m2]^T   (lower part)
//   D' = chol(Ad)^{-1} -> X[k1:k1+m2, k1:k1+m2]
// L21's first m2 rows are staged transposed (lt[k][i] = L21[i][k]); thread
// (r4, c4) accumulates the 4 x 4 block rows 4 r4.., columns 4 c4.. with two
// 16-byte reads per k.
struct LeafTaskSmem {
  union {
    struct {
      float lt[64][68];
      float blk[64][65];
    } s;
    LeafSmem leaf;
  } u;
  float blk2[64][65];   // the updated block, input of the leaf
};

__device__ inline void leaf_task_run(const LeafTask& t, LeafTaskSmem& sm) {
  const int tid = threadIdx.x;
  const int64_t n = t.n;
  for (int e = tid; e < 64 * 64; e += 256) {
    const int i = e >> 6, j = e & 63;
    sm.u.s.lt[j][i] = (i < t.m2 && j < t.mk) ? t.L21[i * n + j] : 0.f;
    sm.u.s.blk[i][j] = (i < t.m2 && j <= i) ? t.A[(t.k1 + i) * n + t.k1 + j] : 0.f;
  }
  __syncthreads();
  {
    const int r4 = tid >> 4, c4 = tid & 15;
    if (4 * c4 <= 4 * r4 + 3) {   // block touches the lower triangle
      float acc[4][4];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = 0.f;
      for (int k = 0; k < t.mk; ++k) {
        const float4 li = *reinterpret_cast<const float4*>(&sm.u.s.lt[k][4 * r4]);
        const float4 lj = *reinterpret_cast<const float4*>(&sm.u.s.lt[k][4 * c4]);
        const float lv[4] = {li.x, li.y, li.z, li.w}, jv[4] = {lj.x, lj.y, lj.z, lj.w};
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int b = 0; b < 4; ++b) acc[a][b] = fmaf(lv[a], jv[b], acc[a][b]);
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int i = 4 * r4 + a, j = 4 * c4 + b;
          sm.blk2[i][j] = (j <= i) ? sm.u.s.blk[i][j] - acc[a][b] : 0.f;
        }
    }
  }
  __syncthreads();
  leaf_run(&sm.blk2[0][0], 65, t.X, n, t.k1, t.m2, t.perm, t.st, sm.u.leaf);
}

}  // namespace gq
