// Leaf of the factorisation: Cholesky and inverse of one <= 64 x 64
// diagonal block by one workgroup of 4 wavefronts, and the task that first
// applies the preceding panel's update to that block. Included by the
// kernels that run it (device code, inline).
//
// "Resumen Técnico: GPTQ-intrinsic LoRA", "Detalles de Implementación":
// the standard method factorises the regularised Hessian by Cholesky.
//
// Work split (wave w = 0..3, lane = threadIdx.x % 64), in 16 blocks of 4
// consecutive pivots; block b is owned by wave b % 4:
//  * Cholesky, right-looking: lane i holds row i; wave w holds the columns
//    of its blocks, j = 16q + 4w + c (q, c = 0..3), in registers a[q][c].
//    The owner of block b takes its 4 pivots in registers: it reads the
//    block's 4 x 4 lower part once (v_readlane), factors it on wave-uniform
//    values, and every lane forms its entries of the 4 columns from those.
//  * Inverse X = L^{-1}, column-oriented forward substitution: lane c holds
//    column c of X; wave w holds the rows of its blocks, x[q][c'] =
//    X[16q + 4w + c'][lane]. The owner of block b finalises rows 4b..4b+3
//    right after the block's pivots (divide by L_kk, eliminate within the
//    block).
//  * One barrier per block publishes the 4 columns of L and the 4 rows of
//    X; every wave then applies the rank-4 update to its later Cholesky
//    columns and its later X rows. L's columns are stored in the order
//    pos(i) = 16 w_i + 4 q_i + c_i of i = 16 q_i + 4 w_i + c_i, so a wave
//    reads the 16 values of its own index set as four 16-byte broadcasts
//    (and the same values serve both updates).
// A non-positive or non-finite pivot raises kNotPD with the original column
// perm[n-1-(k0+k)] (the matrix is the index-reversed Hessian).
#pragma once
#include "common.h"

#include <utility>

namespace gq {

struct LeafSmem {
  float colw[64][64];   // colw[k][pos(i)] = L[i][k]
  float xrow[64][64];   // xrow[k][c] = X[k][c], final rows of L^{-1}
  int bad;              // first failed pivot (64: none)
};

struct LeafState {
  float a[4][4];        // A[lane][16q + 4w + c] -> Schur complement / L columns
  float x[4][4];        // X[16q + 4w + c][lane]
  int bad;              // first failed pivot of this wave (64: none), wave-uniform
};

__device__ __forceinline__ int leaf_pos(int i) { return 16 * ((i >> 2) & 3) + 4 * (i >> 4) + (i & 3); }

__device__ __forceinline__ float lane_val(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// The owner of block BLK takes its 4 pivots. The block's 4 x 4 lower part
// is read once (10 independent v_readlane) and factored on wave-uniform
// values; each lane then forms its entries of the 4 columns and of X's 4
// rows with those values. Every FMA is the one a lane-by-lane pivot
// sequence would do (same operands, same order), so the results are the
// same; only the v_readlane between dependent steps are gone from the
// chain. A failed pivot (not positive or not finite) is recorded as a
// wave-uniform minimum, off the dependent chain; what follows it is then
// garbage and the caller discards the result.
template <int BLK>
__device__ __forceinline__ void leaf_owner(LeafState& S, int lane) {
  constexpr int qb = BLK / 4, K0 = 4 * BLK;
  float b[4][4];   // b[r][c], c <= r: the block's Schur complement, then L
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c <= r; ++c) b[r][c] = lane_val(S.a[qb][c], K0 + r);
  float inv[4];
#pragma unroll
  for (int C = 0; C < 4; ++C) {
    const float d2 = b[C][C];
    if (!(d2 > 0.f && isfinite(d2))) S.bad = min(S.bad, K0 + C);
    inv[C] = __builtin_amdgcn_rsqf(d2);   // 1 / sqrt(d2)
    b[C][C] = d2 * inv[C];
#pragma unroll
    for (int r = C + 1; r < 4; ++r) b[r][C] *= inv[C];
#pragma unroll
    for (int c2 = C + 1; c2 < 4; ++c2)
#pragma unroll
      for (int r = c2; r < 4; ++r) b[r][c2] = fmaf(-b[r][C], b[c2][C], b[r][c2]);
  }
  // this lane's entries of the 4 columns (rows above the block: zero)
#pragma unroll
  for (int C = 0; C < 4; ++C) {
    const int K = K0 + C;
    float l = (lane > K) ? S.a[qb][C] * inv[C] : 0.f;
    l = (lane == K) ? b[C][C] : l;
    S.a[qb][C] = l;
#pragma unroll
    for (int c2 = C + 1; c2 < 4; ++c2) S.a[qb][c2] = fmaf(-l, b[c2][C], S.a[qb][c2]);
  }
  // rows K0..K0+3 of X: forward substitution inside the block
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    S.x[qb][c] *= inv[c];
#pragma unroll
    for (int c2 = c + 1; c2 < 4; ++c2) S.x[qb][c2] = fmaf(-b[c2][c], S.x[qb][c], S.x[qb][c2]);
  }
}

template <int BLK>
__device__ __forceinline__ void leaf_block(LeafState& S, LeafSmem& sm, int w, int lane) {
  constexpr int qb = BLK / 4, ob = BLK % 4, K0 = 4 * BLK;
  if (w == ob) {
    leaf_owner<BLK>(S, lane);
    const int pl = leaf_pos(lane);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      sm.colw[K0 + c][pl] = S.a[qb][c];
      sm.xrow[K0 + c][lane] = S.x[qb][c];
    }
    // the wave's last block: publish its first failure before the barrier
    if (BLK >= 12 && lane == 0 && S.bad < 64) atomicMin(&sm.bad, S.bad);
  }
  __syncthreads();
  // ---- rank-4 updates of the later blocks of every wave. Blocks with
  // q > qb are later for every wave; block 4 qb + w only for w > ob, which
  // is applied branch-free by zeroing the multipliers of the other waves.
  if constexpr (BLK < 15) {
    const int pl = leaf_pos(lane);
    const bool later = w > ob;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int k = K0 + c;
      const float li = sm.colw[k][pl];
      const float xk = sm.xrow[k][lane];
      const float lq = later ? li : 0.f, xq = later ? xk : 0.f;
#pragma unroll
      for (int q = qb; q < 4; ++q) {
        const float4 t = *reinterpret_cast<const float4*>(&sm.colw[k][16 * w + 4 * q]);
        const float lj[4] = {t.x, t.y, t.z, t.w};
        const float lm = (q == qb) ? lq : li, xm = (q == qb) ? xq : xk;
#pragma unroll
        for (int c2 = 0; c2 < 4; ++c2) {
          S.a[q][c2] = fmaf(-lm, lj[c2], S.a[q][c2]);
          S.x[q][c2] = fmaf(-lj[c2], xm, S.x[q][c2]);
        }
      }
    }
  }
}

template <int... Bs>
__device__ __forceinline__ void leaf_blocks(LeafState& S, LeafSmem& sm, int w, int lane,
                                            std::integer_sequence<int, Bs...>) {
  (leaf_block<Bs>(S, sm, w, lane), ...);
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
  S.bad = 64;
  if (threadIdx.x == 0) sm.bad = 64;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = 16 * q + 4 * w + c;
      const float v = src[min(lane, m - 1) * lds + min(j, m - 1)];   // always in bounds
      S.a[q][c] = (lane < m && j < m) ? ((j <= lane) ? v : 0.f) : ((lane == j) ? 1.f : 0.f);
      S.x[q][c] = (j == lane) ? 1.f : 0.f;
    }
  __syncthreads();   // sm.bad initialised before any pivot can fail
  leaf_blocks(S, sm, w, lane, std::make_integer_sequence<int, 16>{});
  // only the first failing block reports (later ones run on garbage)
  if (threadIdx.x == 0 && sm.bad < m && st->flags == 0) raise_status(st, kNotPD, perm[n - 1 - (k0 + sm.bad)]);
  float* xcol = X + k0 * n + k0 + lane;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int i = 16 * q + 4 * w + c;
      if (i < m && lane < m && lane <= i) xcol[(int64_t)i * n] = S.x[q][c];
    }
}

// Step k's Schur update of the next diagonal block followed by its leaf, for
// the workgroup that runs beside step k's trailing update:
//   Ad = A[k1:k1+m2, k1:k1+m2] - L21[0:m2] L21[0:m2]^T   (lower part)
//   D' = chol(Ad)^{-1} -> X[k1:k1+m2, k1:k1+m2]
// Every global load (L21's first m2 rows, the block) is issued up front with
// clamped, always-valid addresses. L21 is staged row-major (k contiguous);
// waves 0-2 each take one lower 32 x 32 tile of the product on
// v_mfma_f32_32x32x2f32. Within each group of 8 k, lane half h feeds k =
// 4h + t to the t-th MFMA, so a lane reads its 4 k values as one 16-byte
// LDS read; the result is combined with the block read straight into the
// accumulator layout.
typedef float leaf_f32x16 __attribute__((ext_vector_type(16)));

// The three phases reuse one region: lrow is last read by the MFMAs
// (barrier before blk2 is written), blk2 is last read by the leaf's
// register load (barrier before the leaf's first LDS write).
struct LeafTaskSmem {
  union {
    float lrow[64][68];   // L21[i][k], zero outside m2 x mk
    float blk2[64][65];   // the updated block, input of the leaf
    LeafSmem leaf;
  } u;
};

__device__ inline void leaf_task_run(const LeafTask& t, LeafTaskSmem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n = t.n;
  const int m2 = t.m2, mk = t.mk;
  float lv[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int i = (tid >> 6) + 4 * v;
    lv[v] = t.L21[(int64_t)min(i, m2 - 1) * n + min(lane, mk - 1)];
  }
  // tile (ta, tb) of this wave: (0,0), (1,0), (1,1); wave 3 has none
  const int ta = wave >= 1 ? 1 : 0, tb = wave == 2 ? 1 : 0;
  const int lr = lane & 31, lh = lane >> 5;
  float av[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = 32 * ta + 8 * (r >> 2) + 4 * lh + (r & 3), col = 32 * tb + lr;
    av[r] = t.A[(t.k1 + min(row, m2 - 1)) * n + t.k1 + min(col, m2 - 1)];
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int i = (tid >> 6) + 4 * v;
    sm.u.lrow[i][lane] = (i < m2 && lane < mk) ? lv[v] : 0.f;
  }
  __syncthreads();
  leaf_f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  if (wave < 3) {
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const float4 fa = *reinterpret_cast<const float4*>(&sm.u.lrow[32 * ta + lr][8 * p + 4 * lh]);
      const float4 fb = *reinterpret_cast<const float4*>(&sm.u.lrow[32 * tb + lr][8 * p + 4 * lh]);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa.x, fb.x, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa.y, fb.y, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa.z, fb.z, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa.w, fb.w, acc, 0, 0, 0);
    }
  }
  __syncthreads();   // every read of lrow is done
  if (wave < 3) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 32 * ta + 8 * (r >> 2) + 4 * lh + (r & 3), col = 32 * tb + lr;
      sm.u.blk2[row][col] = (col <= row) ? av[r] - acc[r] : 0.f;
    }
  }
  __syncthreads();
  leaf_run(&sm.u.blk2[0][0], 65, t.X, n, t.k1, m2, t.perm, t.st, sm.u.leaf);
}

}  // namespace gq
