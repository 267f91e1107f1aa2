// Upper Cholesky factor of the inverse of the damped Hessian.
//
// "Resumen Técnico: GPTQ-intrinsic LoRA", "Detalles de Implementación":
// standard GPTQ is Cholesky-based on the lambda-regularised Hessian.
//
// With A = J H_d J = L L^T (J = index reversal, L lower), the factor GPTQ's
// sweep needs is U = J L^{-1} J (upper, U^T U = H_d^{-1}).
//
// Phase 1, right-looking Cholesky in 64-column panels p = [k0, k1):
//   leaf:    L11 = chol(A11), D = L11^{-1} -> X[p, p]   (one workgroup)
//   panel:   A[k1:, p] = A[k1:, p] D^T                 (= L21, in place;
//            full 64-column panels only: a panel narrower than 64 is the
//            last one and has no rows below it)
//   update:  A[k1:, k1:] -= L21 L21^T                   (lower part)
// The next panel's leaf runs inside the update launch (see slab.hip).
// Phase 2, X = L^{-1} by recursive doubling over the diagonal blocks: with
// the inverses X_ii, X_jj of two adjacent blocks of h rows,
//   X_ji = -X_jj (L_ji X_ii),
// for h = 64, 128, ... ; every level is two batched GEMM launches (all
// block pairs of the level at once) that skip the zero triangles of X_ii
// and X_jj. The product L_ji X_ii is kept, transposed, in the free upper
// triangle of A.
// All products are fp32 v_mfma_f32_32x32x2f32.
#include "common.h"
#include "dma.h"
#include "leaf.h"

#include <algorithm>
#include <utility>

namespace gq {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

__global__ void __launch_bounds__(256)
k_leaf(const float* __restrict__ A, float* __restrict__ X, int64_t n, int64_t k0, int m,
       const int32_t* __restrict__ perm, DevStatus* st) {
  __shared__ __align__(16) LeafSmem sm;
  leaf_run(A + k0 * n + k0, n, X, n, k0, m, perm, st, sm);
}

hipError_t launch_leaf(hipStream_t s, float* A, float* X, int64_t n, int64_t off, int64_t m,
                       const int32_t* perm, DevStatus* st) {
  hipLaunchKernelGGL(k_leaf, dim3(1), dim3(256), 0, s, A, X, n, off, (int)m, perm, st);
  return hipGetLastError();
}

// ---------------------------------------------------------------- panel solve
// L21 = A21 D^T in place (A21: the r x 64 panel rows below the diagonal
// block, D = L11^{-1} lower, both row pitch ld). A workgroup owns 16 rows;
// wave w computes columns 16w..16w+15 with v_mfma_f32_16x16x4f32 and its
// operands are read straight from memory: for MFMA t of a group of four,
// lane group g = lane / 16 feeds k = 16p + 4g + t to both operands, so each
// lane reads 16-byte pieces of one row of A21 and one row of D. Every read
// of the workgroup's rows completes before any write (the MFMAs consume
// them before the barrier), so the result can overwrite its input.
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 row4(const float* p, bool vec) {
  if (vec) return *reinterpret_cast<const float4*>(p);
  return make_float4(p[0], p[1], p[2], p[3]);
}

__global__ void __launch_bounds__(256)
k_panel_solve(float* A21, const float* __restrict__ D, int64_t ld, int64_t r) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int li = lane & 15, g = lane >> 4;
  const int64_t r0 = (int64_t)blockIdx.x * 16;
  const bool vec = ((ld & 3) == 0) && (((uintptr_t)A21 & 15) == 0) && (((uintptr_t)D & 15) == 0);
  const bool rok = r0 + li < r;
  // rows past the end read the last row (always valid); zeroed below
  const float* pa = A21 + min(r0 + li, r - 1) * ld + 4 * g;
  const float* pb = D + (int64_t)(16 * w + li) * ld + 4 * g;
  float4 a[4], b[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    a[p] = row4(pa + 16 * p, vec);
    b[p] = row4(pb + 16 * p, vec);
    if (!rok) a[p] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[p].x, b[p].x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[p].y, b[p].y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[p].z, b[p].z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[p].w, b[p].w, acc, 0, 0, 0);
  }
  __syncthreads();
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t row = r0 + 4 * g + v;
    if (row < r) A21[row * ld + 16 * w + li] = acc[v];
  }
}

hipError_t launch_panel_solve(hipStream_t s, float* A21, const float* D, int64_t ld, int64_t r) {
  if (r <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_panel_solve, dim3((unsigned)ceil_div(r, 16)), dim3(256), 0, s, A21, D, ld, r);
  return hipGetLastError();
}

// ---------------------------------------------------------------- GEMM
// C = alpha op(A) op(B) + beta C. 256 threads as 2 x 2 waves, each wave a
// (BM/2) x (BN/2) block of 32x32 v_mfma_f32_32x32x2f32 tiles. K is staged
// through LDS in chunks of 32. Each operand keeps its memory layout in LDS,
// so every global->LDS move is a plain 16-byte copy:
//  * k-contiguous operands ([m][k] / [n][k], pitch 36 floats) are read with
//    one ds_read_b128 per four MFMAs;
//  * m- or n-contiguous ones ([k][m] / [k][n], pitch BM+4) with four
//    conflict-free ds_read_b32.
// For MFMA s (0..3) of a group of four, lanes 0-31 take k = 8q + s and
// lanes 32-63 take k = 8q + 4 + s, identically for A and B. The next chunk
// is prefetched into registers while the current one is multiplied; alpha
// is applied while staging A, and beta * C is loaded straight into the
// accumulators, so the epilogue only stores.
constexpr int kGBK = 32;
constexpr int kGP = kGBK + 4;

template <int BM, int BN>
struct GemmSmem {
  static constexpr int SA = (BM * kGP > kGBK * (BM + 4)) ? BM * kGP : kGBK * (BM + 4);
  static constexpr int SB = (BN * kGP > kGBK * (BN + 4)) ? BN * kGP : kGBK * (BN + 4);
  float a[2][SA];
  float b[2][SB];
};

// Load 4 consecutive elements along the contiguous dimension; zero outside.
__device__ inline float4 load4(const float* __restrict__ p, int64_t ld, int64_t r, int64_t c,
                               int64_t R, int64_t C) {
  if (r < R && c + 3 < C) {
    const float* q = p + r * ld + c;
    if (((uintptr_t)q & 15) == 0) return *reinterpret_cast<const float4*>(q);
    return make_float4(q[0], q[1], q[2], q[3]);
  }
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (r < R) {
    const float* q = p + r * ld;
    if (c < C) v.x = q[c];
    if (c + 1 < C) v.y = q[c + 1];
    if (c + 2 < C) v.z = q[c + 2];
  }
  return v;
}

struct GemmPair {
  GemmArgs p[2];
  int ntn[2];     // tiles along N per problem
  int per[2];     // tiles per batch instance
  int nt0;        // tiles of problem 0, all instances (problem 1 follows)
};

// Staging of one operand tile (R rows of the output dimension x kGBK).
// KC: the operand is k-contiguous in memory (M x K for A, N x K for B).
template <int R, bool KC>
struct Operand {
  static constexpr int L = R * kGBK / 4 / 256;   // float4 per thread
  // whole chunk inside the operand, 16-byte aligned rows: no predicates
  __device__ static float4 load_full(const float* p, int64_t ld, int64_t r0, int64_t k0, int idx) {
    if constexpr (KC) {
      const int r = idx / (kGBK / 4), k4 = idx % (kGBK / 4);
      return *reinterpret_cast<const float4*>(p + (r0 + r) * ld + k0 + 4 * k4);
    } else {
      const int k = idx / (R / 4), r4 = idx % (R / 4);
      return *reinterpret_cast<const float4*>(p + (k0 + k) * ld + r0 + 4 * r4);
    }
  }
  __device__ static float4 load(const float* p, int64_t ld, int64_t r0, int64_t k0, int64_t RN,
                                int64_t K, int idx) {
    if constexpr (KC) {
      const int r = idx / (kGBK / 4), k4 = idx % (kGBK / 4);
      return load4(p, ld, r0 + r, k0 + 4 * k4, RN, K);
    } else {
      const int k = idx / (R / 4), r4 = idx % (R / 4);
      return load4(p, ld, k0 + k, r0 + 4 * r4, K, RN);
    }
  }
  __device__ static void store(float* s, int idx, float4 v) {
    if constexpr (KC) {
      const int r = idx / (kGBK / 4), k4 = idx % (kGBK / 4);
      *reinterpret_cast<float4*>(s + r * kGP + 4 * k4) = v;
    } else {
      const int k = idx / (R / 4), r4 = idx % (R / 4);
      *reinterpret_cast<float4*>(s + k * (R + 4) + 4 * r4) = v;
    }
  }
  // the four values of row r for k = kb + 0..3
  __device__ static float4 frag(const float* s, int r, int kb) {
    if constexpr (KC) {
      return *reinterpret_cast<const float4*>(s + r * kGP + kb);
    } else {
      return make_float4(s[kb * (R + 4) + r], s[(kb + 1) * (R + 4) + r], s[(kb + 2) * (R + 4) + r],
                         s[(kb + 3) * (R + 4) + r]);
    }
  }
};

// LATE_C: the product is summed in 32-deep slices, each slice from zero in
// the MFMA accumulator and then added to a running fp32 total, and beta C
// is added once at the end. Each rounding then happens at the magnitude of
// a 32-term slice or of the total so far, never once per k at C's
// magnitude, for long updates of a matrix whose entries are much larger
// than its result (the trailing matrix of a Cholesky factorisation).
template <int BM, int BN, bool TA, bool TB, bool LATE_C = false>
__device__ __forceinline__ void gemm_tile(const GemmArgs& g, int tm, int tn, GemmSmem<BM, BN>& sm) {
  constexpr int WM = BM / 2, WN = BN / 2;          // per-wave block
  constexpr int FM = WM / 32, FN = WN / 32;        // MFMA tiles per wave
  using OA = Operand<BM, !TA>;
  using OB = Operand<BN, TB>;
  static_assert(OA::L >= 1 && OB::L >= 1, "tile too small");
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  int64_t klo = 0, khi = g.K;
  if (g.kmode == 1) khi = min(g.K, n0 + BN);
  else if (g.kmode == 2) klo = (n0 / kGBK) * kGBK;
  else if (g.kmode == 3) khi = min(g.K, m0 + BM);
  else if (g.kmode == 4) klo = (m0 / kGBK) * kGBK;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lk = 4 * (lane >> 5);

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int b = 0; b < FN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = 0.f;
        if (!LATE_C && g.beta != 0.f) {
          const int64_t i = m0 + WM * wm + 32 * a + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int64_t j = n0 + WN * wn + 32 * b + lr;
          if (i < g.M && j < g.N) v = g.beta * g.C[i * g.ldc + j];
        }
        acc[a][b][r] = v;
      }

  f32x16_t tot[LATE_C ? FM : 1][LATE_C ? FN : 1];
  if constexpr (LATE_C) {
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
      for (int b = 0; b < FN; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) tot[a][b][r] = 0.f;
  }

  float4 ra[OA::L], rb[OB::L];
  // interior chunks (the common case) take unpredicated 16-byte loads, so
  // all of a chunk's loads are in flight at once
  const bool vec = ((g.lda & 3) == 0) && ((g.ldb & 3) == 0) && (((uintptr_t)g.A & 15) == 0) &&
                   (((uintptr_t)g.B & 15) == 0) && m0 + BM <= g.M && n0 + BN <= g.N;
  auto gload = [&](int64_t k0) {
    if (vec && k0 + kGBK <= g.K) {
#pragma unroll
      for (int v = 0; v < OA::L; ++v) ra[v] = OA::load_full(g.A, g.lda, m0, k0, tid + 256 * v);
#pragma unroll
      for (int v = 0; v < OB::L; ++v) rb[v] = OB::load_full(g.B, g.ldb, n0, k0, tid + 256 * v);
      return;
    }
#pragma unroll
    for (int v = 0; v < OA::L; ++v) ra[v] = OA::load(g.A, g.lda, m0, k0, g.M, g.K, tid + 256 * v);
#pragma unroll
    for (int v = 0; v < OB::L; ++v) rb[v] = OB::load(g.B, g.ldb, n0, k0, g.N, g.K, tid + 256 * v);
  };
  auto sstore = [&](int buf) {
    const float al = g.alpha;
#pragma unroll
    for (int v = 0; v < OA::L; ++v)
      OA::store(sm.a[buf], tid + 256 * v, make_float4(al * ra[v].x, al * ra[v].y, al * ra[v].z, al * ra[v].w));
#pragma unroll
    for (int v = 0; v < OB::L; ++v) OB::store(sm.b[buf], tid + 256 * v, rb[v]);
  };

  const int64_t nk = khi > klo ? ceil_div(khi - klo, kGBK) : 0;
  if (nk > 0) {
    gload(klo);
    sstore(0);
  }
  __syncthreads();
  for (int64_t it = 0; it < nk; ++it) {
    const int cur = (int)(it & 1);
    const bool more = it + 1 < nk;
    if (more) gload(klo + (it + 1) * kGBK);
#pragma unroll
    for (int kq = 0; kq < kGBK / 8; ++kq) {
      float4 fa[FM], fb[FN];
#pragma unroll
      for (int a = 0; a < FM; ++a) fa[a] = OA::frag(sm.a[cur], WM * wm + 32 * a + lr, 8 * kq + lk);
#pragma unroll
      for (int b = 0; b < FN; ++b) fb[b] = OB::frag(sm.b[cur], WN * wn + 32 * b + lr, 8 * kq + lk);
#pragma unroll
      for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b) {
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[a].x, fb[b].x, acc[a][b], 0, 0, 0);
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[a].y, fb[b].y, acc[a][b], 0, 0, 0);
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[a].z, fb[b].z, acc[a][b], 0, 0, 0);
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[a].w, fb[b].w, acc[a][b], 0, 0, 0);
        }
    }
    if constexpr (LATE_C) {
#pragma unroll
      for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b) {
#pragma unroll
          for (int r = 0; r < 16; ++r) tot[a][b][r] += acc[a][b][r];
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
        }
    }
    if (more) sstore(cur ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int b = 0; b < FN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t i = m0 + WM * wm + 32 * a + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t j = n0 + WN * wn + 32 * b + lr;
        if (i < g.M && j < g.N) {
          float v = LATE_C ? tot[a][b][r] : acc[a][b][r];
          if (LATE_C && g.beta != 0.f) v += g.beta * g.C[i * g.ldc + j];
          g.C[i * g.ldc + j] = v;
        }
      }
}

// One operand layout (TA, TB) per instantiation: the four layouts in one
// kernel would take the register count of the largest (288 at 128 x 128,
// one workgroup per CU), each alone stays within 256 (two per CU).
template <int BM, int BN, bool TA, bool TB>
__global__ void __launch_bounds__(256, BM == 128 ? 2 : 1)
k_gemm_f32(GemmPair gp) {
  __shared__ __align__(16) GemmSmem<BM, BN> sm;
  const int which = (int)blockIdx.x >= gp.nt0;
  int t = (int)blockIdx.x - (which ? gp.nt0 : 0);
  GemmArgs g = gp.p[which];
  const int per = gp.per[which];          // tiles of one batch instance
  // Triangular K ranges make tiles unequal. The tiles are ordered longest
  // first and dealt to the CUs 256 at a time, so the workgroups that share a
  // CU are t, t + 256, ...: every other full round is reversed (a serpentine),
  // which pairs long tiles with short ones on each CU.
  if (g.kmode != 0) {
    const int total = which ? (int)gridDim.x - gp.nt0 : gp.nt0;
    const int q = t >> 8, w = t & 255;
    if ((q & 1) && (q << 8) + 256 <= total) t = (q << 8) + 255 - w;
  }
  const int b = t / per;
  t -= b * per;
  g.A += b * g.sA;
  g.B += b * g.sB;
  g.C += b * g.sC;
  int tm = t / gp.ntn[which];
  const int tn = t % gp.ntn[which];
  // triangular K ranges: dispatch the longest row tiles first
  if (g.kmode == 3) tm = per / gp.ntn[which] - 1 - tm;
  if (g.lower_only && tn * BN > tm * BM + BM - 1) return;
  gemm_tile<BM, BN, TA, TB>(g, tm, tn, sm);
}

template <int BM, int BN>
static hipError_t launch_pair(hipStream_t s, const GemmArgs& a, const GemmArgs* b) {
  GemmPair gp{};
  gp.p[0] = a;
  gp.ntn[0] = (int)ceil_div(a.N, BN);
  gp.per[0] = (int)(ceil_div(a.M, BM) * gp.ntn[0]);
  gp.nt0 = (a.M > 0 && a.N > 0 && a.K >= 0) ? gp.per[0] * std::max(a.batch, 1) : 0;
  int nt1 = 0;
  if (b && b->M > 0 && b->N > 0) {
    gp.p[1] = *b;
    gp.ntn[1] = (int)ceil_div(b->N, BN);
    gp.per[1] = (int)(ceil_div(b->M, BM) * gp.ntn[1]);
    nt1 = gp.per[1] * std::max(b->batch, 1);
  } else {
    gp.p[1] = a;
    gp.ntn[1] = 1;
    gp.per[1] = 1;
  }
  const int total = gp.nt0 + nt1;
  if (total == 0) return hipSuccess;
  const int ta = a.ta != 0, tb = a.tb != 0;
  if (b && b->M > 0 && b->N > 0 && ((b->ta != 0) != ta || (b->tb != 0) != tb)) return hipErrorInvalidValue;
  if (ta) {
    if (tb) hipLaunchKernelGGL((k_gemm_f32<BM, BN, true, true>), dim3(total), dim3(256), 0, s, gp);
    else hipLaunchKernelGGL((k_gemm_f32<BM, BN, true, false>), dim3(total), dim3(256), 0, s, gp);
  } else {
    if (tb) hipLaunchKernelGGL((k_gemm_f32<BM, BN, false, true>), dim3(total), dim3(256), 0, s, gp);
    else hipLaunchKernelGGL((k_gemm_f32<BM, BN, false, false>), dim3(total), dim3(256), 0, s, gp);
  }
  return hipGetLastError();
}

// One launch for one or two independent products with the same operand
// layout (ta, tb); the tile shape follows the larger one.
hipError_t launch_gemm_pair(hipStream_t s, const GemmArgs& a, const GemmArgs* b) {
  // 128 x 128 tiles only when there are enough of them for four rounds of
  // the 256 CUs; otherwise 64 x 64 (four workgroups per CU), which also
  // balances the uneven K ranges of triangular operands
  auto tiles128 = [](const GemmArgs& g) {
    return ceil_div(g.M, 128) * ceil_div(g.N, 128) * std::max(g.batch, 1);
  };
  int64_t t = tiles128(a);
  if (b) t = std::max(t, tiles128(*b));
  if (t >= 1024) return launch_pair<128, 128>(s, a, b);
  return launch_pair<64, 64>(s, a, b);
}

hipError_t launch_gemm_f32(hipStream_t s, const GemmArgs& g) { return launch_gemm_pair(s, g, nullptr); }

// C = beta C + alpha A A^T on the 128 x 128 tiles on or below the diagonal
// only (A is N x K, k-contiguous rows; B = A): the symmetric rank-K update
// of a wide factorisation's trailing matrix, summed in 32-deep slices and
// added to C once (LATE_C). The upper half of a diagonal
// tile is written too (that part of the matrix is never read as L). Tiles
// are numbered row by row over the lower triangle, so no workgroup is
// spent on a tile above it, and dealt to the XCDs in contiguous runs
// (workgroup b runs on XCD b % 8): the tiles resident on one XCD share
// A's row block in its L2.
__global__ void __launch_bounds__(256) k_syrk_f32(GemmArgs g, int ntile) {
  __shared__ __align__(16) GemmSmem<128, 128> sm;
  const int per = (ntile + 7) >> 3;
  const int t = ((int)blockIdx.x & 7) * per + ((int)blockIdx.x >> 3);
  if (t >= ntile) return;
  // t = tm (tm + 1) / 2 + tn, 0 <= tn <= tm
  int tm = (int)((sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
  while ((tm + 1) * (tm + 2) / 2 <= t) ++tm;
  while (tm * (tm + 1) / 2 > t) --tm;
  const int tn = t - tm * (tm + 1) / 2;
  gemm_tile<128, 128, false, true, true>(g, tm, tn, sm);
}

hipError_t launch_syrk_f32(hipStream_t s, const GemmArgs& g) {
  if (g.M != g.N || g.A != g.B || g.lda != g.ldb || g.ta != 0 || g.tb != 1 || g.kmode != 0)
    return hipErrorInvalidValue;
  const int64_t nt = ceil_div(g.N, 128);
  const int64_t ntile = nt * (nt + 1) / 2;
  if (ntile == 0) return hipSuccess;
  if (ntile > (1 << 28)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_syrk_f32, dim3((unsigned)(8 * ((ntile + 7) / 8))), dim3(256), 0, s, g, (int)ntile);
  return hipGetLastError();
}

// ---------------------------------------------------------------- rotate
// U[i][j] = X[n-1-i][n-1-j]: the flat array reversed; optionally with U's
// split-bf16 parts for the far-field update.
__global__ void k_rotate(const float* __restrict__ X, float* __restrict__ U, int64_t nn, uint16_t* __restrict__ hi,
                         uint16_t* __restrict__ lo) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < nn; q += stride) {
    const float v = X[nn - 1 - q];
    U[q] = v;
    if (hi) {
      const uint16_t h = f32_to_bf16_rne(v);
      hi[q] = h;
      lo[q] = f32_to_bf16_rne(v - bf16_to_f32(h));
    }
  }
}

hipError_t launch_rotate(hipStream_t s, const float* X, float* U, int64_t n, uint16_t* hi, uint16_t* lo) {
  const int64_t nn = n * n;
  int64_t blocks = ceil_div(nn, 256);
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(k_rotate, dim3((unsigned)blocks), dim3(256), 0, s, X, U, nn, hi, lo);
  return hipGetLastError();
}

}  // namespace gq
