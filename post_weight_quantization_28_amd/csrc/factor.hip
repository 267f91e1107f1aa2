// Upper Cholesky factor of the inverse of the damped Hessian.
//
// "Resumen Técnico: GPTQ-intrinsic LoRA", "Detalles de Implementación":
// standard GPTQ is Cholesky-based on the lambda-regularised Hessian.
//
// With A = J H_d J = L L^T (J = index reversal, L lower), the factor GPTQ's
// sweep needs is U = J L^{-1} J (upper, U^T U = H_d^{-1}). L and X = L^{-1}
// are built together by recursive halving of A:
//   [A11  .  ]      L11, X11 = rec(A11)
//   [A21 A22 ]      T1 = A21 X11^T          (= L21)
//                   A22 -= T1 T1^T          (Schur complement, lower tiles)
//                   T2 = T1 X11             (= L21 L11^{-1})
//                   L22, X22 = rec(A22)
//                   X21 = -X22 T2
// so L itself is never stored: only X = L^{-1} (lower; its upper part is
// kept zero) and the two temporaries, which live in blocks that are dead at
// that point (T1 in X21's place, T2 in A21's place). Every product is a
// fp32 v_mfma_f32_32x32x2f32 GEMM; leaves of up to 64 columns are factored
// and inverted inside one workgroup in LDS.
#include "common.h"

namespace gq {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------- leaf
// m <= 64 columns at offset off of the flipped matrix (ld = n). Writes the
// lower triangle of X[off:off+m, off:off+m] = L11^{-1}. A non-positive or
// non-finite pivot raises kNotPD with the original column perm[n-1-(off+k)].
__global__ void __launch_bounds__(256)
k_leaf(const float* __restrict__ A, float* __restrict__ X, int64_t n, int64_t off, int m,
       const int32_t* __restrict__ perm, DevStatus* st) {
  __shared__ float sA[64][65];
  __shared__ float sX[64][65];
  __shared__ float sD[64];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  for (int e = tid; e < 64 * 64; e += 256) {
    const int i = e >> 6, j = e & 63;
    float v;
    if (i < m && j < m) v = (j <= i) ? A[(off + i) * n + off + j] : 0.f;
    else v = (i == j) ? 1.f : 0.f;
    sA[i][j] = v;
    sX[i][j] = (i == j) ? 1.f : 0.f;
  }
  __syncthreads();
  // right-looking Cholesky: column k scaled, trailing lower part updated
  for (int k = 0; k < 64; ++k) {
    const float d2 = sA[k][k];
    const bool ok = d2 > 0.f && isfinite(d2);
    if (tid == 0 && k < m && !ok) raise_status(st, kNotPD, perm[n - 1 - (off + k)]);
    const float d = ok ? sqrtf(d2) : 1.f;
    if (tid == 0) sD[k] = d;
    const float inv = 1.f / d;
    if (tid > k && tid < 64) sA[tid][k] *= inv;
    __syncthreads();
    for (int a = 0; a < 4; ++a) {
      const int i = k + 1 + ty + 16 * a;
      if (i >= 64) break;
      const float lik = sA[i][k];
      for (int b = 0; b < 4; ++b) {
        const int j = k + 1 + tx + 16 * b;
        if (j <= i) sA[i][j] -= lik * sA[j][k];
      }
    }
    __syncthreads();
  }
  // X = L^{-1}: forward substitution on the identity, row by row
  for (int i = 0; i < 64; ++i) {
    const float inv = 1.f / sD[i];
    if (tid <= i) sX[i][tid] *= inv;
    __syncthreads();
    for (int a = 0; a < 4; ++a) {
      const int r = i + 1 + ty + 16 * a;
      if (r >= 64) break;
      const float lri = sA[r][i];
      for (int b = 0; b < 4; ++b) {
        const int c = tx + 16 * b;
        if (c <= i) sX[r][c] -= lri * sX[i][c];
      }
    }
    __syncthreads();
  }
  for (int e = tid; e < 64 * 64; e += 256) {
    const int i = e >> 6, j = e & 63;
    if (i < m && j <= i) X[(off + i) * n + off + j] = sX[i][j];
  }
}

hipError_t launch_leaf(hipStream_t s, float* A, float* X, int64_t n, int64_t off, int64_t m,
                       const int32_t* perm, DevStatus* st) {
  hipLaunchKernelGGL(k_leaf, dim3(1), dim3(256), 0, s, A, X, n, off, (int)m, perm, st);
  return hipGetLastError();
}

// ---------------------------------------------------------------- GEMM
// C = alpha op(A) op(B) + beta C with 4 waves (2x2), each wave owning a
// (BM/2) x (BN/2) block of 32x32 MFMA tiles; K staged through LDS in chunks
// of 16 as [k][m] and [k][n] (consecutive lanes read consecutive m or n).
constexpr int kGBK = 16;

template <int BM, int BN>
struct GemmSmem {
  float a[2][kGBK][BM + 4];
  float b[2][kGBK][BN + 4];
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

template <int BM, int BN>
__global__ void __launch_bounds__(256)
k_gemm_f32(GemmArgs g) {
  constexpr int WM = BM / 2, WN = BN / 2;          // per-wave block
  constexpr int FM = WM / 32, FN = WN / 32;        // MFMA tiles per wave
  constexpr int LA = BM * kGBK / 4 / 256;          // float4 loads per thread
  constexpr int LB = BN * kGBK / 4 / 256;
  static_assert(LA >= 1 && LB >= 1, "tile too small");
  __shared__ GemmSmem<BM, BN> sm;

  if (g.st != nullptr && g.st->flags != 0) return;
  const int tm = blockIdx.y, tn = blockIdx.x;
  if (g.lower_only && tn * BN > tm * BM + BM - 1) return;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  int64_t klo = 0, khi = g.K;
  if (g.kmode == 1) khi = min(g.K, n0 + BN);
  else if (g.kmode == 2) klo = (n0 / kGBK) * kGBK;
  else if (g.kmode == 3) khi = min(g.K, m0 + BM);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int b = 0; b < FN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  float4 ra[LA], rb[LB];
  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int v = 0; v < LA; ++v) {
      const int idx = tid + 256 * v;
      if (!g.ta) {   // A is M x K, k contiguous: 4 k values of row m
        const int m = idx / (kGBK / 4), k4 = idx % (kGBK / 4);
        ra[v] = load4(g.A, g.lda, m0 + m, k0 + 4 * k4, g.M, g.K);
      } else {       // A stored K x M, m contiguous: 4 m values of row k
        const int k = idx / (BM / 4), m4 = idx % (BM / 4);
        ra[v] = load4(g.A, g.lda, k0 + k, m0 + 4 * m4, g.K, g.M);
      }
    }
#pragma unroll
    for (int v = 0; v < LB; ++v) {
      const int idx = tid + 256 * v;
      if (!g.tb) {   // B is K x N, n contiguous
        const int k = idx / (BN / 4), n4 = idx % (BN / 4);
        rb[v] = load4(g.B, g.ldb, k0 + k, n0 + 4 * n4, g.K, g.N);
      } else {       // B stored N x K, k contiguous
        const int nn = idx / (kGBK / 4), k4 = idx % (kGBK / 4);
        rb[v] = load4(g.B, g.ldb, n0 + nn, k0 + 4 * k4, g.N, g.K);
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int v = 0; v < LA; ++v) {
      const int idx = tid + 256 * v;
      if (!g.ta) {
        const int m = idx / (kGBK / 4), k4 = idx % (kGBK / 4);
        sm.a[buf][4 * k4 + 0][m] = ra[v].x;
        sm.a[buf][4 * k4 + 1][m] = ra[v].y;
        sm.a[buf][4 * k4 + 2][m] = ra[v].z;
        sm.a[buf][4 * k4 + 3][m] = ra[v].w;
      } else {
        const int k = idx / (BM / 4), m4 = idx % (BM / 4);
        *reinterpret_cast<float4*>(&sm.a[buf][k][4 * m4]) = ra[v];
      }
    }
#pragma unroll
    for (int v = 0; v < LB; ++v) {
      const int idx = tid + 256 * v;
      if (!g.tb) {
        const int k = idx / (BN / 4), n4 = idx % (BN / 4);
        *reinterpret_cast<float4*>(&sm.b[buf][k][4 * n4]) = rb[v];
      } else {
        const int nn = idx / (kGBK / 4), k4 = idx % (kGBK / 4);
        sm.b[buf][4 * k4 + 0][nn] = rb[v].x;
        sm.b[buf][4 * k4 + 1][nn] = rb[v].y;
        sm.b[buf][4 * k4 + 2][nn] = rb[v].z;
        sm.b[buf][4 * k4 + 3][nn] = rb[v].w;
      }
    }
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
    for (int ks = 0; ks < kGBK / 2; ++ks) {
      const int kk = 2 * ks + (lane >> 5);
      float af[FM], bf[FN];
#pragma unroll
      for (int a = 0; a < FM; ++a) af[a] = sm.a[cur][kk][WM * wm + 32 * a + (lane & 31)];
#pragma unroll
      for (int b = 0; b < FN; ++b) bf[b] = sm.b[cur][kk][WN * wn + 32 * b + (lane & 31)];
#pragma unroll
      for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[a], bf[b], acc[a][b], 0, 0, 0);
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
        const int64_t j = n0 + WN * wn + 32 * b + (lane & 31);
        if (i < g.M && j < g.N) {
          float v = g.alpha * acc[a][b][r];
          if (g.beta != 0.f) v += g.beta * g.C[i * g.ldc + j];
          g.C[i * g.ldc + j] = v;
        }
      }
}

hipError_t launch_gemm_f32(hipStream_t s, const GemmArgs& g) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  if (g.M * g.N >= (int64_t)512 * 512) {
    dim3 grid((unsigned)ceil_div(g.N, 128), (unsigned)ceil_div(g.M, 128));
    hipLaunchKernelGGL((k_gemm_f32<128, 128>), grid, dim3(256), 0, s, g);
  } else {
    dim3 grid((unsigned)ceil_div(g.N, 64), (unsigned)ceil_div(g.M, 64));
    hipLaunchKernelGGL((k_gemm_f32<64, 64>), grid, dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- rotate
// U[i][j] = X[n-1-i][n-1-j]: the flat array reversed.
__global__ void k_rotate(const float* __restrict__ X, float* __restrict__ U, int64_t nn) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < nn; q += stride)
    U[q] = X[nn - 1 - q];
}

hipError_t launch_rotate(hipStream_t s, const float* X, float* U, int64_t n) {
  const int64_t nn = n * n;
  int64_t blocks = ceil_div(nn, 256);
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(k_rotate, dim3((unsigned)blocks), dim3(256), 0, s, X, U, nn);
  return hipGetLastError();
}

}  // namespace gq
