// EoRA: rank-r compensation B A of a compressed layer's error in the
// eigenspace of the activation covariance.
//
// "Aumento de la precisión de LLM de 2 bits con EoRA" (7minutos.es),
// "Bucear en el espacio propio en busca de un adaptador": the error
// Delta W = W - W_hat is projected into the eigenspace of the activation
// covariance, Delta W' = Delta W Q Lambda^{1/2}, truncated to rank r by SVD
// and projected back (B = U'_r Sigma'_r, A = V'_r^T Lambda^{-1/2} Q^T).
//
// Computed here without an eigendecomposition of H: for any square root R
// of H = R R^T the rank-r truncation [Delta W R]_r R^{-1} is the same
// product (square roots differ by an orthogonal factor, which commutes with
// the truncation), and its left factor is the top-r eigenspace of
//   G = Delta W H Delta W^T = (Delta W R)(Delta W R)^T   (d_out x d_out).
// With G = U' Sigma'^2 U'^T: B = U'_r Sigma'_r and
// A = Sigma'_r^{-1} U'_r^T Delta W, so B A = U'_r U'_r^T Delta W. The top
// eigenpairs of G come from block subspace iteration with CholeskyQR and a
// Rayleigh-Ritz step whose k x k eigenproblem is solved here by Jacobi
// rotations (the host sequences the GEMMs and the Cholesky factorisations).
#include "common.h"

#include <algorithm>

namespace gq {

// D = W - W_hat (fp32), W bf16 or fp32 with row stride ldw; non-finite
// entries raise kNonFinite with their column.
template <bool kBF16>
__global__ void __launch_bounds__(256)
k_eora_delta(const void* __restrict__ W, int64_t ldw, const float* __restrict__ Wh, int64_t n,
             float* __restrict__ D, DevStatus* st) {
  const int64_t r = blockIdx.y;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < n; c += (int64_t)gridDim.x * 256) {
    float w;
    if (kBF16) w = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(W)[r * ldw + c] << 16);
    else w = reinterpret_cast<const float*>(W)[r * ldw + c];
    const float d = w - Wh[r * n + c];
    if (!isfinite(d)) raise_status(st, kNonFinite, c);
    D[r * n + c] = d;
  }
}

hipError_t launch_eora_delta(hipStream_t s, const void* W, int wbf16, int64_t ldw, const float* Wh,
                             int64_t d_out, int64_t n, float* D, DevStatus* st) {
  if (d_out == 0 || n == 0) return hipSuccess;
  const dim3 grid((unsigned)std::min<int64_t>(ceil_div(n, 256), 64), (unsigned)d_out);
  if (wbf16) hipLaunchKernelGGL(k_eora_delta<true>, grid, dim3(256), 0, s, W, ldw, Wh, n, D, st);
  else hipLaunchKernelGGL(k_eora_delta<false>, grid, dim3(256), 0, s, W, ldw, Wh, n, D, st);
  return hipGetLastError();
}

// The start block of the subspace iteration: Om[i][j] = 1 if i % k == j
// (column j of G Om sums the rows of G congruent to j), a fixed pattern.
__global__ void k_eora_start(float* __restrict__ Om, int64_t d, int k) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= d * k) return;
  const int64_t i = q / k, j = q % k;
  Om[q] = (i % k == j) ? 1.f : 0.f;
}

hipError_t launch_eora_start(hipStream_t s, float* Om, int64_t d, int k) {
  hipLaunchKernelGGL(k_eora_start, dim3((unsigned)ceil_div(d * k, 256)), dim3(256), 0, s, Om, d, k);
  return hipGetLastError();
}

// Y[:, j] /= ||Y[:, j]|| (d x k, row-major; a zero column stays zero): the
// CholeskyQR Gram matrix then has a unit diagonal, so its conditioning is
// that of the columns' directions, not of their lengths. One workgroup per
// column, fixed-order reduction.
__global__ void __launch_bounds__(256)
k_col_normalize(float* __restrict__ Y, int64_t d, int k) {
  __shared__ double red[256];
  const int j = blockIdx.x;
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < d; i += 256) {
    const double v = Y[i * k + j];
    acc += v * v;
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  const double nrm = sqrt(red[0]);
  const float f = nrm > 0.0 ? (float)(1.0 / nrm) : 0.f;
  for (int64_t i = threadIdx.x; i < d; i += 256) Y[i * k + j] *= f;
}

hipError_t launch_col_normalize(hipStream_t s, float* Y, int64_t d, int k) {
  hipLaunchKernelGGL(k_col_normalize, dim3((unsigned)k), dim3(256), 0, s, Y, d, k);
  return hipGetLastError();
}

// C[i] = sum over p of part[p * count + i], in p order (the split-K sums of
// the skinny products below).
__global__ void k_sum_partials(const float* __restrict__ part, int np, int64_t count, float* __restrict__ C) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count) return;
  float v = 0.f;
  for (int p = 0; p < np; ++p) v += part[p * count + i];
  C[i] = v;
}

hipError_t launch_sum_partials(hipStream_t s, const float* part, int np, int64_t count, float* C) {
  hipLaunchKernelGGL(k_sum_partials, dim3((unsigned)ceil_div(count, 256)), dim3(256), 0, s, part, np, count, C);
  return hipGetLastError();
}

// ---- Jacobi eigensolver for one small symmetric matrix (k <= 128, even).
// Cyclic Jacobi in round-robin order: every round rotates k/2 disjoint
// index pairs at once, (r mod m, k-1) and ((r + j) mod m, (r - j) mod m),
// j = 1..k/2-1, m = k - 1, so a sweep of m rounds meets every pair once.
// A rotation J (J_pp = J_qq = c, J_pq = s, J_qp = -s) with
// t = sign(tau) / (|tau| + sqrt(1 + tau^2)), tau = (S_qq - S_pp) / (2 S_pq),
// c = 1 / sqrt(1 + t^2), s = t c zeroes S_pq in J^T S J (Golub and Van
// Loan, the symmetric Schur decomposition); V accumulates the rotations.
// Sweeps stop when the off-diagonal Frobenius norm is at most 1e-7 of the
// whole (or after kJacobiSweeps). Output: eigenvalues in descending order
// (equal values by index) and V's columns in the same order.
constexpr int kJacobiMax = 128;
constexpr int kJacobiSweeps = 16;

struct JacobiSmem {
  float S[kJacobiMax][kJacobiMax + 1];
  float V[kJacobiMax][kJacobiMax + 1];
  float c[kJacobiMax / 2], sn[kJacobiMax / 2];
  int p[kJacobiMax / 2], q[kJacobiMax / 2];
  float red[1024 / 64];
  float diag[kJacobiMax];
};

__global__ void __launch_bounds__(1024)
k_sym_eig_jacobi(const float* __restrict__ Sin, int k, float* __restrict__ theta, float* __restrict__ Vout) {
  __shared__ __align__(16) JacobiSmem sm;
  const int tid = threadIdx.x, nt = blockDim.x;
  const int m = k - 1, half = k / 2;
  for (int e = tid; e < k * k; e += nt) {
    const int i = e / k, j = e % k;
    sm.S[i][j] = 0.5f * (Sin[i * k + j] + Sin[j * k + i]);
    sm.V[i][j] = (i == j) ? 1.f : 0.f;
  }
  __syncthreads();
  for (int sweep = 0; sweep < kJacobiSweeps; ++sweep) {
    // convergence: off-diagonal norm against the whole
    float off = 0.f, all = 0.f;
    for (int e = tid; e < k * k; e += nt) {
      const int i = e / k, j = e % k;
      const float v = sm.S[i][j];
      all += v * v;
      if (i != j) off += v * v;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      off += __shfl_xor(off, o);
      all += __shfl_xor(all, o);
    }
    __syncthreads();
    if ((tid & 63) == 0) sm.red[tid >> 6] = off;
    __syncthreads();
    float offs = 0.f;
    for (int w = 0; w < nt / 64; ++w) offs += sm.red[w];
    __syncthreads();
    if ((tid & 63) == 0) sm.red[tid >> 6] = all;
    __syncthreads();
    float alls = 0.f;
    for (int w = 0; w < nt / 64; ++w) alls += sm.red[w];
    __syncthreads();
    // fp32 rounding leaves off^2 near k eps^2 of the whole once converged
    if (!(offs > 1e-11f * alls)) break;          // uniform across the workgroup
    for (int r = 0; r < m; ++r) {
      if (tid < half) {
        int a, b;
        if (tid == 0) {
          a = r % m;
          b = k - 1;
        } else {
          a = (r + tid) % m;
          b = (r - tid + m) % m;
        }
        const int pp = min(a, b), qq = max(a, b);
        const float apq = sm.S[pp][qq];
        float c = 1.f, s = 0.f;
        if (apq != 0.f) {
          const float tau = (sm.S[qq][qq] - sm.S[pp][pp]) / (2.f * apq);
          const float t = (tau >= 0.f ? 1.f : -1.f) / (fabsf(tau) + sqrtf(1.f + tau * tau));
          c = 1.f / sqrtf(1.f + t * t);
          s = t * c;
        }
        sm.p[tid] = pp;
        sm.q[tid] = qq;
        sm.c[tid] = c;
        sm.sn[tid] = s;
      }
      __syncthreads();
      // rows: S <- J^T S
      for (int e = tid; e < half * k; e += nt) {
        const int pi = e / k, j = e % k;
        const int pp = sm.p[pi], qq = sm.q[pi];
        const float c = sm.c[pi], s = sm.sn[pi];
        const float sp = sm.S[pp][j], sq = sm.S[qq][j];
        sm.S[pp][j] = c * sp - s * sq;
        sm.S[qq][j] = s * sp + c * sq;
      }
      __syncthreads();
      // columns: S <- S J, V <- V J
      for (int e = tid; e < half * k; e += nt) {
        const int pi = e / k, i = e % k;
        const int pp = sm.p[pi], qq = sm.q[pi];
        const float c = sm.c[pi], s = sm.sn[pi];
        const float sp = sm.S[i][pp], sq = sm.S[i][qq];
        sm.S[i][pp] = c * sp - s * sq;
        sm.S[i][qq] = s * sp + c * sq;
        const float vp = sm.V[i][pp], vq = sm.V[i][qq];
        sm.V[i][pp] = c * vp - s * vq;
        sm.V[i][qq] = s * vp + c * vq;
      }
      __syncthreads();
      if (tid < half) {
        const int pp = sm.p[tid], qq = sm.q[tid];
        sm.S[pp][qq] = 0.f;
        sm.S[qq][pp] = 0.f;
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < k; i += nt) sm.diag[i] = sm.S[i][i];
  __syncthreads();
  // descending order, ties by index: output slot of eigenpair i
  for (int i = tid; i < k; i += nt) {
    const float di = sm.diag[i];
    int rank = 0;
    for (int j = 0; j < k; ++j) {
      const float dj = sm.diag[j];
      rank += (dj > di) || (dj == di && j < i);
    }
    theta[rank] = di;
    for (int row = 0; row < k; ++row) Vout[row * k + rank] = sm.V[row][i];
  }
}

hipError_t launch_sym_eig_jacobi(hipStream_t s, const float* S, int k, float* theta, float* V) {
  if (k < 2 || k > kJacobiMax || (k & 1)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_sym_eig_jacobi, dim3(1), dim3(1024), 0, s, S, k, theta, V);
  return hipGetLastError();
}

// sigma_j = sqrt(max(theta_j, 0)); B[:, j] = Ur[:, j] sigma_j (in place,
// d x r, pitch ldb); A's row j = its value / sigma_j (0 when sigma_j = 0).
__global__ void k_eora_sigma(const float* __restrict__ theta, int r, float* __restrict__ sigma) {
  const int j = threadIdx.x;
  if (j < r) sigma[j] = sqrtf(fmaxf(theta[j], 0.f));
}

__global__ void k_eora_scale_cols(float* __restrict__ B, int64_t d, int r, int64_t ldb,
                                  const float* __restrict__ sigma) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= d * r) return;
  const int64_t i = q / r;
  const int j = (int)(q % r);
  B[i * ldb + j] *= sigma[j];
}

__global__ void k_eora_scale_rows(float* __restrict__ A, int r, int64_t n, const float* __restrict__ sigma) {
  const int j = blockIdx.y;
  const float s = sigma[j];
  const float f = s > 0.f ? 1.f / s : 0.f;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < n; c += (int64_t)gridDim.x * 256)
    A[j * n + c] *= f;
}

hipError_t launch_eora_finish(hipStream_t s, const float* theta, int r, float* sigma, float* B, int64_t d,
                              int64_t ldb, float* A, int64_t n) {
  hipLaunchKernelGGL(k_eora_sigma, dim3(1), dim3(128), 0, s, theta, r, sigma);
  hipLaunchKernelGGL(k_eora_scale_cols, dim3((unsigned)ceil_div(d * r, 256)), dim3(256), 0, s, B, d, r, ldb,
                     sigma);
  if (n > 0)
    hipLaunchKernelGGL(k_eora_scale_rows, dim3((unsigned)std::min<int64_t>(ceil_div(n, 256), 64), (unsigned)r),
                       dim3(256), 0, s, A, r, n, sigma);
  return hipGetLastError();
}

}  // namespace gq
