// Bid-Up: coordinate descent over the codes of a low-precision layer on its
// fixed quantization grid, for a fixed target T = W - B A.
//
// "Resumen Técnico: GPTQ-intrinsic LoRA", "Refinamiento Bid-Up": Q is
// optimised for fixed L and R by coordinate updates over the fixed
// quantization grid; with OLrC (the optimal low-rank part for fixed Q) the
// cycle never increases the layer error.
//
// One pass visits the columns in order. With residual d = T - W_hat and
// g = d H, the objective along code j is a parabola whose minimum lies at
// c_j + g_j / (H_jj s); the code moves to the nearest grid point, clamped to
// [0, maxq], and g -= delta H[j, :] with delta = s (c' - c). Lazy batches of
// 128 columns: inside a block each lane (one row) applies delta to the
// block's later columns at once; after the block the host applies
// G[:, later] -= Delta H[block, later] as one GEMM.
#include "common.h"

#include <algorithm>
#include <utility>

namespace gq {

constexpr int kBidB = 128;    // columns per block
constexpr int kBidRows = 64;  // rows per workgroup (one wave, one row per lane)

struct BidSmem {
  float h[kBidB][kBidB];      // H[j0 + a][j0 + b]
  float s[kBidRows][kBidB + 1];   // scale of (row, column); padded: lane-strided reads hit distinct banks
  int gi[kBidB];
};

template <int J>
__device__ __forceinline__ void bid_step(float (&g)[kBidB], BidSmem& sm, int lane, int nb, float maxq,
                                         uint8_t* __restrict__ crow, float* __restrict__ drow) {
  if (J >= nb) return;
  const float h = sm.h[J][J];
  const float s = sm.s[lane][J];
  const float c = (float)crow[J];
  float delta = 0.f;
  if (h > 0.f) {
    const float pre = c + g[J] / (h * s);
    const float cn = fminf(fmaxf(rintf(pre), 0.f), maxq);
    delta = s * (cn - c);
    crow[J] = (uint8_t)cn;
  }
  drow[J] = delta;
#pragma unroll
  for (int K = J + 1; K < kBidB; ++K) g[K] = fmaf(-delta, sm.h[J][K], g[K]);
}

template <int... Js>
__device__ __forceinline__ void bid_all(float (&g)[kBidB], BidSmem& sm, int lane, int nb, float maxq,
                                        uint8_t* crow, float* drow, std::integer_sequence<int, Js...>) {
  (bid_step<Js>(g, sm, lane, nb, maxq, crow, drow), ...);
}

// Block [j0, j0 + nb): G (d_out x n, pitch n) holds d H with every earlier
// change of this pass applied; codes are updated in place; Delta (d_out x
// kBidB) receives the deltas.
__global__ void __launch_bounds__(64)
k_bidup_block(const float* __restrict__ G, int64_t n, const float* __restrict__ H, uint8_t* __restrict__ codes,
              const float* __restrict__ scales, const int32_t* __restrict__ g_idx,
              int64_t ngroups, int64_t d_out, int64_t j0, int nb, float maxq, float* __restrict__ Delta) {
  __shared__ __align__(16) BidSmem sm;
  const int lane = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * kBidRows;
  for (int b = lane; b < kBidB; b += 64) sm.gi[b] = b < nb ? g_idx[j0 + b] : 0;
  for (int e = lane; e < kBidB * kBidB; e += 64) {
    const int a = e / kBidB, b = e % kBidB;
    sm.h[a][b] = (a < nb && b < nb) ? H[(j0 + a) * n + j0 + b] : 0.f;
  }
  __syncthreads();
  for (int e = lane; e < kBidRows * kBidB; e += 64) {
    const int rr = e / kBidB, b = e % kBidB;
    const int64_t row = min(r0 + rr, d_out - 1);
    const int64_t gi = sm.gi[b];
    sm.s[rr][b] = scales[row * ngroups + gi];
  }
  __syncthreads();
  const int64_t row = r0 + lane;
  if (row >= d_out) return;
  float g[kBidB];
  const float* grow = G + row * n + j0;
#pragma unroll
  for (int b = 0; b < kBidB; ++b) g[b] = b < nb ? grow[b] : 0.f;
  bid_all(g, sm, lane, nb, maxq, codes + row * n + j0, Delta + row * kBidB,
          std::make_integer_sequence<int, kBidB>{});
}

hipError_t launch_bidup_block(hipStream_t s, const float* G, int64_t n, const float* H, uint8_t* codes,
                              const float* scales, const int32_t* g_idx, int64_t ngroups,
                              int64_t d_out, int64_t j0, int nb, int bits, float* Delta) {
  if (nb < 1 || nb > kBidB) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_bidup_block, dim3((unsigned)ceil_div(d_out, kBidRows)), dim3(64), 0, s, G, n, H, codes,
                     scales, g_idx, ngroups, d_out, j0, nb, (float)((1 << bits) - 1), Delta);
  return hipGetLastError();
}

// D = T - s (c - z) (T, D: d_out x n; s, z through g_idx), or the
// dequantised codes alone when T is null.
__global__ void k_bid_residual(const float* __restrict__ T, const uint8_t* __restrict__ codes,
                               const float* __restrict__ scales, const uint8_t* __restrict__ zeros,
                               const int32_t* __restrict__ g_idx, int64_t ngroups, int64_t n,
                               float* __restrict__ D) {
  const int64_t r = blockIdx.y;
  for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < n; j += (int64_t)gridDim.x * 256) {
    const int64_t gi = g_idx[j];
    const float wh = scales[r * ngroups + gi] * ((float)codes[r * n + j] - (float)zeros[r * ngroups + gi]);
    D[r * n + j] = T ? T[r * n + j] - wh : wh;
  }
}

hipError_t launch_bid_residual(hipStream_t s, const float* T, const uint8_t* codes, const float* scales,
                               const uint8_t* zeros, const int32_t* g_idx, int64_t ngroups, int64_t d_out,
                               int64_t n, float* D) {
  if (d_out == 0 || n == 0) return hipSuccess;
  const dim3 grid((unsigned)std::min<int64_t>(ceil_div(n, 256), 64), (unsigned)d_out);
  hipLaunchKernelGGL(k_bid_residual, grid, dim3(256), 0, s, T, codes, scales, zeros, g_idx, ngroups, n, D);
  return hipGetLastError();
}

}  // namespace gq
