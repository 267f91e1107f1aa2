// Short-K products C[M x N] = alpha A[M x K] op(B) + beta C with K <= 128:
// the lazy-batch update of the column sweep inside a super-block (K = block
// width) and the trailing update of the factorisation (K = panel width).
//
// "GPTQ" (wikiprompt.org), "Enfoque Técnico": after a block of columns is
// quantized, the remaining weights receive the closed-form correction of all
// of the block's errors at once (W[:, rest] -= E U[block, rest]).
//
// Layout (MI355X): with K this short, every output element is read and
// written once for only 2K flops, so the kernel streams C with little
// per-element work and keeps operand traffic low:
//  * a workgroup covers 64 x 64 outputs; its A rows and B columns (K <= KT
//    deep) are loaded once, with 16-byte coalesced reads, into LDS as
//    [row][k] / [column][k] (pitch KT + 4 floats) and shared by the four
//    waves, so each output costs 8K/64 bytes of operand reads instead of
//    the 24K/64 of per-wave loading;
//  * wave (wm, wn) owns the 32 x 32 block at (32 wm, 32 wn) as 2 x 2
//    v_mfma_f32_16x16x4f32 tiles; for MFMA t of a group of four, lane group
//    g = lane / 16 feeds k = 16p + 4g + t to both operands, so each operand
//    fragment is one 16-byte LDS read;
//  * the C block is requested before the operands are staged, so its
//    latency overlaps the staging; rows and columns past the edge are
//    clamped to valid addresses and never stored.
// The factorisation's update needs only the lower band (j <= i + lower_off);
// workgroups wholly above it exit at once, waves above it after staging.
#include "common.h"
#include "leaf.h"

#include <algorithm>

namespace gq {

typedef float kp_f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kPN = 64;   // columns per workgroup

// RM rows per workgroup: 64 (waves 2 x 2, each 32 x 32) or 32 (waves 1 x 4,
// each 32 x 16, for products too narrow to fill the chip with 64-row tiles)
template <int KT, int RM>
struct KprodSmem {
  float a[RM][KT + 4];    // A[r0 + m][k]
  float b[kPN][KT + 4];   // B(k, c0 + n), stored [n][k]
};

template <int KT, int RM>
__device__ __forceinline__ void kprod_tile(const SlabArgs& g, int64_t b, KprodSmem<KT, RM>& sm) {
  constexpr int kPM = RM;
  constexpr int WC = RM == 64 ? 2 : 4;       // waves across the columns
  constexpr int CT = 2 / (WC / 2);           // 16-column tiles per wave: 2 or 1
  constexpr int Q = KT / 4;                  // float4 per operand row
  constexpr int VA = kPM * Q / 256;          // float4 per thread of A
  constexpr int VB = kPN * Q / 256;          // float4 per thread of B
  const int64_t ncb = ceil_div(g.N, kPN);
  const int64_t r0 = (b / ncb) * kPM, c0 = (b % ncb) * kPN;
  if (g.lower_only && c0 > r0 + kPM - 1 + g.lower_off) return;   // whole workgroup
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w / WC, wn = w % WC;
  const int li = lane & 15, gq = lane >> 4;
  const int64_t M = g.M, N = g.N;
  const int K = (int)g.K;

  // the wave's C block first (clamped, unconditional: no wait per load)
  float cv[2][CT][4];
  const bool beta = g.beta != 0.f;
  if (beta) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int64_t row = std::min<int64_t>(r0 + 32 * wm + 16 * rt + 4 * gq + v, M - 1);
          const int64_t col = std::min<int64_t>(c0 + 16 * CT * wn + 16 * ct + li, N - 1);
          cv[rt][ct][v] = g.C[row * g.ldc + col];
        }
  }

  // stage A rows and B columns
  const bool avec = K == KT && ((g.lda & 3) == 0) && (((uintptr_t)g.A & 15) == 0);
  const bool bvec = K == KT && ((g.ldb & 3) == 0) && (((uintptr_t)g.B & 15) == 0);
  float4 xa[VA], xb[VB];
#pragma unroll
  for (int v = 0; v < VA; ++v) {
    const int idx = tid + 256 * v;
    const int m = idx / Q, k4 = 4 * (idx % Q);
    const float* pa = g.A + std::min<int64_t>(r0 + m, M - 1) * g.lda;
    if (avec) {
      xa[v] = *reinterpret_cast<const float4*>(pa + k4);
    } else {
      float t[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] = (k4 + e < K) ? pa[std::min(k4 + e, K - 1)] : 0.f;
      xa[v] = make_float4(t[0], t[1], t[2], t[3]);
    }
  }
#pragma unroll
  for (int v = 0; v < VB; ++v) {
    const int idx = tid + 256 * v;
    if (g.tb) {            // B stored N x K: rows of k
      const int m = idx / Q, k4 = 4 * (idx % Q);
      const float* pb = g.B + std::min<int64_t>(c0 + m, N - 1) * g.ldb;
      if (bvec) {
        xb[v] = *reinterpret_cast<const float4*>(pb + k4);
      } else {
        float t[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = (k4 + e < K) ? pb[std::min(k4 + e, K - 1)] : 0.f;
        xb[v] = make_float4(t[0], t[1], t[2], t[3]);
      }
    } else {               // B stored K x N: row k, 4 consecutive columns
      const int kr = idx / (kPN / 4), n4 = 4 * (idx % (kPN / 4));
      const float* pb = g.B + (int64_t)std::min(kr, K - 1) * g.ldb;
      if (bvec && c0 + kPN <= N) {
        xb[v] = *reinterpret_cast<const float4*>(pb + c0 + n4);
      } else {
        float t[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = (kr < K) ? pb[std::min<int64_t>(c0 + n4 + e, N - 1)] : 0.f;
        xb[v] = make_float4(t[0], t[1], t[2], t[3]);
      }
    }
  }
#pragma unroll
  for (int v = 0; v < VA; ++v) {
    const int idx = tid + 256 * v;
    const int m = idx / Q, k4 = 4 * (idx % Q);
    *reinterpret_cast<float4*>(&sm.a[m][k4]) = xa[v];
  }
#pragma unroll
  for (int v = 0; v < VB; ++v) {
    const int idx = tid + 256 * v;
    if (g.tb) {
      const int m = idx / Q, k4 = 4 * (idx % Q);
      *reinterpret_cast<float4*>(&sm.b[m][k4]) = xb[v];
    } else {
      const int kr = idx / (kPN / 4), n4 = 4 * (idx % (kPN / 4));
      sm.b[n4][kr] = xb[v].x;
      sm.b[n4 + 1][kr] = xb[v].y;
      sm.b[n4 + 2][kr] = xb[v].z;
      sm.b[n4 + 3][kr] = xb[v].w;
    }
  }
  __syncthreads();
  if (g.lower_only && c0 + 16 * CT * wn > r0 + 32 * wm + 31 + g.lower_off) return;   // this wave's block

  kp_f32x4_t acc[2][CT];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[rt][ct] = (kp_f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < KT / 16; ++p) {
    float4 fa[2], fb[CT];
#pragma unroll
    for (int t = 0; t < 2; ++t)
      fa[t] = *reinterpret_cast<const float4*>(&sm.a[32 * wm + 16 * t + li][16 * p + 4 * gq]);
#pragma unroll
    for (int t = 0; t < CT; ++t)
      fb[t] = *reinterpret_cast<const float4*>(&sm.b[16 * CT * wn + 16 * t + li][16 * p + 4 * gq]);
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[rt].x, fb[ct].x, acc[rt][ct], 0, 0, 0);
        acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[rt].y, fb[ct].y, acc[rt][ct], 0, 0, 0);
        acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[rt].z, fb[ct].z, acc[rt][ct], 0, 0, 0);
        acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[rt].w, fb[ct].w, acc[rt][ct], 0, 0, 0);
      }
  }
  const float al = g.alpha, be = g.beta;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int64_t col = c0 + 16 * CT * wn + 16 * ct + li;
    if (col >= N) continue;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t row = r0 + 32 * wm + 16 * rt + 4 * gq + v;
        if (row < M) g.C[row * g.ldc + col] = fmaf(al, acc[rt][ct][v], beta ? be * cv[rt][ct][v] : 0.f);
      }
  }
}

template <int KT, int RM>
__global__ void __launch_bounds__(256)
k_kprod(SlabArgs g) {
  __shared__ __align__(16) KprodSmem<KT, RM> sm;
  if (g.st != nullptr && g.st->flags != 0) return;
  kprod_tile<KT, RM>(g, blockIdx.x, sm);
}

// The factorisation's trailing update plus, in workgroup 0 (dispatched
// first), the next diagonal block's update and leaf, which then runs while
// the trailing update streams.
__global__ void __launch_bounds__(256)
k_kprod_leaf(SlabArgs g, LeafTask lt) {
  __shared__ __align__(16) union {
    LeafTaskSmem leaf;
    KprodSmem<64, 64> prod;
  } sm;
  if (lt.st != nullptr && lt.st->flags != 0) return;
  if (blockIdx.x == 0) {
    leaf_task_run(lt, sm.leaf);
    return;
  }
  kprod_tile<64, 64>(g, (int64_t)blockIdx.x - 1, sm.prod);
}

static int64_t kprod_tiles(const SlabArgs& g, int rm) {
  if (g.M <= 0 || g.N <= 0) return 0;
  return ceil_div(g.M, rm) * ceil_div(g.N, kPN);
}

hipError_t launch_slab(hipStream_t s, const SlabArgs& g) {
  if (g.K < 1 || g.K > 128) return hipErrorInvalidValue;
  // 64-row tiles unless they leave the 256 CUs with under two workgroups each
  const int rm = kprod_tiles(g, 64) >= 512 ? 64 : 32;
  const int64_t nt = kprod_tiles(g, rm);
  if (nt == 0) return hipSuccess;
  if (nt >= (int64_t)1 << 31) return hipErrorInvalidValue;
  if (g.K <= 64) {
    if (rm == 64) hipLaunchKernelGGL((k_kprod<64, 64>), dim3((unsigned)nt), dim3(256), 0, s, g);
    else hipLaunchKernelGGL((k_kprod<64, 32>), dim3((unsigned)nt), dim3(256), 0, s, g);
  } else {
    if (rm == 64) hipLaunchKernelGGL((k_kprod<128, 64>), dim3((unsigned)nt), dim3(256), 0, s, g);
    else hipLaunchKernelGGL((k_kprod<128, 32>), dim3((unsigned)nt), dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

hipError_t launch_slab_leaf(hipStream_t s, const SlabArgs& g, const LeafTask& lt) {
  if (g.K < 1 || g.K > 64 || lt.mk > 64 || lt.m2 > 64 || lt.m2 < 1 || lt.mk < 1) return hipErrorInvalidValue;
  const int64_t nt = kprod_tiles(g, 64);
  if (nt + 1 >= (int64_t)1 << 31) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_kprod_leaf, dim3((unsigned)(1 + nt)), dim3(256), 0, s, g, lt);
  return hipGetLastError();
}

}  // namespace gq
