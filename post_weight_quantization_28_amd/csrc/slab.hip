// Short-K products C[M x N] = alpha A[M x K] op(B) + beta C with K <= 128:
// the lazy-batch update of the column sweep inside a super-block (K = block
// width) and the trailing update of the factorisation (K = panel width).
//
// "GPTQ" (wikiprompt.org), "Enfoque Técnico": after a block of columns is
// quantized, the remaining weights receive the closed-form correction of all
// of the block's errors at once (W[:, rest] -= E U[block, rest]).
//
// Layout (MI355X): with K this short, every output element is read and
// written once for only 2K flops, so the kernel is built to stream C with
// as little per-element work as possible and enough waves to fill the chip:
//  * a workgroup covers 32 rows x 64 columns; wave w owns columns
//    16w..16w+15 as two 16 x 16 v_mfma_f32_16x16x4f32 tiles, independently
//    of the other waves (no LDS, no barrier);
//  * operands are read straight from memory: for MFMA t of a group of four,
//    lane group g = lane / 16 feeds k = 16p + 4g + t to both operands, so A
//    (and B when stored N x K) arrive as one 16-byte read per lane per 16 k;
//    B stored K x N arrives as four 4-byte reads of consecutive k rows;
//  * every load of a wave (A, B and the C tile) is issued before the first
//    MFMA; rows and columns past the edge are clamped to valid addresses
//    and never stored.
// The factorisation's update needs only the lower band (j <= i + lower_off);
// waves whose columns lie wholly above it exit at once.
#include "common.h"
#include "leaf.h"

#include <algorithm>

namespace gq {

typedef float kp_f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kPM = 32;   // rows per workgroup
constexpr int kPN = 64;   // columns per workgroup (16 per wave)

template <bool TB, int KT>
__device__ __forceinline__ void kprod_wave(const SlabArgs& g, int64_t r0, int64_t c0, int lane) {
  constexpr int P = KT / 16;
  const int li = lane & 15, gq = lane >> 4;
  const int64_t M = g.M, N = g.N;
  const int K = (int)g.K;
  const float* pa0 = g.A + std::min<int64_t>(r0 + li, M - 1) * g.lda + 4 * gq;
  const float* pa1 = g.A + std::min<int64_t>(r0 + 16 + li, M - 1) * g.lda + 4 * gq;
  const int64_t col = std::min<int64_t>(c0 + li, N - 1);
  float4 a0[P], a1[P], b[P];
  const bool vec = K == KT && ((g.lda & 3) == 0) && (((uintptr_t)g.A & 15) == 0) &&
                   (!TB || (((g.ldb & 3) == 0) && (((uintptr_t)g.B & 15) == 0)));
  if (vec) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      a0[p] = *reinterpret_cast<const float4*>(pa0 + 16 * p);
      a1[p] = *reinterpret_cast<const float4*>(pa1 + 16 * p);
      if constexpr (TB) {
        b[p] = *reinterpret_cast<const float4*>(g.B + col * g.ldb + 16 * p + 4 * gq);
      } else {
        const float* q = g.B + (int64_t)(16 * p + 4 * gq) * g.ldb + col;
        b[p] = make_float4(q[0], q[g.ldb], q[2 * g.ldb], q[3 * g.ldb]);
      }
    }
  } else {
    // K below the template width (or unaligned rows): 4-byte reads, k >= K
    // read as zero (the addresses stay inside row k = K - 1)
#pragma unroll
    for (int p = 0; p < P; ++p) {
      float va0[4], va1[4], vb[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int k = 16 * p + 4 * gq + t;
        const int kc = std::min(k, K - 1) - 4 * gq;   // offset from the lane's base
        const bool ok = k < K;
        va0[t] = ok ? pa0[kc] : 0.f;
        va1[t] = ok ? pa1[kc] : 0.f;
        const int kk = std::min(k, K - 1);
        if constexpr (TB) vb[t] = ok ? g.B[col * g.ldb + kk] : 0.f;
        else vb[t] = ok ? g.B[(int64_t)kk * g.ldb + col] : 0.f;
      }
      a0[p] = make_float4(va0[0], va0[1], va0[2], va0[3]);
      a1[p] = make_float4(va1[0], va1[1], va1[2], va1[3]);
      b[p] = make_float4(vb[0], vb[1], vb[2], vb[3]);
    }
  }
  float cv[2][4];
  if (g.beta != 0.f) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t row = std::min<int64_t>(r0 + 16 * rt + 4 * gq + v, M - 1);
        cv[rt][v] = g.C[row * g.ldc + col];
      }
  } else {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v) cv[rt][v] = 0.f;
  }
  kp_f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < P; ++p) {
    acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a0[p].x, b[p].x, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a1[p].x, b[p].x, acc1, 0, 0, 0);
    acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a0[p].y, b[p].y, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a1[p].y, b[p].y, acc1, 0, 0, 0);
    acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a0[p].z, b[p].z, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a1[p].z, b[p].z, acc1, 0, 0, 0);
    acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a0[p].w, b[p].w, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a1[p].w, b[p].w, acc1, 0, 0, 0);
  }
  if (c0 + li >= N) return;
  const float al = g.alpha, be = g.beta;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t row = r0 + 4 * gq + v;
    if (row < M) g.C[row * g.ldc + col] = fmaf(al, acc0[v], be * cv[0][v]);
    if (row + 16 < M) g.C[(row + 16) * g.ldc + col] = fmaf(al, acc1[v], be * cv[1][v]);
  }
}

// Tile b of the product (row-major over 32 x 64 workgroup tiles).
template <int KT>
__device__ __forceinline__ void kprod_tile(const SlabArgs& g, int64_t b) {
  const int64_t ncb = ceil_div(g.N, kPN);
  const int64_t r0 = (b / ncb) * kPM;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t c0 = (b % ncb) * kPN + 16 * w;
  if (c0 >= g.N) return;
  if (g.lower_only && c0 > r0 + kPM - 1 + g.lower_off) return;
  if (g.tb) kprod_wave<true, KT>(g, r0, c0, lane);
  else kprod_wave<false, KT>(g, r0, c0, lane);
}

template <int KT>
__global__ void __launch_bounds__(256)
k_kprod(SlabArgs g) {
  if (g.st != nullptr && g.st->flags != 0) return;
  kprod_tile<KT>(g, blockIdx.x);
}

// The factorisation's trailing update plus, in workgroup 0 (dispatched
// first), the next diagonal block's update and leaf, which then runs while
// the trailing update streams.
__global__ void __launch_bounds__(256)
k_kprod_leaf(SlabArgs g, LeafTask lt) {
  __shared__ __align__(16) LeafTaskSmem sm;
  if (lt.st != nullptr && lt.st->flags != 0) return;
  if (blockIdx.x == 0) {
    leaf_task_run(lt, sm);
    return;
  }
  kprod_tile<64>(g, (int64_t)blockIdx.x - 1);
}

static int64_t kprod_tiles(const SlabArgs& g) {
  if (g.M <= 0 || g.N <= 0) return 0;
  return ceil_div(g.M, kPM) * ceil_div(g.N, kPN);
}

hipError_t launch_slab(hipStream_t s, const SlabArgs& g) {
  if (g.K < 1 || g.K > 128) return hipErrorInvalidValue;
  const int64_t nt = kprod_tiles(g);
  if (nt == 0) return hipSuccess;
  if (nt >= (int64_t)1 << 31) return hipErrorInvalidValue;
  if (g.K <= 64)
    hipLaunchKernelGGL(k_kprod<64>, dim3((unsigned)nt), dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL(k_kprod<128>, dim3((unsigned)nt), dim3(256), 0, s, g);
  return hipGetLastError();
}

hipError_t launch_slab_leaf(hipStream_t s, const SlabArgs& g, const LeafTask& lt) {
  if (g.K < 1 || g.K > 64 || lt.mk > 64 || lt.m2 > 64 || lt.m2 < 1 || lt.mk < 1) return hipErrorInvalidValue;
  const int64_t nt = kprod_tiles(g);
  if (nt + 1 >= (int64_t)1 << 31) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_kprod_leaf, dim3((unsigned)(1 + nt)), dim3(256), 0, s, g, lt);
  return hipGetLastError();
}

}  // namespace gq
