// Short-K products C[M x N] = alpha A[M x K] B[K x N] + beta C with K <= 128:
// the lazy-batch trailing update of the column sweep (K = block width) and
// the panel updates of the factorisation (K = panel width).
//
// "GPTQ" (wikiprompt.org), "Enfoque Técnico": after a block of columns is
// quantized, the remaining weights receive the closed-form correction of all
// of the block's errors at once (W[:, rest] -= E U[block, rest]).
//
// Layout (MI355X): a workgroup owns a 128-row slab of A, staged once into
// LDS (k-contiguous, alpha applied), and walks a range of 64-column tiles of
// B and C. B tiles are double-buffered through registers and LDS; the C tile
// is read while the MFMAs run and combined in the epilogue. Four waves as
// 2 x 2 over the 128 x 64 tile, each two v_mfma_f32_32x32x2f32 accumulators.
// With the slab resident, A is read from memory once per (slab, column
// range) instead of once per tile.
#include "common.h"
#include "leaf.h"

#include <algorithm>

namespace gq {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kSM = 128;         // slab rows
constexpr int kSN = 64;          // column tile
constexpr int kPBn = kSN + 4;    // B pitch when stored [k][n]

// LDS for K <= KT: the A slab [m][k] and two B tiles. KT = 64 needs 69 KiB,
// so two workgroups share a CU; KT = 128 needs 135 KiB.
template <int KT>
struct SlabSmem {
  static constexpr int PA = KT + 4;    // A pitch ([m][k])
  static constexpr int PBt = KT + 4;   // B pitch when stored [n][k]
  static constexpr int BSZ = (kSN * PBt > KT * kPBn) ? kSN * PBt : KT * kPBn;
  float a[kSM * PA];
  float b[2][BSZ];
};

// B tile (K x 64) -> registers: KT/16 float4 per thread. Full, 16-byte
// aligned tiles take a branch-free path.
template <bool TB, int KT>
__device__ __forceinline__ void slab_load_b(const SlabArgs& g, int64_t n0, int tid, float4 (&rb)[KT / 16]) {
  constexpr int V = KT / 16, Q = KT / 4;   // float4 per thread; float4 per B row (TB)
  const bool full = g.bvec && n0 + kSN <= g.N && g.K == KT;
  if (full) {
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int idx = tid + 256 * v;
      if constexpr (TB) {
        const int nn = idx / Q, k4 = idx % Q;
        rb[v] = *reinterpret_cast<const float4*>(g.B + (n0 + nn) * g.ldb + 4 * k4);
      } else {
        const int k = idx >> 4, n4 = idx & 15;
        rb[v] = *reinterpret_cast<const float4*>(g.B + (int64_t)k * g.ldb + n0 + 4 * n4);
      }
    }
    return;
  }
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int idx = tid + 256 * v;
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (TB) {   // B stored N x K
      const int nn = idx / Q, k4 = idx % Q;
      const int64_t n = n0 + nn, k = 4 * k4;
      if (n < g.N && k < g.K) {
        const float* p = g.B + n * g.ldb + k;
        if (k + 3 < g.K && (((uintptr_t)p & 15) == 0)) x = *reinterpret_cast<const float4*>(p);
        else {
          x.x = p[0];
          if (k + 1 < g.K) x.y = p[1];
          if (k + 2 < g.K) x.z = p[2];
          if (k + 3 < g.K) x.w = p[3];
        }
      }
    } else {              // B stored K x N: rows k, 16 float4 per row
      const int k = idx >> 4, n4 = idx & 15;
      const int64_t n = n0 + 4 * n4;
      if (k < g.K && n < g.N) {
        const float* p = g.B + (int64_t)k * g.ldb + n;
        if (n + 3 < g.N && (((uintptr_t)p & 15) == 0)) x = *reinterpret_cast<const float4*>(p);
        else {
          x.x = p[0];
          if (n + 1 < g.N) x.y = p[1];
          if (n + 2 < g.N) x.z = p[2];
          if (n + 3 < g.N) x.w = p[3];
        }
      }
    }
    rb[v] = x;
  }
}

template <bool TB, int KT>
__device__ __forceinline__ void slab_store_b(float* s, int tid, const float4 (&rb)[KT / 16]) {
  constexpr int V = KT / 16, Q = KT / 4;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int idx = tid + 256 * v;
    if constexpr (TB) {
      const int nn = idx / Q, k4 = idx % Q;
      *reinterpret_cast<float4*>(s + nn * SlabSmem<KT>::PBt + 4 * k4) = rb[v];
    } else {
      const int k = idx >> 4, n4 = idx & 15;
      *reinterpret_cast<float4*>(s + k * kPBn + 4 * n4) = rb[v];
    }
  }
}

__device__ __forceinline__ void slab_load_c(const SlabArgs& g, int64_t m0, int64_t n0, int wm, int wn,
                                            int lane, float (&cold)[2][16]) {
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t i = m0 + 64 * wm + 32 * a + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      const int64_t j = n0 + 32 * wn + (lane & 31);
      cold[a][r] = (g.beta != 0.f && i < g.M && j < g.N) ? g.C[i * g.ldc + j] : 0.f;
    }
}

template <bool TB, int KT>
__device__ __forceinline__ void slab_body(const SlabArgs& g, int wg, SlabSmem<KT>& sm) {
  constexpr int PA = SlabSmem<KT>::PA, PBt = SlabSmem<KT>::PBt;
  constexpr int VA = KT / 8, QA = KT / 4;   // A: float4 per thread; float4 per row
  const int slab = wg / g.nsplit, part = wg % g.nsplit;
  const int64_t m0 = (int64_t)slab * kSM;
  int64_t ntile = ceil_div(g.N, kSN);
  if (g.lower_only) ntile = min(ntile, ceil_div(m0 + kSM + g.lower_off, kSN));
  const int64_t per = ceil_div(ntile, g.nsplit);
  const int64_t t0 = part * per, t1 = min(ntile, t0 + per);
  if (t0 >= t1) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lk = 4 * (lane >> 5);

  // prologue: the A slab, the first B tile and the first C tile are all
  // requested before anything waits, so their latencies overlap
  float4 xa[VA];
#pragma unroll
  for (int v = 0; v < VA; ++v) {
    const int idx = tid + 256 * v;
    const int m = idx / QA, k = 4 * (idx % QA);
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    const int64_t row = m0 + m;
    if (row < g.M && k < g.K) {
      const float* p = g.A + row * g.lda + k;
      if (k + 3 < g.K && (((uintptr_t)p & 15) == 0)) x = *reinterpret_cast<const float4*>(p);
      else {
        x.x = p[0];
        if (k + 1 < g.K) x.y = p[1];
        if (k + 2 < g.K) x.z = p[2];
        if (k + 3 < g.K) x.w = p[3];
      }
    }
    xa[v] = x;
  }
  float4 rb[KT / 16];
  slab_load_b<TB, KT>(g, t0 * kSN, tid, rb);
  float cold[2][16];
  slab_load_c(g, m0, t0 * kSN, wm, wn, lane, cold);
  {
    const float al = g.alpha;
#pragma unroll
    for (int v = 0; v < VA; ++v) {
      const int idx = tid + 256 * v;
      const int m = idx / QA, k = 4 * (idx % QA);
      *reinterpret_cast<float4*>(&sm.a[m * PA + k]) =
          make_float4(al * xa[v].x, al * xa[v].y, al * xa[v].z, al * xa[v].w);
    }
  }
  slab_store_b<TB, KT>(sm.b[0], tid, rb);
  __syncthreads();

  for (int64_t t = t0; t < t1; ++t) {
    const int cur = (int)((t - t0) & 1);
    const int64_t n0 = t * kSN;
    const bool more = t + 1 < t1;
    if (more) slab_load_b<TB, KT>(g, n0 + kSN, tid, rb);
    if (t > t0) slab_load_c(g, m0, n0, wm, wn, lane, cold);
    f32x16_t acc[2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][r] = 0.f;
    const float* sb = sm.b[cur];
#pragma unroll
    for (int kq = 0; kq < KT / 8; ++kq) {
      const int kb = 8 * kq + lk;
      float4 fb;
      if constexpr (TB) {
        fb = *reinterpret_cast<const float4*>(sb + (32 * wn + lr) * PBt + kb);
      } else {
        const float* q = sb + kb * kPBn + 32 * wn + lr;
        fb = make_float4(q[0], q[kPBn], q[2 * kPBn], q[3 * kPBn]);
      }
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const float4 fa = *reinterpret_cast<const float4*>(&sm.a[(64 * wm + 32 * a + lr) * PA + kb]);
        acc[a] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa.x, fb.x, acc[a], 0, 0, 0);
        acc[a] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa.y, fb.y, acc[a], 0, 0, 0);
        acc[a] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa.z, fb.z, acc[a], 0, 0, 0);
        acc[a] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa.w, fb.w, acc[a], 0, 0, 0);
      }
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t i = m0 + 64 * wm + 32 * a + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t j = n0 + 32 * wn + lr;
        if (i < g.M && j < g.N) g.C[i * g.ldc + j] = acc[a][r] + g.beta * cold[a][r];
      }
    if (more) slab_store_b<TB, KT>(sm.b[cur ^ 1], tid, rb);
    __syncthreads();
  }
}

struct SlabPair {
  SlabArgs p[2];
  int nwg0;
};

template <int KT>
__global__ void __launch_bounds__(256, KT == 64 ? 2 : 1)
k_slab(SlabPair sp) {
  __shared__ __align__(16) SlabSmem<KT> sm;
  const int which = (int)blockIdx.x >= sp.nwg0;
  const SlabArgs& g = sp.p[which];
  if (g.st != nullptr && g.st->flags != 0) return;
  const int wg = (int)blockIdx.x - (which ? sp.nwg0 : 0);
  if (g.tb) slab_body<true, KT>(g, wg, sm);
  else slab_body<false, KT>(g, wg, sm);
}

// A slab pair plus the next diagonal block's update and leaf in workgroup 0
// (dispatched first, so the leaf runs while the trailing update streams).
__global__ void __launch_bounds__(256, 2)
k_slab_leaf(SlabPair sp, LeafTask lt) {
  __shared__ __align__(16) union {
    SlabSmem<64> slab;
    LeafTaskSmem leaf;
  } sm;
  if (lt.st != nullptr && lt.st->flags != 0) return;
  if (blockIdx.x == 0) {
    leaf_task_run(lt, sm.leaf);
    return;
  }
  const int b = (int)blockIdx.x - 1;
  const int which = b >= sp.nwg0;
  const SlabArgs& g = sp.p[which];
  const int wg = b - (which ? sp.nwg0 : 0);
  if (g.tb) slab_body<true, 64>(g, wg, sm.slab);
  else slab_body<false, 64>(g, wg, sm.slab);
}

static int slab_setup(SlabArgs& g, int max_split) {
  if (g.M <= 0 || g.N <= 0) return 0;
  g.bvec = ((uintptr_t)g.B % 16 == 0) && (g.ldb % 4 == 0);
  const int64_t nslab = ceil_div(g.M, kSM);
  const int64_t ntile = ceil_div(g.N, kSN);
  int64_t split = ceil_div(512, nslab);          // ~2 workgroups per CU in total
  if (split > ntile) split = ntile;
  if (split > max_split) split = max_split;
  if (split < 1) split = 1;
  g.nsplit = (int)split;
  return (int)(nslab * split);
}

hipError_t launch_slab_pair(hipStream_t s, SlabArgs a, int split_a, const SlabArgs* b, int split_b) {
  SlabPair sp{};
  sp.p[0] = a;
  sp.nwg0 = slab_setup(sp.p[0], split_a);
  int n1 = 0;
  if (b) {
    sp.p[1] = *b;
    n1 = slab_setup(sp.p[1], split_b);
  } else {
    sp.p[1] = sp.p[0];
  }
  const int total = sp.nwg0 + n1;
  if (total == 0) return hipSuccess;
  const int64_t kmax = std::max<int64_t>(a.K, b ? b->K : 0);
  if (kmax <= 64)
    hipLaunchKernelGGL(k_slab<64>, dim3(total), dim3(256), 0, s, sp);
  else
    hipLaunchKernelGGL(k_slab<128>, dim3(total), dim3(256), 0, s, sp);
  return hipGetLastError();
}

hipError_t launch_slab_pair_leaf(hipStream_t s, SlabArgs a, int split_a, const SlabArgs* b,
                                 int split_b, const LeafTask& lt) {
  if (a.K > 64 || (b && b->K > 64) || lt.mk > 64 || lt.m2 > 64 || lt.m2 < 1) return hipErrorInvalidValue;
  SlabPair sp{};
  sp.p[0] = a;
  sp.nwg0 = slab_setup(sp.p[0], split_a);
  int n1 = 0;
  if (b) {
    sp.p[1] = *b;
    n1 = slab_setup(sp.p[1], split_b);
  } else {
    sp.p[1] = sp.p[0];
  }
  hipLaunchKernelGGL(k_slab_leaf, dim3(1 + sp.nwg0 + n1), dim3(256), 0, s, sp, lt);
  return hipGetLastError();
}

hipError_t launch_slab(hipStream_t s, SlabArgs g, int max_split) {
  return launch_slab_pair(s, g, max_split, nullptr, 0);
}

}  // namespace gq
