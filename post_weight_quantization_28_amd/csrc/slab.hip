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
#include "dma.h"
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
  if (blockIdx.x == 0) {
    leaf_task_run(lt, sm.leaf);
    return;
  }
  kprod_tile<64, 64>(g, (int64_t)blockIdx.x - 1, sm.prod);
}

// ---- the factorisation's trailing update: persistent and pipelined
//
// K = 64 (one panel) and B stored N x K, i.e. C -= L21[rows] L21[cols]^T
// over the lower band. With K this short each output costs 2K flops for
// 8 bytes of C traffic, so C must keep streaming while the MFMAs run. One
// workgroup of 8 waves per CU walks a strided list of the band's 64 x 64
// tiles through a 3-stage LDS ring (A rows, B rows and C block of a tile
// per stage), with the waves split by role so that each SIMD always has
// one wave issuing MFMAs:
//  * waves 4-7 move data: they stream tile i + 2 into the ring by LDS-DMA
//    and write tile i - 1's results from LDS to C, while
//  * waves 0-3 multiply tile i: wave (wm, wn) owns the 32 x 32 block at
//    (32 wm, 32 wn) as one v_mfma_f32_32x32x2f32 accumulator (for MFMA s of
//    a group of four, lane half h feeds k = 8q + 4h + s to both operands, so
//    a lane's operand piece is one 16-byte LDS read), then adds C and writes
//    the result over C in the stage.
// One barrier per tile hands the stages over. Buffer descriptors end at
// the last row of A, B and C, so rows past the edge read as zeros and
// stores past C are dropped; N % 4 == 0 keeps 16-byte chunks from
// straddling the last column.
//  * A / B tile: row r is 256 bytes, its 16-byte chunk c stored at chunk
//    c ^ (r % 16), so the 16 rows read by one ds_read_b128 phase fall in
//    distinct banks. C tile: chunk c of row r at c ^ (8 ((r / 4) % 2)), so
//    the two rows read by one ds_read_b32 (4 apart) use different banks.
constexpr int kPA = 64 * 64 * 4;          // bytes of A (= B = C) per tile: 16 KiB
constexpr int kPStage = 3 * kPA;          // 48 KiB
constexpr int kPStages = 3;

struct PipeSmem {
  uint8_t stage[kPStages][kPStage];
};

__device__ __forceinline__ int64_t band_prefix(int r, int d) { return (int64_t)r * (r - 1) / 2 + (int64_t)d * r; }

// Tile t of the band (row-major) -> row tile rt, column tile ct.
__device__ __forceinline__ void band_tile(const BandTiles& bt, int t, int& rt, int& ct) {
  if (t >= bt.ps) {
    rt = bt.rs + (int)((t - bt.ps) / bt.nct);
    ct = (int)((t - bt.ps) % bt.nct);
    return;
  }
  // rows below rs hold rt + d tiles: P(r) = r (r - 1) / 2 + d r <= t
  const double b = 2.0 * bt.d - 1.0;
  int r = (int)((-b + sqrt(b * b + 8.0 * (double)t)) * 0.5);
  r = max(0, min(r, bt.rs - 1));
  while (r + 1 < bt.rs && band_prefix(r + 1, bt.d) <= t) ++r;
  while (r > 0 && band_prefix(r, bt.d) > t) --r;
  rt = r;
  ct = (int)(t - band_prefix(r, bt.d));
}

__device__ __forceinline__ int pipe_c_swz(int r) { return ((r >> 2) & 1) << 3; }

typedef int pipe_i32x4_t __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(512)
k_kprod_leaf_pipe(SlabArgs g, LeafTask lt, BandTiles bt) {
  __shared__ __align__(16) union {
    LeafTaskSmem leaf;
    PipeSmem pipe;
  } sm;
  const int tid = threadIdx.x;
  if (blockIdx.x == 0) {
    if (tid >= 256) return;   // the leaf task takes 4 waves
    leaf_task_run(lt, sm.leaf);
    return;
  }
  const int G = (int)gridDim.x - 1;
  const int t0 = (int)blockIdx.x - 1;
  if (t0 >= bt.total) return;
  const int nt = (int)((bt.total - 1 - t0) / G) + 1;   // tiles t0 + G i, i < nt
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int w4 = wave & 3;
  const int64_t M = g.M, N = g.N;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&sm.pipe.stage[0][0]));

  if (wave >= 4) {
    // ---------------- data movers
    // A rows [0, M), B rows [0, N): 64 floats each; C rows [0, M), columns
    // [0, N). Past the ends: loads read zeros, stores are dropped. Every
    // buffer resource starts at its tile (A's and B's first row, C's first
    // element) and spans at most one tile, so the lane offsets stay below
    // 2^31 bytes whatever the size of the matrix.
    const int64_t a_end = ((M - 1) * g.lda + 64) * 4, b_end = ((N - 1) * g.ldb + 64) * 4;
    const int64_t c_end = ((M - 1) * g.ldc + N) * 4;
    const int64_t a_span = (63 * g.lda + 64) * 4, b_span = (63 * g.ldb + 64) * 4;
    const int64_t c_span = (63 * g.ldc + 64) * 4;
    // instruction q of this wave moves tile rows 16 w4 + 4 q + lane / 16;
    // a lane's 16-byte chunk is lane % 16
    const int ch = lane & 15;
    uint32_t voa[4], vob[4], voc[4], lcs[4];
    int rowq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 16 * w4 + 4 * q + (lane >> 4);
      rowq[q] = r;
      voa[q] = (uint32_t)((r * g.lda + 4 * (ch ^ (r & 15))) * 4);
      vob[q] = (uint32_t)((r * g.ldb + 4 * (ch ^ (r & 15))) * 4);
      voc[q] = (uint32_t)((r * g.ldc + 4 * (ch ^ pipe_c_swz(r))) * 4);
      lcs[q] = 2 * kPA + r * 256 + ch * 16;   // holds chunk ch ^ swz(r) of row r
    }
    auto issue = [&](int i, int st) {
      int rt = 0, ct = 0;
      band_tile(bt, t0 + G * min(i, nt - 1), rt, ct);   // past the end: the last tile again
      const int64_t oa = (int64_t)rt * 64 * g.lda, ob = (int64_t)ct * 64 * g.ldb;
      const int64_t oc = (int64_t)rt * 64 * g.ldc + (int64_t)ct * 64;
      const v4i32_t ra = make_rsrc(g.A + oa, min(a_end - 4 * oa, a_span));
      const v4i32_t rb = make_rsrc(g.B + ob, min(b_end - 4 * ob, b_span));
      const v4i32_t rcl = make_rsrc(g.C + oc, min(c_end - 4 * oc, c_span));
      const uint32_t base = lds0 + (uint32_t)st * kPStage + (uint32_t)(4 * w4) * 1024;
#pragma unroll
      for (int q = 0; q < 4; ++q) dma16_rsrc(voa[q], ra, 0u, base + q * 1024);
#pragma unroll
      for (int q = 0; q < 4; ++q) dma16_rsrc(vob[q], rb, 0u, base + kPA + q * 1024);
#pragma unroll
      for (int q = 0; q < 4; ++q) dma16_rsrc(voc[q], rcl, 0u, base + 2 * kPA + q * 1024);
    };
    // tile i's results (stage st) to C; i < 0 stores nothing (offsets past
    // the buffer) but issues the same 4 stores, keeping the wait counts fixed
    auto store = [&](int i, int st) {
      int rt = 0, ct = 0;
      if (i >= 0) band_tile(bt, t0 + G * i, rt, ct);
      const int64_t oc = (int64_t)rt * 64 * g.ldc + (int64_t)ct * 64;
      const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
          g.C + oc, 0, __builtin_amdgcn_readfirstlane((int)min(c_end - 4 * oc, c_span)), 0x00020000);
      const uint32_t sbase = lds0 + (uint32_t)st * kPStage;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const pipe_i32x4_t v = *reinterpret_cast<const __attribute__((address_space(3))) pipe_i32x4_t*>(
            (uintptr_t)(sbase + lcs[q]));
        const int64_t row = (int64_t)rt * 64 + rowq[q];
        const int64_t col = (int64_t)ct * 64 + 4 * (ch ^ pipe_c_swz(rowq[q]));
        // voc[q] is this lane's offset inside the tile; 2^31 lies past every tile's span
        const uint32_t off = (i >= 0 && row < M && col < N) ? voc[q] : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b128(v, rc, off, 0, 0);
      }
    };
    // Per tile a data mover issues 4 stores and 12 DMA; tile i + 1's DMA,
    // issued in the previous round, is older than the newest 16.
    issue(0, 0);
    issue(1, 1);
    asm volatile("s_waitcnt vmcnt(12)\n\ts_barrier" ::: "memory");
    for (int i = 0; i < nt; ++i) {
      const int st = i % 3;
      store(i - 1, st == 0 ? 2 : st - 1);
      issue(i + 2, st == 0 ? 2 : st - 1);
      asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
    }
    store(nt - 1, (nt - 1) % 3);
    // stand-in DMA may still write this workgroup's LDS: land it before the exit
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    return;
  }

  // ---------------- MFMA waves
  const int wm = w4 >> 1, wn = w4 & 1;
  const int lr = lane & 31, lh = lane >> 5;
  const int arow = 32 * wm + lr, brow = 32 * wn + lr;
  uint32_t fa_off[8], fb_off[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    fa_off[q] = arow * 256 + (((2 * q + lh) ^ (arow & 15)) * 16);
    fb_off[q] = kPA + brow * 256 + (((2 * q + lh) ^ (brow & 15)) * 16);
  }
  // C element r of this lane: row 32 wm + 8 (r / 4) + 4 h + r % 4, column 32 wn + lr
  uint32_t fc_off[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = 32 * wm + 8 * (r >> 2) + 4 * lh + (r & 3), col = 32 * wn + lr;
    fc_off[r] = 2 * kPA + row * 256 + ((((col >> 2) ^ pipe_c_swz(row)) * 16) + (col & 3) * 4);
  }
  __syncthreads();   // tile 0 has landed
  for (int i = 0; i < nt; ++i) {
    int rt, ct;
    band_tile(bt, t0 + G * i, rt, ct);
    const int64_t r0 = (int64_t)rt * 64, c0 = (int64_t)ct * 64;
    const bool active = !(g.lower_only && c0 + 32 * wn > r0 + 32 * wm + 31 + g.lower_off);
    const uint32_t sbase = lds0 + (uint32_t)(i % 3) * kPStage;
    float cv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r)
      cv[r] = *reinterpret_cast<const __attribute__((address_space(3))) float*>((uintptr_t)(sbase + fc_off[r]));
    leaf_f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    if (active) {
      kp_f32x4_t fa[8], fb[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        fa[q] = *reinterpret_cast<const __attribute__((address_space(3))) kp_f32x4_t*>((uintptr_t)(sbase + fa_off[q]));
        fb[q] = *reinterpret_cast<const __attribute__((address_space(3))) kp_f32x4_t*>((uintptr_t)(sbase + fb_off[q]));
      }
      __builtin_amdgcn_sched_barrier(0);   // all 16 reads in flight before the first MFMA
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[q].x, fb[q].x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[q].y, fb[q].y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[q].z, fb[q].z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[q].w, fb[q].w, acc, 0, 0, 0);
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r)
      *reinterpret_cast<__attribute__((address_space(3))) float*>((uintptr_t)(sbase + fc_off[r])) =
          fmaf(g.alpha, acc[r], g.beta * cv[r]);
    __syncthreads();   // results of tile i are in the stage; tile i + 1 has landed
  }
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
  // the pipelined kernel: full panels, 16-byte rows, one tile's span of
  // each operand below 2^31 bytes (its buffer resources start at the tile)
  const bool pipe = g.K == 64 && g.tb && g.M > 0 && g.N > 0 && (g.N & 3) == 0 && (g.ldc & 3) == 0 &&
                    ((uintptr_t)g.C & 15) == 0 && (g.lda & 3) == 0 && (g.ldb & 3) == 0 &&
                    ((uintptr_t)g.A & 15) == 0 && ((uintptr_t)g.B & 15) == 0 &&
                    (63 * g.lda + 64) * 4 < ((int64_t)1 << 31) && (63 * g.ldb + 64) * 4 < ((int64_t)1 << 31) &&
                    (63 * g.ldc + 64) * 4 < ((int64_t)1 << 31);
  if (pipe) {
    const BandTiles bt = band_tiles(g.M, g.N, g.lower_only, g.lower_off);
    if (bt.total >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    // one workgroup per CU (the leaf's CU excepted)
    const int64_t wgs = std::min<int64_t>(bt.total, 255);
    hipLaunchKernelGGL(k_kprod_leaf_pipe, dim3((unsigned)(1 + wgs)), dim3(512), 0, s, g, lt, bt);
    return hipGetLastError();
  }
  const int64_t nt = kprod_tiles(g, 64);
  if (nt + 1 >= (int64_t)1 << 31) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_kprod_leaf, dim3((unsigned)(1 + nt)), dim3(256), 0, s, g, lt);
  return hipGetLastError();
}

}  // namespace gq
