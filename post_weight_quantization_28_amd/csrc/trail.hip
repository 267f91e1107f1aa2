// Far-field lazy-batch update of the GPTQ sweep with split-bf16 MFMA:
//   C[M x N] -= A[M x K] B[K x N]
// with A = E (the errors of one super-block of columns, d_out x K) and
// B = U[super-block rows, columns to the right], both given as bf16 pairs
// (x = hi + lo, hi = bf16(x), lo = bf16(x - hi)).
//
// "GPTQ" (wikiprompt.org), "Enfoque Técnico": after columns are quantized,
// the remaining weights receive the closed-form correction of their errors.
//
// Precision: each product is taken as hi*hi + hi*lo + lo*hi (three
// v_mfma_f32_32x32x16_bf16) with fp32 accumulation; the dropped lo*lo term
// and the rounding of the lo parts leave a relative error of about 2^-16
// per product, against 2^-8 for plain bf16 operands.
//
// Layout (MI355X): 128 x 128 output tile per workgroup of 4 waves (2 x 2,
// each 64 x 64 = 2 x 2 accumulators). K streams through a 4-slot LDS ring
// of 32-deep stages filled by LDS-DMA: A_hi, A_lo as [row][k] (64-byte rows,
// chunk index XOR-swizzled with (row / 2) % 4) read with ds_read_b128, and
// B_hi, B_lo as [k][column] (256-byte rows, swizzled like the Hessian tile)
// read with transposing ds_read_b64_tr_b16. Each wave issues the 8 DMA
// instructions of one of the four operand parts per stage.
#include "common.h"
#include "dma.h"

namespace gq {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kTK = 32;                    // k per stage
constexpr int kTSlots = 4;
constexpr int kTPart = 128 * kTK * 2;      // bytes of one operand part per stage (8 KiB)
constexpr int kTSlot = 4 * kTPart;         // Ahi, Alo, Bhi, Blo

__device__ __forceinline__ int swz_a(int row) { return (row >> 1) & 3; }

__global__ void __launch_bounds__(256)
k_trail_x3(TrailArgs g) {
  __shared__ __align__(16) uint8_t sm[kTSlots * kTSlot];
  if (g.st != nullptr && g.st->flags != 0) return;
  const int ntn = (int)ceil_div(g.N, 128);
  const int tm = (int)blockIdx.x / ntn, tn = (int)blockIdx.x % ntn;
  const int64_t m0 = (int64_t)tm * 128, n0 = (int64_t)tn * 128;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(sm));

  // DMA plan: wave w fills part w (0 A_hi, 1 A_lo, 2 B_hi, 3 B_lo) with 8
  // instructions of 64 x 16 bytes.
  //  A: instruction p covers rows 16p .. 16p+15 (4 chunks of 8 k each).
  //  B: instruction p covers k rows 4p .. 4p+3 (16 chunks of 8 columns).
  const bool isA = wave < 2;
  const uint16_t* base = wave == 0 ? g.Ahi : wave == 1 ? g.Alo : wave == 2 ? g.Bhi : g.Blo;
  int rr[8], cc[8];
  bool rowok[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    if (isA) {
      const int r = 16 * p + (lane >> 2);
      rr[p] = r;
      cc[p] = (lane & 3) ^ swz_a(r);
      rowok[p] = m0 + r < g.M;
    } else {
      const int kr = 4 * p + (lane >> 4);
      rr[p] = kr;
      cc[p] = (lane & 15) ^ dma_swz(kr);
      rowok[p] = n0 + 8 * cc[p] < g.N;      // column chunk inside N
    }
  }
  auto issue = [&](int st, uint32_t slot) {
    const int64_t k0 = (int64_t)st * kTK;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const void* src;
      if (isA) {
        const int64_t k = k0 + 8 * cc[p];
        src = (rowok[p] && k < g.K) ? (const void*)(base + (m0 + rr[p]) * g.lda + k) : (const void*)kZeroChunk;
      } else {
        const int64_t k = k0 + rr[p];
        src = (rowok[p] && k < g.K) ? (const void*)(base + k * g.ldb + n0 + 8 * cc[p]) : (const void*)kZeroChunk;
      }
      dma16(src, __builtin_amdgcn_readfirstlane(slot + wave * kTPart + p * 1024));
    }
  };

  // fragment addressing
  const int G = lane >> 4, sl = lane & 15;
  const int trow = 8 * (G >> 1) + (sl >> 2);          // + 16 ks + 4 h
  const int tchunk = 2 * (G & 1) + ((sl >> 1) & 1);   // + (64 wn + 32 nb) / 8
  const int half8 = (sl & 1) * 8;
  const int arow = lane & 31, akc = lane >> 5;          // + 64 wm + 32 mb ; + 2 ks

  f32x16_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  const int nstage = (int)ceil_div(g.K, kTK);
  auto slot_of = [&](int st) { return lds0 + (uint32_t)(st % kTSlots) * kTSlot; };
#pragma unroll
  for (int ps = 0; ps < kTSlots - 1; ++ps)
    if (ps < nstage) issue(ps, slot_of(ps));

  for (int st = 0; st < nstage; ++st) {
    wait_dma_barrier(min(kTSlots - 2, nstage - 1 - st));
    if (st + kTSlots - 1 < nstage) issue(st + kTSlots - 1, slot_of(st + kTSlots - 1));
    const uint32_t slot = slot_of(st);
#pragma unroll
    for (int ks = 0; ks < kTK / 16; ++ks) {
      bf16x8_t ah[2], al[2], bh[2], bl[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int r = 64 * wm + 32 * mb + arow;
        const uint32_t off = r * 64 + (((2 * ks + akc) ^ swz_a(r)) * 16);
        ah[mb] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const __attribute__((address_space(3))) uint4*>(
                                                  (uintptr_t)(slot + off)));
        al[mb] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const __attribute__((address_space(3))) uint4*>(
                                                  (uintptr_t)(slot + kTPart + off)));
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        v4i16_t h0, h1, l0, l1;
        {
          const int t = 16 * ks + trow;
          const uint32_t off = t * 256 + (((8 * wn + 4 * nb + tchunk) ^ dma_swz(t)) * 16) + half8;
          h0 = lds_tr16(slot + 2 * kTPart + off);
          l0 = lds_tr16(slot + 3 * kTPart + off);
        }
        {
          const int t = 16 * ks + 4 + trow;
          const uint32_t off = t * 256 + (((8 * wn + 4 * nb + tchunk) ^ dma_swz(t)) * 16) + half8;
          h1 = lds_tr16(slot + 2 * kTPart + off);
          l1 = lds_tr16(slot + 3 * kTPart + off);
        }
        bh[nb] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
        bl[nb] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[mb], bh[nb], acc[mb][nb], 0, 0, 0);
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[mb], bl[nb], acc[mb][nb], 0, 0, 0);
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[mb], bh[nb], acc[mb][nb], 0, 0, 0);
        }
    }
  }

  // C -= acc: lane holds D[i][j], j = lane % 32, i = 8 (r / 4) + 4 (lane / 32) + r % 4
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t i = m0 + 64 * wm + 32 * mb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t j = n0 + 64 * wn + 32 * nb + (lane & 31);
        if (i < g.M && j < g.N) {
          float* c = g.C + i * g.ldc + j;
          *c = *c - acc[mb][nb][r];
        }
      }
}

hipError_t launch_trail_x3(hipStream_t s, const TrailArgs& g) {
  if (g.M <= 0 || g.N <= 0 || g.K <= 0) return hipSuccess;
  // 16-byte DMA chunks: rows of A and B, and the column origin of B, must be
  // 8-element aligned, and N a multiple of 8 (a chunk never straddles N)
  if ((g.lda % 8) || (g.ldb % 8) || (g.N % 8) || (g.K % 8) || ((uintptr_t)g.Ahi % 16) ||
      ((uintptr_t)g.Alo % 16) || ((uintptr_t)g.Bhi % 16) || ((uintptr_t)g.Blo % 16))
    return hipErrorInvalidValue;
  const int64_t tiles = ceil_div(g.M, 128) * ceil_div(g.N, 128);
  hipLaunchKernelGGL(k_trail_x3, dim3((unsigned)tiles), dim3(256), 0, s, g);
  return hipGetLastError();
}

// ---- bf16 splitting of fp32 arrays: hi = bf16(x), lo = bf16(x - hi)
__global__ void k_split_bf16(const float* __restrict__ x, int64_t count, uint16_t* __restrict__ hi,
                             uint16_t* __restrict__ lo) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < count; q += stride) {
    const float v = x[q];
    const uint16_t h = f32_to_bf16_rne(v);
    hi[q] = h;
    lo[q] = f32_to_bf16_rne(v - bf16_to_f32(h));
  }
}

hipError_t launch_split_bf16(hipStream_t s, const float* x, int64_t count, uint16_t* hi, uint16_t* lo) {
  if (count <= 0) return hipSuccess;
  int64_t blocks = ceil_div(count, 256);
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(k_split_bf16, dim3((unsigned)blocks), dim3(256), 0, s, x, count, hi, lo);
  return hipGetLastError();
}

}  // namespace gq
