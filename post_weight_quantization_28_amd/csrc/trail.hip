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
// Layout (MI355X): 256 x 128 output tile per workgroup of 4 waves (2 x 2,
// each 128 x 64 = 4 x 2 accumulators). K streams through a 3-slot LDS ring
// of 16-deep stages (24 KiB each) filled by buffer LDS-DMA, so a workgroup
// needs 72 KiB and two independent workgroups share a CU: one's barrier and
// DMA waits are covered by the other's MFMAs. A_hi, A_lo are stored
// [row][k] in LDS (32-byte rows, 16-byte chunk index XOR-swizzled with (row
// / 8) % 2) and read with ds_read_b128; B_hi, B_lo as [k][column] (256-byte
// rows, swizzled like the Hessian tile) and read with transposing
// ds_read_b64_tr_b16. In memory A is tiled (eh_index: 256 rows x 16 k per
// 8 KiB block), so a stage of A is one consecutive 8 KiB block and every
// DMA instruction reads 1 KiB of consecutive memory (row-major A gave 32
// rows x 32 bytes per instruction, a quarter of a cache line each). The
// last row block's rows past M hold anything; an output row depends only
// on its own A row, and rows past M are not stored. B's descriptor ends at
// row K, so k past K reads as zeros; B chunks past N get an offset outside
// the buffer. Each wave issues 6 of the 24 DMA instructions of a stage.
#include "common.h"
#include "dma.h"

namespace gq {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kTM = 256, kTN = 128;        // workgroup tile
constexpr int kTK = 16;                    // k per stage
constexpr int kTSlots = 3;
constexpr int kTA = kTM * kTK * 2;         // bytes of A_hi (or A_lo) per stage: 8 KiB
constexpr int kTB = kTK * kTN * 2;         // bytes of B_hi (or B_lo) per stage: 4 KiB
constexpr int kTSlot = 2 * kTA + 2 * kTB;  // 24 KiB
constexpr int kTDma = 6;                   // DMA instructions per wave per stage

// A rows are 32 bytes: rows r and r + 8 share banks, so the 16-byte chunk
// index is XORed with (r / 8) % 2 (16 consecutive rows of one chunk column
// then cover all 64 banks)
__device__ __forceinline__ int swz_a(int row) { return (row >> 3) & 1; }

// Wait until at most `stages` stages of kTDma DMA instructions of this wave
// are outstanding, then barrier (one asm block, as in dma.h).
__device__ __forceinline__ void wait_dma6_barrier(int stages) {
  if (stages <= 0) asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(6)\n\ts_barrier" ::: "memory");
}

__global__ void __launch_bounds__(256, 2)
k_trail_x3(TrailArgs g) {
  __shared__ __align__(16) uint8_t sm[kTSlots * kTSlot];
  // XCD-contiguous tile order: block b runs on XCD b % 8; give each XCD a
  // contiguous run of row-major tiles, so the rows of A it needs stay in its
  // L2 and each column tile of B is fetched once per XCD
  const int ntn = (int)ceil_div(g.N, kTN);
  const int ntiles = (int)ceil_div(g.M, kTM) * ntn;
  const int per = (ntiles + 7) >> 3;
  const int w = ((int)blockIdx.x & 7) * per + ((int)blockIdx.x >> 3);
  if (((int)blockIdx.x >> 3) >= per || w >= ntiles) return;
  const int tm = w / ntn, tn = w % ntn;
  const int64_t m0 = (int64_t)tm * kTM, n0 = (int64_t)tn * kTN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(sm));

  // buffers: A's 256-row block of this tile (all lda / 16 slices), B rows
  // [0, K) from column n0 on
  const int64_t ablk = g.lda / 16 * (kTM * kTK);   // elements of one row block
  const v4i32_t rAh = make_rsrc(g.Ahi + tm * ablk, ablk * 2);
  const v4i32_t rAl = make_rsrc(g.Alo + tm * ablk, ablk * 2);
  const int64_t bbytes = ((g.K - 1) * g.ldb + (g.N - n0)) * 2;
  const v4i32_t rBh = make_rsrc(g.Bhi + n0, bbytes);
  const v4i32_t rBl = make_rsrc(g.Blo + n0, bbytes);

  // DMA plan: instruction idx = 6 w + q, q = 0..5:
  //   0..7 A_hi, 8..15 A_lo: rows 32p .. 32p+31, 2 chunks of 8 k each
  //     (1 KiB of consecutive memory in the stage's 8 KiB block)
  //   16..19 B_hi, 20..23 B_lo: k rows 4p .. 4p+3, 16 chunks of 8 columns
  uint32_t voff[kTDma];
#pragma unroll
  for (int q = 0; q < kTDma; ++q) {
    const int idx = kTDma * wave + q;
    if (idx < 16) {
      const int p = idx & 7;
      const int r = 32 * p + (lane >> 1);
      const int c = (lane & 1) ^ swz_a(r);
      voff[q] = (uint32_t)(r * 32 + 16 * c);
    } else {
      const int p = idx & 3;
      const int kr = 4 * p + (lane >> 4);
      const int c = (lane & 15) ^ dma_swz(kr);
      voff[q] = (n0 + 8 * c < g.N) ? (uint32_t)((kr * g.ldb + 8 * c) * 2) : 0x80000000u;
    }
  }
  auto issue = [&](int st, int slot) {
    const uint32_t sa = __builtin_amdgcn_readfirstlane((uint32_t)(st * kTA));
    const uint32_t sb = __builtin_amdgcn_readfirstlane((uint32_t)(st * kTK * g.ldb * 2));
#pragma unroll
    for (int q = 0; q < kTDma; ++q) {
      const int idx = kTDma * wave + q;
      const uint32_t dst = __builtin_amdgcn_readfirstlane(
          lds0 + slot * kTSlot +
          (idx < 8 ? (idx & 7) * 1024
                   : idx < 16 ? kTA + (idx & 7) * 1024
                              : idx < 20 ? 2 * kTA + (idx & 3) * 1024 : 2 * kTA + kTB + (idx & 3) * 1024));
      const v4i32_t r = idx < 8 ? rAh : idx < 16 ? rAl : idx < 20 ? rBh : rBl;
      dma16_rsrc(voff[q], r, idx < 16 ? sa : sb, dst);
    }
  };

  // fragment bases (per lane, relative to a slot)
  //  A: row 128 wm + 32 mb + lane % 32, k chunk (lane / 32) ^ swz_a(row)
  //  B: k row 4 h + 8 (G/2) + s/4, column chunk (8 wn + 4 nb + 2 (G%2) + (s/2)%2) ^ dma_swz
  const int arow = 128 * wm + (lane & 31);
  const uint32_t offA = arow * 32 + (((lane >> 5) ^ swz_a(arow)) * 16);   // swz_a is the same for every mb
  const int G = lane >> 4, sl = lane & 15;
  const int trow = 8 * (G >> 1) + (sl >> 2);
  const int swzb = dma_swz(trow);
  uint32_t offB[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
    offB[nb] = 2 * kTA + trow * 256 + (((8 * wn + 4 * nb + 2 * (G & 1) + ((sl >> 1) & 1)) ^ swzb) * 16) +
               (sl & 1) * 8;

  f32x16_t acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  const int nstage = (int)ceil_div(g.K, kTK);
#pragma unroll
  for (int ps = 0; ps < kTSlots - 1; ++ps)
    if (ps < nstage) issue(ps, ps);
  for (int st = 0; st < nstage; ++st) {
    wait_dma6_barrier(min(kTSlots - 2, nstage - 1 - st));
    if (st + kTSlots - 1 < nstage) issue(st + kTSlots - 1, (st + kTSlots - 1) % kTSlots);
    const uint32_t sbase = lds0 + (uint32_t)(st % kTSlots) * kTSlot;
    const uint32_t bA = offA + sbase;
    bf16x8_t ah[4], al[4], bh[2], bl[2];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const uint32_t o = bA + mb * 32 * 32;
      ah[mb] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const __attribute__((address_space(3))) uint4*>(
                                                (uintptr_t)o));
      al[mb] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const __attribute__((address_space(3))) uint4*>(
                                                (uintptr_t)(o + kTA)));
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const uint32_t o = offB[nb] + sbase;
      const v4i16_t h0 = lds_tr16(o), h1 = lds_tr16(o + 4 * 256);
      const v4i16_t l0 = lds_tr16(o + kTB), l1 = lds_tr16(o + kTB + 4 * 256);
      bh[nb] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
      bl[nb] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7));
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[mb], bh[nb], acc[mb][nb], 0, 0, 0);
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[mb], bl[nb], acc[mb][nb], 0, 0, 0);
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[mb], bh[nb], acc[mb][nb], 0, 0, 0);
      }
  }

  // C -= acc: lane holds D[i][j], j = lane % 32, i = 8 (r / 4) + 4 (lane / 32) + r % 4.
  // In two halves (mb = 0..1, then 2..3; 64 registers of C next to the 128
  // accumulators), each loading all of its C values, unconditionally (indices
  // clamped into the matrix), before its first store: predicated loads would
  // each end in a wait, and a store followed by a load the compiler cannot
  // prove disjoint would serialise the read-modify-writes on memory latency.
  const int64_t ib = m0 + 128 * wm + 4 * (lane >> 5);
  const int64_t jb = n0 + 64 * wn + (lane & 31);
  if (m0 + kTM <= g.M && n0 + kTN <= g.N && g.ldc < ((int64_t)1 << 22)) {
    // whole tile: a buffer over this wave's 128 rows, a fixed 32-bit lane
    // offset and a scalar offset per row, so no access needs vector
    // address arithmetic
    const uint64_t cwa = (uint64_t)(uintptr_t)(g.C + (m0 + 128 * wm) * g.ldc + n0 + 64 * wn);
    float* cw = reinterpret_cast<float*>(
        ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(cwa >> 32)) << 32) |
        (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)cwa));   // uniform
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        cw, 0, __builtin_amdgcn_readfirstlane((int)(128 * g.ldc * 4)), 0x00020000);
    const int ldc4 = __builtin_amdgcn_readfirstlane((int)(g.ldc * 4));
    const int lob = (4 * (lane >> 5)) * ldc4 + (lane & 31) * 4;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      float cv[2][2][16];
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            cv[m][nb][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                rc, lob, (32 * (2 * half + m) + 8 * (r >> 2) + (r & 3)) * ldc4 + 128 * nb, 0));
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            __builtin_amdgcn_raw_buffer_store_b32(
                __float_as_uint(cv[m][nb][r] - acc[2 * half + m][nb][r]), rc, lob,
                (32 * (2 * half + m) + 8 * (r >> 2) + (r & 3)) * ldc4 + 128 * nb, 0);
    }
    return;
  }
  // edge tiles: one 32 x 32 block at a time
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      float cv[16];
      const int64_t j = jb + 32 * nb;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t i = min(ib + 32 * mb + 8 * (r >> 2) + (r & 3), g.M - 1);
        cv[r] = g.C[i * g.ldc + min(j, g.N - 1)];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t i = ib + 32 * mb + 8 * (r >> 2) + (r & 3);
        if (i < g.M && j < g.N) g.C[i * g.ldc + j] = cv[r] - acc[mb][nb][r];
      }
    }
}

hipError_t launch_trail_x3(hipStream_t s, const TrailArgs& g) {
  if (g.M <= 0 || g.N <= 0 || g.K <= 0) return hipSuccess;
  // 16-byte DMA chunks: rows of A and B, and the column origin of B, must be
  // 8-element aligned, and N a multiple of 8 (a chunk never straddles N)
  if ((g.lda % 16) || g.K > g.lda || (g.ldb % 8) || (g.N % 8) || (g.K % 8) || ((uintptr_t)g.Ahi % 16) ||
      ((uintptr_t)g.Alo % 16) || ((uintptr_t)g.Bhi % 16) || ((uintptr_t)g.Blo % 16))
    return hipErrorInvalidValue;
  // 32-bit buffer offsets
  if (g.lda * kTM * 2 >= ((int64_t)1 << 31) || g.K * g.ldb * 2 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const int64_t tiles = ceil_div(g.M, kTM) * ceil_div(g.N, kTN);
  hipLaunchKernelGGL(k_trail_x3, dim3((unsigned)(8 * ceil_div(tiles, 8))), dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace gq
