// Symmetric rank-K update of a wide factorisation's trailing matrix on the
// bf16 matrix cores, at fp32 accuracy:
//   C[i][j] -= sum_k P[i][k] P[j][k]      (tiles on or below the diagonal)
// with P = the fp32 rows of the finished super-panel.
//
// "Resumen Técnico: GPTQ-intrinsic LoRA", "Detalles de Implementación": the
// standard method factorises the regularised Hessian by Cholesky; this is
// that factorisation's trailing update in its two-level form.
//
// Precision: each fp32 value is split exactly into three bf16 pieces,
// p = p1 + p2 + p3 + r with p1 = bf16(p), p2 = bf16(p - p1), p3 =
// bf16(p - p1 - p2), |r| <= 2^-24 |p| (each subtraction is exact). A
// product of two pieces is exact in fp32. Of the nine piece products the
// six with pieces (1,1), (1,2), (2,1), (2,2), (1,3), (3,1) are taken; the
// dropped ones are below 2^-23 of the product, the size of an fp32
// rounding, so the sum carries fp32-level error, with six bf16 MFMAs in
// place of the fp32 one at 16 times its rate. The six products of a k slice
// are added smallest first, and the MFMA accumulator is folded into an fp32
// total after every 32 k (as in the fp32 update), so no rounding happens at
// the magnitude of C's entries until the single final addition.
//
// Layout (MI355X): 128 x 128 tiles of C, one per workgroup of 4 waves (2 x
// 2, each 64 x 64 = 2 x 2 accumulators of v_mfma_f32_32x32x16_bf16). K
// streams through a 3-slot LDS ring of 16-deep stages (24 KiB: the three
// pieces of the tile's 128 row-operand rows and of its 128 column-operand
// rows, 32 bytes per row and piece) filled by buffer LDS-DMA, so two
// workgroups share a CU. Both operands are rows of P (k contiguous), read
// with ds_read_b128; the 16-byte chunk index of row r is XORed with
// (r / 8) % 2 so 16 consecutive rows of one chunk column cover all banks.
// The pieces are stored tiled, in exactly the order a stage needs them:
// for each 128-row block of P and each 16-deep k slice, piece by piece, a
// 4 KiB block of 128 rows x 32 bytes. Every DMA instruction then reads 1
// KiB of consecutive memory (row-major P would give 32 rows x 32 bytes,
// a quarter of a cache line each: the fill took twice as long). The tiles
// are numbered row by row over the lower triangle and dealt to the XCDs in
// contiguous runs.
#include "common.h"
#include "dma.h"

namespace gq {

typedef __bf16 s6_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float s6_f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kS6T = 128;                    // tile edge
constexpr int kS6K = 16;                     // k per stage
constexpr int kS6Piece = kS6T * kS6K * 2;    // bytes of one piece of one operand per stage: 4 KiB
constexpr int kS6Slot = 6 * kS6Piece;        // 24 KiB
constexpr int kS6Slots = 3;
constexpr int kS6Dma = 6;                    // DMA instructions per wave per stage

// ---------------------------------------------------------------- split
// The three pieces of src (rows x cols fp32, pitch lds; cols % 16 == 0),
// tiled: piece i of element (r, k) goes to
//   dst + (((r / 128) * (cols / 16) + k / 16) * 3 + i) * 2048 + (r % 128) * 16 + k % 16
// (bf16 elements). Rows rows .. 128 ceil(rows / 128) - 1 are written as zeros.
__global__ void k_split3(const float* __restrict__ src, int64_t rows, int64_t cols, int64_t lds,
                         uint16_t* __restrict__ dst) {
  // thread q takes 4 consecutive k of one row, in the order of the tiled
  // output (block (r / 128, k / 16), then row, then the 4-k group), so a
  // wave writes 512 consecutive bytes of each piece and reads 64 bytes of
  // each of its 16 rows
  const int64_t prow = (rows + kS6T - 1) / kS6T * kS6T;
  const int64_t nst = cols / kS6K;
  const int64_t total = prow * (cols / 4);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total; q += stride) {
    const int64_t b = q >> 9, w = q & 511;            // 512 groups of 4 per (block, stage)
    const int64_t tr = b / nst, stg = b - tr * nst;
    const int64_t r = tr * kS6T + (w >> 2), c = stg * kS6K + 4 * (w & 3);
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r < rows) v = *reinterpret_cast<const float4*>(src + r * lds + c);
    const float x[4] = {v.x, v.y, v.z, v.w};
    uint16_t h1[4], h2[4], h3[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h1[e] = f32_to_bf16_rne(x[e]);
      const float r1 = x[e] - bf16_to_f32(h1[e]);
      h2[e] = f32_to_bf16_rne(r1);
      h3[e] = f32_to_bf16_rne(r1 - bf16_to_f32(h2[e]));
    }
    const int64_t blk = ((r / kS6T) * nst + c / kS6K) * 3;
    const int64_t o = (r % kS6T) * kS6K + c % kS6K;
    *reinterpret_cast<uint2*>(dst + blk * 2048 + o) = make_uint2(h1[0] | ((uint32_t)h1[1] << 16), h1[2] | ((uint32_t)h1[3] << 16));
    *reinterpret_cast<uint2*>(dst + (blk + 1) * 2048 + o) = make_uint2(h2[0] | ((uint32_t)h2[1] << 16), h2[2] | ((uint32_t)h2[3] << 16));
    *reinterpret_cast<uint2*>(dst + (blk + 2) * 2048 + o) = make_uint2(h3[0] | ((uint32_t)h3[1] << 16), h3[2] | ((uint32_t)h3[3] << 16));
  }
}

// ---------------------------------------------------------------- SYRK
__device__ __forceinline__ int s6_swz(int row) { return (row >> 3) & 1; }

__device__ __forceinline__ void s6_wait_barrier(int stages) {
  if (stages <= 0) asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(6)\n\ts_barrier" ::: "memory");
}

struct Syrk6Args {
  int64_t N, K;                       // C is N x N (lower tiles), P is N x K
  const uint16_t* Pt;                 // the pieces, tiled as k_split3 writes them
  float* C; int64_t ldc;
};

__device__ __forceinline__ s6_bf16x8_t s6_frag(uint32_t byte_off) {
  return __builtin_bit_cast(s6_bf16x8_t, *reinterpret_cast<const __attribute__((address_space(3))) uint4*>(
                                             (uintptr_t)byte_off));
}

__global__ void __launch_bounds__(256, 2) k_syrk_x6(Syrk6Args g, int ntile) {
  __shared__ __align__(16) uint8_t sm[kS6Slots * kS6Slot];
  const int per = (ntile + 7) >> 3;
  const int t = ((int)blockIdx.x & 7) * per + ((int)blockIdx.x >> 3);
  if (t >= ntile) return;
  // t = tm (tm + 1) / 2 + tn, 0 <= tn <= tm
  int tm = (int)((sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
  while ((tm + 1) * (tm + 2) / 2 <= t) ++tm;
  while (tm * (tm + 1) / 2 > t) --tm;
  const int tn = t - tm * (tm + 1) / 2;
  const int64_t m0 = (int64_t)tm * kS6T, n0 = (int64_t)tn * kS6T;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(sm));

  // one buffer per operand over its 128-row block of the tiled pieces
  // (stage st, piece i at byte (3 st + i) * 4096; rows past N were written
  // as zeros)
  const int64_t nst = g.K / kS6K;
  const int64_t blk_bytes = nst * 3 * kS6Piece;
  const v4i32_t rA = make_rsrc(g.Pt + (int64_t)tm * (blk_bytes / 2), blk_bytes);
  const v4i32_t rB = make_rsrc(g.Pt + (int64_t)tn * (blk_bytes / 2), blk_bytes);
  // DMA plan: instruction idx = 6 wave + q (0..23): operand op = idx / 12
  // (0: the tile's rows, 1: its columns), piece (idx % 12) / 4, rows 32 p ..
  // 32 p + 31 with p = idx % 4; lane l fills row 32 p + l / 2, LDS chunk l % 2,
  // which holds global chunk (l % 2) ^ swz(row): 1 KiB of consecutive memory
  // per instruction
  uint32_t voff[kS6Dma];
#pragma unroll
  for (int q = 0; q < kS6Dma; ++q) {
    const int idx = kS6Dma * wave + q;
    const int piece = (idx % 12) >> 2;
    const int r = 32 * (idx & 3) + (lane >> 1);
    const int c = (lane & 1) ^ s6_swz(r);
    voff[q] = (uint32_t)(piece * kS6Piece + r * 32 + 16 * c);
  }
  auto issue = [&](int st, int slot) {
    const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)(st * 3 * kS6Piece));
#pragma unroll
    for (int q = 0; q < kS6Dma; ++q) {
      const int idx = kS6Dma * wave + q;
      const int op = idx / 12, piece = (idx % 12) >> 2;   // wave-uniform
      const uint32_t dst = __builtin_amdgcn_readfirstlane(lds0 + slot * kS6Slot + (op * 3 + piece) * kS6Piece +
                                                          (idx & 3) * 1024);
      dma16_rsrc(voff[q], op == 0 ? rA : rB, soff, dst);
    }
  };

  // fragment offsets (per lane, within a slot): row 64 w + 32 b + lane % 32,
  // k chunk lane / 32
  uint32_t offA[2], offB[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int ra = 64 * wm + 32 * b + (lane & 31), rb = 64 * wn + 32 * b + (lane & 31);
    offA[b] = ra * 32 + (((lane >> 5) ^ s6_swz(ra)) * 16);
    offB[b] = 3 * kS6Piece + rb * 32 + (((lane >> 5) ^ s6_swz(rb)) * 16);
  }

  s6_f32x16_t acc[2][2], tot[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc[a][b][r] = 0.f;
        tot[a][b][r] = 0.f;
      }
  auto fold = [&]() {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          tot[a][b][r] -= acc[a][b][r];
          acc[a][b][r] = 0.f;
        }
  };

  const int nstage = (int)(g.K / kS6K);
#pragma unroll
  for (int ps = 0; ps < kS6Slots - 1; ++ps)
    if (ps < nstage) issue(ps, ps);
  for (int st = 0; st < nstage; ++st) {
    s6_wait_barrier(min(kS6Slots - 2, nstage - 1 - st));
    if (st + kS6Slots - 1 < nstage) issue(st + kS6Slots - 1, (st + kS6Slots - 1) % kS6Slots);
    const uint32_t sbase = lds0 + (uint32_t)(st % kS6Slots) * kS6Slot;
    s6_bf16x8_t fa[2][3], fb[2][3];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        fa[b][i] = s6_frag(sbase + i * kS6Piece + offA[b]);
        fb[b][i] = s6_frag(sbase + i * kS6Piece + offB[b]);
      }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a][2], fb[b][0], acc[a][b], 0, 0, 0);
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a][0], fb[b][2], acc[a][b], 0, 0, 0);
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a][1], fb[b][1], acc[a][b], 0, 0, 0);
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a][1], fb[b][0], acc[a][b], 0, 0, 0);
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a][0], fb[b][1], acc[a][b], 0, 0, 0);
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a][0], fb[b][0], acc[a][b], 0, 0, 0);
      }
    if (st & 1) fold();
  }
  if (nstage & 1) fold();

  // C += tot (tot holds minus the product); lane holds D[i][j], j = lane % 32,
  // i = 8 (r / 4) + 4 (lane / 32) + r % 4. All 16 values of a block are
  // loaded before its first store.
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t j = n0 + 64 * wn + 32 * b + (lane & 31);
      const int64_t ib = m0 + 64 * wm + 32 * a + 4 * (lane >> 5);
      float cv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t i = min(ib + 8 * (r >> 2) + (r & 3), g.N - 1);
        cv[r] = g.C[i * g.ldc + min(j, g.N - 1)];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t i = ib + 8 * (r >> 2) + (r & 3);
        if (i < g.N && j < g.N) g.C[i * g.ldc + j] = cv[r] + tot[a][b][r];
      }
    }
}

bool syrk_x6_ok(int64_t N, int64_t K, int64_t lda, const float* A, int64_t ldc, const float* C) {
  return N > 0 && K > 0 && K % kS6K == 0 && lda % 4 == 0 && ((uintptr_t)A & 15) == 0 && ldc > 0 &&
         C != nullptr && kS6T * K * 6 < ((int64_t)1 << 31) && N * (N + 1) / 2 / (kS6T * kS6T) < ((int64_t)1 << 28);
}

int64_t syrk_x6_pieces(int64_t N, int64_t K) { return 3 * ((N + kS6T - 1) / kS6T * kS6T) * K; }

hipError_t launch_syrk_x6(hipStream_t s, const float* A, int64_t lda, float* C, int64_t ldc, int64_t N,
                          int64_t K, uint16_t* pieces) {
  if (N <= 0) return hipSuccess;
  if (!syrk_x6_ok(N, K, lda, A, ldc, C) || !pieces || ((uintptr_t)pieces & 15) != 0) return hipErrorInvalidValue;
  {
    int64_t blocks = ceil_div(ceil_div(N, kS6T) * kS6T * (K / 4), 256);
    if (blocks > 16384) blocks = 16384;
    hipLaunchKernelGGL(k_split3, dim3((unsigned)blocks), dim3(256), 0, s, A, N, K, lda, pieces);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  Syrk6Args g{};
  g.N = N; g.K = K; g.Pt = pieces; g.C = C; g.ldc = ldc;
  const int64_t nt = ceil_div(N, kS6T);
  const int64_t ntile = nt * (nt + 1) / 2;
  hipLaunchKernelGGL(k_syrk_x6, dim3((unsigned)(8 * ((ntile + 7) / 8))), dim3(256), 0, s, g, (int)ntile);
  return hipGetLastError();
}

// ---------------------------------------------------------------- general products
// The triangular inverse's block products (X_ji = -X_jj (L_ji X_ii)) in the
// same six-product form. Each operand is split once per launch into the
// tiled piece layout above (128-row blocks, 16-deep k slices, rows past the
// operand and k past K written as zeros), for a batch of instances; the
// product kernel then runs the SYRK's stage loop over the k range its tile
// needs, with each tile's own row block of each operand.

__host__ __device__ int64_t x6_op_elems(int64_t rows, int64_t K) { return 3 * ceil_div(rows, kS6T) * kS6T * ceil_div(K, kS6K) * kS6K; }

struct Split6Args {
  const float* src; int64_t ld, stride;
  int64_t R, K;
  int trans, batch;
  uint16_t* dst;
};

// A workgroup takes one (instance, 128-row block, 16-deep k slice) item at
// a time, 512 groups of 4 consecutive k, two per thread (the index
// arithmetic is done once per item, in 32 bits). Untransposed sources are
// walked as k_split3 walks them (4 threads per row, 16-byte loads when rows
// are 16-byte aligned); transposed ones with the row index fastest, so that
// each of a thread's four loads is one consecutive run of the source across
// the wave.
template <bool TRANS, bool VEC>
__global__ void __launch_bounds__(256) k_split3_op(Split6Args a) {
  const int nst = (int)ceil_div(a.K, kS6K);
  const int nrb = (int)ceil_div(a.R, kS6T);
  const int per = nrb * nst;                       // items per instance
  const int items = per * a.batch;
  const int64_t out_per = x6_op_elems(a.R, a.K);
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int b = it / per, blk = it - b * per;
    const int tr = blk / nst, stg = blk - tr * nst;
    const float* src = a.src + (int64_t)b * a.stride;
    uint16_t* dblk = a.dst + (int64_t)b * out_per + (int64_t)blk * 3 * 2048;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int w = (int)threadIdx.x + 256 * half;
      const int rr = TRANS ? (w & 127) : (w >> 2);
      const int kg = TRANS ? (w >> 7) : (w & 3);
      const int64_t r = (int64_t)tr * kS6T + rr, k = (int64_t)stg * kS6K + 4 * kg;
      float x[4];
      if (VEC && r < a.R && k + 3 < a.K) {
        const float4 v = *reinterpret_cast<const float4*>(src + r * a.ld + k);
        x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t kk = k + e;
          x[e] = (r < a.R && kk < a.K) ? (TRANS ? src[kk * a.ld + r] : src[r * a.ld + kk]) : 0.f;
        }
      }
      uint16_t h1[4], h2[4], h3[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        h1[e] = f32_to_bf16_rne(x[e]);
        const float r1 = x[e] - bf16_to_f32(h1[e]);
        h2[e] = f32_to_bf16_rne(r1);
        h3[e] = f32_to_bf16_rne(r1 - bf16_to_f32(h2[e]));
      }
      uint16_t* d = dblk + rr * kS6K + 4 * kg;
      *reinterpret_cast<uint2*>(d) = make_uint2(h1[0] | ((uint32_t)h1[1] << 16), h1[2] | ((uint32_t)h1[3] << 16));
      *reinterpret_cast<uint2*>(d + 2048) = make_uint2(h2[0] | ((uint32_t)h2[1] << 16), h2[2] | ((uint32_t)h2[3] << 16));
      *reinterpret_cast<uint2*>(d + 4096) = make_uint2(h3[0] | ((uint32_t)h3[1] << 16), h3[2] | ((uint32_t)h3[3] << 16));
    }
  }
}

struct Gemm6Args {
  int64_t M, N, K;
  const uint16_t* Ap; const uint16_t* Bp;   // pieces: M rows of A, N rows of B, per instance
  float* C; int64_t ldc, sC;
  float alpha;
  int kmode, batch, ntm, ntn;
};

// One 128 x 128 tile of one instance per workgroup (the SYRK's layout and
// stage loop). Tiles are numbered row tile by row tile across the batch,
// the longest k ranges first.
__global__ void __launch_bounds__(256, 2) k_gemm_x6(Gemm6Args g) {
  __shared__ __align__(16) uint8_t sm[kS6Slots * kS6Slot];
  const int per_row = g.batch * g.ntn;
  const int t = (int)blockIdx.x;
  const int tmi = t / per_row, rem = t - tmi * per_row;
  const int inst = rem / g.ntn, tn = rem - inst * g.ntn;
  const int tm = g.kmode == 3 ? g.ntm - 1 - tmi : tmi;
  const int64_t m0 = (int64_t)tm * kS6T, n0 = (int64_t)tn * kS6T;
  const int64_t nst = ceil_div(g.K, kS6K);
  int s_lo = 0, s_hi = (int)nst;
  if (g.kmode == 4) s_lo = (int)(m0 / kS6K);
  else if (g.kmode == 3) s_hi = (int)ceil_div(min(g.K, m0 + kS6T), kS6K);
  const int ns = max(s_hi - s_lo, 0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(sm));

  const int64_t blk_elems = nst * 3 * (kS6Piece / 2);   // one 128-row block's pieces
  const uint16_t* pa = g.Ap + (int64_t)inst * ceil_div(g.M, kS6T) * blk_elems + tm * blk_elems;
  const uint16_t* pb = g.Bp + (int64_t)inst * ceil_div(g.N, kS6T) * blk_elems + tn * blk_elems;
  const v4i32_t rA = make_rsrc(pa, blk_elems * 2);
  const v4i32_t rB = make_rsrc(pb, blk_elems * 2);
  uint32_t voff[kS6Dma];
#pragma unroll
  for (int q = 0; q < kS6Dma; ++q) {
    const int idx = kS6Dma * wave + q;
    const int piece = (idx % 12) >> 2;
    const int r = 32 * (idx & 3) + (lane >> 1);
    const int c = (lane & 1) ^ s6_swz(r);
    voff[q] = (uint32_t)(piece * kS6Piece + r * 32 + 16 * c);
  }
  auto issue = [&](int st, int slot) {
    const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)(st * 3 * kS6Piece));
#pragma unroll
    for (int q = 0; q < kS6Dma; ++q) {
      const int idx = kS6Dma * wave + q;
      const int op = idx / 12, piece = (idx % 12) >> 2;
      const uint32_t dst = __builtin_amdgcn_readfirstlane(lds0 + slot * kS6Slot + (op * 3 + piece) * kS6Piece +
                                                          (idx & 3) * 1024);
      dma16_rsrc(voff[q], op == 0 ? rA : rB, soff, dst);
    }
  };
  uint32_t offA[2], offB[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int ra = 64 * wm + 32 * b + (lane & 31), rb = 64 * wn + 32 * b + (lane & 31);
    offA[b] = ra * 32 + (((lane >> 5) ^ s6_swz(ra)) * 16);
    offB[b] = 3 * kS6Piece + rb * 32 + (((lane >> 5) ^ s6_swz(rb)) * 16);
  }

  s6_f32x16_t acc[2][2], tot[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc[a][b][r] = 0.f;
        tot[a][b][r] = 0.f;
      }
  auto fold = [&]() {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          tot[a][b][r] += acc[a][b][r];
          acc[a][b][r] = 0.f;
        }
  };

#pragma unroll
  for (int ps = 0; ps < kS6Slots - 1; ++ps)
    if (ps < ns) issue(s_lo + ps, ps);
  for (int i = 0; i < ns; ++i) {
    s6_wait_barrier(min(kS6Slots - 2, ns - 1 - i));
    if (i + kS6Slots - 1 < ns) issue(s_lo + i + kS6Slots - 1, (i + kS6Slots - 1) % kS6Slots);
    const uint32_t sbase = lds0 + (uint32_t)(i % kS6Slots) * kS6Slot;
    s6_bf16x8_t fa[2][3], fb[2][3];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        fa[b][p] = s6_frag(sbase + p * kS6Piece + offA[b]);
        fb[b][p] = s6_frag(sbase + p * kS6Piece + offB[b]);
      }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a][2], fb[b][0], acc[a][b], 0, 0, 0);
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a][0], fb[b][2], acc[a][b], 0, 0, 0);
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a][1], fb[b][1], acc[a][b], 0, 0, 0);
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a][1], fb[b][0], acc[a][b], 0, 0, 0);
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a][0], fb[b][1], acc[a][b], 0, 0, 0);
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a][0], fb[b][0], acc[a][b], 0, 0, 0);
      }
    if (i & 1) fold();
  }
  if (ns & 1) fold();

  float* C = g.C + (int64_t)inst * g.sC;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t j = n0 + 64 * wn + 32 * b + (lane & 31);
      const int64_t ib = m0 + 64 * wm + 32 * a + 4 * (lane >> 5);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t i = ib + 8 * (r >> 2) + (r & 3);
        if (i < g.M && j < g.N) C[i * g.ldc + j] = g.alpha * tot[a][b][r];
      }
    }
}

static hipError_t split_op(hipStream_t s, const X6Operand& o, int64_t R, int64_t K, int batch, uint16_t* dst) {
  Split6Args a{};
  a.src = o.src; a.ld = o.ld; a.stride = o.stride;
  a.R = R; a.K = K; a.trans = o.trans; a.batch = batch; a.dst = dst;
  const bool vec = !o.trans && o.ld % 4 == 0 && o.stride % 4 == 0 && ((uintptr_t)o.src & 15) == 0;
  const int64_t items = ceil_div(R, kS6T) * ceil_div(K, kS6K) * batch;   // one per workgroup iteration
  if (items >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const unsigned blocks = (unsigned)std::min<int64_t>(items, 16384);
  if (o.trans) hipLaunchKernelGGL((k_split3_op<true, false>), dim3(blocks), dim3(256), 0, s, a);
  else if (vec) hipLaunchKernelGGL((k_split3_op<false, true>), dim3(blocks), dim3(256), 0, s, a);
  else hipLaunchKernelGGL((k_split3_op<false, false>), dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

static bool x6_args_ok(int64_t M, int64_t N, int64_t K, int batch, const uint16_t* pieces, int kmode) {
  if (K <= 0 || !pieces || ((uintptr_t)pieces & 15) != 0 || !(kmode == 0 || kmode == 3 || kmode == 4)) return false;
  // tile count and buffer sizes / stage offsets are 32-bit
  return ceil_div(M, kS6T) * ceil_div(N, kS6T) * batch < ((int64_t)1 << 31) &&
         ceil_div(K, kS6K) * 3 * kS6Piece < ((int64_t)1 << 31);
}

hipError_t x6_split(hipStream_t s, int64_t M, int64_t N, int64_t K, int batch, const X6Operand& a,
                    const X6Operand& b, uint16_t* pieces) {
  if (M <= 0 || N <= 0 || batch <= 0) return hipSuccess;
  if (!x6_args_ok(M, N, K, batch, pieces, 0)) return hipErrorInvalidValue;
  hipError_t e;
  if ((e = split_op(s, a, M, K, batch, pieces)) != hipSuccess) return e;
  return split_op(s, b, N, K, batch, pieces + x6_op_elems(M, K) * batch);
}

hipError_t x6_product(hipStream_t s, int64_t M, int64_t N, int64_t K, int batch, float* C, int64_t ldc,
                      int64_t sC, float alpha, int kmode, const uint16_t* pieces) {
  if (M <= 0 || N <= 0 || batch <= 0) return hipSuccess;
  if (!x6_args_ok(M, N, K, batch, pieces, kmode)) return hipErrorInvalidValue;
  const int64_t ntm = ceil_div(M, kS6T), ntn = ceil_div(N, kS6T);
  Gemm6Args g{};
  g.M = M; g.N = N; g.K = K; g.Ap = pieces; g.Bp = pieces + x6_op_elems(M, K) * batch;
  g.C = C; g.ldc = ldc; g.sC = sC; g.alpha = alpha;
  g.kmode = kmode; g.batch = batch; g.ntm = (int)ntm; g.ntn = (int)ntn;
  hipLaunchKernelGGL(k_gemm_x6, dim3((unsigned)(ntm * ntn * batch)), dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace gq
