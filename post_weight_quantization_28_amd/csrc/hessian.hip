// H += 2 X^T X on gfx950: bf16 MFMA with fp32 accumulation.
//
// "GPTQ" (wikiprompt.org), "Enfoque Técnico": the method works from the
// Hessian of the layer loss built from calibration inputs; for a linear
// layer that is (up to the factor 2 kept here) the Gram matrix of the
// calibration activations X (T tokens x n input channels).
//
// Design (MI355X):
//  * Only output tiles on or above the diagonal are computed (symmetry).
//  * 256x256 output tile per workgroup of 4 waves (2x2), each wave a 128x128
//    block = 4x4 v_mfma_f32_32x32x16_bf16 accumulators (256 fp32 per lane).
//  * X is row-major (tokens x channels) while MFMA wants 8 consecutive
//    tokens per lane: each thread loads an 8-token x 8-channel block with
//    eight 16-byte loads, transposes it in registers with v_perm_b32 and
//    stores eight 16-byte rows into LDS laid out [channel][token]. Row pitch
//    36 dwords keeps both the transposed stores and the fragment reads free
//    of bank conflicts. Two LDS stages (144 KiB) double-buffer the loads.
//  * The token range is split into chunks; each chunk writes an fp32 partial
//    Gram matrix and a second kernel sums the partials in a fixed order,
//    scales by 2, adds to H and mirrors it: deterministic, exactly
//    symmetric, and the chunked sum bounds fp32 accumulation error.
#include "common.h"

namespace gq {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kHT = 256;      // output tile edge
constexpr int kHBK = 64;      // tokens per LDS stage
constexpr int kHPitch = 36;   // dwords per LDS row (32 data + 4 pad)
constexpr int kHStage = kHT * kHPitch;  // dwords per operand per stage

int hessian_splits(int64_t T, int xdt_bf16) {
  // ~16384 tokens per partial (fp32 MFMA accumulation stays ~1e-6 relative),
  // at most 8 partials.
  int64_t s = ceil_div(T, 16384);
  if (s < 1) s = 1;
  if (s > 8) s = 8;
  (void)xdt_bf16;
  return (int)s;
}

__device__ inline void upper_tile(int t, int nt, int& bi, int& bj) {
  // enumerate (bi, bj), bi <= bj, row by row
  int row = 0;
  while (t >= nt - row) { t -= nt - row; ++row; }
  bi = row;
  bj = row + t;
}

// Load an 8(token) x 8(channel) bf16 block: rows X[t0+r][c0..c0+7].
template <bool kAligned>
__device__ inline void load_block(const uint16_t* __restrict__ X, int64_t ldx, int64_t t0,
                                  int64_t tend, int64_t c0, int64_t n, uint4 (&d)[8]) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    int64_t t = t0 + r;
    if (kAligned) {
      if (t < tend && c0 < n) {
        d[r] = *reinterpret_cast<const uint4*>(X + t * ldx + c0);
      } else {
        d[r] = make_uint4(0, 0, 0, 0);
      }
    } else {
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t lo = 0, hi = 0;
        int64_t c = c0 + 2 * q;
        if (t < tend && c < n) lo = X[t * ldx + c];
        if (t < tend && c + 1 < n) hi = X[t * ldx + c + 1];
        w[q] = lo | (hi << 16);
      }
      d[r] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// Transpose the block in registers and store channel rows into LDS.
__device__ inline void store_block_t(uint32_t* __restrict__ s, int row0, int tok_dw,
                                     const uint4 (&d)[8]) {
  uint32_t dd[8][4];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    dd[r][0] = d[r].x; dd[r][1] = d[r].y; dd[r][2] = d[r].z; dd[r][3] = d[r].w;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t ev[4], od[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      // channel 2q is the low half of dword q, channel 2q+1 the high half;
      // pack tokens (2p, 2p+1) into one dword
      ev[p] = __builtin_amdgcn_perm(dd[2 * p + 1][q], dd[2 * p][q], 0x05040100u);
      od[p] = __builtin_amdgcn_perm(dd[2 * p + 1][q], dd[2 * p][q], 0x07060302u);
    }
    *reinterpret_cast<uint4*>(s + (row0 + 2 * q) * kHPitch + tok_dw) =
        make_uint4(ev[0], ev[1], ev[2], ev[3]);
    *reinterpret_cast<uint4*>(s + (row0 + 2 * q + 1) * kHPitch + tok_dw) =
        make_uint4(od[0], od[1], od[2], od[3]);
  }
}

template <bool kAligned>
__global__ void __launch_bounds__(256)
k_hessian_bf16(const uint16_t* __restrict__ X, int64_t T, int64_t n, int64_t ldx,
               float* __restrict__ part, int64_t chunk) {
  __shared__ uint32_t smem[2 * 2 * kHStage];
  const int nt = (int)ceil_div(n, kHT);
  int bi, bj;
  upper_tile(blockIdx.x, nt, bi, bj);
  const int split = blockIdx.y;
  const int64_t kbeg = (int64_t)split * chunk;
  const int64_t kend = min(T, kbeg + chunk);
  const int64_t iA = (int64_t)bi * kHT, iB = (int64_t)bj * kHT;
  float* __restrict__ P = part + (int64_t)split * n * n;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // loader coordinates: 32 channel blocks x 8 token blocks
  const int lb_c = tid >> 3, lb_t = tid & 7;

  f32x16_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  const int64_t nstage = kend > kbeg ? ceil_div(kend - kbeg, kHBK) : 0;
  uint4 ra[8], rb[8];
  if (nstage > 0) {
    load_block<kAligned>(X, ldx, kbeg + 8 * lb_t, kend, iA + 8 * lb_c, n, ra);
    load_block<kAligned>(X, ldx, kbeg + 8 * lb_t, kend, iB + 8 * lb_c, n, rb);
    store_block_t(smem, 8 * lb_c, 4 * lb_t, ra);
    store_block_t(smem + kHStage, 8 * lb_c, 4 * lb_t, rb);
  }
  __syncthreads();

  for (int64_t st = 0; st < nstage; ++st) {
    const int cur = (int)(st & 1);
    const bool more = st + 1 < nstage;
    if (more) {
      const int64_t t0 = kbeg + (st + 1) * kHBK + 8 * lb_t;
      load_block<kAligned>(X, ldx, t0, kend, iA + 8 * lb_c, n, ra);
      load_block<kAligned>(X, ldx, t0, kend, iB + 8 * lb_c, n, rb);
    }
    const uint32_t* sA = smem + cur * 2 * kHStage;
    const uint32_t* sB = sA + kHStage;
#pragma unroll
    for (int ks = 0; ks < kHBK / 16; ++ks) {
      bf16x8_t af[4], bfr[4];
      const int koff = 8 * ks + 4 * (lane >> 5);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int row = 128 * wm + 32 * mb + (lane & 31);
        uint4 v = *reinterpret_cast<const uint4*>(sA + row * kHPitch + koff);
        af[mb] = __builtin_bit_cast(bf16x8_t, v);
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int row = 128 * wn + 32 * nb + (lane & 31);
        uint4 v = *reinterpret_cast<const uint4*>(sB + row * kHPitch + koff);
        bfr[nb] = __builtin_bit_cast(bf16x8_t, v);
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bfr[nb], acc[mb][nb], 0, 0, 0);
    }
    if (more) {
      uint32_t* dA = smem + (cur ^ 1) * 2 * kHStage;
      store_block_t(dA, 8 * lb_c, 4 * lb_t, ra);
      store_block_t(dA + kHStage, 8 * lb_c, 4 * lb_t, rb);
    }
    __syncthreads();
  }

  // epilogue: lane holds D[i][j], j = lane%32, i = 8*(r/4) + 4*(lane/32) + r%4
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t i = iA + 128 * wm + 32 * mb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t j = iB + 128 * wn + 32 * nb + (lane & 31);
        if (i < n && j < n) P[i * n + j] = acc[mb][nb][r];
      }
}

// Same tile with 8 waves (2 per SIMD): wave (wm, wn) in a 2 x 4 grid owns
// 128 x 64 of the tile (4 x 2 accumulators); threads 0-255 stage the A
// block of a stage and threads 256-511 the B block, so each thread keeps one
// 8 x 8 block in flight. Two waves per SIMD let one wave's transposes and
// LDS traffic overlap the other's MFMAs.
template <bool kAligned>
__global__ void __launch_bounds__(512)
k_hessian_bf16_w8(const uint16_t* __restrict__ X, int64_t T, int64_t n, int64_t ldx,
                  float* __restrict__ part, int64_t chunk) {
  __shared__ uint32_t smem[2 * 2 * kHStage];
  const int nt = (int)ceil_div(n, kHT);
  int bi, bj;
  upper_tile(blockIdx.x, nt, bi, bj);
  const int split = blockIdx.y;
  const int64_t kbeg = (int64_t)split * chunk;
  const int64_t kend = min(T, kbeg + chunk);
  const int64_t iA = (int64_t)bi * kHT, iB = (int64_t)bj * kHT;
  float* __restrict__ P = part + (int64_t)split * n * n;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int half = tid >> 8;                     // 0: stages A, 1: stages B
  const int lt = tid & 255;
  const int lb_c = lt >> 3, lb_t = lt & 7;
  const int64_t ibase = half ? iB : iA;

  f32x16_t acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  const int64_t nstage = kend > kbeg ? ceil_div(kend - kbeg, kHBK) : 0;
  uint4 rr[8];
  if (nstage > 0) {
    load_block<kAligned>(X, ldx, kbeg + 8 * lb_t, kend, ibase + 8 * lb_c, n, rr);
    store_block_t(smem + half * kHStage, 8 * lb_c, 4 * lb_t, rr);
  }
  __syncthreads();

  for (int64_t st = 0; st < nstage; ++st) {
    const int cur = (int)(st & 1);
    const bool more = st + 1 < nstage;
    if (more) load_block<kAligned>(X, ldx, kbeg + (st + 1) * kHBK + 8 * lb_t, kend, ibase + 8 * lb_c, n, rr);
    const uint32_t* sA = smem + cur * 2 * kHStage;
    const uint32_t* sB = sA + kHStage;
#pragma unroll
    for (int ks = 0; ks < kHBK / 16; ++ks) {
      bf16x8_t af[4], bfr[2];
      const int koff = 8 * ks + 4 * (lane >> 5);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int row = 128 * wm + 32 * mb + (lane & 31);
        af[mb] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(sA + row * kHPitch + koff));
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int row = 64 * wn + 32 * nb + (lane & 31);
        bfr[nb] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(sB + row * kHPitch + koff));
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bfr[nb], acc[mb][nb], 0, 0, 0);
    }
    if (more) store_block_t(smem + (cur ^ 1) * 2 * kHStage + half * kHStage, 8 * lb_c, 4 * lb_t, rr);
    __syncthreads();
  }

#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t i = iA + 128 * wm + 32 * mb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t j = iB + 64 * wn + 32 * nb + (lane & 31);
        if (i < n && j < n) P[i * n + j] = acc[mb][nb][r];
      }
}

hipError_t launch_hessian_partials_bf16_w8(hipStream_t s, const uint16_t* X, int64_t T, int64_t n,
                                           int64_t ldx, float* part, int splits) {
  const int nt = (int)ceil_div(n, kHT);
  const int64_t chunk = ceil_div(ceil_div(T, splits), kHBK) * kHBK;
  dim3 grid(nt * (nt + 1) / 2, splits);
  const bool aligned = (n % 8 == 0) && (ldx % 8 == 0) && ((uintptr_t)X % 16 == 0);
  if (aligned)
    hipLaunchKernelGGL(k_hessian_bf16_w8<true>, grid, dim3(512), 0, s, X, T, n, ldx, part, chunk);
  else
    hipLaunchKernelGGL(k_hessian_bf16_w8<false>, grid, dim3(512), 0, s, X, T, n, ldx, part, chunk);
  return hipGetLastError();
}

hipError_t launch_hessian_partials_bf16(hipStream_t s, const uint16_t* X, int64_t T, int64_t n,
                                        int64_t ldx, float* part, int splits) {
  const int nt = (int)ceil_div(n, kHT);
  const int64_t chunk = ceil_div(ceil_div(T, splits), kHBK) * kHBK;
  dim3 grid(nt * (nt + 1) / 2, splits);
  const bool aligned = (n % 8 == 0) && (ldx % 8 == 0) && ((uintptr_t)X % 16 == 0);
  if (aligned)
    hipLaunchKernelGGL(k_hessian_bf16<true>, grid, dim3(256), 0, s, X, T, n, ldx, part, chunk);
  else
    hipLaunchKernelGGL(k_hessian_bf16<false>, grid, dim3(256), 0, s, X, T, n, ldx, part, chunk);
  return hipGetLastError();
}

hipError_t launch_hessian_partials_f32(hipStream_t s, const float* X, int64_t T, int64_t n,
                                       int64_t ldx, float* part, int splits) {
  const int64_t chunk = ceil_div(T, splits);
  for (int sp = 0; sp < splits; ++sp) {
    const int64_t kb = sp * chunk, ke = min(T, kb + chunk);
    GemmArgs g{};
    g.M = n; g.N = n; g.K = ke > kb ? ke - kb : 0;
    g.A = X + kb * ldx; g.lda = ldx; g.ta = 1;     // A(m,k) = X[k][m]
    g.B = X + kb * ldx; g.ldb = ldx; g.tb = 0;     // B(k,n) = X[k][n]
    g.C = part + (int64_t)sp * n * n; g.ldc = n;
    g.alpha = 1.f; g.beta = 0.f; g.kmode = 0; g.lower_only = 0; g.st = nullptr;
    hipError_t e = launch_gemm_f32(s, g);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// H[i][j] (i <= j) = base + 2 * sum_s part[s][i][j]; H[j][i] = H[i][j].
__global__ void __launch_bounds__(256)
k_hessian_reduce(const float* __restrict__ part, int splits, int64_t n, float* __restrict__ H,
                 int zero_first) {
  __shared__ float tile[64][65];
  const int nt = (int)ceil_div(n, 64);
  int a, b;
  upper_tile(blockIdx.x, nt, a, b);
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int64_t nn = n * n;
  for (int r = ty; r < 64; r += 4) {
    const int64_t i = (int64_t)a * 64 + r, j = (int64_t)b * 64 + tx;
    float v = 0.f;
    if (i < n && j < n && i <= j) {
      float sum = 0.f;
      for (int sp = 0; sp < splits; ++sp) sum += part[sp * nn + i * n + j];
      v = (zero_first ? 0.f : H[i * n + j]) + 2.f * sum;
      H[i * n + j] = v;
    }
    tile[r][tx] = v;
  }
  __syncthreads();
  // mirror: H[64b + r][64a + tx] = tile[tx][r] where (64a+tx) < (64b+r)
  for (int r = ty; r < 64; r += 4) {
    const int64_t i = (int64_t)b * 64 + r, j = (int64_t)a * 64 + tx;
    if (i < n && j < n && j < i) H[i * n + j] = tile[tx][r];
  }
}

hipError_t launch_hessian_reduce(hipStream_t s, const float* part, int splits, int64_t n,
                                 float* H, int zero_first) {
  const int nt = (int)ceil_div(n, 64);
  hipLaunchKernelGGL(k_hessian_reduce, dim3(nt * (nt + 1) / 2), dim3(256), 0, s, part, splits, n,
                     H, zero_first);
  return hipGetLastError();
}

}  // namespace gq
