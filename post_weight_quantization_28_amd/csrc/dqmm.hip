// Dequantising matrix product of a packed low-bit layer, for inference:
// Y (M x d_out, fp32) = X (M x n, bf16) W_hat^T with
// W_hat[o][k] = s[o][k / g] (q[o][k] - z[o][k / g]) and the codes q read
// from the LSB-first bitstream the quantizer writes.
//
// "El balance de errores de la inferencia de pocos bits", section 6: the
// saving of a low-bit format is only realised by a kernel that unpacks,
// dequantises and multiplies, and decode (few tokens: bound by reading the
// packed weights) and prefill (many tokens: bound by the matrix cores) are
// different regimes. Section 1: the affine reconstruction s (q - z).
//
// One workgroup of 4 waves computes a (32 MB) x 128 block of Y. Wave w owns
// outputs o0 + 32 w .. + 31, the columns of its 32 x 32 MFMA tiles
// (v_mfma_f32_32x32x16_bf16), for all MB row blocks of X.
//  * The scale is factored out of the sum: per group, the MFMAs accumulate
//    sum_k x[m][k] (q[o][k] - z[o][g]) in fp32 (bf16 x small integer
//    products are exact), and the group's sum is then added to the total
//    times s[o][g]. Every lane's 16 accumulator values belong to one output
//    o, so scale and zero point are one value per lane and group. No
//    weight is ever rounded to bf16.
//  * K advances in chunks of 32 codes: exactly `bits` whole words of a row.
//    Lane l (o = l % 32, half h = l / 32) takes codes 16 kk + 8 h .. + 7 of
//    the chunk for the two K slices kk = 0, 1 from those words (a 64-bit
//    window for 3 bits, whose codes straddle words), subtracts z and
//    converts them to bf16, which is exact for these small integers.
//  * The X fragment of a K slice is one 16-byte load per lane (8 consecutive
//    k of row m); rows past M are loaded from the last row and zeroed.
//  * The next chunk's words and X fragments are loaded before the current
//    chunk's MFMAs.
//  * Few output blocks (decode) split the group range over grid.y; the
//    splits write fp32 partials that a second kernel sums in a fixed order,
//    so results do not depend on timing.
#include "common.h"

namespace gq {

typedef __bf16 dq_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float dq_f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int dq_u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kDqBN = 128;   // outputs per workgroup (4 waves x 32)

// Two small integers (|v| <= 15) as packed bf16: the fp32 pattern of such a
// value has zero low 16 bits, so its high half is the exact bf16.
__device__ __forceinline__ uint32_t dq_pack2(int lo, int hi) {
  const uint32_t a = __float_as_uint((float)lo) >> 16;
  const uint32_t b = __float_as_uint((float)hi) & 0xFFFF0000u;
  return a | b;
}

// Codes 8 j .. 8 j + 7 (j = 2 kk + h) of a 32-code chunk held in w[0..BITS),
// minus z, as 8 bf16.
template <int BITS>
__device__ __forceinline__ dq_bf16x8_t dq_unpack8(const uint32_t (&w)[BITS], int j, int z) {
  const int base = 8 * BITS * j;
  const int wi = base >> 5, sh = base & 31;
  uint64_t v = w[wi];
  if constexpr (BITS == 3) {
    // bits 24..47 and 48..71 cross a word boundary
    if (wi + 1 < BITS) v |= (uint64_t)w[wi + 1] << 32;
  }
  v >>= sh;
  constexpr uint32_t mask = (1u << BITS) - 1u;
  uint32_t p[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int q0 = (int)((v >> (BITS * (2 * e))) & mask);
    const int q1 = (int)((v >> (BITS * (2 * e + 1))) & mask);
    p[e] = dq_pack2(q0 - z, q1 - z);
  }
  const dq_u32x4_t u = {p[0], p[1], p[2], p[3]};
  return __builtin_bit_cast(dq_bf16x8_t, u);
}

template <int BITS, int MB>
__global__ void __launch_bounds__(256)
k_dequant_mm(const uint16_t* __restrict__ X, int64_t M, int64_t n, int64_t ldx,
             const uint32_t* __restrict__ qw, const float* __restrict__ scales,
             const uint8_t* __restrict__ zeros, int64_t d_out, int group,
             float* __restrict__ Y, int64_t ldy, int groups_per_split, int64_t split_stride) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = lane >> 5, li = lane & 31;
  const int64_t m0 = (int64_t)blockIdx.z * (32 * MB);
  const int64_t o = (int64_t)blockIdx.x * kDqBN + 32 * wave + li;
  const int64_t oc = o < d_out ? o : d_out - 1;          // rows past d_out read the last row
  const int64_t ngroups = n / group;
  const int64_t g0 = (int64_t)blockIdx.y * groups_per_split;
  const int64_t g1 = min(ngroups, g0 + groups_per_split);
  const int cpg = group / 32;                              // chunks per group
  const int64_t wpr = n / 32 * BITS;                       // words per row

  const uint32_t* __restrict__ qrow = qw + oc * wpr;
  const uint16_t* xrow[MB];
  bool mok[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int64_t m = m0 + 32 * mb + li;
    mok[mb] = m < M;
    xrow[mb] = X + (m < M ? m : M - 1) * ldx + 8 * h;
  }

  dq_f32x16_t tot[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) tot[mb][r] = 0.f;

  // chunk c of the split: words and X fragments
  uint32_t wn[BITS];
  dq_bf16x8_t xn[MB][2];
  auto load = [&](int64_t c) {
#pragma unroll
    for (int i = 0; i < BITS; ++i) wn[i] = qrow[c * BITS + i];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        xn[mb][kk] = *reinterpret_cast<const dq_bf16x8_t*>(xrow[mb] + 32 * c + 16 * kk);
  };
  const int64_t c_begin = g0 * cpg, c_end = g1 * cpg;
  if (c_begin < c_end) load(c_begin);
  for (int64_t g = g0; g < g1; ++g) {
    const float s = scales[oc * ngroups + g];
    const int z = zeros[oc * ngroups + g];
    dq_f32x16_t acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][r] = 0.f;
    for (int cc = 0; cc < cpg; ++cc) {
      const int64_t c = g * cpg + cc;
      uint32_t w[BITS];
      dq_bf16x8_t xa[MB][2];
#pragma unroll
      for (int i = 0; i < BITS; ++i) w[i] = wn[i];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        xa[mb][0] = mok[mb] ? xn[mb][0] : dq_bf16x8_t{};
        xa[mb][1] = mok[mb] ? xn[mb][1] : dq_bf16x8_t{};
      }
      if (c + 1 < c_end) load(c + 1);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const dq_bf16x8_t b = dq_unpack8<BITS>(w, 2 * kk + h, z);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[mb][kk], b, acc[mb], 0, 0, 0);
      }
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) tot[mb][r] = fmaf(s, acc[mb][r], tot[mb][r]);
  }

  if (o >= d_out) return;
  Y += (int64_t)blockIdx.y * split_stride;   // this split's partial (0 without a split)
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t m = m0 + 32 * mb + 8 * (r >> 2) + 4 * h + (r & 3);
      if (m < M) Y[m * ldy + o] = tot[mb][r];
    }
}

// Y[m][o] = sum over the splits, in split order.
__global__ void __launch_bounds__(256)
k_dequant_mm_reduce(const float* __restrict__ part, int splits, int64_t M, int64_t d_out,
                    float* __restrict__ Y, int64_t ldy) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= M * d_out) return;
  float v = 0.f;
  for (int sp = 0; sp < splits; ++sp) v += part[(int64_t)sp * M * d_out + i];
  Y[(i / d_out) * ldy + i % d_out] = v;
}

DqPlan dequant_mm_plan(int64_t M, int64_t n, int64_t d_out, int group) {
  DqPlan p{};
  p.mb = M <= 32 ? 1 : (M <= 64 ? 2 : 4);
  p.mtiles = ceil_div(M, 32 * p.mb);
  p.otiles = ceil_div(d_out, kDqBN);
  const int64_t ngroups = group > 0 ? n / group : 0;
  const int64_t tiles = p.mtiles * p.otiles;
  int64_t s = tiles > 0 ? ceil_div(256, tiles) : 1;
  if (s > ngroups) s = ngroups;
  if (s < 1) s = 1;
  p.groups_per_split = ngroups > 0 ? ceil_div(ngroups, s) : 1;
  p.splits = ngroups > 0 ? ceil_div(ngroups, p.groups_per_split) : 1;
  p.part_bytes = p.splits > 1 ? (size_t)p.splits * M * d_out * sizeof(float) : 0;
  return p;
}

template <int BITS>
static void launch_bits(hipStream_t s, const DqPlan& p, const uint16_t* X, int64_t M, int64_t n,
                        int64_t ldx, const uint32_t* qw, const float* sc, const uint8_t* z,
                        int64_t d_out, int group, float* out, int64_t ldo) {
  const dim3 grid((unsigned)p.otiles, (unsigned)p.splits, (unsigned)p.mtiles);
  const int64_t ss = p.splits > 1 ? M * d_out : 0;
  if (p.mb == 1)
    hipLaunchKernelGGL((k_dequant_mm<BITS, 1>), grid, dim3(256), 0, s, X, M, n, ldx, qw, sc, z, d_out, group,
                       out, ldo, (int)p.groups_per_split, ss);
  else if (p.mb == 2)
    hipLaunchKernelGGL((k_dequant_mm<BITS, 2>), grid, dim3(256), 0, s, X, M, n, ldx, qw, sc, z, d_out, group,
                       out, ldo, (int)p.groups_per_split, ss);
  else
    hipLaunchKernelGGL((k_dequant_mm<BITS, 4>), grid, dim3(256), 0, s, X, M, n, ldx, qw, sc, z, d_out, group,
                       out, ldo, (int)p.groups_per_split, ss);
}

hipError_t launch_dequant_mm(hipStream_t s, const DqPlan& p, const uint16_t* X, int64_t M, int64_t n,
                             int64_t ldx, const uint32_t* qw, const float* sc, const uint8_t* z,
                             int64_t d_out, int bits, int group, float* Y, int64_t ldy, float* part) {
  if (M <= 0 || d_out <= 0) return hipSuccess;
  float* out = p.splits > 1 ? part : Y;
  const int64_t ldo = p.splits > 1 ? d_out : ldy;
  if (bits == 2) launch_bits<2>(s, p, X, M, n, ldx, qw, sc, z, d_out, group, out, ldo);
  else if (bits == 3) launch_bits<3>(s, p, X, M, n, ldx, qw, sc, z, d_out, group, out, ldo);
  else launch_bits<4>(s, p, X, M, n, ldx, qw, sc, z, d_out, group, out, ldo);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits <= 1) return e;
  hipLaunchKernelGGL(k_dequant_mm_reduce, dim3((unsigned)ceil_div(M * d_out, 256)), dim3(256), 0, s, part,
                     (int)p.splits, M, d_out, Y, ldy);
  return hipGetLastError();
}

}  // namespace gq
