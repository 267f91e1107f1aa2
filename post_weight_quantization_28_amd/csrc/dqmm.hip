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

#include <algorithm>
#include <type_traits>

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

// ---- many tokens: the X tile staged once per workgroup
//
// With 128 tokens per workgroup, the four waves of k_dequant_mm<BITS, 4>
// each fetch the same 8 KiB X tile per chunk through L1, which takes
// longer than the chunk's MFMAs. Here the workgroup stages it in LDS
// instead (double buffer, one barrier per chunk): thread t moves 16-byte
// pieces t % 4 of token rows t / 4 and t / 4 + 64 (rows past M are
// zeroed); each wave then reads its fragments with ds_read_b128 (row pitch
// 80 bytes). Global loads (X pieces and packed words) run kPxAhead chunks
// ahead in registers, and a group's zero point and scale one group ahead.
// Two waves per SIMD matter more than depth: 2 or 4 chunks ahead cost the
// registers of the second wave and measured 255 and 444 us against 241 us
// for one chunk (4096 tokens, 4096 x 4096, 4 bits). Codes, scales and the
// per-group scaling are as in k_dequant_mm.
constexpr int kPxPitch = 80;
constexpr int kPxAhead = 1;   // chunks of global loads in flight per thread

template <int BITS>
__global__ void __launch_bounds__(256)
k_dequant_mm_x(const uint16_t* __restrict__ X, int64_t M, int64_t n, int64_t ldx,
               const uint32_t* __restrict__ qw, const float* __restrict__ scales,
               const uint8_t* __restrict__ zeros, int64_t d_out, int group,
               float* __restrict__ Y, int64_t ldy, int groups_per_split, int64_t split_stride) {
  constexpr int MB = 4;
  __shared__ __align__(16) uint8_t xs[2][128 * kPxPitch];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = lane >> 5, li = lane & 31;
  const int64_t m0 = (int64_t)blockIdx.z * 128;
  const int64_t o = (int64_t)blockIdx.x * kDqBN + 32 * wave + li;
  const int64_t oc = o < d_out ? o : d_out - 1;
  const int64_t ngroups = n / group;
  const int64_t g0 = (int64_t)blockIdx.y * groups_per_split;
  const int64_t g1 = min(ngroups, g0 + groups_per_split);
  const int cpg = group / 32;
  const uint32_t* __restrict__ qrow = qw + oc * (n / 32 * BITS);

  // staging: rows sr and sr + 64 of the tile, 16-byte piece sp
  const int sr = threadIdx.x >> 2, sp = threadIdx.x & 3;
  const bool v0 = m0 + sr < M, v1 = m0 + sr + 64 < M;
  const uint16_t* __restrict__ xs0 = X + min(m0 + sr, M - 1) * ldx + 8 * sp;
  const uint16_t* __restrict__ xs1 = X + min(m0 + sr + 64, M - 1) * ldx + 8 * sp;
  const uint32_t so0 = sr * kPxPitch + 16 * sp, so1 = (sr + 64) * kPxPitch + 16 * sp;

  const int64_t c_begin = g0 * cpg, c_end = g1 * cpg;
  constexpr int D = kPxAhead;
  dq_u32x4_t st0[D], st1[D];
  uint32_t wn[D][BITS];
  auto gload = [&](int u, int64_t c) {
    st0[u] = *reinterpret_cast<const dq_u32x4_t*>(xs0 + 32 * c);
    st1[u] = *reinterpret_cast<const dq_u32x4_t*>(xs1 + 32 * c);
#pragma unroll
    for (int i = 0; i < BITS; ++i) wn[u][i] = qrow[c * BITS + i];
  };

  dq_f32x16_t tot[MB], acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) tot[mb][r] = acc[mb][r] = 0.f;
  if (c_begin >= c_end) goto store;
  {
#pragma unroll
    for (int u = 0; u < D; ++u) gload(u, min(c_begin + u, c_end - 1));
    // scale and zero point of the current group, and of the next one
    int64_t g = g0;
    float sc = scales[oc * ngroups + g], sn = scales[oc * ngroups + min(g + 1, g1 - 1)];
    int zc = zeros[oc * ngroups + g], zn = zeros[oc * ngroups + min(g + 1, g1 - 1)];
    int cin = 0;
    for (int64_t c0 = c_begin; c0 < c_end; c0 += D) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        const int64_t c = c0 + u;
        if (c >= c_end) break;
        uint8_t* buf = xs[c & 1];
        *reinterpret_cast<dq_u32x4_t*>(buf + so0) = v0 ? st0[u] : dq_u32x4_t{0u, 0u, 0u, 0u};
        *reinterpret_cast<dq_u32x4_t*>(buf + so1) = v1 ? st1[u] : dq_u32x4_t{0u, 0u, 0u, 0u};
        uint32_t w[BITS];
#pragma unroll
        for (int i = 0; i < BITS; ++i) w[i] = wn[u][i];
        __syncthreads();
        gload(u, min(c + D, c_end - 1));
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const dq_bf16x8_t bq = dq_unpack8<BITS>(w, 2 * kk + h, zc);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            const dq_bf16x8_t a =
                *reinterpret_cast<const dq_bf16x8_t*>(buf + (32 * mb + li) * kPxPitch + 16 * (2 * kk + h));
            acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq, acc[mb], 0, 0, 0);
          }
        }
        if (++cin == cpg) {           // the group is complete
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              tot[mb][r] = fmaf(sc, acc[mb][r], tot[mb][r]);
              acc[mb][r] = 0.f;
            }
          cin = 0;
          ++g;
          sc = sn;
          zc = zn;
          const int64_t gn = min(g + 1, g1 - 1);
          sn = scales[oc * ngroups + gn];
          zn = zeros[oc * ngroups + gn];
        }
      }
    }
  }
store:
  if (o >= d_out) return;
  Y += (int64_t)blockIdx.y * split_stride;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t m = m0 + 32 * mb + 8 * (r >> 2) + 4 * h + (r & 3);
      if (m < M) Y[m * ldy + o] = tot[mb][r];
    }
}

// ---- decode (M <= 16): v_mfma_f32_16x16x32_bf16, one 32-code chunk per MFMA
//
// Few tokens: the cost is reading the packed weights and unpacking them
// (about 3 VALU operations per code, the same total whatever the layout).
// A workgroup of 16 waves owns kDvOB blocks of 16 outputs and splits K
// among its waves: wave w takes steps w, w + 16, ... of 8 chunks each (8 /
// CPG whole groups, CPG = chunks per group) for all its output blocks, so
// no wave loads what another loads and no partial sum goes to memory. The
// 16 partial sums meet in LDS and are added in wave order (fixed order:
// bitwise reproducible). One block per workgroup spreads the unpacking
// over all CUs (measured: 10.5 against 12.7 us per 4096 x 4096 call with
// two blocks, which halves the activation reads instead). Lane l: output
// o = o0 + l % 16 and K group j = l / 16, i.e. codes 8 j .. 8 j + 7 of each
// chunk (one word at 4 and 2 bits, a two-word window at 3) and
// X[l % 16][k0 + 8 j .. + 7] (one 16-byte load); the accumulator holds rows
// 4 j .. 4 j + 3 of column o. The step's packed words (8 chunks = 32 BITS
// bytes per row) are loaded as whole 16-byte pieces (2 BITS per row), so
// every line is requested once, into the wave's own LDS rows (pitch padded
// by 16 bytes against bank conflicts), and each lane then reads its words
// from there. All loads of a step are issued before its first MFMA; the 4
// waves per SIMD cover each other's latency. Needs 16-byte aligned rows:
// n BITS % 128 == 0.
typedef float dq_f32x4_t __attribute__((ext_vector_type(4)));
constexpr int kDvOB = 1;       // 16-output blocks per workgroup
constexpr int kDvOut = 16 * kDvOB;
constexpr int kDvWaves = 16;   // K slices per workgroup
constexpr int kDvStep = 8;     // chunks per step

// the 8 BITS bits of codes 8 j .. 8 j + 7 of chunk c, in the low bits
template <int BITS>
using dv_win_t = typename std::conditional<BITS == 3, uint64_t, uint32_t>::type;

template <int BITS>
__device__ __forceinline__ dv_win_t<BITS> dv_window(const uint32_t* __restrict__ qrow, int64_t c, int j) {
  const int base = 8 * BITS * j;
  const int64_t wi = c * BITS + (base >> 5);
  if constexpr (BITS == 3) {
    const int64_t wj = c * BITS + min((base >> 5) + 1, BITS - 1);
    return ((uint64_t)qrow[wj] << 32 | qrow[wi]) >> (base & 31);
  } else {
    return qrow[wi] >> (base & 31);
  }
}

template <int BITS>
__device__ __forceinline__ dq_bf16x8_t dv_unpack(dv_win_t<BITS> v, int z) {
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

template <int BITS, int CPG>
__global__ void __launch_bounds__(64 * kDvWaves)
k_dequant_mv(const uint16_t* __restrict__ X, int64_t M, int64_t n, int64_t ldx,
             const uint32_t* __restrict__ qw, const float* __restrict__ scales,
             const uint8_t* __restrict__ zeros, int64_t d_out, float* __restrict__ Y, int64_t ldy) {
  constexpr int GPS = kDvStep / CPG;                       // groups per step
  constexpr int RB = 32 * BITS;                            // bytes of a row per step
  constexpr int PITCH = RB + 16;
  constexpr int PIECES = 2 * BITS;                         // 16-byte pieces per row per step
  __shared__ __align__(16) uint8_t wbuf[kDvWaves][kDvOut * PITCH];
  __shared__ float red[kDvWaves][kDvOB][4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane >> 4, li = lane & 15;
  const int64_t ngroups = n / (32 * CPG);
  const int64_t nsteps = ngroups / GPS;                    // ngroups % GPS == 0
  const int64_t wpr = n / 32 * BITS;
  const float* srow[kDvOB];
  const uint8_t* zrow[kDvOB];
#pragma unroll
  for (int b = 0; b < kDvOB; ++b) {
    const int64_t o = (int64_t)blockIdx.x * kDvOut + 16 * b + li;
    const int64_t oc = o < d_out ? o : d_out - 1;
    srow[b] = scales + oc * ngroups;
    zrow[b] = zeros + oc * ngroups;
  }
  // the pieces this lane moves: piece p = 64 i + lane < NP -> row p / PIECES,
  // piece p % PIECES of that row
  constexpr int NP = kDvOut * PIECES;                      // pieces per step
  constexpr int NI = (NP + 63) / 64;
  const uint8_t* gsrc[NI];
  uint32_t ldst[NI];
  bool pv[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int p = 64 * i + lane;
    pv[i] = p < NP;
    const int row = pv[i] ? p / PIECES : 0, pc = pv[i] ? p % PIECES : 0;
    const int64_t o = (int64_t)blockIdx.x * kDvOut + row;
    const int64_t oc = o < d_out ? o : d_out - 1;
    gsrc[i] = reinterpret_cast<const uint8_t*>(qw + oc * wpr) + 16 * pc;
    ldst[i] = row * PITCH + 16 * pc;
  }
  uint8_t* wb = wbuf[wave];
  const bool mok = li < M;
  const uint16_t* __restrict__ xrow = X + (mok ? li : M - 1) * ldx + 8 * j;

  dq_f32x4_t tot[kDvOB];
#pragma unroll
  for (int b = 0; b < kDvOB; ++b) tot[b] = (dq_f32x4_t){0.f, 0.f, 0.f, 0.f};
  for (int64_t st = wave; st < nsteps; st += kDvWaves) {
    const int64_t g = st * GPS;
    dq_bf16x8_t xa[kDvStep];
    float sc[kDvOB][GPS];
    int zc[kDvOB][GPS];
    dq_u32x4_t piece[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i)
      if (pv[i]) piece[i] = *reinterpret_cast<const dq_u32x4_t*>(gsrc[i] + st * RB);
#pragma unroll
    for (int s = 0; s < kDvStep; ++s)
      xa[s] = *reinterpret_cast<const dq_bf16x8_t*>(xrow + 32 * (g * CPG + s));
#pragma unroll
    for (int b = 0; b < kDvOB; ++b)
#pragma unroll
      for (int q = 0; q < GPS; ++q) {
        sc[b][q] = srow[b][g + q];
        zc[b][q] = zrow[b][g + q];
      }
#pragma unroll
    for (int s = 0; s < kDvStep; ++s)
      if (!mok) xa[s] = dq_bf16x8_t{};
#pragma unroll
    for (int i = 0; i < NI; ++i)
      if (pv[i]) *reinterpret_cast<dq_u32x4_t*>(wb + ldst[i]) = piece[i];
    // this lane's windows: row 16 b + li, chunk s, K group j
    dv_win_t<BITS> w[kDvOB][kDvStep];
#pragma unroll
    for (int b = 0; b < kDvOB; ++b) {
      const uint32_t* rw = reinterpret_cast<const uint32_t*>(wb + (16 * b + li) * PITCH);
#pragma unroll
      for (int s = 0; s < kDvStep; ++s) w[b][s] = dv_window<BITS>(rw, s, j);
    }
#pragma unroll
    for (int b = 0; b < kDvOB; ++b)
#pragma unroll
      for (int q = 0; q < GPS; ++q) {
        dq_f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cc = 0; cc < CPG; ++cc)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[q * CPG + cc],
                                                        dv_unpack<BITS>(w[b][q * CPG + cc], zc[b][q]), acc, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) tot[b][r] = fmaf(sc[b][q], acc[r], tot[b][r]);
      }
  }
#pragma unroll
  for (int b = 0; b < kDvOB; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][b][r][lane] = tot[b][r];
  __syncthreads();
  // threads 0..511: one (block, row-in-lane, lane) each; sum in wave order
  const int t = threadIdx.x;
  if (t >= kDvOB * 4 * 64) return;
  const int b = t >> 8, r = (t >> 6) & 3, l = t & 63;
  float v = 0.f;
#pragma unroll
  for (int w = 0; w < kDvWaves; ++w) v += red[w][b][r][l];
  const int64_t o = (int64_t)blockIdx.x * kDvOut + 16 * b + (l & 15);
  const int64_t m = 4 * (l >> 4) + r;
  if (o < d_out && m < M) Y[m * ldy + o] = v;
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

// ---- act-order layers
//
// The product is invariant to one permutation applied to the columns of both
// X and W_hat, so a layer whose groups are not contiguous in the original
// column order (act-order) is used through any order that makes them
// contiguous: pi lists the columns of group 0, then of group 1, ..., each
// group's members in original order (a stable sort of g_idx).

// perm[g * group + r] = the r-th column k (in original order) with
// g_idx[k] == g; one thread per group. Entries of a group with fewer than
// `group` members keep their prior (zero) value.
__global__ void __launch_bounds__(256)
k_group_order(const int32_t* __restrict__ g_idx, int64_t n, int group, int64_t ngroups,
              int32_t* __restrict__ perm) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= ngroups) return;
  int64_t r = 0;
  for (int64_t k = 0; k < n && r < group; ++k)
    if (g_idx[k] == g) perm[g * group + r++] = (int32_t)k;
}

hipError_t launch_group_order(hipStream_t s, const int32_t* g_idx, int64_t n, int group, int32_t* perm) {
  const int64_t ngroups = n / group;
  if (ngroups == 0) return hipSuccess;
  hipLaunchKernelGGL(k_group_order, dim3((unsigned)ceil_div(ngroups, 256)), dim3(256), 0, s, g_idx, n, group,
                     ngroups, perm);
  return hipGetLastError();
}

// Xp[m][p] = X[m][perm[p]] (bf16 bits), Xp dense with row pitch n.
__global__ void __launch_bounds__(256)
k_gather_cols(const uint16_t* __restrict__ X, int64_t ldx, int64_t n, const int32_t* __restrict__ perm,
              uint16_t* __restrict__ Xp) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t m = blockIdx.y;
  if (p >= n) return;
  Xp[m * n + p] = X[m * ldx + perm[p]];
}

hipError_t launch_gather_cols(hipStream_t s, const uint16_t* X, int64_t M, int64_t ldx, int64_t n,
                              const int32_t* perm, uint16_t* Xp) {
  if (M <= 0 || n <= 0) return hipSuccess;
  for (int64_t m0 = 0; m0 < M; m0 += 65535) {
    const int64_t rows = std::min<int64_t>(65535, M - m0);
    hipLaunchKernelGGL(k_gather_cols, dim3((unsigned)ceil_div(n, 256), (unsigned)rows), dim3(256), 0, s,
                       X + m0 * ldx, ldx, n, perm, Xp + m0 * n);
  }
  return hipGetLastError();
}

DqPlan dequant_mm_plan(int64_t M, int64_t n, int64_t d_out, int bits, int group) {
  DqPlan p{};
  const int64_t ngroups = group > 0 ? n / group : 0;
  const int cpg = group / 32;
  // decode kernel: up to 16 tokens, groups of 32..256 codes, whole 8-chunk
  // steps in every split
  const int gps = cpg > 0 && cpg <= kDvStep && kDvStep % cpg == 0 ? kDvStep / cpg : 0;
  if (M <= 16 && gps > 0 && ngroups >= gps && ngroups % gps == 0 && (n * bits) % 128 == 0) {
    p.decode = 1;
    p.mb = 1;
    p.mtiles = 1;
    p.otiles = ceil_div(d_out, kDvOut);
    p.groups_per_split = ngroups;
    p.splits = 1;
  } else {
    p.decode = 0;
    p.mb = M <= 32 ? 1 : (M <= 64 ? 2 : 4);
    p.mtiles = ceil_div(M, 32 * p.mb);
    p.otiles = ceil_div(d_out, kDqBN);
    const int64_t tiles = p.mtiles * p.otiles;
    int64_t s = tiles > 0 ? ceil_div(256, tiles) : 1;
    if (s > ngroups) s = ngroups;
    if (s < 1) s = 1;
    p.groups_per_split = ngroups > 0 ? ceil_div(ngroups, s) : 1;
    p.splits = ngroups > 0 ? ceil_div(ngroups, p.groups_per_split) : 1;
  }
  p.part_bytes = p.splits > 1 ? (size_t)p.splits * M * d_out * sizeof(float) : 0;
  return p;
}

template <int BITS, int CPG>
static void launch_mv(hipStream_t s, const DqPlan& p, const uint16_t* X, int64_t M, int64_t n, int64_t ldx,
                      const uint32_t* qw, const float* sc, const uint8_t* z, int64_t d_out, float* out,
                      int64_t ldo, int64_t) {
  hipLaunchKernelGGL((k_dequant_mv<BITS, CPG>), dim3((unsigned)p.otiles), dim3(64 * kDvWaves), 0, s,
                     X, M, n, ldx, qw, sc, z, d_out, out, ldo);
}

template <int BITS>
static void launch_bits(hipStream_t s, const DqPlan& p, const uint16_t* X, int64_t M, int64_t n,
                        int64_t ldx, const uint32_t* qw, const float* sc, const uint8_t* z,
                        int64_t d_out, int group, float* out, int64_t ldo) {
  const dim3 grid((unsigned)p.otiles, (unsigned)p.splits, (unsigned)p.mtiles);
  const int64_t ss = p.splits > 1 ? M * d_out : 0;
  if (p.decode) {
    const int cpg = group / 32;
    if (cpg == 1) launch_mv<BITS, 1>(s, p, X, M, n, ldx, qw, sc, z, d_out, out, ldo, ss);
    else if (cpg == 2) launch_mv<BITS, 2>(s, p, X, M, n, ldx, qw, sc, z, d_out, out, ldo, ss);
    else if (cpg == 4) launch_mv<BITS, 4>(s, p, X, M, n, ldx, qw, sc, z, d_out, out, ldo, ss);
    else launch_mv<BITS, 8>(s, p, X, M, n, ldx, qw, sc, z, d_out, out, ldo, ss);
    return;
  }
  if (p.mb == 1)
    hipLaunchKernelGGL((k_dequant_mm<BITS, 1>), grid, dim3(256), 0, s, X, M, n, ldx, qw, sc, z, d_out, group,
                       out, ldo, (int)p.groups_per_split, ss);
  else if (p.mb == 2)
    hipLaunchKernelGGL((k_dequant_mm<BITS, 2>), grid, dim3(256), 0, s, X, M, n, ldx, qw, sc, z, d_out, group,
                       out, ldo, (int)p.groups_per_split, ss);
  else
    hipLaunchKernelGGL((k_dequant_mm_x<BITS>), grid, dim3(256), 0, s, X, M, n, ldx, qw, sc, z, d_out, group,
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
