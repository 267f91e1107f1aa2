// One lazy batch of the GPTQ column sweep.
//
// "GPTQ" (wikiprompt.org), "Enfoque Técnico": columns are quantized one at a
// time and the columns not yet quantized are corrected in closed form (the
// Optimal-Brain step) after each one; groups of weights share a scale.
// "El balance de errores de la inferencia de pocos bits", section 1: affine
// format with scale and zero point (rounding, range and group rules are the
// ones stated in gptq.h).
//
// For block [i0, i0+ncols) and every row independently, in column order j:
//   at a group start: (s, z) from the group's current values
//   q_j = clamp(rint(w_j / s) + z, 0, top), w_hat_j = s (q_j - z)
// (top = maxq; on the symmetric alphabet {-A..A} of the GPTQ-intrinsic LoRA
// page's finite-alphabet bounds, s = max|v| / A, z = A and top = 2A)
//   e_j = (w_j - w_hat_j) / U_jj
//   w_k -= e_j U_jk for the later columns k of the block
// E (d_out x B) collects e_j for the trailing update of the later blocks.
//
// Layout (MI355X): a wavefront holds 4 rows; the 16 lanes of a DPP row own
// one weight row, column 16c + L in register slot c of lane L (c < CPL =
// B/16, cyclic). Column j is decided by lane j % 16 from slot j / 16: the
// value is broadcast to its 16 lanes with DPP row_newbcast (no LDS round
// trip), every lane rounds it redundantly and applies the rank-1 feedback to
// its own slots with U's row j read from LDS. Because the layout is cyclic,
// every slot below (j + 1) / 16 holds only finished columns and is skipped
// at compile time: the feedback costs half of a dense row update. The loop
// over j is fully unrolled (owner lane and slots are compile-time
// constants) and branch-free, so the U row for step j + 2 is in flight
// while step j computes. Codes and errors are kept by a select with a
// constant lane mask; w_hat and the row loss are formed once at the end.
//
// With B = 128 the block's share of the lazy-batch update inside its
// super-block can be taken here, left-looking: before the sweep, W_blk -=
// E[:, :kb] U[i0 - kb : i0, blk] for the kb columns of the super-block
// already quantized (fp32 MFMA, see near_update). That replaces the
// separate right-looking near-field launches.
#include "common.h"
#include "dma.h"
#include <utility>

namespace gq {

template <int O>
__device__ __forceinline__ float bcast16(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x150 + O, 0xF, 0xF, false));
}

// Reductions over the 16 lanes of a DPP row by rotations of 8, 4, 2, 1 (all
// lanes end with the full result; no LDS round trip)
template <int N>
__device__ __forceinline__ float ror16(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x120 + N, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_min16(float v) {
  v = fminf(v, ror16<8>(v));
  v = fminf(v, ror16<4>(v));
  v = fminf(v, ror16<2>(v));
  return fminf(v, ror16<1>(v));
}
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, ror16<8>(v));
  v = fmaxf(v, ror16<4>(v));
  v = fmaxf(v, ror16<2>(v));
  return fmaxf(v, ror16<1>(v));
}
__device__ __forceinline__ float row_sum16(float v) {
  v += ror16<8>(v);
  v += ror16<4>(v);
  v += ror16<2>(v);
  return v + ror16<1>(v);
}

// r = (lane is lane O of its 16-lane row) ? a : b, with the lane mask a
// compile-time constant in an SGPR pair (no per-step compare)
template <int O>
__device__ __forceinline__ float sel_owner(float a, float b) {
  constexpr uint64_t mask = 0x0001000100010001ull << O;
  float r;
  asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(b), "v"(a), "s"(mask));
  return r;
}

// LDS position of slot c of lane L in U row r: slots in groups of V =
// min(4, CPL), group-major, so a V-wide vector read by the 16 lanes of a row
// covers consecutive banks. The lane index is XOR-swizzled by the row and
// group parity: the prologue's scalar stores (4 columns of one row per
// thread) then hit 64 distinct banks per instruction, and each row read is
// still a permutation of whole chunks.
template <int CPL>
__device__ __forceinline__ constexpr int upos(int r, int c, int L) {
  constexpr int V = CPL < 4 ? CPL : 4;
  const int g = c / V;
  const int sw = (r & 1) | ((g & 1) << 1);
  return r * 16 * CPL + g * 16 * V + V * (L ^ sw) + (c % V);
}

template <int CPL>
struct SweepState {
  float w[CPL];
  float ev[CPL];       // e of the lane's columns (0 until decided)
  float qv[CPL];       // codes as floats
  float gs[CPL], gz[CPL];   // (s, z) of each slot's group, for w_hat at the end
  float un[3][CPL];    // U rows of steps j, j+1, j+2 (ring of three)
  float invn[3];       // 1 / U_jj for the same steps
  float s, inv_s, z;
  float nz, mz;        // -z and maxq - z: the clamp range of rint(w / s)
  int nc, gmask;   // columns in this block; group-1 when groups split the block, else -1
};

struct Grid {
  float s, z, inv_s;
};

// (s, z) from the current values of columns [lo, hi) of this block's row
// (the lane's slots) plus, when the group runs past the block, columns
// [i0 + B, i0 + hi) read from Wf. Groups are at least 8 columns wide, so
// inside a block this code is instantiated only at every 8th unrolled step.
template <int CPL, int LO>
__device__ __forceinline__ Grid group_start(const float (&w)[CPL], const SweepArgs& a, int L,
                                            int64_t row, bool row_ok, int hi, float maxq) {
  constexpr int B = 16 * CPL;
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int c = LO / 16; c < CPL; ++c) {
    const int col = 16 * c + L;
    if (col >= LO && col < hi) {
      mn = fminf(mn, w[c]);
      mx = fmaxf(mx, w[c]);
    }
  }
  if (hi > B && row_ok) {
    const float* p = a.Wf + row * a.ldw + a.i0;
    for (int col = B + L; col < hi; col += 16) {
      const float v = p[col];
      mn = fminf(mn, v);
      mx = fmaxf(mx, v);
    }
  }
  mn = row_min16(mn);
  mx = row_max16(mx);
  float xmin = fminf(mn, 0.f), xmax = fmaxf(mx, 0.f);
  Grid g;
  if (a.sym) {
    // symmetric alphabet {-A..A}: s = max|v| / A, codes q + A (z = A)
    const float A = 0.5f * (maxq - 1.f);
    float amax = fmaxf(-xmin, xmax);
    if (amax == 0.f) amax = 1.f;
    g.s = amax / A;
  } else {
    if (xmin == xmax) {
      xmin = -1.f;
      xmax = 1.f;
    }
    g.s = (xmax - xmin) / maxq;
  }
  if (a.scale16) {
    // binary16 scale precision: round to nearest even; a scale that rounds
    // to 0 takes the smallest subnormal 2^-24
    const float s16 = static_cast<float>(static_cast<_Float16>(g.s));
    g.s = s16 > 0.f ? s16 : 5.9604644775390625e-8f;
  }
  g.z = a.sym ? 0.5f * (maxq - 1.f) : rintf(-xmin / g.s);
  g.inv_s = 1.f / g.s;
  if (row_ok && L == 0) {
    const int64_t gi = a.gbase + (LO >> a.gshift);
    a.scales[row * a.ngroups + gi] = g.s;
    a.zeros[row * a.ngroups + gi] = (uint8_t)g.z;
  }
  return g;
}

template <int CPL, int LO>
__device__ __forceinline__ void start_group(SweepState<CPL>& S, const SweepArgs& a, int L, int64_t row,
                                            bool row_ok, float maxq) {
  const int hi = LO + a.group;
  const Grid g = group_start<CPL, LO>(S.w, a, L, row, row_ok, hi, maxq);
  S.s = g.s;
  S.z = g.z;
  S.inv_s = g.inv_s;
  S.nz = -g.z;
  S.mz = (a.sym ? maxq - 1.f : maxq) - g.z;   // the largest code: 2A on the symmetric alphabet
#pragma unroll
  for (int c = LO / 16; c < CPL; ++c) {
    const int col = 16 * c + L;
    const bool in = col >= LO && col < hi;
    S.gs[c] = in ? g.s : S.gs[c];
    S.gz[c] = in ? g.z : S.gz[c];
  }
}

// U row j (slots c >= C0 only; earlier slots are finished for every lane)
template <int CPL, int P, int C0>
__device__ __forceinline__ void load_urow(SweepState<CPL>& S, const float* sU, const float* sInv, int L,
                                          int j) {
  constexpr int V = CPL < 4 ? CPL : 4;
#pragma unroll
  for (int g = C0 / V; g < CPL / V; ++g) {
    const float* p = sU + upos<CPL>(j, g * V, L);
    if constexpr (V == 4) {
      const float4 u = *reinterpret_cast<const float4*>(p);
      S.un[P][4 * g] = u.x; S.un[P][4 * g + 1] = u.y; S.un[P][4 * g + 2] = u.z; S.un[P][4 * g + 3] = u.w;
    } else {
      const float2 u = *reinterpret_cast<const float2*>(p);
      S.un[P][2 * g] = u.x; S.un[P][2 * g + 1] = u.y;
    }
  }
  S.invn[P] = sInv[j];
}

template <int CPL, int J>
__device__ __forceinline__ void sweep_step(SweepState<CPL>& S, const SweepArgs& a, const float* sU,
                                           const float* sInv, int L, int64_t row, bool row_ok, float maxq) {
  constexpr int B = 16 * CPL;
  constexpr int O = J % 16, C = J / 16;   // owner lane and slot of column J
  constexpr int C0 = (J + 1) / 16;        // first slot with a column after J
  if constexpr (J > 0 && (J % 8) == 0) {
    if (J < S.nc && (J & S.gmask) == 0) start_group<CPL, J>(S, a, L, row, row_ok, maxq);
  }
  constexpr int P = J % 3;
  if constexpr (J + 2 < B) load_urow<CPL, (J + 2) % 3, (J + 3) / 16>(S, sU, sInv, L, J + 2);
  // keep those reads here (two steps ahead of their use): only ALU work may
  // be scheduled across this point
  __builtin_amdgcn_sched_barrier(0x407);
  const float* u = S.un[P];
  const float invd = S.invn[P];
  // q - z = clamp(rint(w / s), -z, maxq - z) exactly (z is an integer), so
  // the dependent chain is mul, round, med3, fma, mul
  const float wj = bcast16<O>(S.w[C]);
  const float qz = __builtin_amdgcn_fmed3f(rintf(wj * S.inv_s), S.nz, S.mz);
  const float e = fmaf(-S.s, qz, wj) * invd;   // (w - s (q - z)) / U_jj
  const float q = qz + S.z;
#pragma unroll
  for (int c = C0; c < CPL; ++c) S.w[c] = fmaf(-e, u[c], S.w[c]);
  S.qv[C] = sel_owner<O>(q, S.qv[C]);
  S.ev[C] = sel_owner<O>(e, S.ev[C]);
}

template <int CPL, int... Js>
__device__ __forceinline__ void sweep_all(SweepState<CPL>& S, const SweepArgs& a, const float* sU,
                                          const float* sInv, int L, int64_t row, bool row_ok, float maxq,
                                          std::integer_sequence<int, Js...>) {
  (sweep_step<CPL, Js>(S, a, sU, sInv, L, row, row_ok, maxq), ...);
}


// ---------------------------------------------------------------- near field
// upd[16][128] = E[rows, :kb] U[i0 - kb : i0, i0 : i0 + 128] for this
// workgroup's 16 rows (kb = 32 NCH, at most 384). E's rows and the first
// kNearDepth 32-row chunks of U are requested up front and every later
// chunk kNearDepth chunks ahead (four 16-byte pieces per thread, held in
// registers; one wave per SIMD leaves room for them), so the chunks do not
// each wait a full L2 round trip. They pass through a double buffer in
// LDS. Wave w computes columns 32w..32w+31 as two v_mfma_f32_16x16x4f32
// tiles; for MFMA t of a group of four, lane group g = lane / 16 feeds k =
// 16p + 4g + t to both operands (E as one 16-byte read, U as four 4-byte
// reads).
constexpr int kNearMax = 384;   // largest kb: a 512-column super-block
constexpr int kNearEP = kNearMax + 4;
constexpr int kNearUP = 128 + 4;
constexpr int kNearLds = 16 * kNearEP + 2 * 32 * kNearUP;   // floats (fits the U tile's region)
constexpr int kUpdP = 128 + 4;
constexpr int kNearDepth = 6;   // U chunks in flight

typedef float nf_f32x4_t __attribute__((ext_vector_type(4)));

struct NearCtx {
  float* sE;        // [16][kNearEP]
  float* sUc;       // [2][32][kNearUP]
  const float* src; // this thread's first piece of chunk 0
  int64_t ldu;
  int tid, li, g, w;
};

// The chunk index C is a template argument, so the ring slot C % kNearDepth
// is a compile-time index and the ring stays in registers.
template <int C, int NCH>
__device__ __forceinline__ void near_chunk(const NearCtx& x, nf_f32x4_t (&uc)[kNearDepth][4], nf_f32x4_t (&acc)[2]) {
  constexpr int cur = C & 1, slot = C % kNearDepth;
  float* dst = &x.sUc[(cur * 32 + (x.tid >> 5)) * kNearUP + 4 * (x.tid & 31)];
#pragma unroll
  for (int q = 0; q < 4; ++q) *reinterpret_cast<nf_f32x4_t*>(dst + 8 * q * kNearUP) = uc[slot][q];
  if constexpr (C + kNearDepth < NCH) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      uc[slot][q] = *reinterpret_cast<const nf_f32x4_t*>(x.src + (int64_t)(32 * (C + kNearDepth) + 8 * q) * x.ldu);
  }
  __syncthreads();   // chunk C (and, the first time, E) staged; buffer cur ^ 1 no longer read
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const float4 fa = *reinterpret_cast<const float4*>(&x.sE[x.li * kNearEP + 32 * C + 16 * p + 4 * x.g]);
    const float* ub = &x.sUc[(cur * 32 + 16 * p + 4 * x.g) * kNearUP + 32 * x.w + x.li];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const float* q = ub + 16 * ct;
      acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa.x, q[0], acc[ct], 0, 0, 0);
      acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa.y, q[kNearUP], acc[ct], 0, 0, 0);
      acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa.z, q[2 * kNearUP], acc[ct], 0, 0, 0);
      acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa.w, q[3 * kNearUP], acc[ct], 0, 0, 0);
    }
  }
}

template <int NCH, int... Cs>
__device__ __forceinline__ void near_chunks(const NearCtx& x, nf_f32x4_t (&uc)[kNearDepth][4], nf_f32x4_t (&acc)[2],
                                            std::integer_sequence<int, Cs...>) {
  (near_chunk<Cs, NCH>(x, uc, acc), ...);
}

template <int NCH>
__device__ __forceinline__ void near_update(const SweepArgs& a, float* stage, float* upd) {
  constexpr int kb = 32 * NCH;
  const int tid = threadIdx.x, lane = tid & 63;
  NearCtx x;
  x.tid = tid;
  x.w = tid >> 6;
  x.li = lane & 15;
  x.g = lane >> 4;
  x.sE = stage;
  x.sUc = stage + 16 * kNearEP;
  x.ldu = a.ldu;
  const int64_t r0 = (int64_t)blockIdx.x * 16;
  const float* Ub = a.U + (a.i0 - kb) * a.ldu + a.i0;
  x.src = Ub + (int64_t)(tid >> 5) * a.ldu + 4 * (tid & 31);
  // E rows (clamped to the last row; those results are never used)
  constexpr int q4 = kb / 4;                // float4 per E row
  constexpr int NE = (16 * q4 + 255) / 256;
  float4 ev[NE];
#pragma unroll
  for (int v = 0; v < NE; ++v) {
    const int idx = min(tid + 256 * v, 16 * q4 - 1);
    const int rr = idx / q4, k4 = idx % q4;
    const int64_t row = min(r0 + rr, a.d_out - 1);
    ev[v] = *reinterpret_cast<const float4*>(a.Esb + row * a.lde + 4 * k4);
  }
  nf_f32x4_t uc[kNearDepth][4];
#pragma unroll
  for (int c = 0; c < kNearDepth && c < NCH; ++c)
#pragma unroll
    for (int q = 0; q < 4; ++q) uc[c][q] = *reinterpret_cast<const nf_f32x4_t*>(x.src + (int64_t)(32 * c + 8 * q) * a.ldu);
#pragma unroll
  for (int v = 0; v < NE; ++v) {
    const int idx = tid + 256 * v;
    if (idx < 16 * q4) *reinterpret_cast<float4*>(&x.sE[(idx / q4) * kNearEP + 4 * (idx % q4)]) = ev[v];
  }
  nf_f32x4_t acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  near_chunks<NCH>(x, uc, acc, std::make_integer_sequence<int, NCH>{});
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int v = 0; v < 4; ++v) upd[(4 * x.g + v) * kUpdP + 32 * x.w + 16 * ct + x.li] = acc[ct][v];
  __syncthreads();   // the staging region is free again
}

// One wave per SIMD is all a d_out = 4096 layer provides (16 lanes per row),
// so the scheduler is told to favour latency over occupancy.
template <int CPL>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
k_sweep(SweepArgs a) {
  constexpr int B = 16 * CPL;
  constexpr bool kNear = CPL == 8;   // the fused near field (B = 128)
  static_assert(!kNear || kNearLds <= B * B, "near-field staging must fit the U tile's region");
  // one array, 1 / U_jj first: the per-step diagonal read then takes a
  // constant offset from a single base register
  __shared__ float smem[B + B * B + (kNear ? 16 * kUpdP : 0)];
  float* sInv = smem;
  float* sU = smem + B;
  float* upd = smem + B + B * B;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int L = lane & 15;
  const int64_t row = (int64_t)blockIdx.x * 16 + wave * 4 + (lane >> 4);
  const bool row_ok = row < a.d_out;
  const int nc = (int)a.ncols;
  const float maxq = (float)((1 << a.bits) - 1);

  // strictly-upper U tile of the block and 1 / U_jj (float4 loads; the
  // tile's rows start 16-byte aligned when ldu and i0 are multiples of 4)
  const float* Ublk = a.U + a.i0 * a.ldu + a.i0;
  const bool vec = ((a.ldu & 3) == 0) && ((a.i0 & 3) == 0) && (((uintptr_t)a.U & 15) == 0);
  constexpr int NV = B * B / 4 / 256;   // float4 per thread
  // issue every prologue load (U tile, its diagonal, this row's weights)
  // before the first store so the latencies overlap
  float ut[NV][4];
  if (vec && nc == B) {   // whole tile, aligned: no per-lane predicates
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int e4 = tid + 256 * v;
      const int r = e4 / (B / 4), c0 = 4 * (e4 % (B / 4));
      const float4 t = *reinterpret_cast<const float4*>(Ublk + (int64_t)r * a.ldu + c0);
      ut[v][0] = t.x; ut[v][1] = t.y; ut[v][2] = t.z; ut[v][3] = t.w;
    }
  } else {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int e4 = tid + 256 * v;
      const int r = e4 / (B / 4), c0 = 4 * (e4 % (B / 4));
      const float* src = Ublk + (int64_t)min(r, nc - 1) * a.ldu;
#pragma unroll
      for (int q = 0; q < 4; ++q) ut[v][q] = (r < nc && c0 + q < nc) ? src[min(c0 + q, nc - 1)] : 0.f;
    }
  }
  const float diag = (tid < B && tid < nc) ? Ublk[(int64_t)tid * a.ldu + tid] : 1.f;
  const float loss0 = (row_ok && L == 0) ? a.row_loss[row] : 0.f;
  SweepState<CPL> S;
  S.nc = nc;
  S.gmask = (a.group < B) ? a.group - 1 : -1;   // groups nest: a power of two below B
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int col = 16 * c + L;
    S.w[c] = (row_ok && col < nc) ? a.Wf[row * a.ldw + a.i0 + col] : 0.f;
    S.ev[c] = 0.f;
    S.qv[c] = 0.f;
  }
  // checked after the loads above are issued (they only read valid buffers):
  // nothing is stored when an earlier step failed
  if (a.st->flags != 0) return;
  // the in-super-block update runs while those loads are in flight
  const bool near = kNear && a.kb > 0;
  if (near) {
    // kb is 128, 256 or 384 (a multiple of the 128-column block)
    if (a.kb == 128) near_update<4>(a, sU, upd);
    else if (a.kb == 256) near_update<8>(a, sU, upd);
    else near_update<12>(a, sU, upd);   // each ends with a barrier: sU is free again
  }
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int e4 = tid + 256 * v;
    const int r = e4 / (B / 4), c0 = 4 * (e4 % (B / 4));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int col = c0 + q;
      sU[upos<CPL>(r, col / 16, col % 16)] = (col > r) ? ut[v][q] : 0.f;
    }
  }
  if (tid < B) sInv[tid] = tid < nc ? 1.f / diag : 0.f;
  __syncthreads();
  if (near) {
    const float* ur = upd + (wave * 4 + (lane >> 4)) * kUpdP + L;
#pragma unroll
    for (int c = 0; c < CPL; ++c) S.w[c] -= ur[16 * c];
  }

  if ((a.i0 % a.group) == 0) {
    start_group<CPL, 0>(S, a, L, row, row_ok, maxq);
  } else {
    const int64_t gi = a.gbase;
    S.s = row_ok ? a.scales[row * a.ngroups + gi] : 1.f;
    S.z = row_ok ? (float)a.zeros[row * a.ngroups + gi] : 0.f;
    S.inv_s = 1.f / S.s;
    S.nz = -S.z;
    S.mz = (a.sym ? maxq - 1.f : maxq) - S.z;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      S.gs[c] = S.s;
      S.gz[c] = S.z;
    }
  }

  load_urow<CPL, 0, 0>(S, sU, sInv, L, 0);
  load_urow<CPL, 1, 0>(S, sU, sInv, L, 1);
  sweep_all<CPL>(S, a, sU, sInv, L, row, row_ok, maxq, std::make_integer_sequence<int, B>{});

  float loss = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) loss = fmaf(S.ev[c], S.ev[c], loss);
  loss = row_sum16(loss);
  if (row_ok) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int col = 16 * c + L;
      if (col < nc) {
        a.Wf[row * a.ldw + a.i0 + col] = S.gs[c] * (S.qv[c] - S.gz[c]);
        a.codes[row * a.n_quant + a.i0 + col] = (uint8_t)S.qv[c];
      }
      a.E[row * a.lde + col] = S.ev[c];
      if (a.Ehi) {
        const uint16_t h = f32_to_bf16_rne(S.ev[c]);
        const int64_t o = eh_index(row, a.ehcol + col, a.ldeh);
        a.Ehi[o] = h;
        a.Elo[o] = f32_to_bf16_rne(S.ev[c] - bf16_to_f32(h));
      }
    }
    if (L == 0) a.row_loss[row] = loss0 + loss;
  }
}

// A whole super-block of the fused path in one launch (B = 128, whole
// blocks, groups inside a block): each workgroup keeps its 16 rows for the
// super-block's blocks b = 0 .. ncols / 128 - 1, with the same arithmetic,
// in the same order, as one k_sweep<8> launch per block. Block b + 1's U
// tile, diagonal and weights are requested before block b's chain starts,
// so their latency hides behind it (they are not written in this launch:
// the weights of later blocks change only through the near field below).
// Block b + 1's near field reads the errors this workgroup stored for
// blocks 0..b; the workgroup barrier after each block orders those stores
// before the reads (all waves of a workgroup share one CU and its L1).
// The prefetch needs a wave's whole register file (one workgroup per CU):
// layers with more rows than one round of that (4096) take PF = false,
// which requests each block's operands at its own start and fits two
// workgroups per CU, so one's waits are covered by the other's work.
template <bool PF>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(PF ? 1 : 2, PF ? 1 : 2)))
k_sweep_sb(SweepArgs a) {
  constexpr int CPL = 8, B = 128;
  constexpr int NV = B * B / 4 / 256;   // float4 of the U tile per thread
  __shared__ float smem[B + B * B + 16 * kUpdP];
  float* sInv = smem;
  float* sU = smem + B;
  float* upd = smem + B + B * B;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int L = lane & 15;
  const int64_t row = (int64_t)blockIdx.x * 16 + wave * 4 + (lane >> 4);
  const bool row_ok = row < a.d_out;
  const float maxq = (float)((1 << a.bits) - 1);
  const int64_t s0 = a.i0;
  const int nblk = (int)(a.ncols / B);

  float ut[NV][4];
  float dg;
  float wn[CPL];
  // U tile, 1 / U_jj source and this row's weights of the block at i0 (the
  // launcher guarantees 16-byte aligned tile rows)
  auto fetch = [&](int64_t i0) {
    const float* Ublk = a.U + i0 * a.ldu + i0;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int e4 = tid + 256 * v;
      const int r = e4 / (B / 4), c0 = 4 * (e4 % (B / 4));
      const float4 t = *reinterpret_cast<const float4*>(Ublk + (int64_t)r * a.ldu + c0);
      ut[v][0] = t.x; ut[v][1] = t.y; ut[v][2] = t.z; ut[v][3] = t.w;
    }
    dg = tid < B ? Ublk[(int64_t)tid * a.ldu + tid] : 1.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) wn[c] = row_ok ? a.Wf[row * a.ldw + i0 + 16 * c + L] : 0.f;
  };
  if (PF) fetch(s0);
  float lossacc = (row_ok && L == 0) ? a.row_loss[row] : 0.f;
  if (a.st->flags != 0) return;

  SweepState<CPL> S;
  S.nc = B;
  S.gmask = (a.group < B) ? a.group - 1 : -1;
  for (int b = 0; b < nblk; ++b) {
    SweepArgs ab = a;
    const int64_t i0 = s0 + (int64_t)b * B;
    ab.i0 = i0;
    ab.kb = (int64_t)b * B;
    ab.gbase = a.gbase + (int64_t)b * (B / a.group);
    if (b == 1) near_update<4>(ab, sU, upd);
    else if (b == 2) near_update<8>(ab, sU, upd);
    else if (b == 3) near_update<12>(ab, sU, upd);   // each ends with a barrier: sU is free again
    // without the prefetch, this block's operands are requested after its
    // near field, so they are not live across that field's register ring
    if (!PF) fetch(i0);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      S.w[c] = wn[c];
      S.ev[c] = 0.f;
      S.qv[c] = 0.f;
    }
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int e4 = tid + 256 * v;
      const int r = e4 / (B / 4), c0 = 4 * (e4 % (B / 4));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = c0 + q;
        sU[upos<CPL>(r, col / 16, col % 16)] = (col > r) ? ut[v][q] : 0.f;
      }
    }
    if (tid < B) sInv[tid] = 1.f / dg;
    __syncthreads();
    if (b > 0) {
      const float* ur = upd + (wave * 4 + (lane >> 4)) * kUpdP + L;
#pragma unroll
      for (int c = 0; c < CPL; ++c) S.w[c] -= ur[16 * c];
    }
    start_group<CPL, 0>(S, ab, L, row, row_ok, maxq);
    if (PF && b + 1 < nblk) fetch(i0 + B);

    load_urow<CPL, 0, 0>(S, sU, sInv, L, 0);
    load_urow<CPL, 1, 0>(S, sU, sInv, L, 1);
    sweep_all<CPL>(S, ab, sU, sInv, L, row, row_ok, maxq, std::make_integer_sequence<int, B>{});

    float loss = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) loss = fmaf(S.ev[c], S.ev[c], loss);
    lossacc += row_sum16(loss);
    if (row_ok) {
      float* Eb = a.E + ab.kb;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int col = 16 * c + L;
        a.Wf[row * a.ldw + i0 + col] = S.gs[c] * (S.qv[c] - S.gz[c]);
        a.codes[row * a.n_quant + i0 + col] = (uint8_t)S.qv[c];
        Eb[row * a.lde + col] = S.ev[c];
        if (a.Ehi) {
          const uint16_t h = f32_to_bf16_rne(S.ev[c]);
          const int64_t o = eh_index(row, a.ehcol + ab.kb + col, a.ldeh);
          a.Ehi[o] = h;
          a.Elo[o] = f32_to_bf16_rne(S.ev[c] - bf16_to_f32(h));
        }
      }
    }
    // every wave is done with sU, and this block's errors are stored,
    // before the next near field stages its operands over sU and reads them
    if (b + 1 < nblk) __syncthreads();
  }
  if (row_ok && L == 0) a.row_loss[row] = lossacc;
}

hipError_t launch_sweep_super(hipStream_t s, const SweepArgs& a) {
  if (a.d_out == 0 || a.ncols == 0) return hipSuccess;
  if (a.block != 128 || a.ncols % 128 != 0 || a.ncols > 512 || a.group > 128 || 128 % a.group != 0 ||
      a.i0 % 128 != 0 || a.ldu % 4 != 0 || ((uintptr_t)a.U & 15) != 0 || a.Esb != a.E)
    return hipErrorInvalidValue;
  const int64_t wgs = ceil_div(a.d_out, 16);
  if (wgs <= 256)
    hipLaunchKernelGGL(k_sweep_sb<true>, dim3((unsigned)wgs), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_sweep_sb<false>, dim3((unsigned)wgs), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sweep(hipStream_t s, const SweepArgs& a) {
  if (a.d_out == 0 || a.ncols == 0) return hipSuccess;
  dim3 grid((unsigned)ceil_div(a.d_out, 16));
  switch (a.block) {
    case 32: hipLaunchKernelGGL(k_sweep<2>, grid, dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL(k_sweep<4>, grid, dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL(k_sweep<8>, grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gq
