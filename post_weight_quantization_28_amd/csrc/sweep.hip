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
//   q_j = clamp(rint(w_j / s) + z, 0, maxq), w_hat_j = s (q_j - z)
//   e_j = (w_j - w_hat_j) / U_jj
//   w_k -= e_j U_jk for the later columns k of the block
// E (d_out x B) collects e_j for the trailing update of the later blocks.
//
// Layout (MI355X): a wavefront holds 4 rows; the 16 lanes of a DPP row own
// one weight row, CPL = B/16 consecutive columns each, in registers. The
// value being decided is broadcast to its 16 lanes with DPP row_newbcast
// (no LDS round trip), every lane rounds it redundantly and applies the
// rank-1 feedback to its own columns with U's row j read from LDS (the
// block's strictly-upper U tile, 64 KiB at B = 128, shared by the 16 rows of
// the workgroup). The loop over j is fully unrolled so the owner lane and
// the register slot are compile-time constants.
#include "common.h"
#include <utility>

namespace gq {

template <int O>
__device__ inline float bcast16(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + O, 0xF, 0xF, false));
}

__device__ inline float row_min16(float v) {
#pragma unroll
  for (int m = 8; m > 0; m >>= 1) v = fminf(v, __shfl_xor(v, m, 16));
  return v;
}
__device__ inline float row_max16(float v) {
#pragma unroll
  for (int m = 8; m > 0; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 16));
  return v;
}

template <int CPL>
struct Regs {
  float v[CPL];
};

template <int CPL>
struct SweepState {
  float w[CPL];
  float ev[CPL];
  uint32_t qv[CPL];
  float un[2][CPL];  // U rows, loaded one step ahead (even / odd steps)
  float invn[2];     // 1 / U_jj for the same steps
  float s, inv_s, z, loss;
  int nc, gmask;   // columns in this block; group-1 when groups split the block, else -1
};

struct Grid {
  float s, z, inv_s;
};

// (s, z) from the current values of columns [lo, hi) of this block's row
// (the lane's CPL registers, passed by value) plus, when the group runs past
// the block, columns [i0 + B, i0 + hi) read from Wf. Groups are at least 8
// columns wide, so inside a block this code is instantiated only at every
// 8th unrolled step (inlining it into every step would overflow the
// instruction cache).
template <int CPL>
__device__ __forceinline__ Grid group_start(const Regs<CPL>& w, const SweepArgs& a, int L,
                                            int64_t row, bool row_ok, int lo, int hi, float maxq) {
  constexpr int B = 16 * CPL;
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int col = L * CPL + c;
    if (col >= lo && col < hi) {
      mn = fminf(mn, w.v[c]);
      mx = fmaxf(mx, w.v[c]);
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
  if (xmin == xmax) {
    xmin = -1.f;
    xmax = 1.f;
  }
  Grid g;
  g.s = (xmax - xmin) / maxq;
  g.z = rintf(-xmin / g.s);
  g.inv_s = 1.f / g.s;
  if (row_ok && L == 0) {
    const int64_t gi = a.gbase + (lo >> a.gshift);
    a.scales[row * a.ngroups + gi] = g.s;
    a.zeros[row * a.ngroups + gi] = (uint8_t)g.z;
  }
  return g;
}

template <int CPL>
__device__ __forceinline__ void start_group(SweepState<CPL>& S, const SweepArgs& a, int L, int64_t row,
                                   bool row_ok, int lo, float maxq) {
  Regs<CPL> r;
#pragma unroll
  for (int c = 0; c < CPL; ++c) r.v[c] = S.w[c];
  const Grid g = group_start<CPL>(r, a, L, row, row_ok, lo, lo + a.group, maxq);
  S.s = g.s;
  S.z = g.z;
  S.inv_s = g.inv_s;
}

template <int CPL, int P>
__device__ __forceinline__ void load_urow(SweepState<CPL>& S, const float (*sU)[16 * CPL],
                                          const float* sInv, int L, int j) {
  const float* ur = &sU[j][L * CPL];
#pragma unroll
  for (int c = 0; c < CPL; c += 2) {
    const float2 u = *reinterpret_cast<const float2*>(ur + c);
    S.un[P][c] = u.x;
    S.un[P][c + 1] = u.y;
  }
  S.invn[P] = sInv[j];
}

template <int CPL, int J>
__device__ inline void sweep_step(SweepState<CPL>& S, const SweepArgs& a, const float (*sU)[16 * CPL],
                                  const float* sInv, int L, int64_t row, bool row_ok, float maxq) {
  constexpr int B = 16 * CPL;
  constexpr int O = J / CPL, C = J % CPL;
  if (J >= S.nc) return;
  if constexpr (J > 0 && (J % 8) == 0) {
    if ((J & S.gmask) == 0) start_group<CPL>(S, a, L, row, row_ok, J, maxq);
  }
  // this step's U row was loaded by the previous step; start the next load
  constexpr int P = J & 1;
  const float* u = S.un[P];
  const float invd = S.invn[P];
  if constexpr (J + 1 < B) load_urow<CPL, P ^ 1>(S, sU, sInv, L, J + 1);
  const float wj = bcast16<O>(S.w[C]);
  const float q = fminf(fmaxf(rintf(wj * S.inv_s) + S.z, 0.f), maxq);
  const float what = S.s * (q - S.z);
  const float e = (wj - what) * invd;
  S.loss = fmaf(e, e, S.loss);
#pragma unroll
  for (int c = 0; c < CPL; ++c) S.w[c] = fmaf(-e, u[c], S.w[c]);
  const bool own = L == O;
  S.w[C] = own ? what : S.w[C];
  S.qv[C] = own ? (uint32_t)q : S.qv[C];
  S.ev[C] = own ? e : S.ev[C];
}

template <int CPL, int... Js>
__device__ inline void sweep_all(SweepState<CPL>& S, const SweepArgs& a, const float (*sU)[16 * CPL],
                                 const float* sInv, int L, int64_t row, bool row_ok, float maxq,
                                 std::integer_sequence<int, Js...>) {
  (sweep_step<CPL, Js>(S, a, sU, sInv, L, row, row_ok, maxq), ...);
}

template <int CPL>
__global__ void __launch_bounds__(256)
k_sweep(SweepArgs a) {
  constexpr int B = 16 * CPL;
  __shared__ float sU[B][B];
  __shared__ float sInv[B];
  if (a.st->flags != 0) return;

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
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int e4 = tid + 256 * v;
    const int r = e4 / (B / 4), c0 = 4 * (e4 % (B / 4));
#pragma unroll
    for (int q = 0; q < 4; ++q) ut[v][q] = 0.f;
    if (r < nc) {
      const float* src = Ublk + (int64_t)r * a.ldu + c0;
      if (vec && c0 + 3 < nc) {
        const float4 t = *reinterpret_cast<const float4*>(src);
        ut[v][0] = t.x; ut[v][1] = t.y; ut[v][2] = t.z; ut[v][3] = t.w;
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) ut[v][q] = (c0 + q < nc) ? src[q] : 0.f;
      }
    }
  }
  const float diag = (tid < B && tid < nc) ? Ublk[(int64_t)tid * a.ldu + tid] : 1.f;
  SweepState<CPL> S;
  S.loss = 0.f;
  S.nc = nc;
  S.gmask = (a.group < B) ? a.group - 1 : -1;   // groups nest: a power of two below B
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int col = L * CPL + c;
    S.w[c] = (row_ok && col < nc) ? a.Wf[row * a.ldw + a.i0 + col] : 0.f;
    S.ev[c] = 0.f;
    S.qv[c] = 0;
  }
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int e4 = tid + 256 * v;
    const int r = e4 / (B / 4), c0 = 4 * (e4 % (B / 4));
#pragma unroll
    for (int q = 0; q < 4; ++q) sU[r][c0 + q] = (c0 + q > r) ? ut[v][q] : 0.f;
  }
  if (tid < B) sInv[tid] = tid < nc ? 1.f / diag : 0.f;
  __syncthreads();

  if ((a.i0 % a.group) == 0) {
    start_group<CPL>(S, a, L, row, row_ok, 0, maxq);
  } else {
    const int64_t gi = a.gbase;
    S.s = row_ok ? a.scales[row * a.ngroups + gi] : 1.f;
    S.z = row_ok ? (float)a.zeros[row * a.ngroups + gi] : 0.f;
    S.inv_s = 1.f / S.s;
  }

  load_urow<CPL, 0>(S, sU, sInv, L, 0);
  sweep_all<CPL>(S, a, sU, sInv, L, row, row_ok, maxq, std::make_integer_sequence<int, B>{});

  if (row_ok) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int col = L * CPL + c;
      if (col < nc) {
        a.Wf[row * a.ldw + a.i0 + col] = S.w[c];
        a.codes[row * a.n_quant + a.i0 + col] = (uint8_t)S.qv[c];
      }
      a.E[row * a.lde + col] = S.ev[c];
    }
    if (L == 0) a.row_loss[row] += S.loss;
  }
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
