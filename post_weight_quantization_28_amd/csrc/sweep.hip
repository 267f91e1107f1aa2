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
struct SweepState {
  float w[CPL];
  float ev[CPL];
  uint32_t qv[CPL];
  float s, inv_s, z, loss;
};

// (s, z) from the current values of columns [lo, hi) of this block's row
// (registers) plus, when the group runs past the block, columns
// [i0 + B, i0 + hi) read from Wf.
template <int CPL>
__device__ inline void group_start(SweepState<CPL>& S, const SweepArgs& a, int L, int64_t row,
                                   bool row_ok, int lo, int hi, float maxq) {
  constexpr int B = 16 * CPL;
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int col = L * CPL + c;
    if (col >= lo && col < hi) {
      mn = fminf(mn, S.w[c]);
      mx = fmaxf(mx, S.w[c]);
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
  S.s = (xmax - xmin) / maxq;
  S.z = rintf(-xmin / S.s);
  S.inv_s = 1.f / S.s;
  if (row_ok && L == 0) {
    const int64_t gi = (a.i0 + lo) / a.group;
    a.scales[row * a.ngroups + gi] = S.s;
    a.zeros[row * a.ngroups + gi] = (uint8_t)S.z;
  }
}

template <int CPL, int J>
__device__ inline void sweep_step(SweepState<CPL>& S, const SweepArgs& a, const float (*sU)[16 * CPL],
                                  const float* sInv, int L, int64_t row, bool row_ok, float maxq) {
  constexpr int O = J / CPL, C = J % CPL;
  if (J >= a.ncols) return;
  if (J > 0 && ((a.i0 + J) % a.group) == 0) group_start<CPL>(S, a, L, row, row_ok, J, J + a.group, maxq);
  const float wj = bcast16<O>(S.w[C]);
  const float q = fminf(fmaxf(rintf(wj * S.inv_s) + S.z, 0.f), maxq);
  const float what = S.s * (q - S.z);
  const float e = (wj - what) * sInv[J];
  S.loss = fmaf(e, e, S.loss);
  const float* ur = &sU[J][L * CPL];
#pragma unroll
  for (int c = 0; c < CPL; c += 2) {
    const float2 u = *reinterpret_cast<const float2*>(ur + c);
    S.w[c + 0] = fmaf(-e, u.x, S.w[c + 0]);
    S.w[c + 1] = fmaf(-e, u.y, S.w[c + 1]);
  }
  if (L == O) {
    S.w[C] = what;
    S.qv[C] = (uint32_t)q;
    S.ev[C] = e;
  }
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

  // strictly-upper U tile of the block and 1 / U_jj
  for (int e = tid; e < B * B; e += 256) {
    const int r = e / B, c = e % B;
    float v = 0.f;
    if (c > r && c < nc) v = a.U[(a.i0 + r) * a.ldu + a.i0 + c];
    sU[r][c] = v;
  }
  for (int r = tid; r < B; r += 256) sInv[r] = r < nc ? 1.f / a.U[(a.i0 + r) * a.ldu + a.i0 + r] : 0.f;

  SweepState<CPL> S;
  S.loss = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int col = L * CPL + c;
    S.w[c] = (row_ok && col < nc) ? a.Wf[row * a.ldw + a.i0 + col] : 0.f;
    S.ev[c] = 0.f;
    S.qv[c] = 0;
  }
  __syncthreads();

  if ((a.i0 % a.group) == 0) {
    group_start<CPL>(S, a, L, row, row_ok, 0, a.group, maxq);
  } else {
    const int64_t gi = a.i0 / a.group;
    S.s = row_ok ? a.scales[row * a.ngroups + gi] : 1.f;
    S.z = row_ok ? (float)a.zeros[row * a.ngroups + gi] : 0.f;
    S.inv_s = 1.f / S.s;
  }

  sweep_all<CPL>(S, a, sU, sInv, L, row, row_ok, maxq, std::make_integer_sequence<int, B>{});

  if (row_ok) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int col = L * CPL + c;
      if (col < nc) {
        a.Wf[row * a.ldw + a.i0 + col] = S.w[c];
        a.codes[row * a.n_quant + a.i0 + col] = (uint8_t)S.qv[c];
      }
      a.E[row * B + col] = S.ev[c];
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
