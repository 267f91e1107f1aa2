// Internal declarations shared by the HIP translation units of libgptq.
// Each .hip file owns its kernels and exposes host-side launchers; the C ABI
// in gptq_abi.cpp only calls launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace gq {

// Device-side status written by kernels: flags (bit 0: not positive
// definite, bit 1: non-finite input) and the smallest
// ORIGINAL column that raised it.
struct DevStatus {
  int flags;
  int pad;
  unsigned long long col;
};
constexpr int kNotPD = 1;
constexpr int kNonFinite = 2;

__device__ inline void raise_status(DevStatus* st, int flag, long long col) {
  atomicOr(&st->flags, flag);
  atomicMin(&st->col, (unsigned long long)col);
}

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---- hessian.hip
// Token-chunk splits used for n x n fp32 partials (fixed per (T, n)).
int hessian_splits(int64_t T, int64_t n);
hipError_t launch_hessian_partials_bf16(hipStream_t s, const uint16_t* X, int64_t T,
                                        int64_t n, int64_t ldx, float* part, int splits);
hipError_t launch_hessian_partials_f32(hipStream_t s, const float* X, int64_t T,
                                       int64_t n, int64_t ldx, float* part, int splits);
hipError_t launch_hessian_reduce(hipStream_t s, const float* part, int splits, int64_t n,
                                 float* H, int zero_first);

// ---- prep.hip
hipError_t launch_fill_f32(hipStream_t s, float* p, size_t count, float v);
hipError_t launch_prep_diag(hipStream_t s, const float* H, int64_t n, float* diag,
                            double* lam_out, float damp, DevStatus* st);
hipError_t launch_order(hipStream_t s, const float* diag, int64_t n, int64_t n_quant,
                        int act_order, int32_t* perm, int32_t* invperm);
hipError_t launch_build_flipped(hipStream_t s, const float* H, int64_t n, const int32_t* perm,
                                const float* diag, const double* lam, float* A,
                                DevStatus* st);
hipError_t launch_w_prep(hipStream_t s, const void* W, int wdt_bf16, int64_t d_out,
                         int64_t n, int64_t ldw, const int32_t* perm, float* Wf,
                         DevStatus* st);
hipError_t launch_status_init(hipStream_t s, DevStatus* st);

// ---- factor.hip
constexpr int kLeaf = 64;
hipError_t launch_leaf(hipStream_t s, float* A, float* X, int64_t n, int64_t off, int64_t m,
                       const int32_t* perm, DevStatus* st);
// L21 = A21 D^T in place for a 64-column panel (r rows, row pitch ld).
hipError_t launch_panel_solve(hipStream_t s, float* A21, const float* D, int64_t ld, int64_t r);
// The next diagonal block's update and leaf, run beside a trailing update.
struct LeafTask {
  const float* L21;      // rows k1.., columns of panel k (row pitch n)
  float* A;              // flipped matrix (lower part used)
  float* X;              // L^{-1} being built
  int64_t n, k1;
  int m2, mk;            // next block size, panel-k width
  const int32_t* perm;
  DevStatus* st;
};

// C[M x N] = alpha * op(A) * op(B) + beta * C, fp32 MFMA.
//  ta: A stored K x M (element (m,k) at A[k*lda + m]) instead of M x K
//  tb: B stored N x K (element (k,n) at B[n*ldb + k]) instead of K x N
//  kmode: 0 full K; 1 k < (column-tile end); 2 k >= (column-tile start);
//         3 k < (row-tile end); 4 k >= (row-tile start)
//         (triangular operands whose other part is zero)
//  lower_only: skip tiles strictly above the diagonal (square tiles)
//  batch: number of independent instances; instance b uses A + b*sA,
//         B + b*sB, C + b*sC (batch 0 is treated as 1)
struct GemmArgs {
  int64_t M, N, K;
  const float* A; int64_t lda; int ta;
  const float* B; int64_t ldb; int tb;
  float* C; int64_t ldc;
  float alpha, beta;
  int kmode, lower_only;
  int batch;
  int64_t sA, sB, sC;
};
hipError_t launch_gemm_f32(hipStream_t s, const GemmArgs& g);
hipError_t launch_gemm_pair(hipStream_t s, const GemmArgs& a, const GemmArgs* b);
// lower tiles of C = beta C + alpha A A^T (M == N, B == A, ta = 0, tb = 1)
hipError_t launch_syrk_f32(hipStream_t s, const GemmArgs& g);

// ---- syrk.hip
// Lower tiles of C (N x N, ldc) -= A A^T for fp32 A (N x K, lda) on the bf16
// matrix cores at fp32 accuracy (three bf16 pieces per value, six piece
// products). `pieces` is scratch of syrk_x6_pieces(N, K) bf16 (16-byte
// aligned): the pieces of N rows rounded up to a whole 128-row block.
bool syrk_x6_ok(int64_t N, int64_t K, int64_t lda, const float* A, int64_t ldc, const float* C);
int64_t syrk_x6_pieces(int64_t N, int64_t K);
hipError_t launch_syrk_x6(hipStream_t s, const float* A, int64_t lda, float* C, int64_t ldc, int64_t N,
                          int64_t K, uint16_t* pieces);
// The same six-product scheme for a batch of general products
//   C_b (M x N) = alpha op(A_b) B_b^T  over the k that kmode leaves
// (kmode 0: all k; 3: k < m0 + 128; 4: k >= m0, m0 the first row of a
// 128-row tile: the zero triangles of a triangular operand are skipped).
// An operand is given as fp32 rows of K values (or, when trans, as K rows of
// M values read down their columns). x6_split writes both operands' pieces
// into scratch of (x6_op_elems(M, K) + x6_op_elems(N, K)) * batch bf16 at
// `pieces`; x6_product then reads them there.
struct X6Operand {
  const float* src; int64_t ld, stride;   // instance b at src + b * stride
  int trans;                              // element (r, k) at src[k * ld + r]
};
__host__ __device__ int64_t x6_op_elems(int64_t rows, int64_t K);
hipError_t x6_split(hipStream_t s, int64_t M, int64_t N, int64_t K, int batch, const X6Operand& a,
                    const X6Operand& b, uint16_t* pieces);
hipError_t x6_product(hipStream_t s, int64_t M, int64_t N, int64_t K, int batch, float* C, int64_t ldc,
                      int64_t sC, float alpha, int kmode, const uint16_t* pieces);
// U = X with both indices reversed; if hi is non-null, also U's split-bf16
// parts hi = bf16(U), lo = bf16(U - hi).
hipError_t launch_rotate(hipStream_t s, const float* X, float* U, int64_t n, uint16_t* hi = nullptr,
                         uint16_t* lo = nullptr);

// ---- slab.hip
// C[M x N] = alpha A[M x K] B + beta C for 1 <= K <= 128 (B: K x N, or N x K
// when tb). With lower_only, only columns j <= i + lower_off are needed
// (whole 16-column pieces above that band are skipped). C must not alias A
// or B.
struct SlabArgs {
  int64_t M, N, K;
  const float* A; int64_t lda;
  const float* B; int64_t ldb; int tb;
  float* C; int64_t ldc;
  float alpha, beta;
  int lower_only;
  int64_t lower_off;
};
hipError_t launch_slab(hipStream_t s, const SlabArgs& g);
// The 64 x 64 tiles of C that the lower band needs, row-major: row tile rt
// holds column tiles 0 .. min(nct, rt + d) - 1, d = (63 + lower_off) / 64 + 1
// (d = nct without the band); rows from rs on are full, ps tiles precede
// them.
struct BandTiles {
  int nrt, nct, d, rs;
  int64_t ps, total;
};
inline BandTiles band_tiles(int64_t M, int64_t N, int lower_only, int64_t lower_off) {
  BandTiles b;
  b.nrt = (int)ceil_div(M, 64);
  b.nct = (int)ceil_div(N, 64);
  const int64_t d = lower_only ? (63 + lower_off) / 64 + 1 : (int64_t)b.nct;
  b.d = (int)(d < b.nct ? d : b.nct);
  const int rs = b.nct - b.d;
  b.rs = rs < 0 ? 0 : (rs > b.nrt ? b.nrt : rs);
  b.ps = (int64_t)b.rs * (b.rs - 1) / 2 + (int64_t)b.d * b.rs;
  b.total = b.ps + (int64_t)(b.nrt - b.rs) * b.nct;
  return b;
}
// launch_slab (K <= 64) plus one more workgroup (dispatched first) running `lt`.
hipError_t launch_slab_leaf(hipStream_t s, const SlabArgs& g, const LeafTask& lt);

// ---- trail.hip
// E's split-bf16 parts (the far field's A operand) are stored tiled, in the
// order the far field's LDS stages hold them: for each block of kEhRows rows
// and each 16-column slice of the ld columns, a kEhRows x 16 block (8 KiB),
// row-major. Element (row, col) of a tiled matrix with ld columns (ld a
// multiple of 16) is at eh_index(row, col, ld); the last row block is
// allocated whole.
constexpr int64_t kEhRows = 256;
__host__ __device__ inline int64_t eh_index(int64_t row, int64_t col, int64_t ld) {
  return ((row / kEhRows) * (ld / 16) + col / 16) * (kEhRows * 16) + (row % kEhRows) * 16 + col % 16;
}
__host__ __device__ inline int64_t eh_elems(int64_t rows, int64_t ld) {
  return (rows + kEhRows - 1) / kEhRows * kEhRows * ld;
}

// C[M x N] -= (Ahi + Alo)(Bhi + Blo) without the lo*lo term: split-bf16
// products, fp32 accumulation. A is M x K, tiled with lda columns (see
// eh_index; columns from 0); B is K x N (row-major, ldb), all bf16 bits.
// Requires lda a multiple of 16, ldb, N and K multiples of 8 and 16-byte
// aligned A/B bases (hipErrorInvalidValue otherwise).
struct TrailArgs {
  int64_t M, N, K;
  const uint16_t *Ahi, *Alo; int64_t lda;
  const uint16_t *Bhi, *Blo; int64_t ldb;
  float* C; int64_t ldc;
};
hipError_t launch_trail_x3(hipStream_t s, const TrailArgs& g);

// ---- sweep.hip
struct SweepArgs {
  float* Wf; int64_t ldw;       // d_out x n working weights (processing order)
  const float* U; int64_t ldu;  // n x n upper factor
  int64_t d_out, i0, ncols;     // block [i0, i0 + ncols)
  int block;                    // B
  int group, bits;
  int sym;                      // 1: symmetric alphabet {-A..A}, z = A = 2^(bits-1) - 1
  int scale16;                  // 1: group scales rounded to binary16 before use
  int64_t gbase;                // group index of column i0
  int gshift;                   // log2(group) when groups split a block, else 31
  float* scales; uint8_t* zeros; int64_t ngroups;
  uint8_t* codes; int64_t n_quant;   // processing order, d_out x n_quant
  float* E; int64_t lde;        // d_out x B block errors (row pitch lde)
  // fused near field (B = 128 only): W_blk -= Esb[:, :kb] U[i0 - kb : i0, blk]
  // before the sweep; Esb is the super-block's error matrix (pitch lde),
  // kb = 128, 256 or 384; 0 = none
  const float* Esb; int64_t kb;
  float* row_loss;
  // if non-null, E's split-bf16 parts are written there, tiled with ldeh
  // columns (eh_index), this launch's column 0 at column ehcol
  uint16_t *Ehi, *Elo;
  int64_t ldeh, ehcol;
  const DevStatus* st;
};
hipError_t launch_sweep(hipStream_t s, const SweepArgs& a);
// the fused path's whole super-block [i0, i0 + ncols) in one launch (B = 128,
// ncols a multiple of 128 up to 512, groups inside a block, E == Esb)
hipError_t launch_sweep_super(hipStream_t s, const SweepArgs& a);

// ---- pack.hip
hipError_t launch_pack(hipStream_t s, const uint8_t* codes, int64_t ldc, const int32_t* invperm,
                       int64_t d_out, int64_t n_quant, int bits, uint32_t* qweight);
hipError_t launch_unpack(hipStream_t s, const uint32_t* qweight, int64_t d_out, int64_t n_quant,
                         int bits, uint8_t* codes);
// round-to-nearest on the quantizer's affine grid, groups along rows (2 <= bits <= 8)
hipError_t launch_rtn(hipStream_t s, const float* X, int64_t ldx, int64_t rows, int64_t cols, int bits, int group,
                      uint8_t* codes, float* scales, uint8_t* zeros, float* xh);
hipError_t launch_finish(hipStream_t s, const float* Wf, const uint8_t* codes_p,
                         const int32_t* invperm, int64_t d_out, int64_t n, int64_t n_quant,
                         int group, float* w_hat, uint8_t* codes_out, int32_t* g_idx);

// ---- dqmm.hip: Y = X W_hat^T from the packed codes (inference)
struct DqPlan {
  int decode;                // 1: the 16-token kernel (16 x 16 x 32 MFMA, 8 chunks in flight)
  int mb;                    // 32-row blocks of X per workgroup: 1, 2 or 4
  int64_t mtiles, otiles;    // workgroups along M and along d_out
  int64_t groups_per_split, splits;
  size_t part_bytes;         // fp32 partials when splits > 1
};
DqPlan dequant_mm_plan(int64_t M, int64_t n, int64_t d_out, int bits, int group);
hipError_t launch_group_order(hipStream_t s, const int32_t* g_idx, int64_t n, int group, int32_t* perm);
hipError_t launch_gather_cols(hipStream_t s, const uint16_t* X, int64_t M, int64_t ldx, int64_t n,
                              const int32_t* perm, uint16_t* Xp);
hipError_t launch_dequant_mm(hipStream_t s, const DqPlan& p, const uint16_t* X, int64_t M, int64_t n,
                             int64_t ldx, const uint32_t* qw, const float* scales, const uint8_t* zeros,
                             int64_t d_out, int bits, int group, float* Y, int64_t ldy, float* part);

// ---- eora.hip: rank-r compensation of a layer's error
hipError_t launch_eora_delta(hipStream_t s, const void* W, int wbf16, int64_t ldw, const float* Wh,
                             int64_t d_out, int64_t n, float* D, DevStatus* st);
hipError_t launch_eora_start(hipStream_t s, float* Om, int64_t d, int k);
hipError_t launch_col_normalize(hipStream_t s, float* Y, int64_t d, int k);
hipError_t launch_sum_partials(hipStream_t s, const float* part, int np, int64_t count, float* C);
// eigenvalues (descending) and eigenvectors (columns, same order) of the
// symmetric part of the k x k matrix S; k even, 2 <= k <= 128
hipError_t launch_sym_eig_jacobi(hipStream_t s, const float* S, int k, float* theta, float* V);
hipError_t launch_eora_finish(hipStream_t s, const float* theta, int r, float* sigma, float* B, int64_t d,
                              int64_t ldb, float* A, int64_t n);

// ---- bidup.hip: coordinate descent over codes on a fixed grid
hipError_t launch_bidup_block(hipStream_t s, const float* G, int64_t n, const float* H, uint8_t* codes,
                              const float* scales, const int32_t* g_idx, int64_t ngroups,
                              int64_t d_out, int64_t j0, int nb, int bits, float* Delta);
hipError_t launch_bid_residual(hipStream_t s, const float* T, const uint8_t* codes, const float* scales,
                               const uint8_t* zeros, const int32_t* g_idx, int64_t ngroups, int64_t d_out,
                               int64_t n, float* D);

}  // namespace gq
