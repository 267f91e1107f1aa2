/*
 * gptq.h - C ABI of the MI355X (gfx950) GPTQ layer quantizer.
 *
 * The method (pages cited by title and section):
 *  - "GPTQ" (wikiprompt.org), "Enfoque Técnico": second-order (Hessian)
 *    information of the layer loss; weight columns are quantized one at a
 *    time and the columns not yet quantized receive a closed-form correction
 *    derived from Optimal Brain Quantization; grouped quantization with a
 *    scale per group; 4, 3 and 2 bits.
 *  - "El balance de errores de la inferencia de pocos bits" (auturnal.com),
 *    section 1: uniform affine format with a scale and a zero point; a
 *    format must state its signed range, grouping direction, group size,
 *    scale precision, rounding rule, clipping method and packing layout.
 *  - "Resumen Técnico: GPTQ-intrinsic LoRA" (gist.science 2606.01412),
 *    "Declaración del Problema": the objective ||X W - X W_hat||_F^2 over a
 *    calibration matrix X; "Metodología" 2: standard GPTQ factorises the
 *    regularised Hessian by Cholesky with a parameter lambda, and the
 *    augmented variant appends full-precision columns that are never rounded.
 *
 * Format fixed by this library (the pages leave these open):
 *  - H = 2 X^T X, fp32, full symmetric n x n, row-major.
 *  - lambda = damp * mean(diag H); a zero diagonal entry is replaced by 1
 *    before ordering and damping.
 *  - groups: g consecutive columns of one output row, in processing order;
 *    range = [min(0, min v), max(0, max v)] of the group's current values
 *    when the sweep reaches its first column, (-1, 1) if degenerate; no
 *    clipping search. s = (xmax - xmin) / (2^b - 1) (fp32),
 *    z = rint(-xmin / s) stored as uint8 in [0, 2^b - 1],
 *    q = clamp(rint(w / s) + z, 0, 2^b - 1), rint = round half to even,
 *    reconstruction s * (q - z). Codes are unsigned.
 *  - act_order: columns 0..n_quant-1 processed by descending diag(H)
 *    (stable); columns n_quant..n-1 stay last.
 *  - packing: per row, code k (original column order) occupies bits
 *    [k*b, k*b + b) of an LSB-first stream of little-endian uint32 words;
 *    ceil(n_quant*b/32) words per row; codes may straddle two words.
 *
 * Conventions for every call:
 *  - Matrices are row-major. W is d_out x n (PyTorch Linear layout), X is
 *    T x n. All data pointers are DEVICE pointers owned by the caller; the
 *    library never allocates or frees device memory. Scratch memory is the
 *    caller's ``workspace`` (size from the matching *_workspace_bytes call,
 *    256-byte aligned base).
 *  - ``stream`` is a hipStream_t (NULL = the legacy default stream). Work is
 *    enqueued on it in order.
 *  - Argument errors return GPTQ_EINVAL before anything is enqueued.
 *  - HIP launch or runtime errors return GPTQ_EHIP; gptq_last_error() gives
 *    the text (thread-local).
 */
#ifndef GPTQ_MI355X_H
#define GPTQ_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GPTQ_OK = 0,
  GPTQ_EINVAL = -1,      /* bad argument; nothing enqueued */
  GPTQ_ENOTPD = -2,      /* damped Hessian not positive definite */
  GPTQ_ENONFINITE = -3,  /* NaN/Inf in W or H */
  GPTQ_EHIP = -4,        /* HIP runtime or launch failure */
  GPTQ_EWORKSPACE = -5   /* workspace NULL, misaligned or too small */
} gptq_status;

typedef enum { GPTQ_BF16 = 0, GPTQ_F32 = 1 } gptq_dtype;

typedef struct {
  uint32_t struct_size; /* sizeof(gptq_params); at least offsetof(sym); a
                           field is read only when struct_size covers it */
  int32_t bits;         /* 2, 3 or 4 */
  int32_t group;        /* g >= 8; n_quant % g == 0; g % block == 0 or block % g == 0 */
  float damp;           /* lambda = damp * mean(diag H); >= 0, finite */
  int32_t block;        /* lazy-batch width B: 32, 64 or 128 */
  int32_t act_order;    /* 0 or 1 */
  int64_t n_quant;      /* 1..n; columns n_quant..n-1 receive feedback only */
  int32_t sym;          /* 0: affine grid (scale and zero point per group);
                           1: symmetric alphabet {-A..A}, A = 2^(bits-1) - 1,
                           s = max|v| / A over the group's current values
                           (1 / A for a group of zeros), stored as codes
                           q + A with zeros = A. Read only when struct_size
                           covers it (older callers: 0). ("Resumen Técnico:
                           GPTQ-intrinsic LoRA": a finite integer alphabet of
                           size 2B + 1.) */
  int32_t scale_fp16;   /* 0: scales in fp32; 1: each group's scale is rounded
                           to binary16 (nearest, ties to even; 0 -> 2^-24)
                           before the zero point, the codes and w_hat use it,
                           so the fp32 scales output holds binary16 values
                           that convert exactly. Read only when struct_size
                           covers it (older callers: 0). ("El balance de
                           errores de la inferencia de pocos bits", section
                           1: the precision of the scales is part of the
                           format.) */
  int32_t reserved;     /* 0. (With it the block grew from 40 to 48 bytes, so a
                           caller built before scale_fp16 existed, whose
                           struct_size is 40, never has its padding read.) */
} gptq_params;

typedef struct {
  /* all device pointers, caller-allocated; NULL = not wanted (except where noted) */
  uint32_t *qweight; /* d_out x ceil(n_quant*bits/32) packed codes, original column order */
  uint8_t *codes;    /* d_out x n_quant unpacked codes, original column order */
  float *scales;     /* REQUIRED: d_out x (n_quant/group), group order (processing order) */
  uint8_t *zeros;    /* REQUIRED: d_out x (n_quant/group), integer zero points */
  int32_t *g_idx;    /* n_quant: group index of each original column */
  float *w_hat;      /* d_out x n: s*(q-z) for quantized columns, the fp32
                        feedback-updated values for columns >= n_quant;
                        original column order */
  float *row_loss;   /* d_out: sum over the row's columns of e_j^2,
                        e_j = (w_j - w_hat_j) / U_jj */
} gptq_outputs;

/* ---- Hessian accumulation ------------------------------------------------
 * H (n x n fp32, row-major, ld = n) += 2 X^T X, or H = 2 X^T X when
 * zero_first != 0. X: T x n, row stride ldx >= n elements, dtype xdt
 * (bf16 products are exact in fp32; accumulation is fp32, split over token
 * chunks and summed in a fixed order: results are bitwise reproducible).
 * H stays exactly symmetric. T == 0 only applies zero_first.
 * Asynchronous on ``stream``. Workspace: gptq_hessian_workspace_bytes.
 * ("GPTQ", "Enfoque Técnico": second-order information; factor 2 and fp32
 * storage are this library's convention.) */
gptq_status gptq_hessian_workspace_bytes(int64_t T, int64_t n, gptq_dtype xdt,
                                         size_t *bytes);
gptq_status gptq_accumulate_hessian(void *stream, const void *X, gptq_dtype xdt,
                                    int64_t T, int64_t n, int64_t ldx, float *H,
                                    int zero_first, void *workspace,
                                    size_t workspace_bytes);

/* ---- Layer quantization ----------------------------------------------------
 * GPTQ of W (d_out x n, dtype wdt, row stride ldw >= n) against H (n x n fp32,
 * symmetric, not modified). Steps: dead-column fix and damping, optional
 * act-order, upper Cholesky factor U of (H + lambda I)^-1 (U^T U = H_d^-1),
 * column sweep in blocks of B with in-block error feedback and a lazy-batch
 * trailing update, then un-permutation and packing.
 * Synchronises ``stream`` before returning to read the device status:
 * GPTQ_ENOTPD / GPTQ_ENONFINITE set *fail_col (if fail_col != NULL) to the
 * first offending ORIGINAL column (-1 if unknown); outputs are then
 * unspecified. d_out == 0 is a no-op.
 * Workspace: gptq_workspace_bytes(d_out, n, p) bytes, 256-byte aligned,
 * owned by the caller, not read before it is written (its contents on entry
 * do not matter). It holds the factorisation (two n x n fp32 matrices and
 * U's split-bf16 parts; for n >= 6144 also the bf16 pieces of one
 * 2048-column super-panel, and for the inverse's block products of 1024 or
 * more output tiles the pieces of the largest one's operands: 2.8 GB at
 * n = 28672), the fp32 working weights, one super-block of errors and the
 * processing-order codes.
 * ("GPTQ" (wikiprompt.org), "Enfoque Técnico": the columns are quantized in
 * turn and the columns not yet quantized get the closed-form Optimal Brain
 * Quantization correction, with groups of weights sharing a scale;
 * "El balance de errores de la inferencia de pocos bits", section 1: scale,
 * zero point, rounding and packing fields of the format; "Resumen Técnico:
 * GPTQ-intrinsic LoRA", "Detalles de Implementación": the Cholesky
 * factorisation of the lambda-regularised Hessian; "Metodología" 2: appended
 * columns n_quant..n-1 that absorb the feedback unrounded.) */
gptq_status gptq_workspace_bytes(int64_t d_out, int64_t n, const gptq_params *p,
                                 size_t *bytes);
gptq_status gptq_quantize_layer(void *stream, const void *W, gptq_dtype wdt,
                                int64_t d_out, int64_t n, int64_t ldw,
                                const float *H, const gptq_params *p,
                                void *workspace, size_t workspace_bytes,
                                const gptq_outputs *out, int64_t *fail_col);

/* ---- The factorisation alone (steps 2-3 of quantize_layer) ----------------
 * U_out (n x n fp32 row-major): upper Cholesky factor U of the inverse of
 * the damped, dead-fixed, (optionally) act-order-permuted H, in processing
 * order (U^T U = H_d^-1; strict lower part zero). perm_out (n int32, may be
 * NULL): original column at each processing position. Uses p->damp,
 * p->act_order and p->n_quant only; workspace: gptq_workspace_bytes(0, n, p).
 * Synchronises like quantize_layer.
 * ("Resumen Técnico: GPTQ-intrinsic LoRA", "Detalles de Implementación":
 * Cholesky of the regularised Hessian.) */
gptq_status gptq_factor_hinv(void *stream, const float *H, int64_t n,
                             const gptq_params *p, void *workspace,
                             size_t workspace_bytes, float *U_out,
                             int32_t *perm_out, int64_t *fail_col);

/* ---- Packing (the layout above) -------------------------------------------
 * codes: d_out x n_quant uint8 (values must be < 2^bits; higher bits are
 * masked off), qweight: d_out x ceil(n_quant*bits/32) uint32. Asynchronous. */
gptq_status gptq_pack_codes(void *stream, const uint8_t *codes, int64_t d_out,
                            int64_t n_quant, int32_t bits, uint32_t *qweight);
gptq_status gptq_unpack_codes(void *stream, const uint32_t *qweight,
                              int64_t d_out, int64_t n_quant, int32_t bits,
                              uint8_t *codes);

/* ---- Inference: dequantising product of a packed layer ---------------------
 * Y (M x d_out fp32, row pitch ldy >= d_out) = X W_hat^T for X (M x n, bf16
 * only: xdt must be GPTQ_BF16, row pitch ldx >= n with ldx % 8 == 0, 16-byte
 * aligned base) and W_hat[o][k] = scales[o][k/group] * (q[o][k] -
 * zeros[o][k/group]), the codes q read from qweight in the layout above
 * (d_out x n*bits/32 words, 16-byte aligned base, n_quant = n). Groups must
 * be contiguous in qweight's column order: a layer quantized without
 * act-order as it is, an act-order layer after gptq_repack_act_order (then
 * pass its perm). group must be a positive multiple of 32 that divides n.
 * Products of bf16 activations and the integers q - z are exact in fp32 and
 * each group's sum is scaled once (the weights are never rounded to bf16);
 * sums are fp32 in a fixed order, so results are bitwise reproducible.
 * Workspace: gptq_dequant_matmul_workspace_bytes (the gathered activations
 * when permuted, and fp32 partials when few output tiles split the groups;
 * 0 when neither applies).
 * Asynchronous on ``stream``. M == 0 or d_out == 0 enqueues nothing; n == 0
 * writes zeros.
 * ("El balance de errores de la inferencia de pocos bits", section 6: the
 * saving is realised by a kernel that unpacks, dequantises and multiplies;
 * decode and prefill are separate regimes. Section 1: reconstruction
 * s (q - z).) */
gptq_status gptq_dequant_matmul_workspace_bytes(int64_t M, int64_t n, int64_t d_out,
                                                int32_t bits, int32_t group,
                                                int32_t permuted, size_t *bytes);
/* perm: NULL, or n int32 column indices (see gptq_repack_act_order): the
 * product is then X[:, perm] W_hat^T with qweight, scales and zeros in that
 * column order; X is gathered into the workspace (permuted = 1 in the size
 * call), so its rows need no alignment then. */
gptq_status gptq_dequant_matmul(void *stream, const void *X, int32_t xdt, int64_t M,
                                int64_t n, int64_t ldx, const uint32_t *qweight,
                                const float *scales, const uint8_t *zeros,
                                const int32_t *perm, int64_t d_out, int32_t bits,
                                int32_t group, float *Y, int64_t ldy, void *workspace,
                                size_t ws_bytes);

/* ---- The product without a workspace -----------------------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, serving loops that must not call hipMalloc, harnesses that
 * forbid it. Same arguments, result and errors as gptq_dequant_matmul (the
 * same kernels, bit-identical Y), but its scratch (the gathered activations
 * of a permuted product, the fp32 partials of a split product) lives in a
 * static device array of GPTQ_NOALLOC_SCRATCH_BYTES that the library holds
 * on every GPU it runs on until the process ends; nothing is allocated or
 * freed. A product whose scratch, gptq_dequant_matmul_workspace_bytes(M, n,
 * d_out, bits, group, perm != NULL), exceeds that size returns GPTQ_EINVAL
 * before anything is enqueued. The array belongs to the current device
 * (hipGetDevice): ``stream`` must be a stream of that device. Every call on
 * one GPU shares that GPU's array, so calls that may overlap on one GPU
 * (concurrent streams, several host threads) race and give wrong results:
 * serialise them. The array keeps the last call's contents; every value a
 * call reads from it was written by the same call. */
#define GPTQ_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
gptq_status gptq_dequant_matmul_noalloc(void *stream, const void *X, int32_t xdt,
                                        int64_t M, int64_t n, int64_t ldx,
                                        const uint32_t *qweight, const float *scales,
                                        const uint8_t *zeros, const int32_t *perm,
                                        int64_t d_out, int32_t bits, int32_t group,
                                        float *Y, int64_t ldy);

/* ---- Act-order layers for the product ---------------------------------------
 * A layer quantized with act-order has, in the original column order, groups
 * that are not contiguous (g_idx). The product is invariant to one
 * permutation of the columns of both X and W_hat, so such a layer is used
 * through the order perm that lists group 0's columns, then group 1's, ...
 * (a stable sort of g_idx): perm_out (n int32) receives it, qweight_out (same
 * size as qweight) the codes repacked in that order, whose groups are then
 * contiguous and match scales and zeros as quantize_layer wrote them. g_idx
 * must give every group exactly `group` columns (as quantize_layer's does);
 * otherwise perm is not a permutation and the product is wrong (entries of a
 * short group stay 0; nothing is read out of bounds). Workspace:
 * gptq_repack_act_order_workspace_bytes (d_out x n bytes of codes).
 * Asynchronous. ("El balance de errores de la inferencia de pocos bits",
 * section 1: the grouping direction is part of the format.) */
gptq_status gptq_repack_act_order_workspace_bytes(int64_t d_out, int64_t n, size_t *bytes);
gptq_status gptq_repack_act_order(void *stream, const uint32_t *qweight,
                                  const int32_t *g_idx, int64_t d_out, int64_t n,
                                  int32_t bits, int32_t group, uint32_t *qweight_out,
                                  int32_t *perm_out, void *workspace, size_t ws_bytes);

/* ---- EoRA: rank-r compensation of the compression error ----------------------
 * B (d_out x rank fp32, row-major) and A (rank x n fp32, row-major) such that
 * W_hat + B A is the best rank-r correction of W_hat in the layer loss
 * tr((W - W_hat - B A) H (W - W_hat - B A)^T), and sigma (rank fp32,
 * descending) the singular values of the error projected into the
 * eigenspace of H. H == NULL: the plain SVD of W - W_hat (B = U_r Sigma_r,
 * A = V_r^T). W: d_out x n, dtype wdt, row stride ldw >= n; W_hat: d_out x n
 * fp32 (e.g. quantize_layer's w_hat); H: n x n fp32 symmetric (e.g. the
 * Hessian 2 X^T X). 1 <= rank <= min(64, d_out). The r largest eigenpairs of
 * D H D^T (D = W - W_hat) come from iters steps of block subspace iteration
 * (0: 24) on a block of min(rank + 64, 128) columns and a Rayleigh-Ritz
 * step; B A = U_r U_r^T D, B = U_r diag(sigma), A = diag(1/sigma) U_r^T D
 * (a zero sigma gives zero rows of A). Workspace:
 * gptq_eora_workspace_bytes(d_out, n, rank, H != NULL). Synchronises the
 * stream; GPTQ_ENONFINITE if W - W_hat or H is not finite.
 * ("Aumento de la precisión de LLM de 2 bits con EoRA" (7minutos.es), "Bucear
 * en el espacio propio en busca de un adaptador": the error projected by the
 * eigendecomposition of the activation covariance, truncated by SVD and
 * projected back; the plain-SVD adapter B = U Sigma, A = V^T beside it. Any
 * square root of H gives the same product B A as Q Lambda^{1/2}.) */
gptq_status gptq_eora_workspace_bytes(int64_t d_out, int64_t n, int32_t rank, int32_t with_h,
                                      size_t *bytes);
gptq_status gptq_eora(void *stream, const void *W, gptq_dtype wdt, const float *W_hat,
                      int64_t d_out, int64_t n, int64_t ldw, const float *H, int32_t rank,
                      int32_t iters, float *B, float *A, float *sigma, void *workspace,
                      size_t workspace_bytes);

/* ---- OLrC / Bid-Up refinement of a low-precision plus low-rank layer ---------
 * W ~ W_hat + B A with W_hat = s (q - z) the codes on a fixed grid: each of
 * `cycles` cycles first sets B (d_out x rank) and A (rank x n) to the best
 * rank-r correction of W - W_hat (OLrC: the computation of gptq_eora), then
 * runs `passes` Bid-Up passes over the codes for the target W - B A: the
 * columns in order, each code moved to the grid point nearest the minimiser
 * of tr((W - B A - W_hat) H (...)^T) along it, clamped to [0, 2^bits - 1]
 * (columns with H_jj <= 0 unchanged). Every step lowers or keeps the layer
 * error (up to fp32 rounding). codes: d_out x n uint8, in/out (e.g.
 * quantize_layer's codes); scales / zeros: d_out x (n / group) with g_idx (n
 * int32) mapping each column to its group, as quantize_layer writes them;
 * H: n x n fp32; W: d_out x n, dtype wdt, row stride ldw. Outputs B, A and,
 * if w_hat != NULL, the dequantised codes (d_out x n fp32). bits 2..8,
 * 1 <= rank <= min(64, d_out), cycles and passes 1..100. Workspace:
 * gptq_refine_workspace_bytes. Synchronises the stream.
 * ("Resumen Técnico: GPTQ-intrinsic LoRA", "Refinamiento Bid-Up": OLrC
 * optimises L and R for a fixed Q, Bid-Up optimises Q on the fixed grid by
 * coordinate updates; the alternation never increases the layer error.) */
gptq_status gptq_refine_workspace_bytes(int64_t d_out, int64_t n, int32_t rank, size_t *bytes);
gptq_status gptq_refine_lowrank(void *stream, const void *W, gptq_dtype wdt, int64_t d_out,
                                int64_t n, int64_t ldw, const float *H, int32_t bits,
                                int32_t group, const int32_t *g_idx, const float *scales,
                                const uint8_t *zeros, uint8_t *codes, int32_t rank,
                                int32_t cycles, int32_t passes, float *B, float *A,
                                float *w_hat, void *workspace, size_t workspace_bytes);

/* ---- Round-to-nearest on the same grid ---------------------------------------
 * codes (rows x cols uint8), scales / zeros (rows x cols/group fp32 / uint8)
 * and, if x_hat != NULL, x_hat = s (q - z) (rows x cols fp32) for X (rows x
 * cols fp32, row stride ldx): the quantizer's affine grid per group of
 * `group` consecutive columns of a row, with no error feedback. For the
 * low-rank factors of an adapter (B at 8 bits, A at 4 bits) and as the
 * round-to-nearest baseline. bits 2..8; group divides cols; rows <= 65535.
 * Asynchronous. ("Resumen Técnico: GPTQ-intrinsic LoRA", "Resultados
 * Clave": quantizing the low-rank factors L and R to 4 and 8 bits is often
 * lossless; "GPTQ", "Rendimiento y Precisión": round-to-nearest as the
 * baseline.) */
gptq_status gptq_quantize_rtn(void *stream, const float *X, int64_t rows, int64_t cols,
                              int64_t ldx, int32_t bits, int32_t group, uint8_t *codes,
                              float *scales, uint8_t *zeros, float *x_hat);

/* ---- Diagnostics ------------------------------------------------------------ */
const char *gptq_status_string(int status);
const char *gptq_last_error(void); /* thread-local detail of the last failure */

/* Timing with hipEvents recorded on the caller's stream: around the
 * Hessian Gram kernel, around the Hessian reduction, and around a whole
 * quantize_layer call (events are deliberately coarse: an event record
 * between every pair of small kernels costs microseconds of GPU time).
 * enable == 1 starts recording those (and clears what was recorded);
 * enable >= 2 also records the phases of quantize_layer: the factorisation
 * (preparation of H included), the W preparation and the final un-permute /
 * pack, every sweep launch (with its near-field update), every far-field
 * update, and every block product of the factorisation's inverse that runs
 * on the six-product bf16 kernel (the product alone, not its operand
 * splits; those products are also inside the factorisation's interval);
 * that adds a few microseconds per launch and is meant for one untimed
 * breakdown pass. The arrays given to gptq_profile_collect hold
 * GPTQ_PROF_NCLASSES entries. enable == 0 stops. gptq_profile_collect
 * synchronises the recorded events and returns, for class c in
 * [0, GPTQ_PROF_NCLASSES), the summed milliseconds and the number of timed
 * intervals, then clears. */
enum {
  GPTQ_PROF_HESSIAN_SYRK = 0,
  GPTQ_PROF_HESSIAN_REDUCE = 1,
  GPTQ_PROF_QUANTIZE = 2,
  GPTQ_PROF_FACTOR = 3,
  GPTQ_PROF_PREP_FINISH = 4,
  GPTQ_PROF_SWEEP = 5,
  GPTQ_PROF_FARFIELD = 6,
  GPTQ_PROF_INVERSE_X6 = 7,
  GPTQ_PROF_NCLASSES = 8
};
gptq_status gptq_profile_enable(int enable);
gptq_status gptq_profile_collect(double *ms, int64_t *count);

#ifdef __cplusplus
}
#endif
#endif /* GPTQ_MI355X_H */
