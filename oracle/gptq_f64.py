"""GPTQ in plain float64 numpy: the definition the GPU path is checked against.

TEST INFRASTRUCTURE (see the package docstring): only tests, the smoke check
and the benchmark's CPU-baseline leg use this module.

What the pages fix
------------------
* Objective: choose low-precision weights that minimise the squared Frobenius
  norm of the layer-output difference over calibration inputs X
  ([GIL] "Declaración del Problema"; [EORA] "Bucear en el espacio propio").
* GPTQ uses second-order (Hessian) information of that loss, quantizes the
  weight matrix column by column and, after each column, updates the columns
  not yet quantized with a closed-form correction derived from Optimal Brain
  Quantization; it picks the weights to quantize greedily
  ([GPTQ] "Enfoque Técnico").
* Weights are split into groups, each with its own scale ([GPTQ] "Enfoque
  Técnico"); the format is uniform affine with a scale and a zero point
  ([BAL] section 1).
* Standard GPTQ factorises the regularised Hessian by Cholesky with a
  regularisation parameter lambda ([GIL] "Metodología" 2, "Detalles de
  Implementación").
* The augmented variant appends full-precision columns to the calibration
  matrix and zero weights to W; the appended coordinates are not quantized
  and absorb the error feedback ([GIL] "Metodología" 2, "Hessiano Aumentado",
  "Optimización Conjunta").

Readings where the pages are silent (each applies everywhere below)
------------------------------------------------------------------
R1  H = 2 X^T X, unnormalised, full symmetric.
R2  lambda = damp * mean(diag H) over all n diagonal entries; H_d = H + lambda I.
R3  A zero diagonal entry of H is set to 1 before ordering and damping.
R4  Group range: min-max of the group's current values, widened to include 0;
    no clipping search; a degenerate range (min == max) becomes (-1, +1).
R5  Integer zero point z = rint(-xmin / s), scale s = (xmax - xmin) / maxq.
R6  q = clamp(rint(w / s) + z, 0, maxq) with rint = round half to even;
    reconstruction s * (q - z).
R7  A group is one output row times g consecutive columns in processing order;
    its (s, z) are taken when the sweep reaches its first column, from the
    error-updated values at that moment.
R8  n_quant % g == 0 and (g % B == 0 or B % g == 0).
R9  act-order: stable sort of the (dead-fixed) diagonal in descending order
    over the first n_quant columns; appended columns keep their place.
R10 Columns n_quant..n-1 (augmented) are never rounded; they keep the
    feedback they receive and are returned in full precision.

Orientation: W is d_out x n (PyTorch Linear layout), X is T x n, the layer
output is X W^T and the sweep runs over the n input columns of W.
"""
import numpy as np


# ---------------------------------------------------------------------------
# Step 1: Hessian
# ---------------------------------------------------------------------------
def hessian(X, chunk=8192, out=None):
    """H = 2 X^T X in float64, summed over token chunks (R1).

    [GPTQ] "Enfoque Técnico": second-order information of the layer loss;
    [BAL] section 2: the output error depends on the second-order statistics
    of the input. ``X`` may be any float array (bf16 values given as float32
    upcast exactly); ``out`` lets a caller stream further chunks into one H.
    """
    X = np.asarray(X)
    n = X.shape[1]
    H = np.zeros((n, n), np.float64) if out is None else out
    for t0 in range(0, X.shape[0], chunk):
        Xc = X[t0:t0 + chunk].astype(np.float64)
        H += 2.0 * (Xc.T @ Xc)
    return H


# ---------------------------------------------------------------------------
# Step 2: prepare (dead columns, order, damping)
# ---------------------------------------------------------------------------
def prepare(H, damp, act_order=False, n_quant=None):
    """Return (H_d, perm): the damped Hessian in processing order.

    R3 dead columns, R9 greedy order ([GPTQ] "Enfoque Técnico": weights are
    picked greedily), R2 damping ([GIL] "Detalles de Implementación": the
    standard method regularises with lambda before the Cholesky).
    ``perm[p]`` is the original column processed at position p.
    """
    H = np.array(H, dtype=np.float64, copy=True)
    n = H.shape[0]
    nq = n if n_quant is None else int(n_quant)
    d = np.diagonal(H).copy()
    dead = d == 0.0
    H[dead, dead] = 1.0
    perm = np.arange(n)
    if act_order:
        d = np.diagonal(H)
        perm[:nq] = np.argsort(-d[:nq], kind="stable")
    H = H[np.ix_(perm, perm)]
    lam = damp * np.mean(np.diagonal(H))
    H[np.diag_indices(n)] += lam
    return H, perm


def upper_chol_of_inverse(Hd):
    """U upper triangular with U^T U = H_d^{-1} (the Cholesky factor the sweep
    uses; [GIL] "Detalles de Implementación"). LAPACK via numpy."""
    G = np.linalg.inv(Hd)
    G = 0.5 * (G + G.T)
    L = np.linalg.cholesky(G)        # G = L L^T, L lower
    return L.T


def upper_chol_of_inverse_by_reversal(Hd):
    """The same factor U (upper, U^T U = H_d^{-1}) from one Cholesky of H_d
    with its indices reversed, for layers too wide for an explicit inverse
    (about a third of the flops of inv + cholesky).

    With J the index reversal, J H_d J = L L^T (L lower, LAPACK dpotrf) gives
    H_d^{-1} = J L^{-T} L^{-1} J = (J L^{-1} J)^T (J L^{-1} J), and J L^{-1} J
    is upper triangular with a positive diagonal: it is the unique upper
    Cholesky factor of H_d^{-1}. L^{-1} is LAPACK dtrtri.
    """
    from scipy.linalg import lapack
    n = Hd.shape[0]
    # Hd[::-1, ::-1].T is J H_d J read in Fortran order (H_d is symmetric)
    A = np.array(np.asarray(Hd, np.float64)[::-1, ::-1], order="F", copy=True)
    L, info = lapack.dpotrf(A, lower=1, clean=1, overwrite_a=1)
    del A
    if info != 0:
        raise np.linalg.LinAlgError(f"damped Hessian not positive definite (dpotrf info {info})")
    Li, info = lapack.dtrtri(L, lower=1, overwrite_c=1)
    del L
    if info != 0:
        raise np.linalg.LinAlgError(f"dtrtri info {info}")
    return np.ascontiguousarray(Li[::-1, ::-1]).reshape(n, n)


# ---------------------------------------------------------------------------
# The quantization grid ([BAL] section 1; R4-R6)
# ---------------------------------------------------------------------------
def round_fp16(s):
    """(s16, t, ulp): positive values rounded to IEEE binary16 (10 fraction
    bits, round to nearest, ties to even), from the format's definition.
    The binade of s is 2^e with e = floor(log2 s) (exact, through frexp),
    held at -14 below the normal range, where the subnormals share the
    spacing 2^-24; ulp = 2^(e - 10), t = s / ulp is the value the rounding
    decides on and s16 = rint(t) ulp ("El balance de errores de la
    inferencia de pocos bits", section 1: the precision of the scales is
    part of the format). Reading: a value that rounds to 0 takes the
    smallest subnormal, 2^-24, so that a group always has a positive
    scale."""
    s = np.asarray(s, np.float64)
    _, ex = np.frexp(s)
    e = np.maximum(ex - 1, -14).astype(np.float64)
    ulp = np.exp2(e - 10.0)
    t = s / ulp
    s16 = np.rint(t) * ulp
    return np.where(s16 == 0.0, 2.0 ** -24, s16), t, ulp


def group_grid(v, maxq, sym=False, scale_fp16=False, alt_scale_rows=None):
    """Per-row (s, z, zpre, smargin) from the group's current values ``v``
    (rows x g).

    zpre = -xmin / s is the value rint() decides the zero point from.
    scale_fp16: the scale is rounded to binary16 (round_fp16) before it is
    used, and smargin is that rounding's tie distance in binary16 steps
    (0.5 without the option: no decision); the rows in alt_scale_rows take
    the other binary16 neighbour (the other branch of a scale tie). The
    zero point and the codes use the rounded scale.

    sym: the symmetric alphabet {-A, ..., A} with A = (maxq - 1) / 2 =
    2^(b-1) - 1 levels on each side of zero ("Resumen Técnico:
    GPTQ-intrinsic LoRA", "Límites Inferiores de la Teoría de la
    Información": a finite integer alphabet of size 2B + 1). Reading: the
    scale maps the group's largest magnitude to A, s = max|v| / A (a group
    of zeros takes max|v| = 1, as the affine rule takes the range (-1, 1));
    codes are stored as q + A, i.e. with the fixed zero point z = A, so the
    reconstruction s (code - z) and the packing stay those of the affine
    format. zpre is A itself (no rounding decision).
    """
    xmin = np.minimum(v.min(axis=1), 0.0)
    xmax = np.maximum(v.max(axis=1), 0.0)
    if sym:
        A = (maxq - 1.0) / 2.0
        amax = np.maximum(-xmin, xmax)
        amax = np.where(amax == 0.0, 1.0, amax)
        s = amax / A
    else:
        same = xmin == xmax
        xmin = np.where(same, -1.0, xmin)
        xmax = np.where(same, 1.0, xmax)
        s = (xmax - xmin) / maxq
    smargin = np.full_like(s, 0.5)
    if scale_fp16:
        s16, t, ulp = round_fp16(s)
        if alt_scale_rows:
            rows = list(alt_scale_rows)
            s16[rows] = np.maximum(other_neighbour(t[rows]), 1.0) * ulp[rows]
        s = s16
        smargin = tie_distance(t)
    if sym:
        z = np.full_like(s, A)
        return s, z, z.copy(), smargin
    zpre = -xmin / s
    z = np.rint(zpre)
    return s, z, zpre, smargin


def code_top(maxq, sym):
    """Largest code: maxq on the affine grid, 2A = maxq - 1 on the symmetric
    alphabet (codes q + A for q in {-A..A}; a value pushed past A by the
    feedback clamps to A)."""
    return maxq - 1.0 if sym else maxq


def quantize_column(w, s, z, maxq):
    """(q, w_hat, pre): q = clamp(rint(w/s) + z, 0, maxq), w_hat = s (q - z),
    pre = w / s (the value the rounding decides on)."""
    pre = w / s
    q = np.clip(np.rint(pre) + z, 0.0, maxq)
    return q, s * (q - z), pre


def other_neighbour(x):
    """The integer next to ``x`` on the far side from rint(x): the rounding
    a decision takes when it goes the other way at a tie."""
    r = np.rint(x)
    return np.where(x >= r, r + 1.0, r - 1.0)


def tie_distance(pre):
    """Distance of a pre-rounding value to the nearest half-integer, in
    quantization steps (0 means an exact tie)."""
    f = pre - np.floor(pre)
    return np.abs(f - 0.5)


def _check_params(n, bits, group, block, n_quant):
    if bits not in (2, 3, 4):
        raise ValueError("bits must be 2, 3 or 4")
    if not (1 <= n_quant <= n):
        raise ValueError("n_quant out of range")
    if n_quant % group != 0:
        raise ValueError("group must divide n_quant (R8)")
    if block is not None and not (group % block == 0 or block % group == 0):
        raise ValueError("group and block must nest (R8)")


def _finish(W, Wp, perm, codes_p, scales, zeros, loss, n_quant, group,
            margins, zmargins, smargins):
    d_out, n = W.shape
    w_hat = np.empty_like(Wp)
    w_hat[:, perm] = Wp
    codes = np.empty((d_out, n_quant), np.uint8)
    codes[:, perm[:n_quant]] = codes_p
    g_idx = np.empty(n_quant, np.int32)
    g_idx[perm[:n_quant]] = np.arange(n_quant) // group
    return dict(codes=codes, scales=scales, zeros=zeros.astype(np.uint8),
                g_idx=g_idx, w_hat=w_hat, row_loss=loss, perm=perm,
                codes_proc=codes_p, margins=margins, zmargins=zmargins, smargins=smargins)


# ---------------------------------------------------------------------------
# O2: Cholesky of the inverse + lazy batches (the scalable form)
# ---------------------------------------------------------------------------
def gptq_o2(W, H, bits=4, group=128, damp=0.01, block=128, act_order=False,
            n_quant=None, U=None, perm=None, alt=None, sym=False, scale_fp16=False):
    """GPTQ sweep with the upper Cholesky factor U of H_d^{-1} and lazy
    batches of ``block`` columns ([GPTQ] "Enfoque Técnico"; [GIL]
    "Detalles de Implementación").

    Per row, in processing order, for column j: at a group start take (s, z)
    from the current values (R7); round (R6); e_j = (w_j - w_hat_j) / U_jj;
    subtract e_j U[j, k] from every later column k of the same block at once,
    and the whole block's E U[block, rest] from the later columns after the
    block. Columns >= n_quant only receive feedback (R10).

    ``U``/``perm`` may be passed in to reuse a factorisation (the oracle
    still computes them with :func:`prepare` and LAPACK).
    ``alt`` = (codes, zeros[, scales]), collections of (row, processing
    position) and (row, group) pairs whose rounding takes the other
    neighbour of its pre-rounding value instead of the nearest one: the
    other branch of a decision that sits at a tie, where either rounding is
    correct at the precision of the inputs. Everything after such a
    decision follows from it by the same rules.
    ``scale_fp16``: scales rounded to binary16 before use (group_grid).
    Returns codes (original order), scales/zeros (group order), g_idx,
    w_hat, row_loss = sum_j e_j^2, and the tie distances of every decision.
    """
    W = np.asarray(W, np.float64)
    d_out, n = W.shape
    nq = n if n_quant is None else int(n_quant)
    _check_params(n, bits, group, block, nq)
    maxq = float(2 ** bits - 1)
    qtop = code_top(maxq, sym)
    if U is None:
        Hd, perm = prepare(H, damp, act_order, nq)
        U = upper_chol_of_inverse(Hd)
    Wp = W[:, perm].copy()
    ng = nq // group
    codes = np.zeros((d_out, nq), np.uint8)
    scales = np.zeros((d_out, ng))
    zeros = np.zeros((d_out, ng))
    margins = np.zeros((d_out, nq))
    zmargins = np.zeros((d_out, ng))
    smargins = np.zeros((d_out, ng))
    loss = np.zeros(d_out)
    alt_c, alt_z, alt_s = {}, {}, {}
    for src, dst in zip(alt or ((), (), ()), (alt_c, alt_z, alt_s)):
        for r, k in src:
            dst.setdefault(int(k), []).append(int(r))
    s = z = None
    for i0 in range(0, nq, block):
        i1 = min(i0 + block, nq)
        E = np.zeros((d_out, i1 - i0))
        for j in range(i0, i1):
            if j % group == 0:
                s, z, zpre, smg = group_grid(Wp[:, j:j + group], maxq, sym, scale_fp16,
                                             alt_s.get(j // group))
                rz = alt_z.get(j // group)
                if rz:
                    z[rz] = np.clip(other_neighbour(zpre[rz]), 0.0, qtop)
                scales[:, j // group] = s
                zeros[:, j // group] = z
                zmargins[:, j // group] = tie_distance(zpre)
                smargins[:, j // group] = smg
            q, what, pre = quantize_column(Wp[:, j], s, z, qtop)
            rc = alt_c.get(j)
            if rc:
                q[rc] = np.clip(other_neighbour(pre[rc]) + z[rc], 0.0, qtop)
                what[rc] = s[rc] * (q[rc] - z[rc])
            e = (Wp[:, j] - what) / U[j, j]
            Wp[:, j + 1:i1] -= np.outer(e, U[j, j + 1:i1])
            Wp[:, j] = what
            E[:, j - i0] = e
            loss += e * e
            codes[:, j] = q.astype(np.uint8)
            margins[:, j] = tie_distance(pre)
        Wp[:, i1:] -= E @ U[i0:i1, i1:]
    return _finish(W, Wp, perm, codes, scales, zeros, loss, nq, group,
                   margins, zmargins, smargins)


# ---------------------------------------------------------------------------
# O1: the Optimal-Brain definition with explicit inverse downdates
# ---------------------------------------------------------------------------
def gptq_o1(W, H, bits=4, group=128, damp=0.01, act_order=False, n_quant=None, sym=False,
            scale_fp16=False):
    """Column-by-column OBS form, eager updates ([GPTQ] "Enfoque Técnico").

    G is the inverse of H_d restricted to the columns not yet quantized.
    Quantizing column j with error delta moves the remaining weights by
    -delta / G_00 * G_0,rest (the closed-form optimal correction), adds
    delta^2 / G_00 to the row loss, and G loses its first row and column by
    the Schur-complement downdate G' = G_rr - G_r0 G_0r / G_00.
    O(n^3) per layer: meant for n up to a few hundred.
    """
    W = np.asarray(W, np.float64)
    d_out, n = W.shape
    nq = n if n_quant is None else int(n_quant)
    _check_params(n, bits, group, None, nq)
    maxq = float(2 ** bits - 1)
    qtop = code_top(maxq, sym)
    Hd, perm = prepare(H, damp, act_order, nq)
    G = np.linalg.inv(Hd)
    Wp = W[:, perm].copy()
    ng = nq // group
    codes = np.zeros((d_out, nq), np.uint8)
    scales = np.zeros((d_out, ng))
    zeros = np.zeros((d_out, ng))
    margins = np.zeros((d_out, nq))
    zmargins = np.zeros((d_out, ng))
    smargins = np.zeros((d_out, ng))
    loss = np.zeros(d_out)
    s = z = None
    for j in range(nq):
        if j % group == 0:
            s, z, zpre, smg = group_grid(Wp[:, j:j + group], maxq, sym, scale_fp16)
            scales[:, j // group] = s
            zeros[:, j // group] = z
            zmargins[:, j // group] = tie_distance(zpre)
            smargins[:, j // group] = smg
        q, what, pre = quantize_column(Wp[:, j], s, z, qtop)
        g00 = G[0, 0]
        delta = Wp[:, j] - what
        Wp[:, j + 1:] -= np.outer(delta / g00, G[0, 1:])
        Wp[:, j] = what
        loss += delta * delta / g00
        codes[:, j] = q.astype(np.uint8)
        margins[:, j] = tie_distance(pre)
        G = G[1:, 1:] - np.outer(G[1:, 0], G[0, 1:]) / g00
    return _finish(W, Wp, perm, codes, scales, zeros, loss, nq, group,
                   margins, zmargins, smargins)


# ---------------------------------------------------------------------------
# Round-to-nearest and brute force
# ---------------------------------------------------------------------------
def rtn(W, bits=4, group=128, sym=False, scale_fp16=False):
    """Round-to-nearest on the same grid rules (R4-R6), no feedback: the
    baseline GPTQ is compared with ([GPTQ] "Rendimiento y Precisión")."""
    W = np.asarray(W, np.float64)
    d_out, n = W.shape
    maxq = float(2 ** bits - 1)
    qtop = code_top(maxq, sym)
    ng = n // group
    codes = np.zeros((d_out, n), np.uint8)
    w_hat = np.zeros_like(W)
    scales = np.zeros((d_out, ng))
    zeros = np.zeros((d_out, ng))
    for gi in range(ng):
        sl = slice(gi * group, (gi + 1) * group)
        s, z, _, _ = group_grid(W[:, sl], maxq, sym, scale_fp16)
        scales[:, gi] = s
        zeros[:, gi] = z
        for j in range(sl.start, sl.stop):
            q, what, _ = quantize_column(W[:, j], s, z, qtop)
            codes[:, j] = q.astype(np.uint8)
            w_hat[:, j] = what
    return dict(codes=codes, w_hat=w_hat, scales=scales,
                zeros=zeros.astype(np.uint8))


def row_objective(w, w_hat, H):
    """(w - w_hat)^T H (w - w_hat) for each row: the per-row term of the
    layer objective ([GIL] "Declaración del Problema")."""
    D = np.atleast_2d(np.asarray(w, np.float64) - np.asarray(w_hat, np.float64))
    return ((D @ np.asarray(H, np.float64)) * D).sum(axis=1)


def brute_force_rows(W, H, s, z, bits):
    """Exhaustive minimum of the per-row objective over every code vector on
    the fixed per-row grid (s, z): tiny n only (4^n candidates at 2 bits)."""
    W = np.asarray(W, np.float64)
    d_out, n = W.shape
    levels = np.arange(2 ** bits, dtype=np.float64)
    grids = np.stack(np.meshgrid(*([levels] * n), indexing="ij"), -1).reshape(-1, n)
    best = np.zeros(d_out)
    best_q = np.zeros((d_out, n))
    for r in range(d_out):
        cand = s[r] * (grids - z[r])
        obj = row_objective(np.broadcast_to(W[r], cand.shape), cand, H)
        k = int(np.argmin(obj))
        best[r] = obj[k]
        best_q[r] = grids[k]
    return best, best_q


def layer_error(W, W_hat, H):
    """r = tr(D H D^T) / tr(W H W^T), D = W - W_hat, undamped H: the relative
    layer reconstruction error ||X (W - W_hat)^T||^2 / ||X W^T||^2
    ([GIL] "Declaración del Problema")."""
    W = np.asarray(W, np.float64)
    H = np.asarray(H, np.float64)
    num = row_objective(W, W_hat, H).sum()
    den = row_objective(W, np.zeros_like(W), H).sum()
    return float(num / den)
