"""Refinement of a low-precision plus low-rank layer W ~ Q + L R: OLrC and
Bid-Up cycles, in plain float64 numpy.

TEST INFRASTRUCTURE (see the package docstring): only tests, the smoke check
and the benchmark's CPU-baseline leg use this module.

What the page fixes ("Resumen Técnico: GPTQ-intrinsic LoRA" (gist.science
2606.01412), "Metodología" 4 "Refinamiento Bid-Up"; the objective from
"Declaración del Problema"):
  * the objective is the layer's reconstruction error
    ||X W - X (Q + L R)||_F^2 over the calibration matrix X;
  * OLrC (optimal low-rank compensation) optimises L and R for a fixed Q;
  * Bid-Up optimises Q for fixed L and R by coordinate updates on the
    fixed quantization grid;
  * the two alternate, and since every step minimises the objective over a
    subset of the variables (or over the fixed grid), the layer error never
    increases.
Readings:
  B1  Orientation: W is d_out x n, the layer output X W^T, so the objective
      is tr((W - W_hat - B A) H (W - W_hat - B A)^T) / 2 with H = 2 X^T X,
      W_hat = s (q - z) the dequantised codes, and the low-rank term B A
      (B d_out x r, A r x n). OLrC for a fixed W_hat is the unconstrained
      best rank-r B A for that loss: the EoRA problem on the error
      W - W_hat (oracle.eora), whose optimality is pinned there.
  B2  The grid stays fixed: each row's groups keep GPTQ's scale and zero
      point; a code is an integer in [0, 2^b - 1] (the affine grid).
  B3  A Bid-Up pass visits the columns in original order 0..n-1 (Gauss-
      Seidel); per row, coordinate j moves to the grid point nearest the
      one-dimensional minimiser: with target t = W - B A, residual
      d = t - W_hat and g = (d H)_j, the objective along q_j is a parabola
      with minimum at q_j + g / H_jj, so the new code is
      clamp(rint(c_j + g / (H_jj s)), 0, maxq), rint half to even (R6).
      A column with H_jj = 0 is left unchanged.
  B4  A cycle is OLrC, then Bid-Up (the page alternates them and starts
      from GPTQ-intrinsic LoRA's own Q, L, R, whose low-rank part is not
      yet optimal for its Q).
"""
import numpy as np

from . import eora as E
from . import gptq_f64 as O


def dequant(codes, scales, zeros, g_idx):
    """W_hat[r, j] = s[r, g] (q[r, j] - z[r, g]) with g = g_idx[j]."""
    g = np.asarray(g_idx)
    return np.asarray(scales, np.float64)[:, g] * (np.asarray(codes, np.float64) - np.asarray(zeros, np.float64)[:, g])


def objective(W, W_hat, H, B=None, A=None):
    """tr(R H R^T), R = W - W_hat - B A (B1)."""
    return E.layer_loss(W, W_hat, H, B, A)


def bidup(T, codes, scales, zeros, g_idx, H, bits, passes=1):
    """Bid-Up passes (B2, B3) for the target T = W - B A: returns
    (codes, margins, history). margins[p][r, j] is the tie distance of the
    decision of pass p at (r, j) (oracle.gptq_f64.tie_distance of the
    pre-rounding value c + g / (H_jj s)); history lists the objective
    tr((T - W_hat) H (T - W_hat)^T) before the first pass and after each."""
    T = np.asarray(T, np.float64)
    H = np.asarray(H, np.float64)
    c = np.asarray(codes, np.float64).copy()
    g_idx = np.asarray(g_idx)
    S = np.asarray(scales, np.float64)[:, g_idx]
    Z = np.asarray(zeros, np.float64)[:, g_idx]
    maxq = float(2 ** bits - 1)
    D = T - S * (c - Z)
    G = D @ H
    hist = [float((G * D).sum())]
    margins = []
    for _ in range(passes):
        mg = np.full(c.shape, 0.5)
        for j in range(T.shape[1]):
            h = H[j, j]
            if h <= 0.0:
                continue
            pre = c[:, j] + G[:, j] / (h * S[:, j])
            cn = np.clip(np.rint(pre), 0.0, maxq)
            delta = S[:, j] * (cn - c[:, j])
            c[:, j] = cn
            G -= np.outer(delta, H[j])
            mg[:, j] = O.tie_distance(pre)
        margins.append(mg)
        D = T - S * (c - Z)
        hist.append(float(((D @ H) * D).sum()))
    return c.astype(np.uint8), margins, hist


def refine(W, H, codes, scales, zeros, g_idx, bits, rank, cycles=1, passes=1):
    """OLrC / Bid-Up cycles (B4). Returns (codes, B, A, losses) where losses
    lists the layer objective at the start and after every OLrC and every
    Bid-Up step (non-increasing by the page's argument)."""
    W = np.asarray(W, np.float64)
    c = np.asarray(codes).copy()
    W_hat = dequant(c, scales, zeros, g_idx)
    losses = [objective(W, W_hat, H)]
    B = A = None
    for _ in range(cycles):
        B, A, _ = E.eora(W, W_hat, H, rank)
        losses.append(objective(W, W_hat, H, B, A))
        c, _, _ = bidup(W - B @ A, c, scales, zeros, g_idx, H, bits, passes)
        W_hat = dequant(c, scales, zeros, g_idx)
        losses.append(objective(W, W_hat, H, B, A))
    return c, B, A, losses
