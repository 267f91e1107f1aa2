"""EoRA: low-rank compensation of a compressed layer in the eigenspace of the
activation covariance, in plain float64 numpy.

TEST INFRASTRUCTURE (see the package docstring): only tests, the smoke check
and the benchmark's CPU-baseline leg use this module.

What the page fixes ("Aumento de la precisión de LLM de 2 bits con EoRA"
(7minutos.es), section "Bucear en el espacio propio en busca de un
adaptador"):
  * the compression error is Delta W = W - W_hat;
  * the plain baseline decomposes it by SVD, U Sigma V^T, and keeps rank r:
    B = U_r Sigma_r, A = V_r^T (the two factors of a LoRA adapter);
  * EoRA first projects the error into the eigenspace of the activation
    covariance X~ X~^T = Q Lambda Q^T, Delta W' = Delta W Q', takes the
    rank-r SVD of Delta W' and projects the result back to the original
    space, adjusting the factors; the projection weighs each direction by
    its contribution to the layer output (through the eigenvalues), so the
    truncation minimises the layer's compression loss itself.

Readings (the page is garbled or silent here):
  E1  Q' = Q Lambda^{1/2}. The page prints "Q' = Q lambda"; with
      Lambda^{1/2} the Frobenius norm of Delta W' equals the layer loss
      ||X Delta W^T||_F^2 = tr(Delta W H Delta W^T) / 2 and the rank-r
      truncation of Delta W' is the loss-optimal rank-r correction, which
      is what the page says the projection achieves; with Lambda itself it
      is not (pinned: the mutant with Lambda fails the optimality pin).
  E2  The covariance is H = 2 X^T X, the Hessian GPTQ uses (its scale does
      not change the result). Directions with Lambda = 0 carry no
      activation; the back-projection uses the pseudo-inverse there
      (Lambda^{-1/2} := 0), so A has no component along them.
  E3  Back-projection: Delta W ~ U'_r Sigma'_r V'_r^T (Q')^{-1}, i.e.
      B = U'_r Sigma'_r (d_out x r) and A = V'_r^T Lambda^{-1/2} Q^T (r x n).
      The compensated layer is W_hat + B A.
Orientation: W is d_out x n (PyTorch Linear layout), X is T x n, the layer
output is X W^T.
"""
import numpy as np


def eigen_basis(H, rel_tol=1e-12):
    """(Q, sqrt(Lambda), pseudo-inverse of sqrt(Lambda)) of the symmetric
    covariance H (E2): numpy eigh in float64."""
    H = np.asarray(H, np.float64)
    lam, Q = np.linalg.eigh(0.5 * (H + H.T))
    lam = np.where(lam > rel_tol * max(lam.max(), 0.0), lam, 0.0)
    sq = np.sqrt(lam)
    inv = np.where(sq > 0.0, 1.0 / np.where(sq > 0.0, sq, 1.0), 0.0)
    return Q, sq, inv


def eora(W, W_hat, H, rank):
    """(B, A, sigma): the rank-r EoRA adapter of the error W - W_hat, the
    page's steps in its order (E1-E3): eigendecomposition of H, projection
    Delta W' = Delta W Q Lambda^{1/2}, SVD, rank-r truncation, projection
    back. sigma holds the r largest singular values of Delta W'."""
    D = np.asarray(W, np.float64) - np.asarray(W_hat, np.float64)
    Q, sq, inv = eigen_basis(H)
    Dp = D @ (Q * sq[None, :])                     # Delta W' = Delta W Q'
    U, S, Vt = np.linalg.svd(Dp, full_matrices=False)
    r = int(rank)
    B = U[:, :r] * S[None, :r]
    A = (Vt[:r] * inv[None, :]) @ Q.T
    return B, A, S[:r]


def svd_baseline(W, W_hat, rank):
    """The page's plain baseline: rank-r SVD of Delta W, B = U_r Sigma_r,
    A = V_r^T."""
    D = np.asarray(W, np.float64) - np.asarray(W_hat, np.float64)
    U, S, Vt = np.linalg.svd(D, full_matrices=False)
    r = int(rank)
    return U[:, :r] * S[None, :r], Vt[:r].copy(), S[:r]


def layer_loss(W, W_hat, H, B=None, A=None):
    """tr(R H R^T) with R = W - W_hat - B A (R = W - W_hat without an
    adapter): twice the layer loss ||X R^T||_F^2 when H = 2 X^T X ("Resumen
    Técnico: GPTQ-intrinsic LoRA", "Declaración del Problema")."""
    R = np.asarray(W, np.float64) - np.asarray(W_hat, np.float64)
    if B is not None:
        R = R - np.asarray(B, np.float64) @ np.asarray(A, np.float64)
    return float(((R @ np.asarray(H, np.float64)) * R).sum())
