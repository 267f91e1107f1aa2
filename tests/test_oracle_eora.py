"""Pins of the EoRA oracle (oracle/eora.py) against what the page and the
mathematics fix ("Aumento de la precisión de LLM de 2 bits con EoRA",
"Bucear en el espacio propio en busca de un adaptador"): a hand-worked case
where EoRA and plain SVD differ, full rank, the closed form of the optimal
weighted rank-r error (eigenvalues of a different matrix), the page's claim
that EoRA's layer loss is below plain SVD's, the reduction to plain SVD at
isotropic activations, scale invariance, local optimality, and a singular
covariance. Planted mistakes in a copy of the oracle must fail the pins."""
import inspect
import types

import numpy as np
import pytest

import oracle.eora as E


def _problem(seed, d_out=12, n=16, T=200):
    r = np.random.default_rng(seed)
    X = r.standard_t(4, (T, n))
    X[:, r.integers(0, n)] *= 8.0
    W = r.standard_normal((d_out, n)) * 0.02
    W_hat = np.round(W / 0.01) * 0.01          # a coarse grid: a compression error
    return W, W_hat, 2.0 * X.T @ X


def test_hand_worked_eora_differs_from_svd():
    """Delta W = diag(1, 1.5), H = diag(4, 1), rank 1. Plain SVD keeps the
    larger weight error (1.5 on row 2): residual diag(1, 0), loss 4 * 1 = 4.
    EoRA weighs column 1 by sqrt(4) = 2: Delta W' = diag(2, 1.5), so it
    keeps row 1: B A = diag(1, 0), residual diag(0, 1.5), loss 1.5^2 = 2.25,
    sigma = 2."""
    W = np.diag([1.0, 1.5])
    Z = np.zeros((2, 2))
    H = np.diag([4.0, 1.0])
    B, A, s = E.eora(W, Z, H, 1)
    assert np.allclose(B @ A, np.diag([1.0, 0.0]), atol=1e-14)
    assert s == pytest.approx([2.0], rel=1e-14)
    assert E.layer_loss(W, Z, H, B, A) == pytest.approx(2.25, rel=1e-14)
    Bs, As, ss = E.svd_baseline(W, Z, 1)
    assert np.allclose(Bs @ As, np.diag([0.0, 1.5]), atol=1e-14)
    assert E.layer_loss(W, Z, H, Bs, As) == pytest.approx(4.0, rel=1e-14)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_full_rank_removes_the_error(seed):
    W, W_hat, H = _problem(seed)
    B, A, _ = E.eora(W, W_hat, H, min(W.shape))
    assert np.allclose(B @ A, W - W_hat, atol=1e-12)
    assert E.layer_loss(W, W_hat, H, B, A) <= 1e-20 * E.layer_loss(W, W_hat, H) + 1e-24


@pytest.mark.parametrize("seed,rank", [(4, 1), (5, 3), (6, 8)])
def test_closed_form_of_the_optimal_rank_r_loss(seed, rank):
    """The best rank-r correction in the loss tr(R H R^T) leaves exactly the
    sum of the d_out - r smallest eigenvalues of Delta W H Delta W^T, and its
    singular values are the square roots of the r largest (Eckart-Young in
    the H-weighted norm; computed here with eigvalsh of that other matrix)."""
    W, W_hat, H = _problem(seed)
    D = W - W_hat
    lam = np.sort(np.linalg.eigvalsh(D @ H @ D.T))[::-1]
    B, A, s = E.eora(W, W_hat, H, rank)
    assert E.layer_loss(W, W_hat, H, B, A) == pytest.approx(lam[rank:].sum(), rel=1e-9)
    assert np.allclose(s, np.sqrt(lam[:rank]), rtol=1e-10)
    assert E.layer_loss(W, W_hat, H) == pytest.approx(lam.sum(), rel=1e-10)


def test_eora_loss_not_above_plain_svd():
    """The page: plain SVD does not minimise the layer's compression loss,
    EoRA's eigenspace projection does. On every seed and rank, EoRA's layer
    loss is at most plain SVD's, and strictly below on most."""
    below = 0
    for seed in range(20):
        W, W_hat, H = _problem(100 + seed)
        for r in (1, 2, 4):
            le = E.layer_loss(W, W_hat, H, *E.eora(W, W_hat, H, r)[:2])
            ls = E.layer_loss(W, W_hat, H, *E.svd_baseline(W, W_hat, r)[:2])
            assert le <= ls * (1 + 1e-12)
            below += le < ls * (1 - 1e-6)
    assert below >= 50


def test_isotropic_activations_give_plain_svd():
    W, W_hat, _ = _problem(7)
    B, A, s = E.eora(W, W_hat, 3.0 * np.eye(W.shape[1]), 4)
    Bs, As, ss = E.svd_baseline(W, W_hat, 4)
    assert np.allclose(B @ A, Bs @ As, atol=1e-13)
    assert np.allclose(s, np.sqrt(3.0) * ss, rtol=1e-12)


def test_scale_invariance():
    W, W_hat, H = _problem(8)
    B, A, s = E.eora(W, W_hat, H, 3)
    B7, A7, s7 = E.eora(W, W_hat, 7.0 * H, 3)
    assert np.allclose(B @ A, B7 @ A7, atol=1e-13)
    assert np.allclose(s7, np.sqrt(7.0) * s, rtol=1e-12)


def test_no_rank_r_perturbation_lowers_the_loss():
    W, W_hat, H = _problem(9, d_out=6, n=8)
    B, A, _ = E.eora(W, W_hat, H, 2)
    base = E.layer_loss(W, W_hat, H, B, A)
    r = np.random.default_rng(10)
    for _ in range(200):
        eps = 10.0 ** r.uniform(-4, -1)
        Bp = B + eps * r.standard_normal(B.shape) * np.abs(B).max()
        Ap = A + eps * r.standard_normal(A.shape) * np.abs(A).max()
        assert E.layer_loss(W, W_hat, H, Bp, Ap) >= base * (1 - 1e-12)


def test_singular_covariance_uses_the_pseudo_inverse():
    """A column no token activates: its direction has Lambda = 0, A has no
    component along it and the loss still equals the closed form."""
    W, W_hat, _ = _problem(11)
    r = np.random.default_rng(12)
    X = r.standard_normal((200, W.shape[1]))
    X[:, 5] = 0.0
    H = 2.0 * X.T @ X
    B, A, _ = E.eora(W, W_hat, H, 3)
    assert np.abs(A[:, 5]).max() <= 1e-12 * np.abs(A).max()
    D = W - W_hat
    lam = np.sort(np.linalg.eigvalsh(D @ H @ D.T))[::-1]
    assert E.layer_loss(W, W_hat, H, B, A) == pytest.approx(lam[3:].sum(), rel=1e-9)


# ---- planted mistakes ------------------------------------------------------
def _mutant(old, new):
    src = inspect.getsource(E)
    assert src.count(old) == 1, old
    m = types.ModuleType("eora_mutant")
    exec(compile(src.replace(old, new), "eora_mutant", "exec"), m.__dict__)
    return m


def _battery(M):
    W = np.diag([1.0, 1.5])
    Z = np.zeros((2, 2))
    H = np.diag([4.0, 1.0])
    B, A, s = M.eora(W, Z, H, 1)
    assert np.allclose(B @ A, np.diag([1.0, 0.0]), atol=1e-12)
    W, W_hat, H = _problem(4)
    D = W - W_hat
    lam = np.sort(np.linalg.eigvalsh(D @ H @ D.T))[::-1]
    B, A, s = M.eora(W, W_hat, H, 3)
    assert M.layer_loss(W, W_hat, H, B, A) == pytest.approx(lam[3:].sum(), rel=1e-9)
    B, A, _ = M.eora(W, W_hat, H, min(W.shape))
    assert np.allclose(B @ A, D, atol=1e-12)


MUTANTS = [
    ("Lambda instead of its square root (the page's literal Q' = Q Lambda)",
     "Dp = D @ (Q * sq[None, :])", "Dp = D @ (Q * (sq * sq)[None, :])"),
    ("no back-projection scale", "A = (Vt[:r] * inv[None, :]) @ Q.T", "A = Vt[:r] @ Q.T"),
    ("back-projection with Q instead of Q^T", "A = (Vt[:r] * inv[None, :]) @ Q.T",
     "A = (Vt[:r] * inv[None, :]) @ Q"),
    ("smallest singular directions kept", "B = U[:, :r] * S[None, :r]", "B = U[:, -r:] * S[None, -r:]"),
    ("singular values dropped from B", "B = U[:, :r] * S[None, :r]", "B = U[:, :r]"),
]


def test_battery_passes_on_the_oracle():
    _battery(E)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutation_is_caught(name, old, new):
    m = _mutant(old, new)
    with pytest.raises((AssertionError, ValueError, np.linalg.LinAlgError)):
        _battery(m)
