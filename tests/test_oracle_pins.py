"""Pins of the float64 oracle against what the pages and the mathematics fix.

Every check here is independent of the oracle's own arithmetic: a library
routine used differently (linear solves instead of the inverse-downdate or
Cholesky machinery), brute force over tiny inputs, hand-worked values of the
format, closed forms, invariants, and the pages' printed numbers.
"""
import json
import os

import numpy as np
import pytest

from oracle import gptq_f64 as O
from oracle import memory as M
from oracle import packing as P
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _tiny(seed, d_out, n, T, heavy=False):
    r = np.random.default_rng(seed)
    X = r.standard_t(4, (T, n)) if heavy else r.standard_normal((T, n))
    X[:, r.integers(0, n)] *= 10.0
    W = r.standard_normal((d_out, n)) * 0.02
    return W, X


# ---------------------------------------------------------------- Hessian
def test_hessian_is_sum_of_token_outer_products():
    """P-H: 2 X^T X equals 2 * sum_t x_t x_t^T written out per token."""
    r = np.random.default_rng(1)
    X = r.standard_normal((37, 6))
    H = O.hessian(X, chunk=5)
    ref = np.zeros((6, 6))
    for t in range(X.shape[0]):
        for i in range(6):
            for j in range(6):
                ref[i, j] += 2.0 * X[t, i] * X[t, j]
    assert np.allclose(H, ref, rtol=1e-13, atol=1e-13)
    assert np.array_equal(H, H.T)


def test_hessian_bf16_products_exact():
    """bf16 inputs: every product and the whole sum is exact in float64 for
    small T (8+8 mantissa bits, few terms), so chunking cannot change it."""
    wl = synth.make_workload("c2", d_out=4, n=24, T=64, group=8)
    a = O.hessian(wl.X, chunk=1)
    b = O.hessian(wl.X, chunk=64)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------- grid
def test_grid_hand_worked_3bit():
    """Format readings R4-R6 worked by hand with dyadic values (3-bit,
    maxq = 7, one group of four per row):
      [1.5,-0.25,0.125,0.375]: range [-0.25,1.5] -> s=1.75/7=0.25, z=rint(1)=1;
          w/s = 6,-1,0.5,1.5 -> rint (half to even) 6,-1,0,2 -> +z 7,0,1,3
      [0.5,1.75,0.25,1.0]: range widened to 0 -> [0,1.75], s=0.25, z=0;
          codes 2,7,1,4
      [-0.5,-1.75,-0.25,-1.0]: range [-1.75,0], s=0.25, z=rint(7)=7;
          w/s = -2,-7,-1,-4 -> codes 5,0,6,3
      [0,0,0,0]: degenerate -> (-1,1), s=2/7, z=rint(3.5)=4 (half to even);
          codes 4, reconstruction 0
    """
    W = np.array([[1.5, -0.25, 0.125, 0.375],
                  [0.5, 1.75, 0.25, 1.0],
                  [-0.5, -1.75, -0.25, -1.0],
                  [0.0, 0.0, 0.0, 0.0]])
    res = O.rtn(W, bits=3, group=4)
    assert res["codes"].tolist() == [[7, 0, 1, 3], [2, 7, 1, 4], [5, 0, 6, 3], [4, 4, 4, 4]]
    assert res["zeros"][:, 0].tolist() == [1, 0, 7, 4]
    assert np.allclose(res["scales"][:, 0], [0.25, 0.25, 0.25, 2.0 / 7.0])
    assert np.array_equal(res["w_hat"][0], [1.5, -0.25, 0.0, 0.5])
    assert np.array_equal(res["w_hat"][3], [0.0, 0.0, 0.0, 0.0])


# ---------------------------------------------------------------- symmetric alphabet
def test_symmetric_grid_hand_worked():
    """4 bits: alphabet {-7 .. 7}, s = max|v| / 7, codes stored as q + 7.
    Group [-0.7, 0.35, 0.1, 0]: s = 0.1, w / s = [-7, 3.5, 1, 0], rint (half
    to even) = [-7, 4, 1, 0], codes [0, 11, 8, 7], w_hat [-0.7, 0.4, 0.1, 0].
    A group of zeros takes s = 1 / 7."""
    W = np.array([[-0.7, 0.35, 0.1, 0.0, 0.0, 0.0, 0.0, 0.0]])
    o = O.rtn(W, 4, 4, sym=True)
    assert np.array_equal(o["codes"][0, :4], [0, 11, 8, 7])
    assert np.allclose(o["scales"][0], [0.1, 1.0 / 7.0], rtol=0, atol=1e-15)
    assert np.array_equal(o["zeros"][0], [7, 7])
    assert np.allclose(o["w_hat"][0, :4], [-0.7, 0.4, 0.1, 0.0], rtol=0, atol=1e-15)
    assert np.array_equal(o["codes"][0, 4:], [7, 7, 7, 7])


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_symmetric_alphabet_levels_and_odd_symmetry(bits):
    """Codes stay in [0, 2A] (2A + 1 levels, A = 2^(b-1) - 1); the
    reconstruction is an odd function of the weights (rint to even is
    odd-symmetric and the scale depends on |v| only)."""
    r = np.random.default_rng(40 + bits)
    W = r.standard_normal((12, 64)) * 0.02
    A = 2 ** (bits - 1) - 1
    a = O.rtn(W, bits, 16, sym=True)
    b = O.rtn(-W, bits, 16, sym=True)
    assert a["codes"].max() <= 2 * A and np.all(a["zeros"] == A)
    assert np.array_equal(a["w_hat"], -b["w_hat"])
    assert np.array_equal(a["codes"].astype(int), 2 * A - b["codes"].astype(int))
    # every group's largest magnitude is reproduced exactly as s * A
    g = np.abs(W).reshape(12, 4, 16).max(axis=2)
    assert np.allclose(a["scales"] * A, g, rtol=1e-15, atol=0)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_symmetric_alphabet_holds_under_feedback(bits):
    """With feedback the later columns of a group can move past the scale's
    range; their codes clamp to the alphabet's end, never to 2A + 1."""
    W, X = _tiny(50 + bits, 24, 128, 600, heavy=True)
    o = O.gptq_o2(W, O.hessian(X), bits, 64, 0.01, 32, sym=True)
    A = 2 ** (bits - 1) - 1
    assert o["codes"].max() <= 2 * A and np.all(o["zeros"] == A)
    assert o["codes"].max() == 2 * A          # the clamp is reached on this input
    q = o["w_hat"] / o["scales"][:, np.arange(128) // 64]
    assert np.allclose(q, np.rint(q), atol=1e-9) and np.abs(np.rint(q)).max() <= A


# ---------------------------------------------------------------- RTN special case
@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_diagonal_hessian_is_rtn(bits, sym):
    """P-RTN: with orthonormal-column calibration (one nonzero per token, so
    X^T X is diagonal) there is no feedback and O1, O2 and round-to-nearest
    agree bitwise."""
    r = np.random.default_rng(bits)
    n, d_out, T = 64, 16, 256
    X = np.zeros((T, n))
    X[np.arange(T), np.arange(T) % n] = r.standard_normal(T)   # one-hot tokens
    H = O.hessian(X)
    assert np.count_nonzero(H - np.diag(np.diagonal(H))) == 0
    W = r.standard_normal((d_out, n)) * 0.02
    ref = O.rtn(W, bits, 16, sym=sym)
    o2 = O.gptq_o2(W, H, bits, 16, 0.01, 32, sym=sym)
    o1 = O.gptq_o1(W, H, bits, 16, 0.01, sym=sym)
    for o in (o1, o2):
        assert np.array_equal(o["codes"], ref["codes"])
        assert np.array_equal(o["w_hat"], ref["w_hat"])
    o3 = O.gptq_o2(W, 2.0 * np.eye(n), bits, 16, 0.01, 8, sym=sym)
    assert np.array_equal(o3["codes"], ref["codes"])


# ---------------------------------------------------------------- closed forms
def test_single_column_is_rtn_and_optimal():
    """P-N1: n = 1 -> GPTQ = RTN = exhaustive optimum."""
    r = np.random.default_rng(3)
    W = r.standard_normal((20, 1))
    H = np.array([[3.0]])
    o2 = O.gptq_o2(W, H, 2, 1, 0.01, 1)
    ref = O.rtn(W, 2, 1)
    assert np.array_equal(o2["codes"], ref["codes"])
    best, best_q = O.brute_force_rows(W, H, ref["scales"][:, 0], ref["zeros"][:, 0].astype(float), 2)
    assert np.array_equal(best_q[:, 0].astype(np.uint8), o2["codes"][:, 0])


def test_two_columns_closed_form_update():
    """P-N2: after column 0 is rounded, the optimal continuous column 1 given
    w_hat_0 is w1 + (w0 - w_hat0) Hd01 / Hd11; GPTQ rounds exactly that."""
    r = np.random.default_rng(4)
    for _ in range(50):
        W = r.standard_normal((8, 2))
        A = r.standard_normal((5, 2))
        H = 2 * A.T @ A
        Hd = H + 0.01 * np.mean(np.diag(H)) * np.eye(2)
        o = O.gptq_o2(W, H, 4, 2, 0.01, 2)
        s, z = o["scales"][:, 0], o["zeros"][:, 0].astype(float)
        w1p = W[:, 1] + (W[:, 0] - o["w_hat"][:, 0]) * Hd[0, 1] / Hd[1, 1]
        q1 = np.clip(np.rint(w1p / s) + z, 0, 15)
        assert np.array_equal(q1.astype(np.uint8), o["codes"][:, 1])


def _sequential_ls_codes(W, Hd, bits, group, out):
    """Independent characterisation of the sweep: at column j the value
    GPTQ rounds is the j-th coordinate of the minimiser of (w-w0)^T Hd (w-w0)
    over w with w_<j fixed to the already-rounded values (linear solve), and
    at a group start the group's grid comes from that same minimiser."""
    d_out, n = W.shape
    maxq = 2 ** bits - 1
    codes = np.zeros((d_out, n), np.uint8)
    what = out["w_hat"]                       # identity permutation here
    for r_ in range(d_out):
        w0 = W[r_]
        s = z = None
        for j in range(n):
            d = what[r_, :j] - w0[:j]
            if j:
                x = -np.linalg.solve(Hd[j:, j:], Hd[j:, :j] @ d)
            else:
                x = np.zeros(n)
            cur = w0[j:] + x
            if j % group == 0:
                g = cur[:group]
                lo, hi = min(g.min(), 0.0), max(g.max(), 0.0)
                if lo == hi:
                    lo, hi = -1.0, 1.0
                s = (hi - lo) / maxq
                z = np.rint(-lo / s)
            codes[r_, j] = np.clip(np.rint(cur[0] / s) + z, 0, maxq)
    return codes


@pytest.mark.parametrize("bits,group,block", [(4, 16, 8), (3, 8, 16), (2, 32, 32)])
def test_sweep_is_sequential_constrained_least_squares(bits, group, block):
    """P-LS: O2's codes equal the codes of the sequential constrained
    least-squares characterisation (solved with np.linalg.solve, no inverse
    downdates, no Cholesky)."""
    W, X = _tiny(10 + bits, 6, 32, 200)
    H = O.hessian(X)
    Hd = H + 0.01 * np.mean(np.diag(H)) * np.eye(32)
    o = O.gptq_o2(W, H, bits, group, 0.01, block)
    ref = _sequential_ls_codes(W, Hd, bits, group, o)
    ok = (ref == o["codes"]) | (o["margins"] < 1e-9)
    assert ok.all()


# ---------------------------------------------------------------- loss identity
@pytest.mark.parametrize("act_order", [False, True])
def test_row_loss_equals_quadratic_form(act_order):
    """P-LOSS: sum_j e_j^2 = delta^T Hd delta (processing order), delta = w - w_hat."""
    W, X = _tiny(5, 12, 48, 300, heavy=True)
    H = O.hessian(X)
    o = O.gptq_o2(W, H, 3, 16, 0.01, 16, act_order=act_order)
    Hd, perm = O.prepare(H, 0.01, act_order)
    D = (W - o["w_hat"])[:, perm]
    q = np.einsum("ri,ij,rj->r", D, Hd, D)
    assert np.allclose(o["row_loss"], q, rtol=1e-9)
    o1 = O.gptq_o1(W, H, 3, 16, 0.01, act_order=act_order)
    assert np.allclose(o1["row_loss"], q, rtol=1e-9)


# ---------------------------------------------------------------- tie branches
def test_other_neighbour():
    x = np.array([2.5, 3.5, 2.4999, 2.5001, -0.5, 0.0004, 6.9])
    assert np.array_equal(O.other_neighbour(x), [3.0, 3.0, 3.0, 2.0, -1.0, 1.0, 6.0])


@pytest.mark.parametrize("act_order", [False, True])
def test_tie_branch_is_a_valid_gptq_run(act_order):
    """The other branch at a decision: every earlier decision unchanged, that
    code one level away from the plain run's, and the branch is still a GPTQ
    run of the same problem (its row loss equals its own quadratic form)."""
    W, X = _tiny(6, 9, 64, 400, heavy=True)
    H = O.hessian(X)
    Hd, perm = O.prepare(H, 0.01, act_order)
    U = O.upper_chol_of_inverse(Hd)
    plain = O.gptq_o2(W, H, 3, 16, 0.01, 16, act_order, U=U, perm=perm)
    assert _same_run(plain, O.gptq_o2(W, H, 3, 16, 0.01, 16, act_order, U=U, perm=perm, alt=((), ())))
    # the closest decision whose other neighbour is not clipped away
    cp = plain["codes_proc"]
    m = np.where((cp > 0) & (cp < 7), plain["margins"], np.inf)
    r, j = np.unravel_index(np.argmin(m), m.shape)
    br = O.gptq_o2(W, H, 3, 16, 0.01, 16, act_order, U=U, perm=perm, alt=([(r, j)], ()))
    cb = br["codes_proc"]
    assert np.array_equal(np.delete(cp, r, 0), np.delete(cb, r, 0))
    assert np.array_equal(cp[r, :j], cb[r, :j])
    assert abs(int(cb[r, j]) - int(cp[r, j])) == 1
    D = (W - br["w_hat"])[:, perm]
    assert np.allclose(br["row_loss"], np.einsum("ri,ij,rj->r", D, Hd, D), rtol=1e-9)
    # a zero point's other branch: z moves by one, the group's scale does not
    g = 1
    bz = O.gptq_o2(W, H, 3, 16, 0.01, 16, act_order, U=U, perm=perm, alt=((), [(r, g)]))
    assert abs(int(bz["zeros"][r, g]) - int(plain["zeros"][r, g])) == 1
    assert np.array_equal(bz["codes_proc"][r, :16 * g], cp[r, :16 * g])
    assert bz["scales"][r, g] == plain["scales"][r, g]
    D = (W - bz["w_hat"])[:, perm]
    assert np.allclose(bz["row_loss"], np.einsum("ri,ij,rj->r", D, Hd, D), rtol=1e-9)


def _same_run(a, b):
    return all(np.array_equal(a[k], b[k]) for k in ("codes", "zeros", "scales", "w_hat", "row_loss"))


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("shape,T", [((2, 3), 8), ((3, 4), 16)])
def test_gptq_not_better_than_exhaustive_optimum(shape, T):
    """P-BF: at 2 bits the exhaustive optimum of the layer objective over the
    GPTQ grid is never above GPTQ's own objective; GPTQ's codes lie on it."""
    d_out, n = shape
    r = np.random.default_rng(7 + n)
    W = r.standard_normal(shape)
    X = r.standard_normal((T, n))
    H = O.hessian(X)
    o = O.gptq_o2(W, H, 2, n, 0.01, n)
    s, z = o["scales"][:, 0], o["zeros"][:, 0].astype(float)
    best, _ = O.brute_force_rows(W, H, s, z, 2)
    mine = O.row_objective(W, o["w_hat"], H)
    assert np.all(best <= mine + 1e-12)
    rt = O.rtn(W, 2, n)
    best_rtn, _ = O.brute_force_rows(W, H, rt["scales"][:, 0], rt["zeros"][:, 0].astype(float), 2)
    assert np.all(best_rtn <= O.row_objective(W, rt["w_hat"], H) + 1e-12)


def test_two_column_greedy_choice_is_optimal_given_first():
    """With column 0 fixed to GPTQ's choice, GPTQ's column-1 code is the
    exhaustive optimum of the damped objective over column 1 (when the
    optimum is not clamped)."""
    r = np.random.default_rng(8)
    for _ in range(30):
        W = r.standard_normal((4, 2))
        X = r.standard_normal((6, 2))
        H = O.hessian(X)
        Hd = H + 0.01 * np.mean(np.diag(H)) * np.eye(2)
        o = O.gptq_o2(W, H, 3, 2, 0.01, 2)
        for i in range(4):
            s, z = o["scales"][i, 0], float(o["zeros"][i, 0])
            cands = s * (np.arange(8) - z)
            objs = [O.row_objective(W[i:i + 1], np.array([[o["w_hat"][i, 0], c]]), Hd)[0] for c in cands]
            assert int(np.argmin(objs)) == int(o["codes"][i, 1])


# ---------------------------------------------------------------- invariants
def test_block_size_invariance():
    """P-B: lazy batching is exact: every block size gives the same codes."""
    W, X = _tiny(11, 10, 128, 600, heavy=True)
    H = O.hessian(X)
    base = O.gptq_o2(W, H, 4, 32, 0.01, 128)
    for B in (1, 2, 4, 8, 32, 64):
        o = O.gptq_o2(W, H, 4, 32, 0.01, B)
        ok = (o["codes"] == base["codes"]) | (base["margins"][:, :] < 1e-9)
        assert ok.all(), B
        assert np.allclose(o["w_hat"], base["w_hat"], atol=1e-12)


@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("act_order", [False, True])
def test_o1_equals_o2(bits, act_order, sym):
    """P-O1O2: the OBS inverse-downdate definition and the Cholesky/lazy-batch
    form agree to float64 rounding."""
    W, X = _tiny(20 + bits, 16, 96, 500, heavy=True)
    H = O.hessian(X)
    o1 = O.gptq_o1(W, H, bits, 32, 0.01, act_order=act_order, sym=sym)
    o2 = O.gptq_o2(W, H, bits, 32, 0.01, 16, act_order=act_order, sym=sym)
    assert np.array_equal(o1["perm"], o2["perm"])
    ok = (o1["codes"] == o2["codes"]) | (o2["margins"][:, np.argsort(o2["perm"])] < 1e-8)
    assert ok.all()
    assert np.allclose(o1["w_hat"], o2["w_hat"], atol=1e-10)
    assert np.allclose(o1["row_loss"], o2["row_loss"], rtol=1e-8)


def test_cholesky_factor_of_inverse():
    """P-CHOL: U upper, positive diagonal, U^T U Hd = I."""
    _, X = _tiny(30, 1, 64, 400)
    Hd, _ = O.prepare(O.hessian(X), 0.01)
    U = O.upper_chol_of_inverse(Hd)
    assert np.array_equal(U, np.triu(U))
    assert np.all(np.diag(U) > 0)
    assert np.abs(U.T @ U @ Hd - np.eye(64)).max() < 1e-10


@pytest.mark.parametrize("n", [1, 7, 64, 333])
def test_cholesky_factor_by_reversal(n):
    """P-CHOL for the route used on the widest layer (one Cholesky of the
    index-reversed H_d and a triangular inverse): U upper, positive
    diagonal, U^T U H_d = I, and equal to the explicit-inverse route."""
    _, X = _tiny(35 + n, 1, n, 4 * n + 8)
    Hd, _ = O.prepare(O.hessian(X), 0.01)
    U = O.upper_chol_of_inverse_by_reversal(Hd)
    assert np.array_equal(U, np.triu(U))
    assert np.all(np.diag(U) > 0)
    assert np.abs(U.T @ U @ Hd - np.eye(n)).max() < 1e-10
    assert np.abs(U - O.upper_chol_of_inverse(Hd)).max() <= 1e-12 * np.abs(U).max()
    with pytest.raises(np.linalg.LinAlgError):
        O.upper_chol_of_inverse_by_reversal(-Hd)


def test_act_order_is_permuted_problem():
    """P-PERM: act-order = plain GPTQ on the problem permuted by descending
    diag(H) (stable), un-permuted afterwards."""
    W, X = _tiny(31, 8, 64, 300, heavy=True)
    H = O.hessian(X)
    d = np.diag(H)
    perm = sorted(range(64), key=lambda i: (-d[i], i))
    a = O.gptq_o2(W, H, 3, 16, 0.01, 16, act_order=True)
    b = O.gptq_o2(W[:, perm], H[np.ix_(perm, perm)], 3, 16, 0.01, 16)
    assert list(a["perm"]) == perm
    inv = np.argsort(perm)
    assert np.array_equal(a["codes"], b["codes"][:, inv])
    assert np.allclose(a["w_hat"], b["w_hat"][:, inv], atol=1e-14)
    assert np.array_equal(a["g_idx"], (inv // 16).astype(np.int32))


def test_dead_column_reading():
    """R3 end to end on a tiny layer: the result is finite and O1 and O2 agree
    (the decoupling and the round-to-nearest code of the dead column are
    asserted by test_dead_column_is_decoupled_unit_curvature)."""
    W, X = _tiny(32, 4, 16, 100)
    X[:, 5] = 0.0
    H = O.hessian(X)
    o = O.gptq_o2(W, H, 4, 16, 0.01, 16)
    assert np.isfinite(o["w_hat"]).all()
    o1 = O.gptq_o1(W, H, 4, 16, 0.01)
    assert np.array_equal(o["codes"], o1["codes"])


# ---------------------------------------------------------------- augmented Hessian
def test_augmented_identities():
    """P-AUG ([GIL] Metodología 2): X~ W~^T = X W^T at W~ = [W, 0]; with r = 0
    the augmented call is plain GPTQ; the codes do not depend on the sign of
    the appended basis; Q_deq + R V^T reproduces X~ W_hat~^T."""
    r = np.random.default_rng(40)
    T, n, rk, d_out = 400, 32, 4, 6
    X = r.standard_t(4, (T, n))
    W = r.standard_normal((d_out, n)) * 0.02
    _, _, Vt = np.linalg.svd(X, full_matrices=False)
    V = Vt[:rk].T
    Xa = np.concatenate([X, X @ V], axis=1)
    Wa = np.concatenate([W, np.zeros((d_out, rk))], axis=1)
    assert np.allclose(Xa @ Wa.T, X @ W.T, atol=1e-12)
    plain = O.gptq_o2(W, O.hessian(X), 2, 16, 0.01, 16)
    same = O.gptq_o2(W, O.hessian(X), 2, 16, 0.01, 16, n_quant=n)
    assert np.array_equal(plain["codes"], same["codes"])
    o = O.gptq_o2(Wa, O.hessian(Xa), 2, 16, 0.01, 16, n_quant=n)
    Xb = np.concatenate([X, -(X @ V)], axis=1)
    ob = O.gptq_o2(Wa, O.hessian(Xb), 2, 16, 0.01, 16, n_quant=n)
    assert np.array_equal(o["codes"], ob["codes"])
    assert np.allclose(o["w_hat"][:, n:], -ob["w_hat"][:, n:], atol=1e-12)
    Q, R = o["w_hat"][:, :n], o["w_hat"][:, n:]
    assert np.allclose(Xa @ o["w_hat"].T, X @ (Q + R @ V.T).T, atol=1e-10)
    # the appended coordinates help: layer error with R <= without
    e_aug = O.layer_error(Wa, o["w_hat"], O.hessian(Xa))
    e_plain = O.layer_error(W, plain["w_hat"], O.hessian(X))
    assert e_aug <= e_plain * 1.0001


# ---------------------------------------------------------------- GPTQ vs RTN
def test_gptq_not_worse_than_rtn_tiny_seeds():
    """P-RTN>= ([GPTQ] "Rendimiento y Precisión": GPTQ lowers the error of
    round-to-nearest). GPTQ is a greedy heuristic, not a minimiser: on
    4-row problems it loses to RTN on some seeds (the sequential
    least-squares pin above shows the oracle is the algorithm). The claim is
    therefore checked in aggregate over 100 tiny seeds per width (mean ratio
    and share of seeds improved) and per seed on the workload recipes."""
    for bits in (2, 3, 4):
        ratios = []
        for seed in range(100):
            W, X = _tiny(1000 + seed, 8, 64, 256, heavy=True)
            H = O.hessian(X)
            o = O.gptq_o2(W, H, bits, 32, 0.01, 32)
            rt = O.rtn(W, bits, 32)
            ratios.append(O.layer_error(W, o["w_hat"], H) / O.layer_error(W, rt["w_hat"], H))
        ratios = np.array(ratios)
        assert ratios.mean() < 0.95, bits
        assert (ratios < 1).mean() >= 0.9, bits


@pytest.mark.parametrize("name,kw", [
    ("c1", dict()),
    ("c2", dict(d_out=64, n=256, T=4096)),
    ("c3", dict(d_out=64, n=384, T=4096)),
    ("c5", dict(d_out=64, n=256, T=4096, aug_rank=16)),
])
def test_gptq_not_worse_than_rtn_config_recipes(name, kw):
    wl = synth.make_workload(name, **kw)
    H = O.hessian(wl.X)
    p = wl.params
    o = O.gptq_o2(wl.W, H, p["bits"], p["group"], p["damp"], p["block"],
                  p["act_order"], wl.n_quant)
    rt = O.rtn(wl.W[:, :wl.n_quant], p["bits"], p["group"])
    what_rtn = np.concatenate([rt["w_hat"], wl.W[:, wl.n_quant:]], axis=1)
    assert O.layer_error(wl.W, o["w_hat"], H) < O.layer_error(wl.W, what_rtn, H)


def test_c4_recipe_reduced_given_hessian():
    """The given-Hessian recipe at reduced shape: fp32 H from float64 sums."""
    wl = synth.make_workload("c4", d_out=32, n=256, T=2048,
                             H_fn=lambda chunks: sum(O.hessian(x) for _, x, _ in chunks))
    assert wl.H.dtype == np.float32 and wl.H.shape == (256, 256)
    o = O.gptq_o2(wl.W, wl.H, 2, 64, 0.01, 128)
    rt = O.rtn(wl.W, 2, 64)
    assert O.layer_error(wl.W, o["w_hat"], wl.H) < O.layer_error(wl.W, rt["w_hat"], wl.H)


# ---------------------------------------------------------------- packing
def test_pack_roundtrip_all_widths():
    r = np.random.default_rng(50)
    for bits in (2, 3, 4):
        for nq in (1, 7, 32, 33, 96, 200):
            c = r.integers(0, 2 ** bits, (5, nq)).astype(np.uint8)
            w = P.pack(c, bits)
            assert w.shape == (5, P.words_per_row(nq, bits))
            assert np.array_equal(P.unpack(w, nq, bits), c)


def test_pack_3bit_hand_words():
    """R17 by hand: codes 0..31 -> 1,2,3,...: code k at bit 3k.
    word0 = codes 0..9 in bits 0..29, code 10's low 2 bits in bits 30..31;
    code 10 = 3 = 0b011 -> bits 30,31 = 1,1, its high bit (0) starts word1."""
    c = (np.arange(32) % 8).astype(np.uint8)[None, :]
    w = P.pack(c, 3)
    word0 = sum(int(c[0, k]) << (3 * k) for k in range(10)) | ((int(c[0, 10]) & 3) << 30)
    assert int(w[0, 0]) == word0
    assert int(w[0, 1]) & 1 == (int(c[0, 10]) >> 2) & 1
    assert w.shape[1] == 3
    one = np.zeros((1, 11), np.uint8)
    one[0, 10] = 7                               # straddles bits 30..32
    w1 = P.pack(one, 3)
    assert int(w1[0, 0]) == 0xC0000000 and int(w1[0, 1]) == 1


def test_pack_4bit_is_nibbles():
    c = np.array([[1, 2, 3, 4, 5, 6, 7, 8, 15]], np.uint8)
    w = P.pack(c, 4)
    assert int(w[0, 0]) == 0x87654321 and int(w[0, 1]) == 0xF


def test_words_per_row_for_recipes():
    assert [P.words_per_row(nq, b) for nq, b in
            [(128, 4), (4096, 4), (11008, 3), (28672, 2), (5120, 2)]] == [16, 512, 1032, 1792, 320]


# ---------------------------------------------------------------- storage (pages' numbers)
def test_storage_examples_from_pages():
    g = json.load(open(os.path.join(GOLD, "pages_storage_examples.json")))
    ex = g["worked_example_7b_4bit"]
    b = M.raw_weight_bytes(ex["n_params"], ex["bits"])
    assert M.gb(b) == ex["gb"]
    assert round(M.gib(b), ex["gib_decimals"]) == ex["gib_approx"]
    opt = g["opt175b_4bit"]
    assert M.gb(M.raw_weight_bytes(opt["n_params"], opt["bits"])) == opt["gb_approx"]
    assert M.gb(M.raw_weight_bytes(opt["n_params"], 16)) == opt["float_reference_gb"]
    bp = g["bytes_per_param"]
    assert M.raw_weight_bytes(1, 4) == bp["int4_bytes"] and M.raw_weight_bytes(1, 32) == bp["fp32_bytes"]
    ll = g["llama70b_fp16"]
    assert M.gb(M.raw_weight_bytes(ll["n_params"], 16)) == ll["fp16_gb_approx"]
    assert M.gb(M.raw_weight_bytes(ll["n_params"], 4)) < ll["int4_total_gb_approx"]
    assert M.bits_per_weight(4, 128) == 4.28125


# ---------------------------------------------------------------- tie distance
def test_tie_distance_hand_values():
    """The distance of a pre-rounding value to the nearest half-integer, in
    steps, worked by hand: exact half-integers (positive, negative, a
    zero-point value) are 0, integers are 0.5, and a value 0.01 below a
    half-integer is 0.01, on either side of zero."""
    x = np.array([0.5, 1.0, -0.5, 2.49, 3.0, -1.25, -0.75, 7.5, -2.0, 0.0, -2.51, 14.5])
    want = np.array([0.0, 0.5, 0.0, 0.01, 0.5, 0.25, 0.25, 0.0, 0.5, 0.5, 0.01, 0.0])
    assert np.allclose(O.tie_distance(x), want, atol=1e-12, rtol=0)


def test_tie_distance_is_distance_to_the_rounding_boundary():
    """Brute force: the distance equals min over k of |x - (k + 1/2)|, and it
    is the decision's margin: moving x by less than it never changes rint(x),
    moving it slightly past it (towards the nearest half-integer) does."""
    r = np.random.default_rng(3)
    x = np.concatenate([r.uniform(-20, 20, 4000), np.arange(-12, 12) + 0.5 + r.uniform(-1e-3, 1e-3, 24)])
    halves = np.arange(-40, 41) + 0.5
    ref = np.abs(x[:, None] - halves[None, :]).min(1)
    d = O.tie_distance(x)
    assert np.allclose(d, ref, atol=1e-12, rtol=0)
    keep = d > 1e-6
    xs, ds = x[keep], d[keep]
    near = np.where(xs - np.floor(xs) < 0.5, 1.0, -1.0)   # direction of the nearest half-integer
    assert np.array_equal(np.rint(xs + near * ds * 0.999), np.rint(xs))
    assert np.array_equal(np.rint(xs - near * ds * 0.999), np.rint(xs))
    assert np.all(np.rint(xs + near * (ds + 1e-7)) != np.rint(xs))


def test_zero_point_margin_hand_worked():
    """The margin of a zero-point decision: 3-bit (maxq 7), a row whose range
    is [-0.625, 1.125] gives s = 0.25 and -xmin/s = 2.5 exactly (a tie, z =
    rint(2.5) = 2, half to even); a row with range [-0.25, 1.5] gives
    -xmin/s = 1 (margin 0.5). H = 2I: no feedback, the grid is the input's."""
    W = np.array([[-0.625, 1.125, 0.0, 0.5], [1.5, -0.25, 0.125, 0.375]])
    o = O.gptq_o2(W, 2.0 * np.eye(4), 3, 4, 0.01, 4)
    assert np.array_equal(o["scales"][:, 0], [0.25, 0.25])
    assert np.array_equal(o["zeros"][:, 0], [2, 1])
    assert np.allclose(o["zmargins"][:, 0], [0.0, 0.5], atol=1e-15)
    # code margins: row 1 is w / s = 6, -1, 0.5, 1.5
    assert np.allclose(o["margins"][1], [0.5, 0.5, 0.0, 0.0], atol=1e-15)


# ---------------------------------------------------------------- layer error
def test_layer_error_hand_worked():
    """r = ||X (W - W_hat)^T||^2 / ||X W^T||^2 ("Resumen Técnico:
    GPTQ-intrinsic LoRA", "Declaración del Problema"), by hand:
    X = [[1, 0], [1, 1]], W = [1, 2], W_hat = [1, 1]: X W^T = (1, 3), norm^2
    10; X (W - W_hat)^T = (0, 1), norm^2 1; r = 0.1. Any positive scale of H
    gives the same r."""
    X = np.array([[1.0, 0.0], [1.0, 1.0]])
    W = np.array([[1.0, 2.0]])
    Wh = np.array([[1.0, 1.0]])
    assert O.layer_error(W, Wh, O.hessian(X)) == pytest.approx(0.1, rel=1e-15)
    assert O.layer_error(W, Wh, X.T @ X) == pytest.approx(0.1, rel=1e-15)


def test_layer_error_from_activations():
    """The same ratio formed from X directly, on a random layer: the
    undamped H, all rows, the output-space norm."""
    r = np.random.default_rng(12)
    X = r.standard_t(4, (300, 24))
    W = r.standard_normal((7, 24)) * 0.02
    o = O.gptq_o2(W, O.hessian(X), 3, 8, 0.01, 8)
    ref = np.linalg.norm(X @ (W - o["w_hat"]).T) ** 2 / np.linalg.norm(X @ W.T) ** 2
    assert O.layer_error(W, o["w_hat"], O.hessian(X)) == pytest.approx(ref, rel=1e-12)


# ---------------------------------------------------------------- dead columns (R3)
def _dead_problem(seed, n=16, j=5):
    r = np.random.default_rng(seed)
    X = r.standard_normal((200, n))
    X[:, j] = 0.0
    W = r.standard_normal((6, n)) * 0.02
    W[:, j] = 0.5 * W[:, 0]          # inside every row's range: the grid does not depend on it
    return W, O.hessian(X), j


@pytest.mark.parametrize("damp", [0.0, 0.01])
def test_dead_column_is_decoupled_unit_curvature(damp):
    """R3: a column no token activates (H_jj = 0) takes H_jj := 1 before
    damping. Then it couples to no other column: the other columns' codes
    and w_hat equal GPTQ on the problem with that column removed (with the
    damping matched: lambda = damp * mean of the diagonal including the 1);
    its own code is round-to-nearest of its original value on its group's
    grid; and the row loss gains exactly (w_j - w_hat_j)^2 (1 + lambda)."""
    W, H, j = _dead_problem(33)
    n = H.shape[0]
    keep = np.delete(np.arange(n), j)
    d = np.diag(H)
    lam = damp * (d.sum() + 1.0) / n
    damp_red = lam / (d[keep].sum() / (n - 1))
    for run in (lambda W_, H_, g, dm: O.gptq_o2(W_, H_, 4, g, dm, g),
                lambda W_, H_, g, dm: O.gptq_o1(W_, H_, 4, g, dm)):
        full = run(W, H, n, damp)
        red = run(W[:, keep], H[np.ix_(keep, keep)], n - 1, damp_red)
        assert np.array_equal(full["codes"][:, keep], red["codes"])
        assert np.allclose(full["w_hat"][:, keep], red["w_hat"], atol=1e-13, rtol=0)
        s, z = full["scales"][:, 0], full["zeros"][:, 0].astype(np.float64)
        assert np.array_equal(full["scales"][:, 0], red["scales"][:, 0])
        q = np.clip(np.rint(W[:, j] / s) + z, 0, 15)
        assert np.array_equal(full["codes"][:, j], q.astype(np.uint8))
        assert np.array_equal(full["w_hat"][:, j], s * (q - z))
        extra = (W[:, j] - full["w_hat"][:, j]) ** 2 * (1.0 + lam)
        assert np.allclose(full["row_loss"], red["row_loss"] + extra, rtol=1e-10, atol=0)


def test_dead_column_in_act_order():
    """With act-order the fixed diagonal value 1 takes its place in the
    stable descending sort like any other entry."""
    W, H, j = _dead_problem(34)
    d = np.diag(H).copy()
    d[j] = 1.0
    want = sorted(range(len(d)), key=lambda i: (-d[i], i))
    _, perm = O.prepare(H, 0.01, act_order=True)
    assert list(perm) == want


# ---------------------------------------------------------------- fp16 scales
def test_round_fp16_is_binary16_rounding():
    """The oracle's binary16 rounding (written from the format) equals
    numpy's float16 conversion (a library routine) on values across the
    normal and subnormal ranges, and the reading for values that round to
    zero gives the smallest subnormal."""
    r = np.random.default_rng(14)
    s = np.concatenate([10.0 ** r.uniform(-7.5, 4.5, 20000), 2.0 ** np.arange(-24, 15, dtype=np.float64),
                        (1.0 + (2 * np.arange(1, 200) + 1) * 2.0 ** -11)])
    s16, t, ulp = O.round_fp16(s)
    ref = s.astype(np.float16).astype(np.float64)
    ok = ref > 0
    assert np.array_equal(s16[ok], ref[ok])
    assert np.all(s16[~ok] == 2.0 ** -24)
    assert np.all(s16 > 0)


def test_round_fp16_hand_values():
    """1 is exact (t = 1024, margin 0.5); 1 + 2^-11 is an exact tie that goes
    to the even neighbour 1 (margin 0); 1 + 3 * 2^-11 ties to 1 + 2^-9;
    3 * 2^-26 lies in the subnormal range (ulp 2^-24, t = 0.75) and rounds
    to 2^-24; 0.1 rounds to 1638 * 2^-14."""
    s16, t, _ = O.round_fp16(np.array([1.0, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 3 * 2.0 ** -26, 0.1]))
    assert s16.tolist() == [1.0, 1.0, 1 + 2.0 ** -9, 2.0 ** -24, 1638 * 2.0 ** -14]
    assert np.allclose(O.tie_distance(t[:3]), [0.5, 0.0, 0.0], atol=1e-12)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_fp16_scales_diagonal_hessian_is_rtn(bits):
    """With binary16 scales GPTQ on a diagonal H is round-to-nearest on the
    same binary16 grid, and every stored scale is a binary16 value."""
    r = np.random.default_rng(15 + bits)
    W = r.standard_normal((9, 64)) * 0.02
    o = O.gptq_o2(W, 2.0 * np.eye(64), bits, 16, 0.01, 16, scale_fp16=True)
    rt = O.rtn(W, bits, 16, scale_fp16=True)
    assert np.array_equal(o["codes"], rt["codes"])
    assert np.array_equal(o["scales"], rt["scales"])
    assert np.array_equal(o["scales"], o["scales"].astype(np.float16).astype(np.float64))
    assert np.array_equal(o["w_hat"], rt["w_hat"])


def test_fp16_scales_hand_worked_group():
    """One 4-bit group (maxq 15) with range [-0.5, 1.0]: s = 0.1 exactly in
    float64, binary16 0.0999755859375 (1638 * 2^-14); z = rint(0.5 / s16)
    = rint(5.0012...) = 5; w = 0.3 -> rint(0.3 / s16) = 3 -> code 8,
    w_hat = 3 s16."""
    W = np.array([[-0.5, 1.0, 0.3, 0.0]])
    rt = O.rtn(W, 4, 4, scale_fp16=True)
    s16 = 1638 * 2.0 ** -14
    assert rt["scales"][0, 0] == s16
    assert rt["zeros"][0, 0] == 5
    assert rt["codes"][0].tolist() == [0, 15, 8, 5]
    assert rt["w_hat"][0, 2] == 3 * s16
    plain = O.rtn(W, 4, 4)
    assert plain["scales"][0, 0] == 0.1


@pytest.mark.parametrize("act_order", [False, True])
def test_fp16_scales_o1_equals_o2(act_order):
    W, X = _tiny(41, 12, 96, 500, heavy=True)
    H = O.hessian(X)
    o1 = O.gptq_o1(W, H, 3, 32, 0.01, act_order=act_order, scale_fp16=True)
    o2 = O.gptq_o2(W, H, 3, 32, 0.01, 16, act_order=act_order, scale_fp16=True)
    ok = (o1["codes"] == o2["codes"]) | (o2["margins"][:, np.argsort(o2["perm"])] < 1e-8)
    assert ok.all()
    assert np.array_equal(o1["scales"], o2["scales"]) or np.all(o2["smargins"] < 1e-8)
    assert np.allclose(o1["w_hat"], o2["w_hat"], atol=1e-10)
    D = (W - o2["w_hat"])[:, o2["perm"]]
    Hd, _ = O.prepare(H, 0.01, act_order)
    assert np.allclose(o2["row_loss"], np.einsum("ri,ij,rj->r", D, Hd, D), rtol=1e-9)


def test_fp16_scale_tie_branch():
    """The other branch of a scale decision: that group's scale moves to the
    other binary16 neighbour, earlier decisions are unchanged, and the run is
    still a GPTQ run (loss identity)."""
    W, X = _tiny(42, 6, 64, 400, heavy=True)
    H = O.hessian(X)
    Hd, perm = O.prepare(H, 0.01)
    U = O.upper_chol_of_inverse(Hd)
    a = O.gptq_o2(W, H, 3, 16, 0.01, 16, U=U, perm=perm, scale_fp16=True)
    r, g = 2, 1
    b = O.gptq_o2(W, H, 3, 16, 0.01, 16, U=U, perm=perm, scale_fp16=True, alt=((), (), [(r, g)]))
    s_a, s_b = a["scales"][r, g], b["scales"][r, g]
    assert s_a != s_b and abs(s_a - s_b) <= 2.0 ** -10 * s_a
    assert np.array_equal(a["codes_proc"][r, :16 * g], b["codes_proc"][r, :16 * g])
    assert np.array_equal(np.delete(a["codes_proc"], r, 0), np.delete(b["codes_proc"], r, 0))
    D = (W - b["w_hat"])[:, perm]
    assert np.allclose(b["row_loss"], np.einsum("ri,ij,rj->r", D, Hd, D), rtol=1e-9)
