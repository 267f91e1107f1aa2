"""Pins of the OLrC / Bid-Up refinement oracle (oracle/intrinsic.py) against
what the page and the mathematics fix ("Resumen Técnico: GPTQ-intrinsic
LoRA", "Refinamiento Bid-Up": coordinate updates on a fixed grid, OLrC for
fixed Q, a layer error that never increases): a hand-worked pass, the
diagonal case against exhaustive search per coordinate, monotonicity after
every coordinate step, a coordinate-wise optimum at the fixed point
(exhaustive over every code of every coordinate), and non-increasing
losses over whole cycles. Planted mistakes must fail."""
import inspect
import types

import numpy as np
import pytest

import oracle.intrinsic as IN
from oracle import eora as E
from oracle import gptq_f64 as O


def _grid(seed, d_out, n, bits, group):
    r = np.random.default_rng(seed)
    W = r.standard_normal((d_out, n)) * 0.02
    rt = O.rtn(W, bits, group)
    return W, rt["codes"], rt["scales"], rt["zeros"].astype(np.float64), np.arange(n) // group


def _H(seed, n, T=None):
    r = np.random.default_rng(seed)
    X = r.standard_t(4, (T or 4 * n, n))
    X[:, r.integers(0, n)] *= 6.0
    return 2.0 * X.T @ X


def test_hand_worked_pass():
    """One row, two columns, 2-bit grid s = 1, z = 0, H = [[2, 1], [1, 2]],
    target (1.6, 0.2), codes (0, 0). Column 0: g = (dH)_0 = 3.4, minimiser
    0 + 3.4 / 2 = 1.7 -> code 2, g_1 becomes 2.0 - 2 * 1 = 0. Column 1:
    0 + 0 / 2 -> code 0. Objective 0.24, the minimum over all 16 code pairs;
    a second pass changes nothing."""
    H = np.array([[2.0, 1.0], [1.0, 2.0]])
    T = np.array([[1.6, 0.2]])
    c, mg, hist = IN.bidup(T, np.zeros((1, 2), np.uint8), np.ones((1, 1)), np.zeros((1, 1)), [0, 0], H, 2,
                           passes=2)
    assert c.tolist() == [[2, 0]]
    assert hist[1] == pytest.approx(0.24, abs=1e-12) and hist[2] == pytest.approx(0.24, abs=1e-12)
    best = min(float(((T - np.array([[a, b]])) @ H @ (T - np.array([[a, b]])).T)[0, 0])
               for a in range(4) for b in range(4))
    assert best == pytest.approx(0.24, abs=1e-12)
    assert mg[0][0, 0] == pytest.approx(0.2, abs=1e-12) and mg[0][0, 1] == pytest.approx(0.5, abs=1e-12)


def test_diagonal_H_is_nearest_grid_point():
    """With a diagonal H the coordinates decouple: one pass puts every code
    on the grid point nearest the target (exhaustive over the codes)."""
    W, codes, sc, z, gi = _grid(1, 16, 64, 3, 16)
    H = np.diag(np.random.default_rng(2).uniform(0.5, 3.0, 64))
    T = W + 0.003 * np.random.default_rng(3).standard_normal(W.shape)
    c, _, _ = IN.bidup(T, codes, sc, z, gi, H, 3)
    S, Z = sc[:, gi], z[:, gi]
    levels = np.arange(8.0)
    err = (T[:, :, None] - S[:, :, None] * (levels[None, None, :] - Z[:, :, None])) ** 2
    assert np.array_equal(c, np.argmin(err, axis=2).astype(np.uint8))


def test_every_coordinate_step_is_non_increasing():
    W, codes, sc, z, gi = _grid(4, 5, 24, 2, 8)
    H = _H(5, 24)
    T = W + 0.004 * np.random.default_rng(6).standard_normal(W.shape)
    prev = IN.objective(T, IN.dequant(codes, sc, z, gi), H)
    # single-column passes: Bid-Up restricted to column j is one coordinate step
    c = codes.copy()
    for p in range(2):
        for j in range(24):
            before = IN.objective(T, IN.dequant(c, sc, z, gi), H)
            keep = np.arange(24) != j
            # a non-positive curvature makes a pass skip a column (B3): only column j moves,
            # and its gradient still sees H's true coupling
            cj, _, _ = IN.bidup(T, c, sc, z, gi, np.where(np.eye(24, dtype=bool) & keep[:, None], -1.0, H), 2)
            assert np.array_equal(np.delete(cj, j, 1), np.delete(c, j, 1))
            after = IN.objective(T, IN.dequant(cj, sc, z, gi), H)
            assert after <= before * (1 + 1e-12)
            c = cj
    c2, _, hist = IN.bidup(T, codes, sc, z, gi, H, 2, passes=3)
    assert all(b <= a * (1 + 1e-12) for a, b in zip(hist, hist[1:]))
    assert hist[-1] < prev


def test_fixed_point_is_coordinatewise_optimal():
    """After enough passes no code changes, and no single code change of any
    coordinate lowers the objective (exhaustive over every code)."""
    W, codes, sc, z, gi = _grid(7, 4, 20, 2, 10)
    H = _H(8, 20)
    T = W + 0.005 * np.random.default_rng(9).standard_normal(W.shape)
    c, _, hist = IN.bidup(T, codes, sc, z, gi, H, 2, passes=20)
    c2, _, _ = IN.bidup(T, c, sc, z, gi, H, 2, passes=1)
    assert np.array_equal(c, c2)
    base = ((T - IN.dequant(c, sc, z, gi)) @ H * (T - IN.dequant(c, sc, z, gi))).sum(1)
    for r in range(4):
        for j in range(20):
            for v in range(4):
                cc = c.copy()
                cc[r, j] = v
                D = T - IN.dequant(cc, sc, z, gi)
                assert (D[r] @ H @ D[r]) >= base[r] * (1 - 1e-12) - 1e-18


def test_refine_losses_never_increase():
    """Cycles of OLrC then Bid-Up starting from round-to-nearest codes: the
    layer objective never increases, OLrC lowers it, and the first OLrC is
    the EoRA adapter of the current error."""
    for seed in range(5):
        W, codes, sc, z, gi = _grid(20 + seed, 12, 48, 2, 16)
        H = _H(30 + seed, 48)
        c, B, A, losses = IN.refine(W, H, codes, sc, z, gi, 2, rank=3, cycles=3, passes=2)
        assert all(b <= a * (1 + 1e-12) for a, b in zip(losses, losses[1:])), losses
        assert losses[1] < losses[0]
        B0, A0, _ = E.eora(W, IN.dequant(codes, sc, z, gi), H, 3)
        assert losses[1] == pytest.approx(IN.objective(W, IN.dequant(codes, sc, z, gi), H, B0, A0), rel=1e-12)


# ---- planted mistakes ------------------------------------------------------
def _mutant(old, new):
    src = inspect.getsource(IN)
    assert src.count(old) == 1, old
    m = types.ModuleType("oracle.intrinsic_mutant")
    m.__package__ = "oracle"
    exec(compile(src.replace(old, new), "intrinsic_mutant", "exec"), m.__dict__)
    return m


def _battery(M):
    H = np.array([[2.0, 1.0], [1.0, 2.0]])
    T = np.array([[1.6, 0.2]])
    c, _, hist = M.bidup(T, np.zeros((1, 2), np.uint8), np.ones((1, 1)), np.zeros((1, 1)), [0, 0], H, 2, passes=2)
    assert c.tolist() == [[2, 0]]
    W, codes, sc, z, gi = _grid(7, 4, 20, 2, 10)
    H = _H(8, 20)
    T = W + 0.005 * np.random.default_rng(9).standard_normal(W.shape)
    c, _, hist = M.bidup(T, codes, sc, z, gi, H, 2, passes=20)
    assert all(b <= a * (1 + 1e-12) for a, b in zip(hist, hist[1:]))
    base = ((T - M.dequant(c, sc, z, gi)) @ H * (T - M.dequant(c, sc, z, gi))).sum(1)
    for r in range(4):
        for j in range(20):
            for v in range(4):
                cc = c.copy()
                cc[r, j] = v
                D = T - M.dequant(cc, sc, z, gi)
                assert (D[r] @ H @ D[r]) >= base[r] * (1 - 1e-12) - 1e-18


MUTANTS = [
    ("step against the gradient", "pre = c[:, j] + G[:, j] / (h * S[:, j])", "pre = c[:, j] - G[:, j] / (h * S[:, j])"),
    ("step without the scale", "pre = c[:, j] + G[:, j] / (h * S[:, j])", "pre = c[:, j] + G[:, j] / h"),
    ("gradient not updated", "G -= np.outer(delta, H[j])", "G -= 0.0 * np.outer(delta, H[j])"),
    ("gradient update sign", "G -= np.outer(delta, H[j])", "G += np.outer(delta, H[j])"),
    ("step of twice the minimiser", "pre = c[:, j] + G[:, j] / (h * S[:, j])",
     "pre = c[:, j] + 2.0 * G[:, j] / (h * S[:, j])"),
]


def test_battery_passes_on_the_oracle():
    _battery(IN)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutation_is_caught(name, old, new):
    with pytest.raises(AssertionError):
        _battery(_mutant(old, new))
