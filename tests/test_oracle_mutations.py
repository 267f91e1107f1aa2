"""Planted mistakes: each test edits one line of a copy of the oracle (on the
CPU, in memory) and checks that the pin battery rejects the copy. This shows
the pins are sensitive to the plausible errors (sign, dropped term, wrong
index, transposed operand, wrong rounding) rather than passing vacuously."""
import inspect
import types

import numpy as np
import pytest

import oracle.gptq_f64 as ORIG
import oracle.packing as PORIG


def _mutant(module, old, new):
    src = inspect.getsource(module)
    assert src.count(old) >= 1, old
    src = src.replace(old, new)
    m = types.ModuleType(module.__name__ + "_mutant")
    exec(compile(src, module.__name__ + "_mutant", "exec"), m.__dict__)
    return m


def _tiny(seed, d_out, n, T):
    r = np.random.default_rng(seed)
    X = r.standard_t(4, (T, n))
    X[:, r.integers(0, n)] *= 10.0
    return r.standard_normal((d_out, n)) * 0.02, X


# ---- the battery (each returns normally if the pin holds) ----------------
def pin_hessian(O):
    r = np.random.default_rng(1)
    X = r.standard_normal((9, 3))
    ref = sum(2.0 * np.outer(x, x) for x in X)
    assert np.allclose(O.hessian(X), ref, rtol=1e-13)


def pin_grid(O):
    W = np.array([[1.5, -0.25, 0.125, 0.375], [0.5, 1.75, 0.25, 1.0],
                  [-0.5, -1.75, -0.25, -1.0], [0.0, 0.0, 0.0, 0.0]])
    res = O.rtn(W, bits=3, group=4)
    assert res["codes"].tolist() == [[7, 0, 1, 3], [2, 7, 1, 4], [5, 0, 6, 3], [4, 4, 4, 4]]
    assert np.array_equal(res["w_hat"][0], [1.5, -0.25, 0.0, 0.5])


def pin_o1_o2(O):
    W, X = _tiny(5, 8, 64, 300)
    H = O.hessian(X)
    for ao in (False, True):
        a = O.gptq_o1(W, H, 3, 16, 0.01, act_order=ao)
        b = O.gptq_o2(W, H, 3, 16, 0.01, 16, act_order=ao)
        assert np.allclose(a["w_hat"], b["w_hat"], atol=1e-10)


def pin_loss(O):
    W, X = _tiny(6, 8, 48, 300)
    H = O.hessian(X)
    Hd = H + 0.01 * np.mean(np.diag(H)) * np.eye(48)
    for f in (lambda: O.gptq_o2(W, H, 3, 16, 0.01, 16), lambda: O.gptq_o1(W, H, 3, 16, 0.01)):
        o = f()
        D = W - o["w_hat"]
        assert np.allclose(o["row_loss"], np.einsum("ri,ij,rj->r", D, Hd, D), rtol=1e-9)


def pin_n2(O):
    r = np.random.default_rng(4)
    for _ in range(20):
        W = r.standard_normal((8, 2))
        A = r.standard_normal((5, 2))
        H = 2 * A.T @ A
        Hd = H + 0.01 * np.mean(np.diag(H)) * np.eye(2)
        o = O.gptq_o2(W, H, 4, 2, 0.01, 2)
        s, z = o["scales"][:, 0], o["zeros"][:, 0].astype(float)
        w1p = W[:, 1] + (W[:, 0] - o["w_hat"][:, 0]) * Hd[0, 1] / Hd[1, 1]
        assert np.array_equal(np.clip(np.rint(w1p / s) + z, 0, 15).astype(np.uint8), o["codes"][:, 1])


def pin_perm(O):
    W, X = _tiny(7, 4, 32, 200)
    H = O.hessian(X)
    d = np.diag(H)
    perm = sorted(range(32), key=lambda i: (-d[i], i))
    a = O.gptq_o2(W, H, 3, 8, 0.01, 8, act_order=True)
    assert list(a["perm"]) == perm


def pin_rtn_special(O):
    n = 32
    r = np.random.default_rng(2)
    W = r.standard_normal((6, n)) * 0.02
    ref = O.rtn(W, 2, 8)
    o = O.gptq_o2(W, 2.0 * np.eye(n), 2, 8, 0.01, 8)
    assert np.array_equal(o["codes"], ref["codes"])


def pin_block_inv(O):
    W, X = _tiny(8, 6, 64, 300)
    H = O.hessian(X)
    a = O.gptq_o2(W, H, 4, 16, 0.01, 64)
    b = O.gptq_o2(W, H, 4, 16, 0.01, 16)
    assert np.allclose(a["w_hat"], b["w_hat"], atol=1e-12)


def pin_tie_distance(O):
    x = np.array([0.5, 1.0, -0.5, 2.49, 3.0, -1.25, -0.75, 7.5, -2.0, -2.51])
    want = [0.0, 0.5, 0.0, 0.01, 0.5, 0.25, 0.25, 0.0, 0.5, 0.01]
    assert np.allclose(O.tie_distance(x), want, atol=1e-12, rtol=0)


def pin_layer_error(O):
    r = np.random.default_rng(12)
    X = r.standard_t(4, (300, 24))
    W = r.standard_normal((7, 24)) * 0.02
    Wh = O.rtn(W, 3, 8)["w_hat"]
    ref = np.linalg.norm(X @ (W - Wh).T) ** 2 / np.linalg.norm(X @ W.T) ** 2
    assert abs(O.layer_error(W, Wh, O.hessian(X)) - ref) <= 1e-12 * ref


def pin_dead_column(O):
    r = np.random.default_rng(33)
    n, j = 16, 5
    X = r.standard_normal((200, n))
    X[:, j] = 0.0
    W = r.standard_normal((6, n)) * 0.02
    W[:, j] = 0.5 * W[:, 0]
    H = O.hessian(X)
    keep = np.delete(np.arange(n), j)
    d = np.diag(H)
    lam = 0.01 * (d.sum() + 1.0) / n
    full = O.gptq_o2(W, H, 4, n, 0.01, n)
    red = O.gptq_o2(W[:, keep], H[np.ix_(keep, keep)], 4, n - 1, lam / (d[keep].sum() / (n - 1)), n - 1)
    assert np.allclose(full["w_hat"][:, keep], red["w_hat"], atol=1e-13, rtol=0)
    extra = (W[:, j] - full["w_hat"][:, j]) ** 2 * (1.0 + lam)
    assert np.allclose(full["row_loss"], red["row_loss"] + extra, rtol=1e-10, atol=0)


def pin_chol_reversal(O):
    r = np.random.default_rng(9)
    A = r.standard_normal((80, 24))
    Hd = 2.0 * A.T @ A + 0.1 * np.eye(24)
    U = O.upper_chol_of_inverse_by_reversal(Hd)
    assert np.array_equal(U, np.triu(U)) and np.all(np.diag(U) > 0)
    assert np.abs(U.T @ U @ Hd - np.eye(24)).max() < 1e-10


def pin_fp16(O):
    s16, t, _ = O.round_fp16(np.array([1.0, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 3 * 2.0 ** -26, 0.1, 7e-5, 3e-6]))
    ref = np.array([1.0, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 3 * 2.0 ** -26, 0.1, 7e-5, 3e-6]).astype(np.float16)
    assert np.array_equal(s16, ref.astype(np.float64))
    W = np.array([[-0.5, 1.0, 0.3, 0.0]])
    assert O.rtn(W, 4, 4, scale_fp16=True)["codes"][0].tolist() == [0, 15, 8, 5]


BATTERY = [pin_hessian, pin_grid, pin_o1_o2, pin_loss, pin_n2, pin_perm,
           pin_rtn_special, pin_block_inv, pin_tie_distance, pin_layer_error, pin_dead_column,
           pin_chol_reversal, pin_fp16]


def _caught(O):
    failures = []
    for pin in BATTERY:
        try:
            pin(O)
        except (AssertionError, np.linalg.LinAlgError, ValueError, IndexError, FloatingPointError):
            failures.append(pin.__name__)
    return failures


def test_battery_passes_on_the_oracle():
    assert _caught(ORIG) == []


MUTATIONS = [
    ("in-block feedback sign", "Wp[:, j + 1:i1] -= np.outer(e, U[j, j + 1:i1])",
     "Wp[:, j + 1:i1] += np.outer(e, U[j, j + 1:i1])"),
    ("trailing update dropped", "Wp[:, i1:] -= E @ U[i0:i1, i1:]", "Wp[:, i1:] -= 0.0 * (E @ U[i0:i1, i1:])"),
    ("trailing update sign", "Wp[:, i1:] -= E @ U[i0:i1, i1:]", "Wp[:, i1:] += E @ U[i0:i1, i1:]"),
    ("error not scaled by U_jj", "e = (Wp[:, j] - what) / U[j, j]", "e = (Wp[:, j] - what)"),
    ("U transposed (lower factor)", "    return L.T\n", "    return L\n"),
    ("range not widened to 0", "xmin = np.minimum(v.min(axis=1), 0.0)", "xmin = v.min(axis=1)"),
    ("round half up", "q = np.clip(np.rint(pre) + z, 0.0, maxq)", "q = np.clip(np.floor(pre + 0.5) + z, 0.0, maxq)"),
    ("zero point dropped in reconstruction", "return q, s * (q - z), pre", "return q, s * q, pre"),
    ("damping dropped", "H[np.diag_indices(n)] += lam", "H[np.diag_indices(n)] += 0.0 * lam"),
    ("act-order ascending", 'np.argsort(-d[:nq], kind="stable")', 'np.argsort(d[:nq], kind="stable")'),
    ("Hessian factor 2 dropped", "H += 2.0 * (Xc.T @ Xc)", "H += (Xc.T @ Xc)"),
    ("O1 downdate sign", "G = G[1:, 1:] - np.outer(G[1:, 0], G[0, 1:]) / g00",
     "G = G[1:, 1:] + np.outer(G[1:, 0], G[0, 1:]) / g00"),
    ("O1 update without 1/G00", "Wp[:, j + 1:] -= np.outer(delta / g00, G[0, 1:])",
     "Wp[:, j + 1:] -= np.outer(delta, G[0, 1:])"),
    ("group start off by one", "if j % group == 0:", "if j % group == 1 or j == 0:"),
    ("tie distance without floor", "f = pre - np.floor(pre)", "f = pre - np.trunc(pre)"),
    ("tie distance to the integer", "return np.abs(f - 0.5)", "return np.minimum(f, 1.0 - f)"),
    ("tie distance signed", "return np.abs(f - 0.5)", "return f - 0.5"),
    ("layer error on damped H", "num = row_objective(W, W_hat, H).sum()",
     "num = row_objective(W, W_hat, H + 0.01 * np.mean(np.diag(H)) * np.eye(len(H))).sum()"),
    ("layer error over the weight norm", "den = row_objective(W, np.zeros_like(W), H).sum()",
     "den = float((W * W).sum())"),
    ("dead-column fix skipped", "H[dead, dead] = 1.0", "H[dead, dead] = 0.0"),
    ("dead-column value 2", "H[dead, dead] = 1.0", "H[dead, dead] = 2.0"),
    ("reversal route without the reversal", "A = np.array(np.asarray(Hd, np.float64)[::-1, ::-1], order=",
     "A = np.array(np.asarray(Hd, np.float64), order="),
    ("binary16 with 11 fraction bits", "ulp = np.exp2(e - 10.0)", "ulp = np.exp2(e - 11.0)"),
    ("binary16 without the subnormal floor", "e = np.maximum(ex - 1, -14).astype(np.float64)",
     "e = (ex - 1).astype(np.float64)"),
    ("binary16 rounding by truncation", "s16 = np.rint(t) * ulp", "s16 = np.floor(t) * ulp"),
    ("reversal route returns the lower factor", "return np.ascontiguousarray(Li[::-1, ::-1]).reshape(n, n)",
     "return np.ascontiguousarray(Li).reshape(n, n)"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(name, old, new):
    m = _mutant(ORIG, old, new)
    assert _caught(m), name


def test_packing_mutation_is_caught():
    m = _mutant(PORIG, "val = (codes[:, k] & np.uint64((1 << bits) - 1)) << np.uint64(sh)",
                "val = (codes[:, k] & np.uint64((1 << bits) - 1)) << np.uint64(sh + 1)")
    c = np.zeros((1, 11), np.uint8)
    c[0, 10] = 7
    w = m.pack(c, 3)
    assert not (int(w[0, 0]) == 0xC0000000 and int(w[0, 1]) == 1)
