"""The acceptance rules of the GPU parity tests, exercised on the CPU with
results the oracle itself produces (no GPU): a result that took the other
rounding at one of the oracle's ties is accepted, one that flipped a code
that is not a tie is rejected, and the branch reruns of the rule touch only
the rows that need them."""
import numpy as np

from oracle import gptq_f64 as O
import parity


def _problem(seed=3, d_out=32, n=128):
    r = np.random.default_rng(seed)
    X = r.standard_t(4, (600, n))
    W = r.standard_normal((d_out, n)) * 0.02
    H = O.hessian(X)
    p = dict(bits=3, group=32, damp=0.01, block=32, act_order=True)
    orc = O.gptq_o2(W, H, p["bits"], p["group"], p["damp"], p["block"], p["act_order"])
    return W, H, p, orc


def _closest_inner_decision(orc, maxq):
    cp = orc["codes_proc"]
    m = np.where((cp > 0) & (cp < maxq), orc["margins"], np.inf)
    return np.unravel_index(np.argmin(m), m.shape), m


def test_other_branch_at_a_tie_is_accepted():
    W, H, p, orc = _problem()
    (r, j), m = _closest_inner_decision(orc, 7)
    tau = 2.0 * m[r, j] + 1e-12
    br = O.gptq_o2(W, H, p["bits"], p["group"], p["damp"], p["block"], p["act_order"], alt=([(r, j)], ()))
    assert not np.array_equal(br["codes"], orc["codes"])
    rate, nrows, bad = parity.first_mismatch_report(br["codes"], br["zeros"], orc, p["group"], tau=tau)
    assert nrows == 1 and bad == []
    brate, ties, bbad = parity.tie_branch_report(br["codes"], br["zeros"], W, H, orc, p, W.shape[1], tau=tau)
    assert brate == 1.0 and bbad == [] and ties[r] == 1 and ties.sum() == 1


def test_flip_away_from_a_tie_is_rejected():
    W, H, p, orc = _problem()
    cp = orc["codes_proc"]
    m = np.where((cp > 0) & (cp < 7), orc["margins"], -np.inf)
    r, j = np.unravel_index(np.argmax(m), m.shape)       # the least tied decision
    assert m[r, j] > 0.3
    fake = orc["codes"].copy()
    col = orc["perm"][j]
    fake[r, col] = fake[r, col] + 1
    rate, nrows, bad = parity.first_mismatch_report(fake, orc["zeros"], orc, p["group"])
    assert bad == [r]
    brate, ties, bbad = parity.tie_branch_report(fake, orc["zeros"], W, H, orc, p, W.shape[1])
    assert bbad == [r] and brate < 1.0


def test_zero_point_flip_away_from_a_tie_is_rejected():
    W, H, p, orc = _problem()
    zr = np.where(orc["zeros"] < 7, orc["zmargins"], -np.inf)
    r, g = np.unravel_index(np.argmax(zr), zr.shape)
    assert zr[r, g] > 0.3
    fz = orc["zeros"].copy()
    fz[r, g] += 1
    _, _, bad = parity.first_mismatch_report(orc["codes"], fz, orc, p["group"])
    assert bad == [int(r)]


def test_binary16_scale_branch_is_accepted_and_a_flip_away_is_not():
    """With binary16 scales the scale is a rounding decision too: a result
    that took the other binary16 neighbour at the oracle's closest scale tie
    is accepted (first mismatch rule and tie branches); one whose scale moved
    where the oracle's decision is far from a tie is rejected."""
    r = np.random.default_rng(8)
    X = r.standard_t(4, (600, 128))
    W = r.standard_normal((48, 128)) * 0.02
    H = O.hessian(X)
    p = dict(bits=3, group=32, damp=0.01, block=32, act_order=False, scale_fp16=True)
    orc = O.gptq_o2(W, H, 3, 32, 0.01, 32, scale_fp16=True)
    sm = orc["smargins"]
    rr, gg = np.unravel_index(np.argmin(sm), sm.shape)
    tau = 2.0 * sm[rr, gg] + 1e-12
    br = O.gptq_o2(W, H, 3, 32, 0.01, 32, scale_fp16=True, alt=((), (), [(rr, gg)]))
    assert br["scales"][rr, gg] != orc["scales"][rr, gg]
    _, nrows, bad = parity.first_mismatch_report(br["codes"], br["zeros"], orc, 32, tau=tau,
                                                 gpu_scales=br["scales"])
    assert nrows == 1 and bad == []
    brate, ties, bbad = parity.tie_branch_report(br["codes"], br["zeros"], W, H, orc, p, 128, tau=tau,
                                                 gpu_scales=br["scales"])
    assert brate == 1.0 and bbad == [] and ties.sum() >= 1
    rf, gf = np.unravel_index(np.argmax(sm), sm.shape)
    assert sm[rf, gf] > 0.3
    fake = orc["scales"].copy()
    fake[rf, gf] *= 1.0 + 2.0 ** -10
    _, _, bad = parity.first_mismatch_report(orc["codes"], orc["zeros"], orc, 32, gpu_scales=fake)
    assert bad == [int(rf)]
