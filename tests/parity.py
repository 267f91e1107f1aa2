"""Parity helpers shared by the GPU tests: move seeded inputs to the GPU,
run the oracle on the same values, and apply the acceptance rules.

Acceptance (float decides the integer codes; the oracle is float64, the GPU
path fp32, so decisions can differ only where the oracle's pre-rounding value
sits next to a half-integer):
  * H: relative Frobenius error <= 1e-5.
  * codes: identical on >= 99.9% of entries, and in every row the first
    differing decision (zero point at a group start, or code) in processing
    order is a tie for the oracle: its pre-rounding value lies within
    TAU = 1e-3 quantization steps of a half-integer. Later differences in
    the same row are the cascade of that tie.
  * layer error r within 1e-3 (relative) of the oracle's.
"""
import numpy as np
import torch

from oracle import gptq_f64 as O

TAU = 1e-3


def to_dev(wl_vals, bits=None, dtype="f32"):
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(wl_vals, dtype=np.float32))
    return t.cuda()


def w_dev(wl):
    return to_dev(wl.W, wl.W_bits, "bf16" if wl.W_bits is not None else "f32")


def x_dev(wl):
    return to_dev(wl.X, wl.X_bits, "bf16" if wl.X_bits is not None else "f32")


def rel_fro(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def first_mismatch_report(gpu_codes_orig, gpu_zeros, orc, group, tau=TAU):
    """Returns (identity_rate, rows_with_mismatch, bad_rows) where bad_rows
    lists rows whose first differing decision is not an oracle tie."""
    perm = orc["perm"]
    nq = gpu_codes_orig.shape[1]
    g = np.asarray(gpu_codes_orig)[:, perm[:nq]]
    o = orc["codes_proc"]
    cm = g != o
    zm = np.asarray(gpu_zeros) != orc["zeros"]
    rate = 1.0 - cm.mean()
    bad = []
    rows = np.nonzero(cm.any(1) | zm.any(1))[0]
    for r in rows:
        jc = int(np.argmax(cm[r])) if cm[r].any() else nq
        gz = int(np.argmax(zm[r])) if zm[r].any() else nq
        jz = gz * group if gz < zm.shape[1] else nq
        if jz <= jc:
            ok = orc["zmargins"][r, gz] < tau
        else:
            ok = orc["margins"][r, jc] < tau
        if not ok:
            bad.append(int(r))
    return rate, len(rows), bad


def check_quant(res, wl, H64, orc, params, nq, report=None):
    """Apply the acceptance rules to a QuantResult against oracle output."""
    codes = res.codes.cpu().numpy()
    zeros = res.zeros.cpu().numpy()
    rate, nrows, bad = first_mismatch_report(codes, zeros, orc, params["group"])
    w_hat = res.w_hat.cpu().numpy().astype(np.float64)
    r_gpu = O.layer_error(wl.W, w_hat, H64)
    r_orc = O.layer_error(wl.W, orc["w_hat"], H64)
    info = dict(identity=rate, rows_mismatch=nrows, bad_rows=bad[:10], r_gpu=r_gpu, r_oracle=r_orc)
    if report is not None:
        report.update(info)
    assert rate >= 0.999, info
    assert not bad, info
    assert abs(r_gpu - r_orc) <= 1e-3 * r_orc, info
    # g_idx is integer work: exact
    assert np.array_equal(res.g_idx.cpu().numpy(), orc["g_idx"]), "g_idx"
    return info
