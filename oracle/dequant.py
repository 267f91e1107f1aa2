"""Dequantising matrix product of a packed low-bit layer (oracle side).

TEST INFRASTRUCTURE (see the package docstring).

[BAL] section 6: a low-bit layer only pays at inference through a kernel
that unpacks, dequantises and multiplies; small-batch decoding and
large-batch prefill are different regimes and are measured separately.
[BAL] section 1: the affine reconstruction w = s (q - z) with the scale and
zero point of the weight's group, and the packing layout of
:mod:`oracle.packing` (reading R17).

The product is Y = X W_hat^T (X: tokens x n, W_hat: d_out x n), written
out in float64 from its definition; nothing here is blocked or factored.
"""
import numpy as np

from oracle.packing import unpack


def dequantize(qweight, scales, zeros, bits, group, n, g_idx=None):
    """W_hat[o][k] = scales[o][g(k)] * (code(o, k) - zeros[o][g(k)]) in float64,
    g(k) = g_idx[k] (k // group when g_idx is None)."""
    codes = unpack(qweight, n, bits).astype(np.float64)
    g = np.arange(n) // group if g_idx is None else np.asarray(g_idx)
    s = np.asarray(scales, np.float64)[:, g]
    z = np.asarray(zeros, np.float64)[:, g]
    return s * (codes - z)


def dequant_matmul(X, qweight, scales, zeros, bits, group, g_idx=None):
    """Y = X W_hat^T in float64 (X given as float values, e.g. bf16 upcast)."""
    X = np.asarray(X, np.float64)
    W = dequantize(qweight, scales, zeros, bits, group, X.shape[1], g_idx)
    return X @ W.T


def dequant_matmul_loops(X, qweight, scales, zeros, bits, group):
    """The same product as explicit sums over every (token, output, input)
    triple with each code read by bit arithmetic from its words: tiny
    inputs only."""
    X = np.asarray(X, np.float64)
    M, n = X.shape
    qw = np.asarray(qweight, np.uint64)
    d_out = qw.shape[0]
    Y = np.zeros((M, d_out))
    for o in range(d_out):
        for k in range(n):
            bit = k * bits
            w, sh = bit // 32, bit % 32
            v = int(qw[o, w]) >> sh
            if sh + bits > 32:
                v |= int(qw[o, w + 1]) << (32 - sh)
            q = v & ((1 << bits) - 1)
            wk = float(scales[o][k // group]) * (q - int(zeros[o][k // group]))
            for m in range(M):
                Y[m, o] += X[m, k] * wk
    return Y
