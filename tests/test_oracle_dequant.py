"""Pins of the dequantising product's oracle (oracle/dequant.py): a
hand-worked example, the explicit-loop definition with codes read by bit
arithmetic, and the sweep's own reconstruction."""
import numpy as np
import pytest

import synth
from oracle import dequant as D
from oracle import gptq_f64 as O
from oracle import packing as P


def test_hand_worked_4bit_two_groups():
    # one output row, 8 inputs, groups of 4, 4-bit codes [0 5 15 7 | 3 3 3 3]
    # packed LSB first: nibble k at bits 4k.. -> 0x33337F50
    qweight = np.array([[0x33337F50]], np.uint32)
    scales = np.array([[0.5, 0.25]])
    zeros = np.array([[7, 1]], np.uint8)
    # w_hat = [-3.5 -1 4 0 | 0.5 0.5 0.5 0.5]
    W = D.dequantize(qweight, scales, zeros, 4, 4, 8)
    assert np.array_equal(W, [[-3.5, -1.0, 4.0, 0.0, 0.5, 0.5, 0.5, 0.5]])
    X = np.array([[1, 2, 3, 4, 1, 1, 1, 1], [0, 0, 0, 0, 2, 0, 0, -2]], np.float64)
    # row 0: -3.5 - 2 + 12 + 0 + 2 = 8.5; row 1: 1 - 1 = 0
    assert np.array_equal(D.dequant_matmul(X, qweight, scales, zeros, 4, 4), [[8.5], [0.0]])


@pytest.mark.parametrize("bits,group", [(2, 8), (3, 8), (4, 16)])
def test_matches_explicit_loops(bits, group):
    r = np.random.default_rng(bits)
    M, d_out, n = 3, 5, 48
    codes = r.integers(0, 2 ** bits, (d_out, n)).astype(np.uint8)
    qw = P.pack(codes, bits)
    scales = r.uniform(0.01, 0.1, (d_out, n // group))
    zeros = r.integers(0, 2 ** bits, (d_out, n // group)).astype(np.uint8)
    X = r.standard_normal((M, n))
    a = D.dequant_matmul(X, qw, scales, zeros, bits, group)
    b = D.dequant_matmul_loops(X, qw, scales, zeros, bits, group)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("act_order", [False, True])
def test_reconstructs_the_sweeps_w_hat(act_order):
    """Unpacking what the sweep emits and dequantising gives its w_hat
    exactly, so the product is the quantized layer's output."""
    wl = synth.make_workload("c3", d_out=24, n=256, T=2048, group=64, bits=3)
    H = O.hessian(wl.X)
    o = O.gptq_o2(wl.W, H, 3, 64, 0.01, 128, act_order)
    qw = P.pack(o["codes"], 3)
    W = D.dequantize(qw, o["scales"], o["zeros"], 3, 64, 256, g_idx=o["g_idx"])
    assert np.array_equal(W, o["w_hat"])
    X = wl.X[:7].astype(np.float64)
    assert np.allclose(D.dequant_matmul(X, qw, o["scales"], o["zeros"], 3, 64, g_idx=o["g_idx"]),
                       X @ o["w_hat"].T, rtol=1e-13, atol=1e-13)
