"""Host-side checks of the benchmark's contract and bookkeeping (no GPU):
it refuses more than one GPU with a message, the profile classes of the
binding match the header's count, and its count of the inverse's
six-product block products follows the recursive doubling's levels."""
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_profile_classes_match_the_header():
    from post_weight_quantization_28_amd import gptq
    src = open(os.path.join(ROOT, "include", "gptq.h")).read()
    n = int(re.search(r"GPTQ_PROF_NCLASSES\s*=\s*(\d+)", src).group(1))
    assert len(gptq.PROF_CLASSES) == n
    assert gptq.PROF_CLASSES[int(re.search(r"GPTQ_PROF_INVERSE_X6\s*=\s*(\d+)", src).group(1))] == "inverse_x6"


def _levels(n):
    """(h, hj, batch) of every set of pairs of the inverse's recursive
    doubling: blocks of h rows paired with the next h (or the hj left)."""
    out, h = [], 64
    while h < n:
        full = n // (2 * h)
        if full:
            out.append((h, h, full))
        rest = n - full * 2 * h - h
        if rest > 0:
            out.append((h, rest, 1))
        h *= 2
    return out


def test_six_product_count_and_flops():
    # no level has 1024 output tiles of 128 x 128 below 8065 columns
    for n in (4096, 5184, 6208):
        assert bench.inverse_x6_work(n) == (0.0, 0)
    for n, want in ((10246, 4), (11008, 4), (28672, 10)):
        flops, products = bench.inverse_x6_work(n)
        assert products == want
        # the same flops from the levels, counted as triangular products:
        # T^T = X_ii^T L_ji^T has sum over output rows m of (h - m) terms per
        # column, X_ji = -X_jj T sum over rows m of (m + 1) terms per column
        ref = 0
        for h, hj, batch in _levels(n):
            if h >= 1024 and -(-h // 128) * -(-hj // 128) * batch >= 1024:
                ref += batch * 2 * (hj * sum(h - m for m in range(h)) + h * sum(m + 1 for m in range(hj)))
        assert flops == ref
    # nearly all of the inverse's (1/3) n^3 flops at the widest layer
    flops, _ = bench.inverse_x6_work(28672)
    assert 0.99 < flops / (28672 ** 3 / 3) < 1.0
