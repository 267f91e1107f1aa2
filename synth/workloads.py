"""Seeded synthetic layer workloads.

Five recipes describe the layer shapes and input statistics the quantizer is
exercised on (weights, calibration activations with heavy tails, outlier
channels, gated-MLP inputs, a low-rank spike, an augmented calibration
matrix). Every recipe can be instantiated at its full size or at a reduced
shape with the same statistics, for tests that must finish in seconds.

Random numbers come from ``numpy.random.Generator(PCG64(1000*index + id))``
with tensor ids 0 = W, 1 = X, 2 = outlier-channel choice, 3 = second factor
(gate y or spike Z), 4 = spike basis V; the token-chunked tensors (X, y, Z)
use one generator per chunk of CHUNK tokens, seeded with
``SeedSequence([1000*index + id, chunk])``, whose float64 uniforms are
turned into normals (Box-Muller) and Student-t(4) values (closed-form
inverse CDF) in float64. Samples are drawn in float64,
rounded once to float32 (round to nearest even) and, for bf16 tensors, once
more to bf16 (round to nearest even on the float32 bits). The same bf16 or
float32 values are handed to the GPU path and, upcast exactly, to the oracle.

Nothing here implements the quantization method.
"""
import os
from dataclasses import dataclass, field

import numpy as np
import torch

RECIPES = {
    # tiny layer: fp32 everything, 4 outlier channels x20
    "c1": dict(index=1, d_out=128, n=128, T=512, w_std=0.02, w_dtype="f32",
               x_dtype="f32", x_kind="gauss_outliers", n_outliers=4,
               outlier_scale=20.0, bits=4, group=128, block=128, damp=0.01,
               act_order=False, h_given=False, aug_rank=0),
    # attention projection: Student-t(4) activations, 1% outlier channels x30
    "c2": dict(index=2, d_out=4096, n=4096, T=131072, w_std=0.02,
               w_dtype="bf16", x_dtype="bf16", x_kind="t4_outliers",
               outlier_frac=0.01, outlier_scale=30.0, bits=4, group=128,
               block=128, damp=0.01, act_order=False, h_given=False,
               aug_rank=0),
    # MLP down projection: x*sigmoid(x)*y gated inputs, act-order, 3-bit
    "c3": dict(index=3, d_out=4096, n=11008, T=65536, w_std=0.015,
               w_dtype="bf16", x_dtype="bf16", x_kind="silu_gated", bits=3,
               group=128, block=128, damp=0.01, act_order=True,
               h_given=False, aug_rank=0),
    # large 2-bit layer; H given in fp32 from Gaussian X with a rank-32 spike
    "c4": dict(index=4, d_out=8192, n=28672, T=32768, w_std=0.01,
               w_dtype="bf16", x_dtype="f64", x_kind="gauss_spike",
               spike_rank=32, spike_scale=10.0, bits=2, group=64, block=128,
               damp=0.01, act_order=False, h_given=True, aug_rank=0),
    # augmented calibration matrix [X, X V_r], r = 64 appended columns
    "c5": dict(index=5, d_out=5120, n=5120, T=65536, w_std=0.02,
               w_dtype="bf16", x_dtype="bf16", x_kind="t4", bits=2,
               group=128, block=128, damp=0.01, act_order=False,
               h_given=False, aug_rank=64),
}


def rng(index, tensor_id):
    return np.random.Generator(np.random.PCG64(1000 * index + tensor_id))


def f32_to_bf16_bits(a):
    """float array -> uint16 bf16 bit patterns: round to float32 (nearest
    even), then to bf16 (nearest even on the float32 bits). torch's CPU
    casts implement exactly these roundings and run multi-threaded."""
    t = torch.from_numpy(np.ascontiguousarray(a)).to(torch.float32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b):
    u = np.asarray(b, np.uint16)
    return torch.from_numpy(u.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()


def _round(a, dtype):
    """float64 samples -> (float32 values, uint16 bits or None)."""
    if dtype == "bf16":
        bits = f32_to_bf16_bits(a)
        return bf16_bits_to_f32(bits), bits
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.float32).numpy(), None


def gen_W(recipe, d_out, n):
    """Weights ~ N(0, w_std^2): (float32 values, bf16 bits or None)."""
    r = rng(recipe["index"], 0)
    w = r.standard_normal((d_out, n)) * recipe["w_std"]
    return _round(w, recipe["w_dtype"])


def _outlier_channels(recipe, n):
    if "n_outliers" in recipe:
        k = recipe["n_outliers"]
    elif "outlier_frac" in recipe:
        k = int(round(recipe["outlier_frac"] * n))
    else:
        return np.zeros(0, np.int64)
    k = min(max(k, 1), n)
    return np.sort(rng(recipe["index"], 2).choice(n, k, replace=False))


def _spike_basis(recipe, n):
    k = recipe["spike_rank"]
    g = rng(recipe["index"], 4).standard_normal((n, k))
    q, _ = np.linalg.qr(g)
    return q


CHUNK = 16384   # tokens per calibration chunk; each chunk has its own stream


def chunk_rng(index, tensor_id, c):
    """Generator for chunk c of tensor ``tensor_id``: independent per chunk
    so chunks can be drawn in parallel and in any order."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([1000 * index + tensor_id, c])))


def _uniform_open(r, shape):
    """Uniforms in the open interval (0, 1) from the generator's doubles."""
    return torch.from_numpy(r.random(shape)).add_(2.0 ** -54)


def _normal(r, shape):
    """N(0, 1) by Box-Muller from two uniform fields (float64)."""
    u1 = _uniform_open(r, shape)
    u2 = torch.from_numpy(r.random(shape))
    return torch.sqrt(-2.0 * torch.log(u1)) * torch.cos((2.0 * np.pi) * u2)


def _student_t4(r, shape):
    """Student-t with 4 degrees of freedom by its closed-form inverse CDF:
    t = sign(u - 1/2) * 2 * sqrt(cos(arccos(sqrt(a)) / 3) / sqrt(a) - 1),
    a = 4 u (1 - u)."""
    u = _uniform_open(r, shape)
    a = 4.0 * u * (1.0 - u)
    sa = torch.sqrt(a)
    t = 2.0 * torch.sqrt(torch.clamp(torch.cos(torch.arccos(sa) / 3.0) / sa - 1.0, min=0.0))
    return torch.where(u < 0.5, -t, t)


def _x_chunk(recipe, c, T, n, cols, V):
    kind = recipe["x_kind"]
    t0 = c * CHUNK
    m = min(CHUNK, T - t0)
    rx = chunk_rng(recipe["index"], 1, c)
    if kind == "gauss_outliers":
        x = _normal(rx, (m, n))
    elif kind in ("t4_outliers", "t4"):
        x = _student_t4(rx, (m, n))
    elif kind == "silu_gated":
        a = _normal(rx, (m, n))
        y = _normal(chunk_rng(recipe["index"], 3, c), (m, n))
        x = a * torch.sigmoid(a) * y
    elif kind == "gauss_spike":
        z = _normal(chunk_rng(recipe["index"], 3, c), (m, recipe["spike_rank"]))
        x = _normal(rx, (m, n)) + recipe["spike_scale"] * (z @ torch.from_numpy(V).T)
    else:
        raise ValueError(kind)
    if cols.size:
        x[:, torch.from_numpy(cols)] *= recipe.get("outlier_scale", 1.0)
    x = x.numpy()
    if recipe["x_dtype"] == "f64":
        return t0, x, None
    vals, bits = _round(x, recipe["x_dtype"])
    return t0, vals, bits


def iter_X(recipe, T, n, workers=None):
    """Yield (t0, values float32-or-float64, bf16 bits or None) for the
    calibration matrix in chunks of CHUNK tokens, in order. Chunks are drawn
    in a thread pool (each has its own generator, so the values do not depend
    on the number of workers)."""
    from concurrent.futures import ThreadPoolExecutor
    cols = _outlier_channels(recipe, n)
    V = _spike_basis(recipe, n) if recipe["x_kind"] == "gauss_spike" else None
    nch = (T + CHUNK - 1) // CHUNK
    workers = workers or min(2, max(nch, 1))
    if workers <= 1 or nch <= 1:
        for c in range(nch):
            yield _x_chunk(recipe, c, T, n, cols, V)
        return
    with ThreadPoolExecutor(workers) as ex:
        futs = [ex.submit(_x_chunk, recipe, c, T, n, cols, V) for c in range(min(nch, workers))]
        nxt = len(futs)
        for c in range(nch):
            res = futs[c].result()
            futs[c] = None
            if nxt < nch:
                futs.append(ex.submit(_x_chunk, recipe, nxt, T, n, cols, V))
                nxt += 1
            yield res


def x_full(recipe, T, n, workers=None):
    """Whole calibration matrix: (values, bits or None), filled chunk by chunk."""
    vals = bits = None
    for t0, v, b in iter_X(recipe, T, n, workers):
        if vals is None:
            vals = np.empty((T, n), v.dtype)
            bits = None if b is None else np.empty((T, n), np.uint16)
        vals[t0:t0 + v.shape[0]] = v
        if b is not None:
            bits[t0:t0 + v.shape[0]] = b
    return vals, bits


def augment_basis(x_vals, r):
    """Top-r right singular vectors of X (eigenvectors of X^T X for the r
    largest eigenvalues), float64, each column's largest-magnitude entry made
    positive so the basis is reproducible. Input preparation for the
    augmented-calibration workload: [X, X V_r]."""
    gram = np.zeros((x_vals.shape[1],) * 2)
    for t0 in range(0, x_vals.shape[0], 16384):
        xc = x_vals[t0:t0 + 16384].astype(np.float64)
        gram += xc.T @ xc
    evals, evecs = np.linalg.eigh(gram)
    V = evecs[:, ::-1][:, :r].copy()
    idx = np.argmax(np.abs(V), axis=0)
    V *= np.sign(V[idx, np.arange(r)])
    return V


@dataclass
class Workload:
    """One instantiated layer problem."""
    name: str
    recipe: dict
    d_out: int
    n: int                       # columns of W (augmented width for c5)
    n_quant: int
    T: int
    W: np.ndarray                # float32 values (exact bf16 values if bf16)
    W_bits: np.ndarray = None    # uint16 bf16 bits, or None for fp32
    X: np.ndarray = None         # float32 (exact bf16 values), or None
    X_bits: np.ndarray = None
    H: np.ndarray = None         # float32 given Hessian (h_given recipes)
    params: dict = field(default_factory=dict)


def make_workload(name, d_out=None, n=None, T=None, with_x=True, H_fn=None,
                  aug_rank=None, **overrides):
    """Instantiate recipe ``name`` at full or reduced shape.

    For recipes whose Hessian is given (``h_given``), ``H_fn(X_chunks)`` must
    be supplied by the caller to accumulate it (float64), and the result is
    rounded once to float32 here; this module does not compute it itself.
    ``overrides`` replace quantizer parameters (bits, group, block, damp,
    act_order) for reduced shapes whose width the recipe's group does not
    divide; ``aug_rank`` overrides the number of appended columns.
    """
    rc = RECIPES[name]
    d_out = rc["d_out"] if d_out is None else d_out
    n0 = rc["n"] if n is None else n
    T = rc["T"] if T is None else T
    W, Wb = gen_W(rc, d_out, n0)
    params = dict(bits=rc["bits"], group=rc["group"], block=rc["block"],
                  damp=rc["damp"], act_order=rc["act_order"])
    params.update(overrides)
    wl = Workload(name=name, recipe=rc, d_out=d_out, n=n0, n_quant=n0, T=T,
                  W=W, W_bits=Wb, params=params)
    if rc["h_given"]:
        if H_fn is not None:
            Hd = H_fn(iter_X(rc, T, n0))
            wl.H = np.asarray(Hd, np.float64).astype(np.float32)
        return wl
    if not with_x:
        return wl
    X, Xb = x_full(rc, T, n0)
    r = rc["aug_rank"] if aug_rank is None else aug_rank
    if r:
        V = augment_basis(X, r)
        xa, xab = _round(X.astype(np.float64) @ V, rc["x_dtype"])
        X = np.concatenate([X, xa], axis=1)
        Xb = None if Xb is None else np.concatenate([Xb, xab], axis=1)
        wl.W = np.concatenate([W, np.zeros((d_out, r), np.float32)], axis=1)
        if Wb is not None:
            wl.W_bits = np.concatenate([Wb, np.zeros((d_out, r), np.uint16)], axis=1)
        wl.n = n0 + r
        wl.n_quant = n0
    wl.X, wl.X_bits = X, Xb
    return wl
