"""Benchmark: one GPTQ layer step on one MI355X.

A step is the whole path on the 4096 x 4096 attention-projection workload:
Hessian H = 2 X^T X from 131072 bf16 calibration tokens, then quantize_layer
(damping, factorisation, blocked column sweep with trailing updates, packing)
at 4 bits, group 128, block 128. Inputs are resident in HBM before the timed
region; every step recomputes everything from X and W.

Prints one JSON line: the step throughput, the Hessian kernel against the bf16
MFMA roofline, the phases of quantize_layer (factorisation, sweep, far-field
update) with the sweep's HBM rate and the far field's MFMA rate, the copy and
GEMM rates this box measures, and the float64 oracle timed on the host cores.

`--workload eora` times the EoRA rank-64 adapter of that layer's 4-bit
GPTQ output (the compensation of the quantization error in the eigenspace of
H) and times the float64 oracle beside it.

`--config c3|c4|c5` times the other layer shapes the same way: 4096 x 11008
3-bit act-order, 8192 x 28672 2-bit with H given (the step is quantize_layer
alone; its roofline is the far-field update's), 5120 x 5184 augmented 2-bit.

`--workload dequant_matmul --tokens M` instead times the inference product
Y = X W_hat^T of a packed 4096 x 4096 4-bit g128 layer for M tokens (decode:
M = 16, bound by reading the packed weights; prefill: M = 4096, bound by the
matrix cores) and prints one JSON line for it.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GPTQ layer time & quantized weights/s (4096², 4-bit g128); Hessian TFLOP/s"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
PEAK_FP32_TFLOPS = 157.3      # MI355X dense fp32 MFMA

# HBM bytes moved by one k_hessian_dma launch on this workload, from two
# rocprofv3 counter runs of `bench.py --steps 1 --warmup 0 --no-cpu-baseline
# --copy-calibration` (FETCH_SIZE, then WRITE_SIZE, each scaled by what the
# same counter reads for the 1 GiB copy/fill that --copy-calibration runs).
# Valid only for the kernel source with the recorded SHA-256; reported as
# null once hessian.hip changes.
HESSIAN_TRAFFIC = {
    "bytes": 6567341205,
    "source_sha256": "1bb0fc52d0a4bfe86db77c89b69bbab173366867a7aa8cfedac7d90131647508",
    "profile": "profiles/k_hessian_dma_c2_hbm_traffic.md",
}
HESSIAN_SRC = os.path.join(ROOT, "post_weight_quantization_28_amd", "csrc", "hessian.hip")

# The same record for the 16-token dequantising product (k_dequant_mv on the
# packed 4096 x 4096 4-bit g128 layer), from `bench.py --workload
# dequant_matmul --tokens 16 --steps 20 --warmup 2 --no-cpu-baseline
# --copy-calibration` under the two counter passes.
DEQUANT16_TRAFFIC = {
    "bytes": 10424147,
    "source_sha256": "fd34db3af77fbf5b2cc1c7e18a3f37d1c7d6cdfd05fe5ff447e2adfd781df555",
    "profile": "profiles/k_dequant_mv_4096x4096_4bit_16tok_hbm_traffic.md",
}
DEQUANT_SRC = os.path.join(ROOT, "post_weight_quantization_28_amd", "csrc", "dqmm.hip")


def recorded_traffic(record, src):
    with open(src, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    if record["bytes"] is None or sha != record["source_sha256"]:
        return None
    return record["bytes"]


def hessian_traffic():
    return recorded_traffic(HESSIAN_TRAFFIC, HESSIAN_SRC)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def host_blas():
    """(threads, description) of the BLAS numpy uses on this host, and the CPU model."""
    import numpy  # noqa: F401  (loads the BLAS so that threadpoolctl sees it)
    threads, blas = None, "unknown BLAS"
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            threads = sum(i.get("num_threads", 0) for i in libs) or None
            blas = ", ".join(f"{i.get('internal_api')} {i.get('version')} ({i.get('architecture')}, "
                             f"{i.get('num_threads')} threads)" for i in libs)
    except Exception:
        pass
    cpu = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return threads, f"{cpu}; {os.cpu_count()} logical CPUs; {blas}"


def cpu_baseline(wl, X_vals, p, sample_tokens=4096, sample_rows=64, given_h=False, sub_n=8192):
    """The float64 oracle, untuned, on a bounded sample of the same workload,
    scaled to the whole layer step. With H given (the 28672-wide layer) the
    step has no Hessian, and the factorisation and the sweep run on the
    leading sub_n columns, scaled by (n / sub_n)^3 and (n / sub_n)^2."""
    import numpy as np
    from oracle import gptq_f64 as O
    cores, host = host_blas()
    if given_h:
        n = wl.H.shape[0]
        m = min(sub_n, n)
        Hs = wl.H[:m, :m].astype(np.float64)
        Ws = wl.W[:sample_rows, :m]
        t_h = 0.0
        f_scale, s_scale = (n / m) ** 3, (wl.d_out / sample_rows) * (n / m) ** 2
        nq_s = m
    else:
        T, n = X_vals.shape
        t0 = time.perf_counter()
        Hs = O.hessian(X_vals[:sample_tokens])
        t_h = (time.perf_counter() - t0) * (T / sample_tokens)
        Ws = wl.W[:sample_rows]
        f_scale, s_scale = 1.0, wl.d_out / sample_rows
        nq_s = wl.n_quant
    t0 = time.perf_counter()
    Hd, perm = O.prepare(Hs, p["damp"], p["act_order"], nq_s)
    U = O.upper_chol_of_inverse(Hd)
    t_f = (time.perf_counter() - t0) * f_scale
    t0 = time.perf_counter()
    O.gptq_o2(Ws, Hs, p["bits"], p["group"], p["damp"], p["block"], p["act_order"], nq_s, U=U, perm=perm)
    t_s = (time.perf_counter() - t0) * s_scale
    total = t_h + t_f + t_s
    if given_h:
        sample = (f"H given: factorisation of the leading {m}x{m} block (time x(n/{m})^3) and the sweep of "
                  f"{sample_rows} of {wl.d_out} rows over those {m} columns (time x{wl.d_out // sample_rows}"
                  f" x(n/{m})^2); float64 numpy")
    else:
        sample = (f"Hessian on {sample_tokens} of {T} tokens (time x{T // sample_tokens}); "
                  f"factorisation at full n={n}; sweep on {sample_rows} of {wl.d_out} rows "
                  f"(time x{wl.d_out // sample_rows}); float64 numpy")
    return {
        "value": wl.d_out * wl.n_quant / total, "unit": "weights/s", "cores": cores, "kind": "oracle",
        "sample": sample, "host": host,
        "seconds_est": {"hessian": t_h, "factor": t_f, "sweep": t_s, "step": total},
    }


def bench_dequant(args):
    """The inference product on the 4096 x 4096 4-bit g128 layer (seeded
    random codes, zero points and scales; Student-t(4) bf16 activations)."""
    import numpy as np
    import torch

    import post_weight_quantization_28_amd as G
    import synth

    if not os.path.exists(G.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    G.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    M, n, d_out, bits, group = args.tokens, 4096, 4096, 4, 128
    r = np.random.default_rng(2024)
    codes = r.integers(0, 2 ** bits, (d_out, n)).astype(np.uint8)
    scales = r.uniform(0.002, 0.05, (d_out, n // group)).astype(np.float32)
    zeros = r.integers(0, 2 ** bits, (d_out, n // group)).astype(np.uint8)
    xv = r.standard_t(4, (M, n)).astype(np.float32)
    xb = synth.f32_to_bf16_bits(xv)
    qw_dev = G.pack_codes(torch.from_numpy(codes).to(dev), bits)
    sc_dev = torch.from_numpy(scales).to(dev)
    z_dev = torch.from_numpy(zeros).to(dev)
    X = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
    Y = torch.empty((M, d_out), dtype=torch.float32, device=dev)
    ws = torch.empty(max(G.dequant_matmul_workspace_bytes(M, n, d_out, bits, group), 1), dtype=torch.uint8,
                     device=dev)

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        a.fill_(1)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    def step():
        G.dequant_matmul(X, qw_dev, sc_dev, z_dev, bits, group, out=Y, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # events on the stream the library launches on (torch's current stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    w_bytes = d_out * n * bits // 8 + d_out * (n // group) * 5          # codes, fp32 scales, uint8 zeros
    io_bytes = M * n * 2 + M * d_out * 4
    flops = 2.0 * M * n * d_out
    if M <= 64:
        ach = (w_bytes + io_bytes) / (ms / 1e3) / 1e9
        kern = "k_dequant_mv" if M <= 16 else "k_dequant_mm"
        traffic = recorded_traffic(DEQUANT16_TRAFFIC, DEQUANT_SRC) if M == 16 else None
        roof = {"bound": "hbm", "kernel": kern, "achieved": ach,
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS, "traffic": traffic,
                "work": "packed codes + scales + zeros + X + Y bytes per call; time between HIP events "
                        "around back-to-back calls (launch gaps included)"}
    else:
        ach = flops / (ms / 1e3) / 1e12
        roof = {"bound": "mfma", "kernel": "k_dequant_mm_x", "achieved": ach, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": ach / PEAK_BF16_TFLOPS, "traffic": None,
                "work": "2 M n d_out flop per call"}
    line = {
        "metric": f"packed-layer product Y = X W_hat^T (4096², 4-bit g128), {M} tokens",
        "value": M / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "wall_ms_per_step": 1e3 * elapsed / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"inference product of a packed 4096x4096 4-bit g128 layer, {M} bf16 tokens "
                               f"({'decode' if M <= 64 else 'prefill'})",
                   "tokens": M, "d_in": n, "d_out": d_out, "bits": bits, "group": group,
                   "parallelism": "single GPU"},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        from oracle import dequant as D
        from oracle import packing as P
        cores, host = host_blas()
        ms_rows = min(M, 16)
        qw_host = P.pack(codes, bits)
        xs = synth.bf16_bits_to_f32(xb[:ms_rows])
        t0 = time.perf_counter()
        D.dequant_matmul(xs, qw_host, scales, zeros, bits, group)
        t = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": ms_rows / t, "unit": "tokens/s", "cores": cores, "kind": "oracle",
                                "sample": f"{ms_rows} of {M} tokens: float64 unpack, dequantise and product "
                                          "(numpy)", "host": host}
    print(json.dumps(line), flush=True)


CONFIG_TEXT = {
    "c2": "attention-projection GPTQ layer: W 4096x4096 bf16, X 131072x4096 bf16 Student-t(4) with 41 "
          "outlier channels x30; 4-bit asymmetric, group 128, block 128, damp 0.01, act-order off",
    "c3": "MLP down-projection GPTQ layer: W 4096x11008 bf16, X 65536x11008 bf16 x*sigmoid(x)*y gated; "
          "3-bit asymmetric, group 128, block 128, damp 0.01, act-order on",
    "c4": "large 2-bit GPTQ layer: W 8192x28672 bf16, fp32 H given (2 X^T X of 32768x28672 Gaussian X with "
          "a rank-32 spike x10); 2-bit asymmetric, group 64, block 128, damp 0.01",
    "c5": "GPTQ-intrinsic augmented layer: W 5120x5120 bf16 -> [W, 0] 5120x5184, X~ = [X, X V_64] "
          "65536x5184 bf16 Student-t(4); 2-bit asymmetric, group 128, block 128, damp 0.01, 5120 columns "
          "quantized, 64 kept in fp32",
}


def inverse_x6_work(n):
    """(flops, products) of the triangular inverse's block products that run
    on the six-product bf16 kernel: for every level h of the recursive
    doubling with h >= 1024 whose first product has at least 1024 output
    tiles of 128 x 128, each pair (h rows, partner hj rows) costs
    hj h (h + 1) flop (T^T = X_ii^T L_ji^T, X_ii triangular) plus
    h hj (hj + 1) flop (X_ji = -X_jj T, X_jj triangular)."""
    flops, products = 0.0, 0
    h = 64
    while h < n:
        full = n // (2 * h)
        bp_last = full * 2 * h + h
        hj_last = n - bp_last if bp_last < n else 0
        for hj, batch in ((h, full), (hj_last, 1)):
            if batch <= 0 or hj <= 0 or h < 1024:
                continue
            if -(-h // 128) * -(-hj // 128) * batch < 1024:
                continue
            flops += batch * (hj * h * (h + 1) + h * hj * (hj + 1))
            products += 2
        h *= 2
    return flops, products


def far_field_flops(d_out, n, nq, group, block=128):
    """Algorithmic flops of the far-field updates per quantize call: every
    512-column super-block's errors (K = its width) applied to all columns
    right of it (the library's two-level split for groups <= block)."""
    sw = 512 if group <= block else (group * (512 // group) if group <= 512 else group)
    f = 0.0
    for s0 in range(0, nq, sw):
        s1 = min(s0 + sw, nq)
        if s1 < n:
            f += 2.0 * d_out * (s1 - s0) * (n - s1)
    return f


def measured_peaks(dev):
    """What this machine delivers on two plain reference operations, beside the
    nominal peaks: a 1 GiB device-to-device copy (torch, read + write bytes)
    and an 8192^3 bf16 GEMM (torch -> hipBLASLt)."""
    import torch
    a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    a.fill_(1)
    x = torch.randn((8192, 8192), device=dev).to(torch.bfloat16)
    y = torch.randn((8192, 8192), device=dev).to(torch.bfloat16)
    for _ in range(3):
        b.copy_(a)
        torch.matmul(x, y)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2.0 * (1 << 30) * 10 / (e0.elapsed_time(e1) / 1e3) / 1e9
    e0.record()
    for _ in range(10):
        torch.matmul(x, y)
    e1.record()
    torch.cuda.synchronize()
    gemm_tf = 2.0 * 8192 ** 3 * 10 / (e0.elapsed_time(e1) / 1e3) / 1e12
    del a, b, x, y
    torch.cuda.empty_cache()
    return {"hbm_copy_GBps": copy_gbs, "bf16_gemm_hipblaslt_TFLOPs": gemm_tf,
            "nominal_hbm_GBps": PEAK_HBM_GBS, "nominal_bf16_TFLOPs": PEAK_BF16_TFLOPS,
            "how": "1 GiB device copy (read + write bytes) and an 8192^3 bf16 matmul through torch, "
                   "10 timed repetitions each"}


def gram_f64_on_device(chunks):
    """2 X^T X in float64 over the token chunks of the large layer's X, on the
    device: the recipe's given H (an input of the benchmark, formed before
    the timed region and rounded once to fp32 by the recipe)."""
    import torch
    H = None
    for _, x, _ in chunks:
        xt = torch.from_numpy(x).to("cuda", torch.float64)
        g = xt.T.contiguous() @ xt
        H = g if H is None else H.add_(g)
        del xt, g
    H.mul_(2.0)
    out = H.cpu().numpy()
    del H
    torch.cuda.empty_cache()
    return out


def bench_eora(args):
    """EoRA adapter of the 4096 x 4096 attention projection: the layer's own
    4-bit GPTQ output on the GPU (untimed, as are H and the quantization),
    then gptq_eora at rank 64 timed between HIP events."""
    import numpy as np
    import torch

    import post_weight_quantization_28_amd as G
    import synth

    if not os.path.exists(G.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    G.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    rank = args.rank
    log("bench: generating the c2 workload")
    wl = synth.make_workload("c2")
    p = wl.params
    W = torch.from_numpy(wl.W_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    X = torch.from_numpy(wl.X_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    H = G.accumulate_hessian(X)
    del X
    q = G.quantize_layer(W, H, bits=p["bits"], group=p["group"], damp=p["damp"], block=p["block"])
    d_out, n = W.shape
    ws = torch.empty(G.eora_workspace_bytes(d_out, n, rank), dtype=torch.uint8, device=dev)

    def step():
        return G.eora(W, q.w_hat, H, rank=rank, iters=args.iters, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        B, A, sig = step()
    e1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    k = min(rank + 64, 128, d_out)
    k += k & 1
    iters = args.iters or 24
    flops = (2.0 * d_out * n * n + 2.0 * d_out * d_out * n                 # D H, then (D H) D^T
             + (iters + 3) * (2.0 * d_out * d_out * k + 4.0 * d_out * k * k)   # G Q, Y^T Y, Y U^T
             + 2.0 * d_out * k * k + 2.0 * d_out * k * rank + 2.0 * rank * d_out * n)
    ach = flops / (ms / 1e3) / 1e12
    line = {
        "metric": f"EoRA rank-{rank} adapter of a GPTQ layer (4096², 4-bit g128)",
        "value": d_out * n / (ms / 1e3), "unit": "weights/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "wall_ms_per_step": 1e3 * elapsed / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "EoRA adapter of the 4096x4096 attention-projection layer after 4-bit g128 GPTQ, "
                               f"H = 2 X^T X of 131072 Student-t(4) tokens, rank {rank}, {iters} subspace steps",
                   "d_out": d_out, "d_in": n, "rank": rank, "iters": iters, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": "gptq_eora (k_gemm_f32 products)", "achieved": ach,
                     "peak": 157.3, "unit": "TFLOP/s", "frac": ach / 157.3, "traffic": None,
                     "work": "2 d n^2 + 2 d^2 n (G = D H D^T) + per subspace step 2 d^2 k + 4 d k^2, plus the "
                             "final U_r and A products, per call; fp32 MFMA peak"},
    }
    if not args.no_cpu_baseline:
        from oracle import eora as E
        cores, host = host_blas()
        Wv = wl.W.astype(np.float64)
        Wh = q.w_hat.cpu().numpy().astype(np.float64)
        Hn = H.cpu().numpy().astype(np.float64)
        t0 = time.perf_counter()
        E.eora(Wv, Wh, Hn, rank)
        t = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": d_out * n / t, "unit": "weights/s", "cores": cores, "kind": "oracle",
                                "sample": "the whole layer: float64 eigh of H, projection, SVD, back-projection "
                                          "(numpy)", "host": host, "seconds": t}
    print(json.dumps(line), flush=True)


def bench_refine(args):
    """One OLrC + Bid-Up cycle on the 5120-wide GPTQ-intrinsic layer (the
    augmented 2-bit sweep's codes and grid, H of the original activations),
    rank 64, timed between HIP events; the inputs are made untimed."""
    import numpy as np
    import torch

    import post_weight_quantization_28_amd as G
    import synth

    if not os.path.exists(G.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    G.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("bench: generating the c5 workload")
    wl = synth.make_workload("c5")
    n0 = wl.n_quant
    X = torch.from_numpy(wl.X_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    Wa = torch.from_numpy(wl.W_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    q = G.quantize_layer(Wa, G.accumulate_hessian(X), bits=2, group=128, damp=0.01, block=128, n_quant=n0,
                         want_codes=True)
    H = G.accumulate_hessian(X[:, :n0].contiguous())
    del X
    W = Wa[:, :n0].contiguous()
    d_out = W.shape[0]
    rank = 64
    ws = torch.empty(G.refine_workspace_bytes(d_out, n0, rank), dtype=torch.uint8, device=dev)

    def step():
        return G.refine_lowrank(W, H, q.codes, q.scales, q.zeros, q.g_idx, 2, 128, rank=rank, cycles=1,
                                passes=1, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    line = {
        "metric": "OLrC + Bid-Up refinement cycle of a GPTQ-intrinsic layer (5120x5120, 2-bit g128, rank 64)",
        "value": d_out * n0 / (ms / 1e3), "unit": "weights/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "wall_ms_per_step": 1e3 * elapsed / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "one OLrC (rank-64 EoRA of W - W_hat) and one Bid-Up pass on the 5120x5120 layer's "
                               "codes from the augmented 2-bit g128 sweep (X~ = [X, X V_64], 65536 Student-t(4) "
                               "tokens); H = 2 X^T X of the original columns",
                   "d_out": d_out, "d_in": n0, "rank": rank, "bits": 2, "group": 128, "parallelism": "single GPU"},
        "roofline": None,
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="before warm-up, run one plain 1 GiB device copy and one 1 GiB fill "
                         "(known bytes) for calibrating HBM byte counters")
    ap.add_argument("--workload", choices=["gptq_layer", "dequant_matmul", "eora", "refine"], default="gptq_layer")
    ap.add_argument("--rank", type=int, default=64, help="adapter rank for --workload eora")
    ap.add_argument("--iters", type=int, default=0, help="subspace steps for --workload eora (0: 24)")
    ap.add_argument("--config", choices=sorted(CONFIG_TEXT), default="c2",
                    help="layer workload: c2 4096x4096 4-bit (the metric's), c3 4096x11008 3-bit act-order, "
                         "c4 8192x28672 2-bit with H given, c5 5120x5184 augmented 2-bit")
    ap.add_argument("--no-peaks", action="store_true", help="skip the copy / GEMM peak measurement")
    ap.add_argument("--tokens", type=int, default=16, help="tokens M for --workload dequant_matmul")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported; the library and this benchmark "
              "run on one GPU (a token-sharded Hessian and row-sharded sweep are not implemented)",
              file=sys.stderr)
        sys.exit(2)
    if args.workload == "dequant_matmul":
        bench_dequant(args)
        return
    if args.workload == "eora":
        bench_eora(args)
        return
    if args.workload == "refine":
        bench_refine(args)
        return

    import numpy as np
    import torch

    import post_weight_quantization_28_amd as G
    import synth

    if not os.path.exists(G.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    G.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    cfg = args.config
    log(f"bench: generating the {cfg} workload")
    t0 = time.perf_counter()
    wl = synth.make_workload(cfg, H_fn=gram_f64_on_device if cfg == "c4" else None)
    p = wl.params
    log(f"bench: inputs ready in {time.perf_counter() - t0:.1f} s")
    W = torch.from_numpy(wl.W_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    d_out, n = W.shape
    nq = wl.n_quant
    given_h = wl.H is not None
    if given_h:
        X = None
        T = wl.T
        H = torch.from_numpy(wl.H).to(dev)
        ws_h = None
    else:
        X = torch.from_numpy(wl.X_bits.view(np.int16)).view(torch.bfloat16).to(dev)
        T = X.shape[0]
        H = torch.empty((n, n), dtype=torch.float32, device=dev)
        ws_h = torch.empty(G.hessian_workspace_bytes(T, n, torch.bfloat16), dtype=torch.uint8, device=dev)
    params = G.make_params(p["bits"], p["group"], p["damp"], p["block"], p["act_order"], nq, n)
    ws_q = torch.empty(G.workspace_bytes(d_out, n, params), dtype=torch.uint8, device=dev)
    outs = {
        "qweight": torch.empty((d_out, (nq * p["bits"] + 31) // 32), dtype=torch.int32, device=dev),
        "scales": torch.empty((d_out, nq // p["group"]), dtype=torch.float32, device=dev),
        "zeros": torch.empty((d_out, nq // p["group"]), dtype=torch.uint8, device=dev),
        "g_idx": torch.empty((nq,), dtype=torch.int32, device=dev),
        "w_hat": torch.empty((d_out, n), dtype=torch.float32, device=dev),
        "row_loss": torch.empty((d_out,), dtype=torch.float32, device=dev),
    }

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        a.fill_(1)          # writes 1 GiB
        b.copy_(a)          # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del a, b
        log("bench: ran the 1 GiB fill and copy for counter calibration")

    def step():
        if not given_h:
            G.accumulate_hessian(X, H=H, zero_first=True, workspace=ws_h)
        G.quantize_layer(W, H, bits=p["bits"], group=p["group"], damp=p["damp"], block=p["block"],
                         act_order=p["act_order"], n_quant=nq, workspace=ws_q, outputs=outs)

    for i in range(args.warmup):
        step()
        log(f"bench: warmup {i + 1}/{args.warmup}")
    torch.cuda.synchronize()

    G.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    prof = G.profile_collect()
    G.profile_enable(False)
    log(f"bench: {args.steps} steps in {elapsed:.3f} s")

    # one more, untimed step with the phases of quantize_layer timed
    G.profile_enable(True, phases=True)
    step()
    torch.cuda.synchronize()
    ph = G.profile_collect()
    G.profile_enable(False)

    ms_step = 1e3 * elapsed / args.steps
    per_class = {k: (v[0] / args.steps) for k, v in prof.items()}
    quant_ms = per_class["quantize"]
    sweep_ms, sweep_n = ph["sweep"]
    far_ms, far_n = ph["far_field"]
    sweep_bytes = 13.0 * d_out * nq        # read W 4, write w_hat 4 and E 4, code 1 per weight
    sweep_gbs = sweep_bytes / (sweep_ms / 1e3) / 1e9 if sweep_ms > 0 else None
    ff = far_field_flops(d_out, n, nq, p["group"], p["block"])
    ff_tf = ff / (far_ms / 1e3) / 1e12 if far_ms > 0 else None
    phases = {
        "factor_ms": ph["factor"][0], "sweep_ms": sweep_ms, "sweep_launches": sweep_n,
        "far_field_ms": far_ms, "far_field_launches": far_n, "prep_finish_ms": ph["prep_finish"][0],
        "quantize_ms_with_phase_events": ph["quantize"][0],
        "sweep_GBps": sweep_gbs, "sweep_hbm_frac": sweep_gbs / PEAK_HBM_GBS if sweep_gbs else None,
        "far_field_TFLOPs": ff_tf, "far_field_mfma_frac": ff_tf / PEAK_BF16_TFLOPS if ff_tf else None,
        "far_field_mfma_frac_3_products": 3 * ff_tf / PEAK_BF16_TFLOPS if ff_tf else None,
        "how": "one extra untimed step with an event pair around every phase launch; sweep bytes "
               "13 per weight (read W, write w_hat and E fp32, code), far-field flops "
               "sum 2 d_out K N over the super-blocks",
    }
    line = {
        "metric": METRIC,
        "value": d_out * nq / (ms_step / 1e3),
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": CONFIG_TEXT[cfg], "name": cfg,
                   "d_out": d_out, "d_in": n, "n_quant": nq, "tokens": T, "bits": p["bits"],
                   "group": p["group"], "block": p["block"], "damp": p["damp"], "act_order": p["act_order"],
                   "hessian_given": given_h, "parallelism": "single GPU"},
        "quantize_ms": quant_ms,
        "layer_weights_per_s_quantize_only": d_out * nq / (quant_ms / 1e3),
        "phases": phases,
    }
    if not given_h:
        syrk_ms, syrk_n = prof["hessian_syrk"]
        syrk_avg_s = syrk_ms / max(syrk_n, 1) / 1e3
        hess_flops = float(T) * n * (n + 1)        # symmetric count per launch
        achieved = hess_flops / syrk_avg_s / 1e12
        hess_ms = per_class["hessian_syrk"] + per_class["hessian_reduce"]
        line["hessian_tflops"] = hess_flops / (hess_ms / 1e3) / 1e12
        line["hessian_ms"] = hess_ms
        line["roofline"] = {"bound": "mfma", "kernel": "k_hessian_dma", "achieved": achieved,
                            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                            "traffic": hessian_traffic() if cfg == "c2" else None,
                            "work": "T*n*(n+1) flop per launch (upper triangle of 2 X^T X)"}
    else:
        inv_flops, inv_products = inverse_x6_work(n)
        inv_ms, inv_n = ph["inverse_x6"]
        if inv_products > 0 and inv_n == inv_products and inv_ms > 0:
            # H given: the largest kernel is the six-product block product of
            # the factorisation's triangular inverse (fp32-accurate result
            # from six bf16 MFMA products per value)
            inv_tf = inv_flops / (inv_ms / 1e3) / 1e12
            line["roofline"] = {"bound": "mfma", "kernel": "k_gemm_x6", "achieved": inv_tf,
                                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": inv_tf / PEAK_BF16_TFLOPS,
                                "traffic": None,
                                "frac_six_products": 6 * inv_tf / PEAK_BF16_TFLOPS,
                                "frac_of_fp32_peak": inv_tf / PEAK_FP32_TFLOPS,
                                "work": f"{inv_flops:.4e} flop of fp32-accurate triangular block products per "
                                        f"call over {inv_products} launches, each value taken as six bf16 "
                                        "piece products; frac counts one product against the bf16 peak, "
                                        "frac_six_products all six, frac_of_fp32_peak compares the "
                                        "fp32-accurate rate with the fp32 MFMA peak"}
        else:
            line["roofline"] = {"bound": "mfma", "kernel": "k_trail_x3", "achieved": ff_tf,
                                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                "frac": ff_tf / PEAK_BF16_TFLOPS if ff_tf else None, "traffic": None,
                                "work": "sum over super-blocks of 2 d_out K N flop per call (fp32-accurate "
                                        "product taken as three bf16 products; frac counts one)"}
    if not args.no_peaks:
        line["measured_peaks"] = measured_peaks(dev)
    if not args.no_cpu_baseline:
        log("bench: timing the float64 oracle on a bounded sample (cpu_baseline)")
        line["cpu_baseline"] = cpu_baseline(wl, wl.X, p, given_h=given_h)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
