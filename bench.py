"""Benchmark: one GPTQ layer step on one MI355X.

A step is the whole path on the 4096 x 4096 attention-projection workload:
Hessian H = 2 X^T X from 131072 bf16 calibration tokens, then quantize_layer
(damping, factorisation, blocked column sweep with trailing updates, packing)
at 4 bits, group 128, block 128. Inputs are resident in HBM before the timed
region; every step recomputes everything from X and W.

Prints one JSON line: the step throughput, the Hessian kernel against the bf16
MFMA roofline, and the float64 oracle timed on the host cores.

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

# HBM bytes moved by one k_hessian_dma launch on this workload, from two
# rocprofv3 counter runs of `bench.py --steps 1 --warmup 0 --no-cpu-baseline
# --copy-calibration` (FETCH_SIZE, then WRITE_SIZE, each scaled by what the
# same counter reads for the 1 GiB copy/fill that --copy-calibration runs).
# Valid only for the kernel source with the recorded SHA-256; reported as
# null once hessian.hip changes.
HESSIAN_TRAFFIC = {
    "bytes": 7004416590,
    "source_sha256": "5927485f2d042b6424abe06a23069140f40e97b2f4cd8c42293731090d34503d",
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


def cpu_baseline(wl, X_vals, p, sample_tokens=4096, sample_rows=64):
    """The float64 oracle, untuned, on a bounded sample of the same workload,
    scaled to the whole layer step."""
    import numpy as np
    from oracle import gptq_f64 as O
    try:
        from threadpoolctl import threadpool_info
        cores = sum(i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas") or None
    except Exception:
        cores = None
    T, n = X_vals.shape
    t0 = time.perf_counter()
    Hs = O.hessian(X_vals[:sample_tokens])
    t_h = (time.perf_counter() - t0) * (T / sample_tokens)
    t0 = time.perf_counter()
    Hd, perm = O.prepare(Hs, p["damp"], p["act_order"], wl.n_quant)
    U = O.upper_chol_of_inverse(Hd)
    t_f = time.perf_counter() - t0
    t0 = time.perf_counter()
    O.gptq_o2(wl.W[:sample_rows], Hs, p["bits"], p["group"], p["damp"], p["block"], p["act_order"],
              wl.n_quant, U=U, perm=perm)
    t_s = (time.perf_counter() - t0) * (wl.d_out / sample_rows)
    total = t_h + t_f + t_s
    return {
        "value": wl.d_out * wl.n_quant / total, "unit": "weights/s", "cores": cores, "kind": "oracle",
        "sample": (f"Hessian on {sample_tokens} of {T} tokens (time x{T // sample_tokens}); "
                   f"factorisation at full n={n}; sweep on {sample_rows} of {wl.d_out} rows "
                   f"(time x{wl.d_out // sample_rows}); float64 numpy"),
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
        try:
            from threadpoolctl import threadpool_info
            cores = sum(i.get("num_threads", 0) for i in threadpool_info()
                        if i.get("user_api") == "blas") or None
        except Exception:
            cores = None
        ms_rows = min(M, 16)
        qw_host = P.pack(codes, bits)
        xs = synth.bf16_bits_to_f32(xb[:ms_rows])
        t0 = time.perf_counter()
        D.dequant_matmul(xs, qw_host, scales, zeros, bits, group)
        t = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": ms_rows / t, "unit": "tokens/s", "cores": cores, "kind": "oracle",
                                "sample": f"{ms_rows} of {M} tokens: float64 unpack, dequantise and product "
                                          "(numpy)"}
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
    ap.add_argument("--workload", choices=["gptq_layer", "dequant_matmul"], default="gptq_layer")
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

    log("bench: generating the 4096x4096 layer and 131072x4096 bf16 calibration tokens")
    t0 = time.perf_counter()
    wl = synth.make_workload("c2")
    p = wl.params
    log(f"bench: inputs ready in {time.perf_counter() - t0:.1f} s")
    W = torch.from_numpy(wl.W_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    X = torch.from_numpy(wl.X_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    T, n = X.shape
    d_out = W.shape[0]
    nq = wl.n_quant

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

    ms_step = 1e3 * elapsed / args.steps
    per_class = {k: (v[0] / args.steps) for k, v in prof.items()}
    syrk_ms, syrk_n = prof["hessian_syrk"]
    syrk_avg_s = syrk_ms / max(syrk_n, 1) / 1e3
    hess_flops = float(T) * n * (n + 1)        # symmetric count per launch
    achieved = hess_flops / syrk_avg_s / 1e12
    hess_ms = per_class["hessian_syrk"] + per_class["hessian_reduce"]
    quant_ms = per_class["quantize"]
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
        "config": {"workload": "attention-projection GPTQ layer: W 4096x4096 bf16, X 131072x4096 bf16 "
                               "Student-t(4) with 41 outlier channels x30; 4-bit asymmetric, group 128, "
                               "block 128, damp 0.01, act-order off",
                   "d_out": d_out, "d_in": n, "tokens": T, "bits": p["bits"], "group": p["group"],
                   "block": p["block"], "damp": p["damp"], "act_order": p["act_order"],
                   "parallelism": "single GPU"},
        "hessian_tflops": hess_flops / (hess_ms / 1e3) / 1e12,
        "hessian_ms": hess_ms,
        "quantize_ms": quant_ms,
        "layer_weights_per_s_quantize_only": d_out * nq / (quant_ms / 1e3),
        "roofline": {"bound": "mfma", "kernel": "k_hessian_dma", "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": hessian_traffic(),
                     "work": "T*n*(n+1) flop per launch (upper triangle of 2 X^T X)"},
    }
    if not args.no_cpu_baseline:
        log("bench: timing the float64 oracle on a bounded sample (cpu_baseline)")
        line["cpu_baseline"] = cpu_baseline(wl, wl.X, p)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
