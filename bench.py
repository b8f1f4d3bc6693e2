"""Throughput of the LaCT layer on one MI355X.

One step = one ``lact_chunked_forward`` call: every chunk's query read,
chunk gradient, optimizer step and row normalisation over one batch of
synthetic input that is already resident in HBM.  The default workload is
the posed-image set (196,608 keys as one chunk, 12 heads, d=64, h=128,
update-then-apply on 4,096 queries, Muon with 5 Newton-Schulz iterations).

Prints ONE JSON line.  ``value`` is the layer's algorithmic TFLOP/s; the
line also carries tokens/s, the fraction of the bf16 MFMA peak, per-phase
kernel times from HIP events recorded on the launch stream, the roofline of
the dominant kernel, and the CPU oracle timed on a bounded sample.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import lact_synth as S  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gradient_flops(w: S.Workload) -> float:
    """Algorithmic flops of one launch of the chunk-gradient kernel (one chunk, all pairs)."""
    return 12.0 * w.chunk_kv * w.d * w.h * w.pairs


def counted_traffic(w: S.Workload):
    """HBM bytes per gradient launch from the committed rocprofv3 counter
    summary, if it was taken on this workload from the current kernel source
    (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"grad_{w.name}_hbm_counters.json")
    try:
        rec = json.load(open(path))
        src = open(os.path.join(ROOT, rec["source"]), "rb").read()
    except (OSError, ValueError, KeyError):
        return None
    if rec.get("workload") != w.name or hashlib.sha256(src).hexdigest() != rec.get("source_sha256"):
        return None
    return rec["bytes_per_dispatch"]


def cpu_baseline(w: S.Workload, x, st, budget_s: float = 15.0):
    """The float32 oracle on a bounded sample: whole pairs of the workload,
    as many as fit the time budget (at least one)."""
    import oracle
    hp = oracle.Hyper(opt=w.opt, beta=w.beta, ns_iters=w.ns_iters, token_block=65536,
                      norm_keep=w.norm == "keep")
    per_pair = w.flops() / w.pairs
    done, t_used, pairs = 0, 0.0, []
    for b in range(w.B):
        for h in range(w.H):
            pairs.append((b, h))
    t0 = time.perf_counter()
    for p in pairs:
        oracle.lact_chunked_forward(st, x["Q"], x["K"], x["V"], x["eta"], w.chunk_kv, w.chunk_q,
                                    w.order, hp, dtype=np.float32, pairs=[p])
        done += 1
        t_used = time.perf_counter() - t0
        if t_used > budget_s:
            break
    tflops = done * per_pair / t_used / 1e12
    # the float64 parity oracle on one pair of the same workload, for context
    hp64 = oracle.Hyper(opt=w.opt, beta=w.beta, ns_iters=w.ns_iters, token_block=65536,
                        norm_keep=w.norm == "keep")
    t1 = time.perf_counter()
    oracle.lact_chunked_forward(st, x["Q"], x["K"], x["V"], x["eta"], w.chunk_kv, w.chunk_q,
                                w.order, hp64, dtype=np.float64, pairs=[pairs[0]])
    t64 = time.perf_counter() - t1
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    threads = int(os.environ.get("OMP_NUM_THREADS", cores))
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": round(tflops, 6), "unit": "TFLOP/s", "cores": min(cores, threads), "kind": "oracle",
        "sample": f"{done} of {w.pairs} (batch, head) pairs of the {w.name} workload, full length, "
                  f"float32 NumPy oracle, {t_used:.1f} s",
        "cpu_model": model,
        "fp64_oracle": {"value": round(per_pair / t64 / 1e12, 6), "unit": "TFLOP/s",
                        "sample": f"1 pair, float64 parity oracle, {t64:.1f} s"},
    }


def gemm_reference(n: int = 8192, reps: int = 30):
    """The vendor BLAS (torch.matmul, bf16 in, fp32 accumulate) on one square
    n x n x n product, timed back to back under the same sustained load as the
    steps: a practical matrix-core rate of this GPU, reported beside the
    published peak (context for the roofline, not part of the layer)."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(0)
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
    c = torch.matmul(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    e1.record()
    e1.synchronize()
    ms = e0.elapsed_time(e1) / reps
    tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    del a, b, c
    return {"what": f"torch.matmul bf16 {n}x{n}x{n}, {reps} back-to-back launches",
            "ms": round(ms, 4), "tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}


def other_mode(args, w, cfg, dev, Q, K, V, eta, O, ws):
    """--mode backward / block: the step is lact_chunked_backward (given dO and the
    cotangents of the final weights) or lact_block_forward (shared Q, K, V); one
    JSON line with tokens/s and the dominant kernel's roofline."""
    import torch
    import chunk_test_amd as L
    if args.mode == "backward":
        g = torch.Generator(device="cuda").manual_seed(1)
        dO = torch.randn(Q.shape, generator=g, device="cuda").to(Q.dtype)
        dWf = {n: 0.1 * torch.randn(dev[n].shape, generator=g, device="cuda") for n in ("W1", "W2", "W3")}
        st0 = {n: dev[n] for n in ("W1", "W2", "W3")}
        bws = torch.empty(L.backward_workspace_bytes(cfg, w.T_kv, w.chunk_kv, w.chunk_q), dtype=torch.uint8,
                          device="cuda")

        def step():
            L.lact_chunked_backward(cfg, st0, Q, K, V, eta, dO, w.chunk_kv, w.chunk_q, w.order, ws=bws,
                                    dW_final=dWf)
        metric = "LaCT layer backward tokens/s"
    else:
        if w.T_q != w.T_kv:
            raise SystemExit("--mode block needs T_q == T_kv (shared Q, K, V)")
        init = {n: t.clone() for n, t in dev.items()}

        def step():
            for n, t in dev.items():
                t.copy_(init[n])
            L.lact_block_forward(cfg, dev, Q, K, V, eta, O, w.chunk_kv, args.window, ws, order=w.order)
        metric = "LaCT block (window attention + layer) tokens/s"
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    attn = None
    if args.mode == "block":
        # the window attention alone: algorithmic flops 4 d per (query, visible key)
        vis = sum(min(t + 1, args.window) for t in range(w.T_kv))
        a_flops = 4.0 * w.d * vis * w.pairs
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        for _ in range(args.steps):
            L.lact_window_attention(cfg, Q, K, V, O, args.window)
        a1.record()
        torch.cuda.synchronize()
        a_ms = a0.elapsed_time(a1) / args.steps
        attn = {"ms": round(a_ms, 5), "flop": a_flops, "tflops": round(a_flops / (a_ms * 1e-3) / 1e12, 3),
                "peak_frac": round(a_flops / (a_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    # the dominant kernel's roofline from the library's per-phase HIP events,
    # over as many steps again: the key-side backward token kernel (24 d h
    # flop per key token and pair: six projections, six token-side products),
    # or the window attention (4 d flop per visible (query, key))
    L.profile_enable(True)
    L.profile_read()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    phases = L.profile_read()
    L.profile_enable(False)
    roof = None
    if args.mode == "backward":
        k_ms, k_n = phases["bw_key_tokens"]
        if k_n:
            per_launch = 24.0 * w.d * w.h * w.chunk_kv * w.pairs
            avg = k_ms / k_n
            ach = per_launch / (avg * 1e-3) / 1e12
            roof = {"kernel": "backward key-side token kernel (VJP of the chunk gradient)", "bound": "mfma",
                    "achieved": round(ach, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": None, "avg_launch_ms": round(avg, 5),
                    "flop_per_launch": per_launch}
    elif attn is not None:
        a_ms, a_n = phases["window_attention"]
        if a_n:
            avg = a_ms / a_n
            ach = attn["flop"] / (avg * 1e-3) / 1e12
            roof = {"kernel": "window attention", "bound": "mfma", "achieved": round(ach, 3),
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                    "traffic": None, "avg_launch_ms": round(avg, 5), "flop_per_launch": attn["flop"]}
    line = {
        "metric": metric, "value": round(w.B * w.T_kv / (ms * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.io_dtype == "bf16" else "fp32", "data": "synthetic",
        "config": {"workload": w.name, "mode": args.mode, "B": w.B, "H": w.H, "d": w.d, "h": w.h,
                   "T_kv": w.T_kv, "T_q": w.T_q, "chunk_kv": w.chunk_kv, "chunk_q": w.chunk_q,
                   "order": w.order, "opt": w.opt, "beta": w.beta, "products": w.products,
                   "window": args.window if args.mode == "block" else None},
        "wall_s_timed": round(wall, 4), "roofline": roof, "cpu_baseline": None,
        "window_attention": attn,
        "phase_ms_per_step": {k: round(v[0] / args.steps, 5) for k, v in phases.items() if v[1]},
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="posed", choices=sorted(S.WORKLOADS))
    ap.add_argument("--norm", default="unit", choices=("unit", "keep"),
                    help="variant: updated rows to unit length (default) or kept at their length")
    ap.add_argument("--eta-per-matrix", action="store_true",
                    help="variant: a learning rate per token and matrix (W1, W2, W3)")
    ap.add_argument("--products", default=None, choices=("auto", "bf16", "split"),
                    help="product precision of bf16 mode (default: the workload's own)")
    ap.add_argument("--mode", default="forward", choices=("forward", "backward", "block"),
                    help="forward: the layer (default); backward: lact_chunked_backward on the "
                         "same workload; block: window attention + the layer on shared Q, K, V")
    ap.add_argument("--window", type=int, default=2048, help="attention window of --mode block")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-gemm-reference", action="store_true",
                    help="skip the vendor-BLAS bf16 GEMM timed after the steps (a practical "
                         "matrix-core rate of this GPU under sustained load, for context)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (a reference for "
                         "hardware byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer is built for a single MI355X).", file=sys.stderr)
        sys.exit(2)

    import torch
    import chunk_test_amd as L

    w = S.WORKLOADS[args.workload]
    if args.norm != "unit" or args.eta_per_matrix:
        # a variant of the workload (its own name: the committed counter
        # summaries belong to the plain workloads)
        w = w.replace(name=w.name + ("-keep" if args.norm == "keep" else "")
                      + ("-eta3" if args.eta_per_matrix else ""),
                      norm=args.norm, eta_per_matrix=args.eta_per_matrix)
    if args.products is not None and args.products != w.products:
        w = w.replace(name=w.name + "-" + args.products, products=args.products)
    log(f"[bench] workload {w.name}: generating inputs")
    st = S.gen_weights(w)
    x = S.gen_inputs(w)
    io = torch.bfloat16 if w.io_dtype == "bf16" else torch.float32
    cfg = L.Config(B=w.B, H=w.H, d=w.d, h=w.h, io_dtype=w.io_dtype, opt=w.opt, beta=w.beta,
                   ns_iters=w.ns_iters, products=w.products, norm=w.norm,
                   eta_per_matrix=w.eta_per_matrix)
    dev = {n: torch.from_numpy(st[n]).cuda() for n in ("W1", "W2", "W3")}
    if cfg.uses_momentum():
        for n in ("M1", "M2", "M3"):
            dev[n] = torch.zeros_like(dev["W" + n[1]])
    Q, K, V = (torch.from_numpy(x[n]).cuda().to(io) for n in ("Q", "K", "V"))
    eta = torch.from_numpy(x["eta"]).cuda()
    O = torch.empty_like(Q)
    ws = L.alloc_workspace(cfg, w.chunk_kv, w.chunk_q)
    torch.cuda.synchronize()

    def step():
        L.lact_chunked_forward(cfg, dev, Q, K, V, eta, O, w.chunk_kv, w.chunk_q, w.order, ws)

    if args.copy_probe_mib:
        src = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.mode != "forward":
        return other_mode(args, w, cfg, dev, Q, K, V, eta, O, ws)

    # every step starts from the initial state: W (and M) are restored before
    # each step, outside its timed span (the kernels' time depends on the data)
    init = {n: t.clone() for n, t in dev.items()}

    def reset():
        for n, t in dev.items():
            t.copy_(init[n])

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        reset()
        step()
    torch.cuda.synchronize()

    log(f"[bench] timing {args.steps} steps")
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        reset()
        starts[i].record()
        step()
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    ms = sum(step_ms) / args.steps

    # per-phase kernel durations: HIP events recorded by the library on the
    # launch stream around each phase, over as many steps again, right after
    # the timed ones (the same sustained-load clock regime)
    log("[bench] per-phase event timing")
    L.profile_enable(True)
    L.profile_read()
    for _ in range(args.steps):
        reset()
        step()
    torch.cuda.synchronize()
    phases = L.profile_read()
    L.profile_enable(False)

    flops = w.flops()
    tflops = flops / (ms * 1e-3) / 1e12
    grad_ms, grad_n = phases["gradient"]
    grad_avg = grad_ms / max(grad_n, 1)
    grad_tflops = gradient_flops(w) / (grad_avg * 1e-3) / 1e12 if grad_n else None
    roof = {
        "kernel": "chunk gradient (key projections, SwiGLU backward, token contractions)",
        "bound": "mfma", "achieved": round(grad_tflops, 3) if grad_tflops else None,
        "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
        "frac": round(grad_tflops / PEAK_BF16_TFLOPS, 4) if grad_tflops else None,
        "traffic": counted_traffic(w), "avg_launch_ms": round(grad_avg, 5),
        "flop_per_launch": gradient_flops(w),
    }
    line = {
        "metric": "LaCT layer TFLOP/s (update+apply)",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.io_dtype == "bf16" else "fp32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "d": w.d, "h": w.h,
                   "T_kv": w.T_kv, "T_q": w.T_q, "chunk_kv": w.chunk_kv, "chunk_q": w.chunk_q,
                   "order": w.order, "opt": w.opt, "beta": w.beta, "ns_iters": w.ns_iters,
                   "products": w.products, "norm": w.norm, "eta_per_matrix": w.eta_per_matrix,
                   "mfma_path": L.mfma_path(w.d, w.h, w.io_dtype)},
        "tokens_per_s": round(w.B * w.T_kv / (ms * 1e-3), 1),
        "query_tokens_per_s": round(w.B * w.T_q / (ms * 1e-3), 1),
        "peak_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "flop_per_step": flops,
        "phase_ms_per_step": {k: round(v[0] / args.steps, 5) for k, v in phases.items()},
        "phase_launches_per_step": {k: v[1] / args.steps for k, v in phases.items()},
        "wall_s_timed": round(wall, 4),
        "ms_per_step_min": round(min(step_ms), 5),
        "ms_per_step_median": round(sorted(step_ms)[len(step_ms) // 2], 5),
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_gemm_reference:
        line["gemm_reference"] = gemm_reference()
        if grad_tflops and line["gemm_reference"]["tflops"]:
            roof["frac_of_gemm_reference"] = round(grad_tflops / line["gemm_reference"]["tflops"], 4)
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle baseline (budget {args.cpu_budget} s)")
        line["cpu_baseline"] = cpu_baseline(w, x, st, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
