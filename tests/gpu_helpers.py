"""Shared pieces of the GPU parity tests: moving the seeded inputs to the
device, running the library through the binding, and running the oracle on
the same (bf16-rounded) inputs."""

from __future__ import annotations

import sys

import numpy as np

import lact_synth as S

FP32_TOL = 1e-4   # fp32 I/O mode vs the float64 oracle
BF16_TOL = 2e-2   # bf16-in / fp32-accumulate mode vs the float64 oracle


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(x, y):
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    den = np.max(np.abs(y))
    return float(np.max(np.abs(x - y)) / (den if den > 0 else 1.0))


def tol_of(w: S.Workload):
    return FP32_TOL if w.io_dtype == "fp32" else BF16_TOL


def config_of(w: S.Workload):
    from chunk_test_amd import Config
    return Config(B=w.B, H=w.H, d=w.d, h=w.h, io_dtype=w.io_dtype, opt=w.opt, beta=w.beta,
                  ns_iters=w.ns_iters, products=w.products, norm=w.norm,
                  eta_per_matrix=w.eta_per_matrix, net=w.net)


def to_dev(x, w: S.Workload, io=True):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    if io and w.io_dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t


def device_state(w: S.Workload, st_np):
    import torch
    cfg = config_of(w)
    wn = ("W1",) if w.net == "linear" else ("W1", "W2", "W3")
    st = {n: to_dev(st_np[n], w, io=False) for n in wn}
    if cfg.uses_momentum():
        for n in tuple("M" + x[1] for x in wn):
            src = st_np.get(n)
            st[n] = (to_dev(src, w, io=False) if src is not None
                     else torch.zeros_like(st["W" + n[1]]))
    return st


def run_gpu(w: S.Workload, x, st_np, ws=None):
    """The whole layer on the GPU; returns (O as float32 numpy, state as numpy)."""
    import torch
    import chunk_test_amd as L
    cfg = config_of(w)
    st = device_state(w, st_np)
    Q, K, V = (to_dev(x[n], w) for n in ("Q", "K", "V"))
    eta = to_dev(x["eta"], w, io=False)
    O = torch.empty_like(Q)
    if ws is None:
        ws = L.alloc_workspace(cfg, w.chunk_kv, w.chunk_q)
    L.lact_chunked_forward(cfg, st, Q, K, V, eta, O, w.chunk_kv, w.chunk_q, w.order, ws)
    torch.cuda.synchronize()
    out = {n: t.cpu().numpy() for n, t in st.items()}
    return O.float().cpu().numpy(), out


def run_oracle(w: S.Workload, x, st_np, pairs=None, token_block=65536):
    import oracle
    hp = oracle.Hyper(opt=w.opt, beta=w.beta, ns_iters=w.ns_iters, token_block=token_block,
                      norm_keep=w.norm == "keep", net=w.net, normalize=w.norm != "none")
    return oracle.lact_chunked_forward(st_np, x["Q"], x["K"], x["V"], x["eta"], w.chunk_kv,
                                       w.chunk_q, w.order, hp, pairs=pairs)


def compare(w: S.Workload, O_gpu, st_gpu, O_ref, st_ref, pairs=None, tol=None):
    """Worst rel err per tensor over the given pairs (all pairs if None)."""
    tol = tol_of(w) if tol is None else tol
    sel = (lambda a: a) if pairs is None else (lambda a: np.stack([a[b, h] for b, h in pairs]))
    errs = {"O": rel_err(sel(O_gpu), sel(O_ref))}
    for n in st_ref:
        if n in st_gpu:
            errs[n] = rel_err(sel(st_gpu[n]), sel(st_ref[n]))
    say(f"  {w.name}: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()) + f" (tol {tol:.0e})")
    bad = {k: v for k, v in errs.items() if not v <= tol}
    return errs, bad
