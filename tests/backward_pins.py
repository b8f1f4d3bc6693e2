"""Pins of the backward oracle (CPU, float64), independent of its code.

* ``torch_scan``: the layer's forward written again with torch float64
  tensors (f_W, the chunk loss, its gradient taken by torch.autograd with
  create_graph so the outer pass differentiates through it, GD / momentum /
  Newton-Schulz, unit rows, both orders); torch.autograd of
  sum(O * dO) + sum(W_N * dW_N) gives the reference cotangents.
* central finite differences of the same objective along random directions
  (through the oracle's own forward, which is pinned separately).
* eta = 0: the chunk gradient vanishes for every K, V, so dK = dV = 0.
"""

from __future__ import annotations

import numpy as np

COEFFS = (3.4445, -4.7750, 2.0315)


def torch_scan(W0, Q, K, V, eta, chunk_kv, chunk_q, order, opt, beta, ns_iters=5, step=1.0,
               norm_eps=1e-12, ns_eps=1e-7):
    """Forward of one pair in torch (inputs are torch float64 tensors that may
    require grad).  Returns (O, W_final)."""
    import torch

    def f(W, X):
        W1, W2, W3 = W
        return (torch.nn.functional.silu(X @ W1.T) * (X @ W3.T)) @ W2.T

    def ns(G):
        a, b, c = COEFFS
        X = G.T if G.shape[0] > G.shape[1] else G
        X = X / (torch.linalg.norm(X) + ns_eps)
        for _ in range(ns_iters):
            A = X @ X.T
            X = a * X + (b * A + c * (A @ A)) @ X
        return X.T if G.shape[0] > G.shape[1] else X

    def rows(W):
        return W / torch.clamp(torch.linalg.norm(W, dim=1, keepdim=True), min=norm_eps)

    W = list(W0)
    mom = opt == "momentum" or (opt == "muon" and beta > 0)
    M = [torch.zeros_like(x) for x in W]
    N = K.shape[0] // chunk_kv
    outs = []
    for c in range(N):
        ks = slice(c * chunk_kv, (c + 1) * chunk_kv)
        qs = slice(c * chunk_q, (c + 1) * chunk_q)
        if order == "apply_then_update":
            outs.append(f(W, Q[qs]))
        loss = -(eta[ks] * (f(W, K[ks]) * V[ks]).sum(1)).sum()
        g = torch.autograd.grad(loss, W, create_graph=True)
        newW = []
        for m in range(3):
            d = g[m]
            if mom:
                M[m] = beta * M[m] + d
                d = M[m]
            if opt == "muon":
                d = ns(d)
            newW.append(rows(W[m] - step * d))
        W = newW
        if order == "update_then_apply":
            outs.append(f(W, Q[qs]))
    return torch.cat(outs, 0), W


def reference_cotangents(W0, Q, K, V, eta, dO, dWf, chunk_kv, chunk_q, order, opt, beta):
    import torch
    t = lambda x: torch.tensor(np.asarray(x, np.float64), dtype=torch.float64, requires_grad=True)
    Wt = [t(x) for x in W0]
    Qt, Kt, Vt, Et = t(Q), t(K), t(V), t(eta)
    O, WN = torch_scan(Wt, Qt, Kt, Vt, Et, chunk_kv, chunk_q, order, opt, beta)
    obj = (O * torch.tensor(dO)).sum() + sum((w * torch.tensor(d)).sum() for w, d in zip(WN, dWf))
    grads = torch.autograd.grad(obj, [Qt, Kt, Vt, Et] + Wt)
    return [g.detach().numpy() for g in grads]


def tiny_case(seed, d=6, h=10, T=12, chunk=4, Tq=6, chunk_q=2):
    r = np.random.default_rng(seed)
    W0 = (r.normal(size=(h, d)) / np.sqrt(d), r.normal(size=(d, h)) / np.sqrt(h),
          r.normal(size=(h, d)) / np.sqrt(d))
    Q, K, V = r.normal(size=(Tq, d)), r.normal(size=(T, d)), r.normal(size=(T, d))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    eta = 0.3 * np.abs(r.normal(size=T))
    dO = r.normal(size=(Tq, d))
    dWf = tuple(r.normal(size=w.shape) for w in W0)
    return W0, Q, K, V, eta, dO, dWf, chunk, chunk_q


def rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def pin_autograd(o, opt, beta, order, seed=5):
    """max rel err of every oracle cotangent against torch.autograd."""
    W0, Q, K, V, eta, dO, dWf, ck, cq = tiny_case(seed)
    hp = o.Hyper(opt=opt, beta=beta)
    dq, dk, dv, de, dw = o.chunked_backward_pair(W0, Q, K, V, eta, dO, ck, cq, order, hp, dWf)
    ref = reference_cotangents(W0, Q, K, V, eta, dO, dWf, ck, cq, order, opt, beta)
    mine = [dq, dk, dv, de, *dw]
    return max(rel(a, b) for a, b in zip(mine, ref))


def pin_finite_differences(o, opt, beta, order, seed=9, h=1e-6):
    """Directional derivatives of sum(O dO) + sum(W_N dW_N) by central
    differences through the oracle's forward, against the oracle's
    cotangents (max rel err over the inputs)."""
    W0, Q, K, V, eta, dO, dWf, ck, cq = tiny_case(seed)
    hp = o.Hyper(opt=opt, beta=beta)

    def obj(W, Q_, K_, V_, e_):
        M = tuple(np.zeros_like(x) for x in W) if hp.uses_momentum() else None
        O, WN, _ = o.chunked_forward_pair(W, M, Q_, K_, V_, e_, ck, cq, order, hp)
        return float(np.sum(O * dO) + sum(np.sum(a * b) for a, b in zip(WN, dWf)))

    dq, dk, dv, de, dw = o.chunked_backward_pair(W0, Q, K, V, eta, dO, ck, cq, order, hp, dWf)
    r = np.random.default_rng(seed + 1)
    worst = 0.0
    args = [W0, Q, K, V, eta]
    grads = [dw, dq, dk, dv, de]
    for i in range(5):
        if i == 0:
            dirs = tuple(r.normal(size=w.shape) for w in W0)
            plus = (tuple(w + h * x for w, x in zip(W0, dirs)),)
            minus = (tuple(w - h * x for w, x in zip(W0, dirs)),)
            analytic = sum(np.sum(g * x) for g, x in zip(dw, dirs))
        else:
            x = r.normal(size=args[i].shape)
            plus = (args[i] + h * x,)
            minus = (args[i] - h * x,)
            analytic = np.sum(grads[i] * x)
        ap = args[:i] + list(plus) + args[i + 1:]
        am = args[:i] + list(minus) + args[i + 1:]
        fd = (obj(*ap) - obj(*am)) / (2 * h)
        worst = max(worst, abs(fd - analytic) / max(abs(analytic), 1e-8))
    return worst


def pin_eta_zero(o, seed=11):
    """eta = 0: the chunk gradient is zero for every K and V, so dK = dV = 0
    (deta does not vanish)."""
    W0, Q, K, V, eta, dO, dWf, ck, cq = tiny_case(seed)
    eta = np.zeros_like(eta)
    hp = o.Hyper(opt="muon", beta=0.5)
    dq, dk, dv, de, dw = o.chunked_backward_pair(W0, Q, K, V, eta, dO, ck, cq, "apply_then_update",
                                                 hp, dWf)
    assert np.max(np.abs(de)) > 0
    return float(max(np.max(np.abs(dk)), np.max(np.abs(dv))))


CONFIGS = [(opt, beta, order) for opt, beta in (("gd", 0.0), ("momentum", 0.9), ("muon", 0.0),
                                               ("muon", 0.6))
           for order in ("apply_then_update", "update_then_apply")]
