"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each ``pin_*`` function takes the oracle module and returns an error figure
(the worst deviation, in the units the pin states) so that the same pins can
be run against deliberately broken copies of the oracle (tests/test_oracle_mutations.py).

Pins:
* gradient: central finite differences of the loss, and torch.autograd
  (an independent backward pass) through a torch forward of f_W;
* additivity of the chunk gradient over any partition of the tokens (the
  pages' context-parallel claim: gradients of parts of a chunk combine);
* set semantics of the large-chunk update (review, "Local attention and
  nonlinear memory work together": tokens of a chunk are a set);
* closed form of the linear fast net: chunk-causal linear attention for
  apply-then-update, its inclusive twin for update-then-apply, and the
  geometric weights of heavy-ball momentum;
* Newton-Schulz = the scalar polynomial map on the singular values
  (numpy.linalg.svd), convergence of the cubic map to the polar factor,
  oddness, scale invariance and orthogonal equivariance;
* unit row norms after every update;
* chunk size 1 == an independently written per-token loop (autograd
  gradient, SVD-form Newton-Schulz);
* eta = 0 special case and split-run resume.
"""

from __future__ import annotations

import numpy as np

try:
    import torch
except ImportError:  # pragma: no cover - torch is part of the image
    torch = None

COEFFS = (3.4445, -4.7750, 2.0315)


def rng(seed):
    return np.random.default_rng(seed)


def rand_weights(r, d, h, scale=1.0):
    W1 = r.normal(0, scale / np.sqrt(d), (h, d))
    W3 = r.normal(0, scale / np.sqrt(d), (h, d))
    W2 = r.normal(0, scale / np.sqrt(h), (d, h))
    return W1, W2, W3


def unit_rows(x):
    return x / np.linalg.norm(x, axis=1, keepdims=True)


def rel_err(x, y):
    """max_i |x_i - y_i| / max_i |y_i|  (the parity metric used throughout)."""
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    den = np.max(np.abs(y))
    return float(np.max(np.abs(x - y)) / (den if den > 0 else 1.0))


# --------------------------------------------------------------------------
# gradient pins
# --------------------------------------------------------------------------

def pin_fd_grad(o, seed=0, d=4, h=8, n=6, step=1e-6):
    """Central differences of the chunk loss vs the oracle's gradient."""
    r = rng(seed)
    W = list(rand_weights(r, d, h, scale=1.5))
    K = r.normal(size=(n, d))
    V = r.normal(size=(n, d))
    eta = np.abs(r.normal(size=n)) + 0.1
    g = o.swiglu_grad(W[0], W[1], W[2], K, V, eta)
    worst = 0.0
    for m in range(3):
        fd = np.zeros_like(W[m])
        for idx in np.ndindex(W[m].shape):
            Wp = [w.copy() for w in W]
            Wm = [w.copy() for w in W]
            Wp[m][idx] += step
            Wm[m][idx] -= step
            lp = o.swiglu_loss(Wp[0], Wp[1], Wp[2], K, V, eta)
            lm = o.swiglu_loss(Wm[0], Wm[1], Wm[2], K, V, eta)
            fd[idx] = (lp - lm) / (2 * step)
        worst = max(worst, rel_err(g[m], fd))
    return worst


def torch_grad(W1, W2, W3, K, V, eta):
    """Gradient of -sum_i eta_i <f_W(k_i), v_i> by torch.autograd (float64, CPU)."""
    t = lambda x, g=False: torch.tensor(np.asarray(x, np.float64), dtype=torch.float64,
                                        requires_grad=g)
    w1, w2, w3 = t(W1, True), t(W2, True), t(W3, True)
    Kt, Vt, et = t(K), t(V), t(eta)
    F = (torch.nn.functional.silu(Kt @ w1.T) * (Kt @ w3.T)) @ w2.T
    L = -(et * (F * Vt).sum(dim=1)).sum()
    L.backward()
    return w1.grad.numpy(), w2.grad.numpy(), w3.grad.numpy()


def pin_autograd_grad(o, seed=1, d=64, h=128, n=256):
    """Oracle gradient vs torch.autograd at the tiny workload's shapes."""
    r = rng(seed)
    W = rand_weights(r, d, h)
    K = unit_rows(r.normal(size=(n, d)))
    V = unit_rows(r.normal(size=(n, d)))
    eta = 0.01 * np.logaddexp(0, r.normal(size=n))
    g = o.swiglu_grad(*W, K, V, eta)
    ref = torch_grad(*W, K, V, eta)
    return max(rel_err(a, b) for a, b in zip(g, ref))


def pin_grad_additive(o, seed=2, d=16, h=32, n=100):
    """Gradient over a chunk == sum of gradients over a random partition."""
    r = rng(seed)
    W = rand_weights(r, d, h)
    K = r.normal(size=(n, d))
    V = r.normal(size=(n, d))
    eta = np.abs(r.normal(size=n))
    full = o.swiglu_grad(*W, K, V, eta)
    perm = r.permutation(n)
    cuts = np.sort(r.choice(np.arange(1, n), size=4, replace=False))
    parts = np.split(perm, cuts)
    acc = [np.zeros_like(x) for x in full]
    for p in parts:
        gp = o.swiglu_grad(*W, K[p], V[p], eta[p])
        acc = [a + b for a, b in zip(acc, gp)]
    return max(rel_err(a, b) for a, b in zip(acc, full))


# --------------------------------------------------------------------------
# linear fast net closed forms
# --------------------------------------------------------------------------

def linear_closed_form(W0, Q, K, V, eta, chunk, order, beta):
    """o_t = W0 q_t + sum_i w(c_t, c_i) eta_i (k_i . q_t) v_i.

    GD (beta = 0): w = 1 for chunks before c_t (apply-then-update) or up to
    and including c_t (update-then-apply).  Heavy-ball momentum: the gradient
    of chunk c'' reaches the weights after chunk c with total weight
    sum_{j=0}^{c-c''} beta^j = (1 - beta^{c-c''+1}) / (1 - beta).
    """
    T = Q.shape[0]
    ct = np.arange(T) // chunk
    ci = np.arange(K.shape[0]) // chunk
    # weights seen by chunk c_t: W after chunk (c_t - 1) or after chunk c_t
    last = ct - 1 if order == "apply_then_update" else ct
    lag = last[:, None] - ci[None, :]            # chunks elapsed since chunk c_i
    valid = lag >= 0
    if beta == 0.0:
        w = valid.astype(np.float64)
    else:
        w = np.where(valid, (1.0 - beta ** (lag + 1)) / (1.0 - beta), 0.0)
    scores = (Q @ K.T) * w * eta[None, :]
    return Q @ W0.T + scores @ V


def pin_linear_closed_form(o, order, opt="gd", beta=0.0, seed=3, d=8, T=48, chunk=8):
    r = rng(seed)
    W0 = r.normal(size=(d, d)) / np.sqrt(d)
    Q = r.normal(size=(T, d))
    K = r.normal(size=(T, d))
    V = r.normal(size=(T, d))
    eta = np.abs(r.normal(size=T)) * 0.3
    hp = o.Hyper(opt=opt, beta=beta, net="linear", normalize=False)
    M = (np.zeros_like(W0),) if hp.uses_momentum() else None
    O, _, _ = o.chunked_forward_pair((W0,), M, Q, K, V, eta, chunk, chunk, order, hp)
    ref = linear_closed_form(W0, Q, K, V, eta, chunk, order, beta if opt == "momentum" else 0.0)
    return rel_err(O, ref)


# --------------------------------------------------------------------------
# Newton-Schulz pins
# --------------------------------------------------------------------------

def ns_by_svd(G, iters, coeffs=COEFFS, eps=1e-7):
    """NS through the SVD: singular values follow p(x) = a x + b x^3 + c x^5."""
    a, b, c = coeffs
    U, s, Vt = np.linalg.svd(G, full_matrices=False)
    x = s / (np.sqrt(np.sum(s * s)) + eps)
    for _ in range(iters):
        x = a * x + b * x ** 3 + c * x ** 5
    return (U * x) @ Vt


def pin_ns_svd(o, seed=4):
    r = rng(seed)
    worst = 0.0
    for shape in [(64, 128), (128, 64), (128, 256), (256, 128), (7, 5), (1, 9)]:
        G = r.normal(size=shape) * 3.0
        for iters in (1, 2, 5):
            worst = max(worst, rel_err(o.newton_schulz(G, iters, COEFFS, 1e-7),
                                       ns_by_svd(G, iters, COEFFS, 1e-7)))
    return worst


def pin_ns_cubic_polar(o, seed=5, m=8, n=16, iters=30):
    """Cubic (1.5, -0.5, 0) on a well-conditioned G converges to U V^T."""
    r = rng(seed)
    U, _ = np.linalg.qr(r.normal(size=(m, m)))
    Vq, _ = np.linalg.qr(r.normal(size=(n, n)))
    s = np.linspace(0.5, 1.0, m)
    G = (U * s) @ Vq[:, :m].T
    X = o.newton_schulz(G, iters, (1.5, -0.5, 0.0), 1e-7)
    polar = U @ Vq[:, :m].T
    return max(rel_err(X, polar), float(np.max(np.abs(X @ X.T - np.eye(m)))))


def quintic_band(lo=0.01, iters=5, coeffs=COEFFS, eps=0.0):
    """Range of the 5-fold scalar map over x in [lo, 1]."""
    a, b, c = coeffs
    x = np.linspace(lo, 1.0, 200001)
    for _ in range(iters):
        x = a * x + b * x ** 3 + c * x ** 5
    return float(x.min()), float(x.max())


def pin_ns_band(o, seed=6):
    """Singular values of NS_5(G) with sigma/||G||_F >= 0.01 lie in the band.

    Returns how far (absolute) any such singular value falls outside the
    band; 0 means inside.
    """
    lo, hi = quintic_band()
    r = rng(seed)
    worst = 0.0
    for shape in [(64, 128), (128, 256)]:
        G = r.normal(size=(shape[0], 32)) @ r.normal(size=(32, shape[1])) + 0.3 * r.normal(size=shape)
        X = o.newton_schulz(G, 5, COEFFS, 1e-7)
        U, sg, Vt = np.linalg.svd(G, full_matrices=False)
        # X's value along each singular direction of G (the map is not
        # monotone, so sorted singular values of X do not line up with G's)
        sx = np.einsum("ik,ij,jk->k", U, X, Vt.T)
        keep = sg / np.linalg.norm(G) >= 0.01
        s = sx[keep]
        worst = max(worst, float(np.max(np.maximum(lo - s, 0.0))),
                    float(np.max(np.maximum(s - hi, 0.0))))
    return worst


def pin_ns_invariances(o, seed=7):
    r = rng(seed)
    G = r.normal(size=(12, 20))
    X = o.newton_schulz(G, 5, COEFFS, 0.0)
    P, _ = np.linalg.qr(r.normal(size=(12, 12)))
    R, _ = np.linalg.qr(r.normal(size=(20, 20)))
    e1 = rel_err(o.newton_schulz(-G, 5, COEFFS, 0.0), -X)
    e2 = rel_err(o.newton_schulz(7.5 * G, 5, COEFFS, 0.0), X)
    e3 = rel_err(o.newton_schulz(P @ G @ R, 5, COEFFS, 0.0), P @ X @ R)
    return max(e1, e2, e3)


# --------------------------------------------------------------------------
# normalisation, set semantics, chunk-1 loop, special cases
# --------------------------------------------------------------------------

def _small_problem(seed, d=8, h=16, T=32):
    r = rng(seed)
    W = rand_weights(r, d, h)
    Q = unit_rows(r.normal(size=(T, d)))
    K = unit_rows(r.normal(size=(T, d)))
    V = unit_rows(r.normal(size=(T, d)))
    eta = 0.5 * np.logaddexp(0, r.normal(size=T))
    return W, Q, K, V, eta


def pin_row_norms(o, seed=8):
    """|| ||r||_2 - 1 || over every row after updates with each optimizer."""
    W, Q, K, V, eta = _small_problem(seed)
    worst = 0.0
    for opt, beta in (("gd", 0.0), ("momentum", 0.9), ("muon", 0.0), ("muon", 0.5)):
        hp = o.Hyper(opt=opt, beta=beta)
        M = tuple(np.zeros_like(x) for x in W) if hp.uses_momentum() else None
        _, Wn, _ = o.chunked_forward_pair(W, M, Q, K, V, eta, 8, 8, "apply_then_update", hp)
        for x in Wn:
            worst = max(worst, float(np.max(np.abs(np.linalg.norm(x, axis=1) - 1.0))))
    return worst


def pin_set_semantics(o, seed=9):
    """Permuting (k, v, eta) inside a chunk keeps W; permuting queries permutes O."""
    W, Q, K, V, eta = _small_problem(seed, T=40)
    hp = o.Hyper(opt="muon")
    O, Wa, _ = o.chunked_forward_pair(W, None, Q, K, V, eta, 40, 40, "update_then_apply", hp)
    p = rng(seed + 100).permutation(40)
    Op, Wb, _ = o.chunked_forward_pair(W, None, Q[p], K[p], V[p], eta[p], 40, 40,
                                       "update_then_apply", hp)
    return max(max(rel_err(a, b) for a, b in zip(Wa, Wb)), rel_err(Op, O[p]))


def per_token_reference(W, Q, K, V, eta, order, opt, beta, iters=5, keep=False):
    """Token-by-token scan written independently of the oracle.

    Gradient by torch.autograd, Newton-Schulz by its SVD form, heavy-ball
    momentum, unit-norm rows after every token (with ``keep``: each row back
    to the length it had before the token's update).
    """
    W = [np.array(x, np.float64) for x in W]
    M = [np.zeros_like(x) for x in W]
    O = np.zeros_like(Q)

    def read(t):
        h1 = W[0] @ Q[t]
        h3 = W[2] @ Q[t]
        return W[1] @ (h1 / (1.0 + np.exp(-h1)) * h3)

    use_m = opt == "momentum" or (opt == "muon" and beta > 0)
    for t in range(Q.shape[0]):
        if order == "apply_then_update":
            O[t] = read(t)
        g = torch_grad(W[0], W[1], W[2], K[t:t + 1], V[t:t + 1], eta[t:t + 1])
        for m in range(3):
            step = g[m]
            if use_m:
                M[m] = beta * M[m] + step
                step = M[m]
            if opt == "muon":
                step = ns_by_svd(step, iters)
            length = np.linalg.norm(W[m], axis=1, keepdims=True) if keep else 1.0
            W[m] = W[m] - step
            W[m] = length * W[m] / np.linalg.norm(W[m], axis=1, keepdims=True)
        if order == "update_then_apply":
            O[t] = read(t)
    return O, W


def pin_chunk1(o, order, opt, beta=0.0, seed=10, keep=False):
    W, Q, K, V, eta = _small_problem(seed, d=4, h=8, T=12)
    hp = o.Hyper(opt=opt, beta=beta, norm_keep=keep)
    M = tuple(np.zeros_like(x) for x in W) if hp.uses_momentum() else None
    O, Wn, _ = o.chunked_forward_pair(W, M, Q, K, V, eta, 1, 1, order, hp)
    Or, Wr = per_token_reference(W, Q, K, V, eta, order, opt, beta, keep=keep)
    return max(rel_err(O, Or), max(rel_err(a, b) for a, b in zip(Wn, Wr)))


def pin_eta_zero(o, seed=11):
    """eta = 0: every update leaves rownorm(W_init); chunk 0 of A->U reads W_init."""
    W, Q, K, V, eta = _small_problem(seed)
    eta = np.zeros_like(eta)
    Wn_ref = [x / np.linalg.norm(x, axis=1, keepdims=True) for x in W]

    def read(Ws, X):
        H1 = X @ Ws[0].T
        return (H1 / (1 + np.exp(-H1)) * (X @ Ws[2].T)) @ Ws[1].T

    worst = 0.0
    for opt, beta in (("gd", 0.0), ("momentum", 0.9), ("muon", 0.0)):
        hp = o.Hyper(opt=opt, beta=beta)
        M = tuple(np.zeros_like(x) for x in W) if hp.uses_momentum() else None
        for order in ("apply_then_update", "update_then_apply"):
            O, Wn, _ = o.chunked_forward_pair(W, M, Q, K, V, eta, 8, 8, order, hp)
            worst = max(worst, max(rel_err(a, b) for a, b in zip(Wn, Wn_ref)))
            ref = read(Wn_ref, Q)
            if order == "apply_then_update":
                ref[:8] = read(W, Q[:8])
            worst = max(worst, rel_err(O, ref))
    return worst


def pin_norm_keep_lengths(o, seed=13):
    """norm_keep: after a scan every row still has its initial length (rows of
    random lengths, every optimizer)."""
    W, Q, K, V, eta = _small_problem(seed)
    worst = 0.0
    for opt, beta in (("gd", 0.0), ("momentum", 0.9), ("muon", 0.0), ("muon", 0.5)):
        hp = o.Hyper(opt=opt, beta=beta, norm_keep=True)
        M = tuple(np.zeros_like(x) for x in W) if hp.uses_momentum() else None
        _, Wn, _ = o.chunked_forward_pair(W, M, Q, K, V, eta, 8, 8, "apply_then_update", hp)
        for x, x0 in zip(Wn, W):
            n0 = np.linalg.norm(x0, axis=1)
            worst = max(worst, float(np.max(np.abs(np.linalg.norm(x, axis=1) - n0) / n0)))
    return worst


def pin_norm_keep_direction(o, seed=14):
    """norm_keep moves only the lengths: one update from the same state gives
    the unit rule's rows scaled by the old lengths; from unit-length rows the
    two rules agree over a whole scan."""
    W, Q, K, V, eta = _small_problem(seed)
    worst = 0.0
    for opt in ("gd", "muon"):
        Wu, _ = o.update_pair(W, None, K, V, eta, o.Hyper(opt=opt))
        Wk, _ = o.update_pair(W, None, K, V, eta, o.Hyper(opt=opt, norm_keep=True))
        for a, b, x0 in zip(Wk, Wu, W):
            worst = max(worst, rel_err(a, b * np.linalg.norm(x0, axis=1, keepdims=True)))
        Wunit = tuple(unit_rows(x) for x in W)
        Ou, Wu, _ = o.chunked_forward_pair(Wunit, None, Q, K, V, eta, 8, 8, "update_then_apply",
                                           o.Hyper(opt=opt))
        Ok, Wk, _ = o.chunked_forward_pair(Wunit, None, Q, K, V, eta, 8, 8, "update_then_apply",
                                           o.Hyper(opt=opt, norm_keep=True))
        worst = max(worst, rel_err(Ok, Ou), max(rel_err(a, b) for a, b in zip(Wk, Wu)))
    return worst


def pin_eta_per_matrix_columns(o, seed=15, d=16, h=32, n=64):
    """A rate per token and matrix: each matrix's gradient equals the shared-rate
    gradient computed with that matrix's column of rates."""
    r = rng(seed)
    W = rand_weights(r, d, h)
    K, V = r.normal(size=(n, d)), r.normal(size=(n, d))
    E = np.abs(r.normal(size=(n, 3)))
    g = o.swiglu_grad(*W, K, V, E, token_block=17)
    return max(rel_err(g[m], o.swiglu_grad(*W, K, V, E[:, m])[m]) for m in range(3))


def pin_eta_per_matrix_special(o, seed=16):
    """Three equal columns reproduce the shared-rate scan; a zero column for W2
    leaves W2 at its normalised initial value while W1 and W3 move (batched
    entry point, [3, B, H, T] rates)."""
    W, Q, K, V, eta = _small_problem(seed)
    hp = o.Hyper(opt="muon")
    st = {n: x[None, None] for n, x in zip(("W1", "W2", "W3"), W)}
    Q4, K4, V4 = (x[None, None] for x in (Q, K, V))
    O_s, S_s = o.lact_chunked_forward(st, Q4, K4, V4, eta[None, None], 8, 8, "apply_then_update", hp)
    E3 = np.stack([eta, eta, eta])[:, None, None]
    O_p, S_p = o.lact_chunked_forward(st, Q4, K4, V4, E3, 8, 8, "apply_then_update", hp)
    worst = max(rel_err(O_p, O_s), max(rel_err(S_p[n], S_s[n]) for n in ("W1", "W2", "W3")))
    E3 = np.stack([eta, np.zeros_like(eta), eta])[:, None, None]
    _, S_z = o.lact_chunked_forward(st, Q4, K4, V4, E3, 8, 8, "apply_then_update", hp)
    worst = max(worst, rel_err(S_z["W2"][0, 0], unit_rows(W[1])))
    moved = min(rel_err(S_z[n][0, 0], unit_rows(x)) for n, x in (("W1", W[0]), ("W3", W[2])))
    return worst if moved > 1e-3 else float("inf")


def pin_resume(o, seed=12):
    """Chunks [0, k) then [k, N) with the state handed over == one run."""
    W, Q, K, V, eta = _small_problem(seed, T=48)
    hp = o.Hyper(opt="momentum", beta=0.9)
    M0 = tuple(np.zeros_like(x) for x in W)
    O, Wn, Mn = o.chunked_forward_pair(W, M0, Q, K, V, eta, 8, 8, "apply_then_update", hp)
    Oa, Wa, Ma = o.chunked_forward_pair(W, M0, Q[:24], K[:24], V[:24], eta[:24], 8, 8,
                                        "apply_then_update", hp)
    Ob, Wb, Mb = o.chunked_forward_pair(Wa, Ma, Q[24:], K[24:], V[24:], eta[24:], 8, 8,
                                        "apply_then_update", hp)
    return max(rel_err(np.concatenate([Oa, Ob]), O),
               max(rel_err(a, b) for a, b in zip(Wb, Wn)),
               max(rel_err(a, b) for a, b in zip(Mb, Mn)))


ALL_PINS = {
    # name: (callable(o) -> err, tolerance)
    "fd_grad": (lambda o: pin_fd_grad(o), 1e-7),
    "autograd_grad": (lambda o: pin_autograd_grad(o), 1e-10),
    "grad_additive": (lambda o: pin_grad_additive(o), 1e-12),
    "linear_atu_gd": (lambda o: pin_linear_closed_form(o, "apply_then_update"), 1e-12),
    "linear_uta_gd": (lambda o: pin_linear_closed_form(o, "update_then_apply"), 1e-12),
    "linear_atu_mom": (lambda o: pin_linear_closed_form(o, "apply_then_update", "momentum", 0.9), 1e-12),
    "linear_uta_mom": (lambda o: pin_linear_closed_form(o, "update_then_apply", "momentum", 0.7), 1e-12),
    "ns_svd": (lambda o: pin_ns_svd(o), 1e-10),
    "ns_cubic_polar": (lambda o: pin_ns_cubic_polar(o), 1e-10),
    "ns_band": (lambda o: pin_ns_band(o), 0.0),
    "ns_invariances": (lambda o: pin_ns_invariances(o), 1e-10),
    "row_norms": (lambda o: pin_row_norms(o), 1e-12),
    "set_semantics": (lambda o: pin_set_semantics(o), 1e-12),
    "chunk1_atu_gd": (lambda o: pin_chunk1(o, "apply_then_update", "gd"), 1e-10),
    "chunk1_uta_mom": (lambda o: pin_chunk1(o, "update_then_apply", "momentum", 0.9), 1e-10),
    "chunk1_atu_muon": (lambda o: pin_chunk1(o, "apply_then_update", "muon"), 1e-10),
    "chunk1_uta_muon_mom": (lambda o: pin_chunk1(o, "update_then_apply", "muon", 0.5), 1e-10),
    "eta_zero": (lambda o: pin_eta_zero(o), 1e-12),
    "resume": (lambda o: pin_resume(o), 0.0),
    "norm_keep_lengths": (lambda o: pin_norm_keep_lengths(o), 1e-12),
    "eta_per_matrix_columns": (lambda o: pin_eta_per_matrix_columns(o), 1e-12),
    "eta_per_matrix_special": (lambda o: pin_eta_per_matrix_special(o), 1e-12),
    "norm_keep_direction": (lambda o: pin_norm_keep_direction(o), 1e-12),
    "chunk1_atu_gd_keep": (lambda o: pin_chunk1(o, "apply_then_update", "gd", keep=True), 1e-10),
    "chunk1_uta_muon_keep": (lambda o: pin_chunk1(o, "update_then_apply", "muon", 0.5, keep=True), 1e-10),
}
