"""Plain CPU oracle of the backward pass of the LaCT layer.

TEST INFRASTRUCTURE ONLY, like ``lact_oracle``: nothing in the product path
may import, call or link this module, and it shares no code with the HIP
library.

What it computes.  The layer is trained through its outputs: the pages'
throughput table is training throughput ("LaCT: Large Chunk Test-Time
Training" review, section "Language modelling: quality and throughput
differ"), and context parallelism is described for training (same review,
"Video and distributed computation").  Given the cotangent dO of the
layer's outputs (and optionally dW_N of the final fast weights), this module
returns the cotangents of every input of ``lact_oracle.lact_chunked_forward``:
dQ, dK, dV, deta and dW_0 (the initial fast weights), by reverse-mode
differentiation of the scan, chunk by chunk in reverse order, with each
chunk's fast weights recomputed by a forward pass (the checkpoints W_c).

Each step of the forward has its vector-Jacobian product written out here
(derived by hand, in the order the forward runs them):
  * the query read O = f_W(Q);
  * the chunk gradient g(W, K, V, eta) of the SwiGLU loss, which is itself a
    gradient: its VJP carries second-order terms (silu'');
  * the optimizer: GD, heavy-ball momentum (the buffer's cotangent is carried
    back through the chunks) and Muon (Newton-Schulz, differentiated
    through every iteration and through the Frobenius pre-scaling);
  * the step W - step * direction and the unit row normalisation.

Scope: the SwiGLU fast net with unit rows (norm_mode unit), one rate per
token, any order and optimizer.  Pinned in ``tests/test_oracle_backward.py``
against torch.autograd through an independently written float64 forward,
and against central finite differences.
"""

from __future__ import annotations

import numpy as np

from . import lact_oracle as F


# --------------------------------------------------------------------------
# elementwise pieces
# --------------------------------------------------------------------------

def silu_d1(z):
    """silu'(z) = s (1 + z (1 - s)), s = sigmoid(z)."""
    s = F.sigmoid(z)
    return s * (1.0 + z * (1.0 - s))


def silu_d2(z):
    """silu''(z) = s (1 - s) (2 + z (1 - 2 s))."""
    s = F.sigmoid(z)
    return s * (1.0 - s) * (2.0 + z * (1.0 - 2.0 * s))


# --------------------------------------------------------------------------
# VJPs of the forward steps
# --------------------------------------------------------------------------

def apply_vjp(W1, W2, W3, Q, dO):
    """Cotangents of O = f_W(Q) = (silu(Q W1^T) * (Q W3^T)) W2^T.

    Returns (dQ, dW1, dW2, dW3)."""
    H1 = Q @ W1.T
    H3 = Q @ W3.T
    A = F.silu(H1)
    G = A * H3
    dW2 = dO.T @ G
    dG = dO @ W2
    dH3 = dG * A
    dH1 = dG * H3 * silu_d1(H1)
    dQ = dH1 @ W1 + dH3 @ W3
    return dQ, dH1.T @ Q, dW2, dH3.T @ Q


def grad_vjp(W1, W2, W3, K, V, eta, P1, P2, P3):
    """VJP of the chunk gradient (gW1, gW2, gW3) = swiglu_grad(W, K, V, eta)
    with cotangents (P1, P2, P3) of (gW1, gW2, gW3).

    Forward (per chunk): H1 = K W1^T, H3 = K W3^T, A = silu(H1), G = A H3,
    U = -eta V, dG = U W2, dH3 = dG A, dH1 = dG H3 silu'(H1),
    gW2 = U^T G, gW1 = dH1^T K, gW3 = dH3^T K.
    Returns (dW1, dW2, dW3, dK, dV, deta)."""
    H1 = K @ W1.T
    H3 = K @ W3.T
    S1 = silu_d1(H1)
    A = F.silu(H1)
    G = A * H3
    U = -eta[:, None] * V
    dG = U @ W2
    dH3 = dG * A
    dH1 = dG * H3 * S1
    # cotangents of the forward's intermediates
    dH1_bar = K @ P1.T              # from gW1 = dH1^T K
    dH3_bar = K @ P3.T              # from gW3 = dH3^T K
    G_bar = U @ P2                  # from gW2 = U^T G
    U_bar = G @ P2.T
    dK = dH1 @ P1 + dH3 @ P3
    # dH3 = dG A;  dH1 = dG H3 S1
    dG_bar = dH3_bar * A + dH1_bar * H3 * S1
    A_bar = dH3_bar * dG + G_bar * H3
    H3_bar = dH1_bar * dG * S1 + G_bar * A
    H1_bar = dH1_bar * dG * H3 * silu_d2(H1) + A_bar * S1
    # dG = U W2
    U_bar = U_bar + dG_bar @ W2.T
    dW2 = U.T @ dG_bar
    # H1 = K W1^T, H3 = K W3^T
    dK = dK + H1_bar @ W1 + H3_bar @ W3
    dW1 = H1_bar.T @ K
    dW3 = H3_bar.T @ K
    # U = -eta V
    dV = -eta[:, None] * U_bar
    deta = -np.sum(U_bar * V, axis=1)
    return dW1, dW2, dW3, dK, dV, deta


def newton_schulz_vjp(G, dX, iters, coeffs=F.MUON_COEFFS, eps=1e-7):
    """Cotangent of G for X = newton_schulz(G) with cotangent dX.

    Reverse of: X0 = G' / (||G'||_F + eps) (G' = G or G^T, rows <= cols),
    X_{k+1} = a X_k + B_k X_k, B_k = b A_k + c A_k A_k, A_k = X_k X_k^T."""
    a, b, c = coeffs
    Gp = np.array(G, copy=True)
    dXp = np.array(dX, copy=True)
    transposed = Gp.shape[0] > Gp.shape[1]
    if transposed:
        Gp, dXp = Gp.T, dXp.T
    nrm = np.linalg.norm(Gp)
    X = Gp / (nrm + eps)
    xs = [X]
    for _ in range(iters):
        A = X @ X.T
        X = a * X + (b * A + c * (A @ A)) @ X
        xs.append(X)
    dY = dXp
    for k in range(iters - 1, -1, -1):
        X = xs[k]
        A = X @ X.T
        B = b * A + c * (A @ A)
        dB = dY @ X.T
        dXk = a * dY + B.T @ dY
        dA = b * dB + c * (dB @ A.T + A.T @ dB)
        dXk = dXk + (dA + dA.T) @ X
        dY = dXk
    # X0 = G' / (n + eps), n = ||G'||_F
    dG = dY / (nrm + eps)
    if nrm > 0:
        dG = dG - (np.sum(dY * Gp) / (nrm + eps) ** 2) * Gp / nrm
    return dG.T if transposed else dG


def row_normalize_vjp(R, Y, dY, eps=1e-12):
    """Cotangent of R for Y = row_normalize(R, eps) with cotangent dY."""
    nrm = np.sqrt(np.sum(R * R, axis=1, keepdims=True))
    big = nrm > eps
    proj = dY - Y * np.sum(Y * dY, axis=1, keepdims=True)
    return np.where(big, proj / np.maximum(nrm, eps), dY / eps)


# --------------------------------------------------------------------------
# the scan on one pair
# --------------------------------------------------------------------------

def chunked_backward_pair(W, Q, K, V, eta, dO, chunk_kv, chunk_q, order, hp, dW_final=None):
    """Reverse-mode pass of ``lact_oracle.chunked_forward_pair`` for one pair.

    W = (W1, W2, W3) initial fast weights; dO cotangent of the outputs;
    dW_final optional cotangent of the final fast weights.  Returns
    (dQ, dK, dV, deta, dW0) with dW0 = (dW1, dW2, dW3)."""
    if hp.net != "swiglu" or not hp.normalize or hp.norm_keep:
        raise ValueError("backward: SwiGLU net with unit rows only")
    T_kv, T_q = K.shape[0], Q.shape[0]
    N = T_kv // chunk_kv
    mom = hp.uses_momentum()
    # forward, keeping the fast weights (and momentum) entering every chunk
    Ws, Ms = [tuple(W)], [tuple(np.zeros_like(x) for x in W) if mom else None]
    Wc, Mc = tuple(W), Ms[0]
    for c in range(N):
        ks = slice(c * chunk_kv, (c + 1) * chunk_kv)
        Wc, Mc = F.update_pair(Wc, Mc, K[ks], V[ks], eta[ks], hp)
        Ws.append(Wc)
        Ms.append(Mc)
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    deta = np.zeros_like(eta)
    dWc = [np.zeros_like(x) for x in W] if dW_final is None else [np.array(x, copy=True) for x in dW_final]
    dMc = [np.zeros_like(x) for x in W]
    for c in range(N - 1, -1, -1):
        ks = slice(c * chunk_kv, (c + 1) * chunk_kv)
        qs = slice(c * chunk_q, (c + 1) * chunk_q)
        W_in, W_out = Ws[c], Ws[c + 1]
        if order == F.UPDATE_THEN_APPLY:
            dq, d1, d2, d3 = apply_vjp(*W_out, Q[qs], dO[qs])
            dQ[qs] += dq
            dWc = [x + y for x, y in zip(dWc, (d1, d2, d3))]
        # recompute this chunk's update and go back through it
        g = F.swiglu_grad(*W_in, K[ks], V[ks], eta[ks])
        dg = []
        dW_in = []
        for m in range(3):
            gm = g[m]
            if mom:
                gm = hp.beta * Ms[c][m] + gm       # the new momentum M_{c+1}
            direction = F.newton_schulz(gm, hp.ns_iters, hp.ns_coeffs, hp.ns_eps) if hp.opt == F.OPT_MUON else gm
            R = W_in[m] - hp.step * direction
            dR = row_normalize_vjp(R, W_out[m], dWc[m], hp.norm_eps)
            dW_in.append(dR)                       # W_in enters R directly
            ddir = -hp.step * dR
            if hp.opt == F.OPT_MUON:
                ddir = newton_schulz_vjp(gm, ddir, hp.ns_iters, hp.ns_coeffs, hp.ns_eps)
            if mom:
                dM_new = ddir + dMc[m]             # cotangent of M_{c+1}
                dg.append(dM_new)
                dMc[m] = hp.beta * dM_new          # cotangent of M_c
            else:
                dg.append(ddir)
        d1, d2, d3, dk, dv, de = grad_vjp(*W_in, K[ks], V[ks], eta[ks], *dg)
        dK[ks] += dk
        dV[ks] += dv
        deta[ks] += de
        dWc = [x + y for x, y in zip(dW_in, (d1, d2, d3))]
        if order == F.APPLY_THEN_UPDATE:
            dq, d1, d2, d3 = apply_vjp(*W_in, Q[qs], dO[qs])
            dQ[qs] += dq
            dWc = [x + y for x, y in zip(dWc, (d1, d2, d3))]
    return dQ, dK, dV, deta, tuple(dWc)


def lact_chunked_backward(state, Q, K, V, eta, dO, chunk_kv, chunk_q, order, hp,
                          dW_final=None, dtype=np.float64, pairs=None):
    """Backward pass over [B, H, T, d] inputs.  Returns a dict with dQ, dK,
    dV, deta and dW1, dW2, dW3 (cotangents of the initial fast weights).
    ``dW_final`` optionally holds cotangents of the final W1, W2, W3.
    ``pairs`` restricts the work to some (b, h) pairs (the rest stay zero)."""
    B, H = K.shape[:2]
    out = {"dQ": np.zeros(Q.shape, dtype), "dK": np.zeros(K.shape, dtype),
           "dV": np.zeros(V.shape, dtype), "deta": np.zeros(eta.shape, dtype)}
    for n in ("W1", "W2", "W3"):
        out["d" + n] = np.zeros(state[n].shape, dtype)
    todo = [(b, h) for b in range(B) for h in range(H)] if pairs is None else list(pairs)
    for b, h in todo:
        cast = lambda x: np.asarray(x[b, h], dtype=dtype)
        W = tuple(cast(state[n]) for n in ("W1", "W2", "W3"))
        dWf = None if dW_final is None else tuple(cast(dW_final[n]) for n in ("W1", "W2", "W3"))
        dq, dk, dv, de, dw = chunked_backward_pair(W, cast(Q), cast(K), cast(V), cast(eta), cast(dO),
                                                   chunk_kv, chunk_q, order, hp, dWf)
        out["dQ"][b, h], out["dK"][b, h], out["dV"][b, h], out["deta"][b, h] = dq, dk, dv, de
        for n, x in zip(("W1", "W2", "W3"), dw):
            out["d" + n][b, h] = x
    return out
