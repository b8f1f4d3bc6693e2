"""Plain CPU oracle of the LaCT large-chunk test-time-training layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library under ``chunk_test_amd/``.

Sources (the text of the pages, cited by page title and section):

* "Test-Time Training Done Right", Abstract (arXiv page and project page):
  fast weights act like a recurrent state that carries memory of earlier
  tokens; one update per very large chunk (2K to ~1M tokens); Muon as an
  online optimizer.
* "LaCT: Large Chunk Test-Time Training" (iplexlaw.co.kr review),
  section "Local attention and nonlinear memory work together": the fast net
  is a three-matrix SwiGLU MLP; the loss is a negative inner product between
  the net's output on a key and its value; the chunk gradient weights each
  token by its own learning rate; queries read the fast weights; the update
  is GD, momentum or Muon (Newton-Schulz on the matrix gradient); updated
  fast weights are L2-normalised; the chunk is treated as a set.
* same review, section "Update order must respect the task": language/video
  chunks read memory holding only earlier chunks and then update it
  (apply-then-update); posed image sets absorb the inputs first and then
  answer target-view queries (update-then-apply).
* project page, Figure 2 caption: the fast weight W passes from chunk to
  chunk (sequential scan).

The pages print no formulas.  The plainest reading used here:

* f_W(x) = W2 (silu(W1 x) * (W3 x)), W1, W3 in R^{h x d}, W2 in R^{d x h};
  silu(z) = z * sigmoid(z).
* chunk loss L(W) = - sum_i eta_i <f_W(k_i), v_i>  (a plain sum, no 1/n).
* GD: W <- W - step * dL/dW.  Momentum (heavy ball): M <- beta M + dL/dW,
  W <- W - step * M.  Muon: the direction is NS(g) with g the gradient (or
  the momentum buffer when beta > 0).
* NS(G): work on the orientation whose Gram matrix is the smaller one,
  X0 = G / (||G||_F + eps), then I times  A = X X^T, X <- a X + (b A + c A A) X.
* after each update every stored row r of W1, W3 (length d) and W2 (length h)
  becomes r / max(||r||_2, norm_eps).  The initial weights are not normalised.
* variant with a learning rate per token and matrix (eta of shape [n, 3],
  columns for W1, W2, W3): each matrix follows the gradient of the loss
  written with its own rates, dW_m = d/dW_m (- sum_i eta_{i,m} <f_W(k_i), v_i>);
  with three equal columns this is the shared-rate rule.
* variant ``norm_keep`` (weight normalisation with the magnitude held: the
  reference list's "Weight Normalization" separates a row's direction from
  its length; here the update moves only the direction): the stepped row u
  is rescaled to the length the row had before the update,
  u * ||r_old||_2 / max(||u||_2, norm_eps), so every row keeps its initial
  length through the scan.
* every query of a chunk reads the same W (no causality inside a chunk).

Every routine takes a ``dtype`` (float64 for parity, float32 for the timed
CPU baseline).  Parity against the pages' own numbers is unpinned (the pages
print no per-layer values); the routines are pinned by the tests in
``tests/test_oracle_pins.py`` (finite differences, autograd, closed forms,
SVD identities and invariants).
"""

from __future__ import annotations

import numpy as np

APPLY_THEN_UPDATE = "apply_then_update"
UPDATE_THEN_APPLY = "update_then_apply"
ORDERS = (APPLY_THEN_UPDATE, UPDATE_THEN_APPLY)

OPT_GD = "gd"
OPT_MOMENTUM = "momentum"
OPT_MUON = "muon"
OPTIMIZERS = (OPT_GD, OPT_MOMENTUM, OPT_MUON)

# Quintic Newton-Schulz coefficients published with the Muon optimizer
# (K. Jordan et al., 2024).  The pages only name Newton-Schulz; the
# coefficients are arguments everywhere.
MUON_COEFFS = (3.4445, -4.7750, 2.0315)


# --------------------------------------------------------------------------
# elementwise pieces
# --------------------------------------------------------------------------

def sigmoid(z):
    """Logistic function, evaluated without overflow for either sign of z."""
    z = np.asarray(z)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def silu(z):
    """silu(z) = z * sigmoid(z), the gate of a SwiGLU MLP."""
    return z * sigmoid(z)


# --------------------------------------------------------------------------
# fast net (review, "Local attention and nonlinear memory work together":
# a three-matrix SwiGLU MLP)
# --------------------------------------------------------------------------

def swiglu_forward(W1, W2, W3, X):
    """Rows of X [n, d] -> rows of f_W(X) [n, d], f_W(x) = W2 (silu(W1 x) * (W3 x))."""
    H1 = X @ W1.T
    H3 = X @ W3.T
    return (silu(H1) * H3) @ W2.T


def swiglu_loss(W1, W2, W3, K, V, eta):
    """L = - sum_i eta_i <f_W(k_i), v_i> over the chunk (a plain sum)."""
    F = swiglu_forward(W1, W2, W3, K)
    return -np.sum(eta * np.sum(F * V, axis=1))


def swiglu_grad(W1, W2, W3, K, V, eta, token_block=None):
    """Gradient of ``swiglu_loss`` with respect to (W1, W2, W3).

    ``eta`` is [n] (one rate per token) or [n, 3] (a rate per token and
    matrix: column m weights the loss whose gradient W1, W2, W3 follow).

    Back-propagation through f_W: with U_i = dL/df(k_i) = -eta_i v_i,
      dW2 = U^T G,  dG = U W2,  dH3 = dG * A,  dH1 = dG * H3 * silu'(H1),
      dW1 = dH1^T K,  dW3 = dH3^T K,
    where H1 = K W1^T, H3 = K W3^T, A = silu(H1), G = A * H3 and
    silu'(z) = s (1 + z (1 - s)), s = sigmoid(z).

    The loss is a sum over tokens, so its gradient is the sum of per-token
    gradients; ``token_block`` only bounds host memory by summing that sum in
    consecutive blocks of tokens.
    """
    n = K.shape[0]
    if token_block is None or token_block >= n:
        blocks = [(0, n)]
    else:
        blocks = [(s, min(n, s + token_block)) for s in range(0, n, token_block)]
    dW1 = np.zeros_like(W1)
    dW2 = np.zeros_like(W2)
    dW3 = np.zeros_like(W3)
    eta = np.asarray(eta)
    for s, e in blocks:
        Kb, Vb = K[s:e], V[s:e]
        H1 = Kb @ W1.T
        H3 = Kb @ W3.T
        S = sigmoid(H1)
        A = H1 * S
        G = A * H3
        dA = S * (1.0 + H1 * (1.0 - S))  # silu'(H1)
        if eta.ndim == 1:
            eb = eta[s:e]
            U = -eb[:, None] * Vb
            dW2 += U.T @ G
            dG = U @ W2
            dH3 = dG * A
            dH1 = dG * H3 * dA
        else:
            # U_m = -eta_{i,m} v_i: the output gradient of the loss matrix m follows
            U1, U2, U3 = (-eta[s:e, m][:, None] * Vb for m in range(3))
            dW2 += U2.T @ G
            dH3 = (U3 @ W2) * A
            dH1 = (U1 @ W2) * H3 * dA
        dW1 += dH1.T @ Kb
        dW3 += dH3.T @ Kb
    return dW1, dW2, dW3


# --------------------------------------------------------------------------
# linear fast net (review, "Large chunks alone do not explain the gains":
# the nonlinear fast net against a linear state).  The closed-form pins use
# it without row normalisation; the GPU variant runs it with every
# normalisation mode.
# --------------------------------------------------------------------------

def linear_forward(W, X):
    """Rows of X [n, d] -> rows of W x."""
    return X @ W.T


def linear_grad(W, K, V, eta):
    """d/dW of -sum_i eta_i <W k_i, v_i>  =  -sum_i eta_i v_i k_i^T."""
    U = -eta[:, None] * V
    return U.T @ K


# --------------------------------------------------------------------------
# update rule pieces
# --------------------------------------------------------------------------

def newton_schulz(G, iters, coeffs=MUON_COEFFS, eps=1e-7):
    """Newton-Schulz orthogonalisation of one matrix (Muon's transform).

    Works on the orientation with the smaller Gram matrix (rows <= cols),
    X0 = G / (||G||_F + eps), then ``iters`` times
        A = X X^T,  X <- a X + (b A + c A A) X,
    and returns the result in G's orientation.
    """
    a, b, c = coeffs
    X = np.array(G, copy=True)
    transposed = X.shape[0] > X.shape[1]
    if transposed:
        X = X.T
    X = X / (np.linalg.norm(X) + eps)
    for _ in range(iters):
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X.T if transposed else X


def row_normalize(W, eps=1e-12):
    """Every row r of W becomes r / max(||r||_2, eps)."""
    nrm = np.sqrt(np.sum(W * W, axis=1, keepdims=True))
    return W / np.maximum(nrm, eps)


def optimizer_step(W, dW, M, *, opt, beta, ns_iters, ns_coeffs, ns_eps, step,
                   norm_eps, normalize=True, norm_keep=False):
    """One update of one fast-weight matrix.  Returns (W_new, M_new).

    GD: direction = dW.  Momentum: M <- beta M + dW, direction = M.
    Muon: direction = NS(dW), or NS(M) after the momentum update when
    beta > 0.  Then W <- W - step * direction, then row-wise L2
    normalisation (unless ``normalize`` is False, used by the linear pins);
    with ``norm_keep`` each row is rescaled to its length before the step
    instead of to 1.
    """
    if opt not in OPTIMIZERS:
        raise ValueError(f"unknown optimizer {opt!r}")
    g = dW
    use_m = opt == OPT_MOMENTUM or (opt == OPT_MUON and beta > 0)
    if use_m:
        if M is None:
            M = np.zeros_like(W)
        M = beta * M + g
        g = M
    if opt == OPT_MUON:
        g = newton_schulz(g, ns_iters, ns_coeffs, ns_eps)
    W_old = W
    W = W - step * g
    if normalize:
        W = row_normalize(W, norm_eps)
        if norm_keep:
            W = W * np.sqrt(np.sum(W_old * W_old, axis=1, keepdims=True))
    return W, M


# --------------------------------------------------------------------------
# the layer on one (batch, head) pair
# --------------------------------------------------------------------------

class Hyper:
    """Arguments of the update rule (defaults follow the readings above).

    ``net`` selects the fast net: "swiglu" (the layer) or "linear" (the test
    mode of the closed-form pins, with a single matrix W in R^{d x d}).
    ``normalize`` turns the row normalisation off for the linear pins;
    ``norm_keep`` rescales every updated row to its length before the update
    instead of to 1.
    """

    def __init__(self, opt=OPT_GD, beta=0.0, ns_iters=5, ns_coeffs=MUON_COEFFS,
                 ns_eps=1e-7, step=1.0, norm_eps=1e-12, token_block=None,
                 net="swiglu", normalize=True, norm_keep=False):
        if opt not in OPTIMIZERS:
            raise ValueError(f"unknown optimizer {opt!r}")
        if net not in ("swiglu", "linear"):
            raise ValueError(f"unknown fast net {net!r}")
        self.opt = opt
        self.beta = float(beta)
        self.ns_iters = int(ns_iters)
        self.ns_coeffs = tuple(float(x) for x in ns_coeffs)
        self.ns_eps = float(ns_eps)
        self.step = float(step)
        self.norm_eps = float(norm_eps)
        self.token_block = token_block
        self.net = net
        self.normalize = bool(normalize)
        self.norm_keep = bool(norm_keep)

    def uses_momentum(self):
        return self.opt == OPT_MOMENTUM or (self.opt == OPT_MUON and self.beta > 0)


def fast_forward(W, X, hp: Hyper):
    """f_W on the rows of X for the selected fast net (W is a tuple)."""
    if hp.net == "linear":
        return linear_forward(W[0], X)
    return swiglu_forward(W[0], W[1], W[2], X)


def fast_grad(W, K, V, eta, hp: Hyper):
    """Chunk gradient of the loss for the selected fast net (a tuple like W)."""
    if hp.net == "linear":
        return (linear_grad(W[0], K, V, eta),)
    return swiglu_grad(W[0], W[1], W[2], K, V, eta, hp.token_block)


def update_pair(W, M, K, V, eta, hp: Hyper):
    """One large-chunk update of one pair's fast weights.

    W = (W1, W2, W3) (or (W,) for the linear net); M is a tuple of the same
    length or None.  Returns (W_new, M_new).
    """
    dW = fast_grad(W, K, V, eta, hp)
    Ms = M if M is not None else (None,) * len(W)
    out_w, out_m = [], []
    for Wx, dWx, Mx in zip(W, dW, Ms):
        Wn, Mn = optimizer_step(Wx, dWx, Mx, opt=hp.opt, beta=hp.beta,
                                ns_iters=hp.ns_iters, ns_coeffs=hp.ns_coeffs,
                                ns_eps=hp.ns_eps, step=hp.step,
                                norm_eps=hp.norm_eps, normalize=hp.normalize,
                                norm_keep=hp.norm_keep)
        out_w.append(Wn)
        out_m.append(Mn)
    return tuple(out_w), (tuple(out_m) if hp.uses_momentum() else None)


def chunked_forward_pair(W, M, Q, K, V, eta, chunk_kv, chunk_q, order, hp: Hyper):
    """Sequential scan over the chunks of one pair (project page, Figure 2).

    Chunk c holds keys/values/rates [c*chunk_kv, (c+1)*chunk_kv) and queries
    [c*chunk_q, (c+1)*chunk_q).  apply-then-update: the chunk's queries read
    W_{c-1}, then W_c is computed; update-then-apply: W_c first, then the
    queries read it.  The last update always runs.  Returns (O, W, M).
    """
    if order not in ORDERS:
        raise ValueError(f"unknown order {order!r}")
    T_kv, T_q = K.shape[0], Q.shape[0]
    if T_kv % chunk_kv or T_q % chunk_q:
        raise ValueError("chunk sizes must divide the sequence lengths")
    N = T_kv // chunk_kv
    if T_q // chunk_q != N:
        raise ValueError("key and query chunk counts differ")
    O = np.zeros_like(Q)
    for c in range(N):
        ks = slice(c * chunk_kv, (c + 1) * chunk_kv)
        qs = slice(c * chunk_q, (c + 1) * chunk_q)
        if order == APPLY_THEN_UPDATE:
            O[qs] = fast_forward(W, Q[qs], hp)
        W, M = update_pair(W, M, K[ks], V[ks], eta[ks], hp)
        if order == UPDATE_THEN_APPLY:
            O[qs] = fast_forward(W, Q[qs], hp)
    return O, W, M


# --------------------------------------------------------------------------
# batched entry points over [B, H, ...] arrays (what the tests compare with)
# --------------------------------------------------------------------------

def _pairs(B, H):
    for b in range(B):
        for h in range(H):
            yield b, h


def lact_apply(state, Q, dtype=np.float64):
    """O[b,h] = f_W(Q[b,h]) for every pair.  ``state`` holds W1, W2, W3."""
    Q = np.asarray(Q, dtype=dtype)
    B, H = Q.shape[:2]
    O = np.zeros_like(Q)
    for b, h in _pairs(B, H):
        W1 = np.asarray(state["W1"][b, h], dtype=dtype)
        W2 = np.asarray(state["W2"][b, h], dtype=dtype)
        W3 = np.asarray(state["W3"][b, h], dtype=dtype)
        O[b, h] = swiglu_forward(W1, W2, W3, Q[b, h])
    return O


def _pair_eta(eta, b, h, dtype):
    """Rates of pair (b, h): eta [B, H, T] -> [T]; per matrix, [3, B, H, T] -> [T, 3]."""
    if eta.ndim == 4:
        return np.asarray(eta[:, b, h], dtype=dtype).T
    return np.asarray(eta[b, h], dtype=dtype)


def lact_update(state, K, V, eta, hp: Hyper, dtype=np.float64):
    """One update of every pair on one chunk.  Returns a new state dict.
    ``eta`` is [B, H, T], or [3, B, H, T] for a rate per token and matrix."""
    K = np.asarray(K, dtype=dtype)
    V = np.asarray(V, dtype=dtype)
    eta = np.asarray(eta)
    B, H = K.shape[:2]
    new = {k: np.array(v, dtype=dtype, copy=True) for k, v in state.items()}
    for b, h in _pairs(B, H):
        W = tuple(new[n][b, h] for n in ("W1", "W2", "W3"))
        M = (tuple(new[n][b, h] for n in ("M1", "M2", "M3"))
             if hp.uses_momentum() and "M1" in new else None)
        W, M = update_pair(W, M, K[b, h], V[b, h], _pair_eta(eta, b, h, dtype), hp)
        for n, x in zip(("W1", "W2", "W3"), W):
            new[n][b, h] = x
        if M is not None:
            for n, x in zip(("M1", "M2", "M3"), M):
                new.setdefault(n, np.zeros_like(new["W" + n[1]]))[b, h] = x
    return new


def lact_chunked_forward(state, Q, K, V, eta, chunk_kv, chunk_q, order, hp: Hyper,
                         dtype=np.float64, pairs=None):
    """The whole layer over [B, H, T, d] inputs.  Returns (O, new_state).

    ``pairs`` optionally restricts the work to a list of (b, h) pairs (the
    other outputs stay zero and their state is copied unchanged); the pairs
    are independent, so this is how large configurations are sampled.
    ``eta`` is [B, H, T_kv], or [3, B, H, T_kv] for a rate per token and matrix.
    With the linear fast net (``hp.net == "linear"``) the state holds one
    matrix per pair, W1 [B, H, d, d] (and M1).
    """
    B, H = K.shape[:2]
    wn = ("W1",) if hp.net == "linear" else ("W1", "W2", "W3")
    mn = tuple("M" + n[1] for n in wn)
    new = {k: np.array(v, dtype=dtype, copy=True) for k, v in state.items()}
    if hp.uses_momentum():
        for n in mn:
            new.setdefault(n, np.zeros_like(new["W" + n[1]]))
    O = np.zeros(Q.shape, dtype=dtype)
    todo = list(_pairs(B, H)) if pairs is None else list(pairs)
    for b, h in todo:
        # inputs are cast one pair at a time to bound host memory
        cast = lambda x: np.asarray(x[b, h], dtype=dtype)
        W = tuple(new[n][b, h] for n in wn)
        M = tuple(new[n][b, h] for n in mn) if hp.uses_momentum() else None
        O[b, h], W, M = chunked_forward_pair(W, M, cast(Q), cast(K), cast(V),
                                             _pair_eta(eta, b, h, dtype), chunk_kv, chunk_q,
                                             order, hp)
        for n, x in zip(wn, W):
            new[n][b, h] = x
        if M is not None:
            for n, x in zip(mn, M):
                new[n][b, h] = x
    return O, new
