"""Plant plausible mistakes in copies of the oracle (CPU only) and check that
at least one pin catches each of them.  The real oracle is never modified."""

import importlib.util
import os
import types

import pytest

from tests import oracle_pins as P

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "lact_oracle.py")

# (description, text in the oracle, replacement)
MUTATIONS = [
    ("silu' drops a term", "(1.0 + H1 * (1.0 - S))", "(1.0 + H1 * S)"),
    ("loss sign flipped", "U = -eb[:, None] * Vb", "U = eb[:, None] * Vb"),
    ("mean instead of sum", "dW1 += dH1.T @ Kb", "dW1 += dH1.T @ Kb / len(Kb)"),
    ("W3 used for the gate input", "H3 = X @ W3.T", "H3 = X @ W1.T"),
    ("gate on the wrong branch", "        G = A * H3\n", "        G = H1 * H3\n"),
    ("NS coefficients swapped", "B = b * A + c * (A @ A)", "B = c * A + b * (A @ A)"),
    ("NS spectral instead of Frobenius scaling", "X = X / (np.linalg.norm(X) + eps)",
     "X = X / (np.linalg.norm(X, 2) + eps)"),
    ("NS one iteration short", "for _ in range(iters):", "for _ in range(iters - 1):"),
    ("normalises columns", "nrm = np.sqrt(np.sum(W * W, axis=1, keepdims=True))",
     "nrm = np.sqrt(np.sum(W * W, axis=0, keepdims=True))"),
    ("dampened momentum", "M = beta * M + g", "M = beta * M + (1.0 - beta) * g"),
    ("order ignored (always update first)", "if order == APPLY_THEN_UPDATE:\n            O[qs]",
     "if False:\n            O[qs]"),
    ("last chunk not updated", "W, M = update_pair(W, M, K[ks], V[ks], eta[ks], hp)",
     "W, M = update_pair(W, M, K[ks], V[ks], eta[ks], hp) if c < N - 1 else (W, M)"),
    ("step sign flipped", "W = W - step * g", "W = W + step * g"),
    ("kept length taken after the step", "W = W * np.sqrt(np.sum(W_old * W_old, axis=1, keepdims=True))",
     "W = W * np.sqrt(np.sum(W * W, axis=1, keepdims=True))"),
    ("per-matrix rates of W1 and W3 swapped",
     "U1, U2, U3 = (-eta[s:e, m][:, None] * Vb for m in range(3))",
     "U3, U2, U1 = (-eta[s:e, m][:, None] * Vb for m in range(3))"),
    ("per-matrix W2 follows the W1 rates",
     "U1, U2, U3 = (-eta[s:e, m][:, None] * Vb for m in range(3))",
     "U1, U2, U3 = (-eta[s:e, m][:, None] * Vb for m in (0, 0, 2))"),
    ("kept length squared", "W = W * np.sqrt(np.sum(W_old * W_old, axis=1, keepdims=True))",
     "W = W * np.sum(W_old * W_old, axis=1, keepdims=True)"),
]


def load_mutant(old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation target not unique: {old!r}"
    text = text.replace(old, new, 1)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(text, "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("desc,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(desc, old, new):
    mutant = load_mutant(old, new)
    caught = []
    for name, (fn, tol) in P.ALL_PINS.items():
        try:
            err = fn(mutant)
        except Exception as e:  # a crash also exposes the mistake
            caught.append(f"{name}: {type(e).__name__}")
            continue
        if not err <= tol:
            caught.append(f"{name}: {err:.2e}")
    assert caught, f"no pin caught: {desc}"
