"""The backward oracle against its pins (CPU, float64), and planted
mistakes in copies of it that the pins must catch."""

import importlib.util
import os
import sys
import types

import numpy as np
import pytest

import oracle
from oracle import lact_backward as BW
from tests import backward_pins as P

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("opt,beta,order", P.CONFIGS)
def test_backward_matches_autograd(opt, beta, order):
    err = P.pin_autograd(_ns(BW), opt, beta, order)
    assert err < 1e-9, err


@pytest.mark.parametrize("opt,beta,order", P.CONFIGS[::3])
def test_backward_matches_finite_differences(opt, beta, order):
    err = P.pin_finite_differences(_ns(BW), opt, beta, order)
    assert err < 1e-6, err


def test_eta_zero_gives_no_key_or_value_cotangent():
    assert P.pin_eta_zero(_ns(BW)) == 0.0


def test_batched_backward_matches_pairwise():
    r = np.random.default_rng(3)
    B, H, d, h, T = 2, 2, 4, 8, 8
    st = {"W1": r.normal(size=(B, H, h, d)), "W2": r.normal(size=(B, H, d, h)),
          "W3": r.normal(size=(B, H, h, d))}
    Q, K, V, dO = (r.normal(size=(B, H, T, d)) for _ in range(4))
    eta = np.abs(r.normal(size=(B, H, T))) * 0.1
    hp = oracle.Hyper(opt="momentum", beta=0.5)
    out = oracle.lact_chunked_backward(st, Q, K, V, eta, dO, 4, 4, "update_then_apply", hp)
    for b in range(B):
        for hh in range(H):
            W = tuple(st[n][b, hh] for n in ("W1", "W2", "W3"))
            dq, dk, dv, de, dw = oracle.chunked_backward_pair(W, Q[b, hh], K[b, hh], V[b, hh], eta[b, hh],
                                                              dO[b, hh], 4, 4, "update_then_apply", hp)
            assert np.array_equal(out["dQ"][b, hh], dq) and np.array_equal(out["deta"][b, hh], de)
            assert np.array_equal(out["dW2"][b, hh], dw[1])


def _ns(mod):
    """A namespace holding the backward entry point and the forward's Hyper."""
    return types.SimpleNamespace(chunked_backward_pair=mod.chunked_backward_pair, Hyper=oracle.Hyper,
                                 chunked_forward_pair=oracle.chunked_forward_pair)


SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "lact_backward.py")

MUTATIONS = [
    ("silu'' drops a term", "(2.0 + z * (1.0 - 2.0 * s))", "(2.0 + z * (1.0 - s))"),
    ("second-order term dropped", "H1_bar = dH1_bar * dG * H3 * silu_d2(H1) + A_bar * S1",
     "H1_bar = A_bar * S1"),
    ("U cotangent misses the W2 path", "U_bar = U_bar + dG_bar @ W2.T", "U_bar = U_bar"),
    ("NS pre-scaling treated as a constant",
     "dG = dG - (np.sum(dY * Gp) / (nrm + eps) ** 2) * Gp / nrm", "dG = dG + 0.0"),
    ("NS Gram cotangent not symmetrised", "dXk = dXk + (dA + dA.T) @ X", "dXk = dXk + 2 * dA @ X"),
    ("momentum cotangent not carried", "dMc[m] = hp.beta * dM_new", "dMc[m] = 0 * dM_new"),
    ("row-norm projection dropped", "proj = dY - Y * np.sum(Y * dY, axis=1, keepdims=True)",
     "proj = dY"),
    ("apply cotangent from the wrong weights (update-then-apply)",
     "dq, d1, d2, d3 = apply_vjp(*W_out, Q[qs], dO[qs])",
     "dq, d1, d2, d3 = apply_vjp(*W_in, Q[qs], dO[qs])"),
    ("rate cotangent sign", "deta = -np.sum(U_bar * V, axis=1)", "deta = np.sum(U_bar * V, axis=1)"),
]


def _mutant(old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, old
    src = src.replace(old, new)
    mod = types.ModuleType("mutant_backward")
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src, "mutant_backward", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("desc,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_backward_mistake_is_caught(desc, old, new):
    mod = _ns(_mutant(old, new))
    caught = False
    for opt, beta, order in P.CONFIGS:
        try:
            if P.pin_autograd(mod, opt, beta, order) > 1e-6:
                caught = True
                break
        except Exception:  # noqa: BLE001 - a crash also counts as caught
            caught = True
            break
    if not caught:
        caught = P.pin_eta_zero(mod) > 0
    assert caught, desc
