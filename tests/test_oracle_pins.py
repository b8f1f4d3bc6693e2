"""The oracle against its pins (CPU only, float64)."""

import numpy as np
import pytest

import oracle
from tests import oracle_pins as P


@pytest.mark.parametrize("name", sorted(P.ALL_PINS))
def test_pin(name):
    fn, tol = P.ALL_PINS[name]
    err = fn(oracle)
    assert err <= tol, f"{name}: error {err:.3e} above {tol:.1e}"


def test_quintic_band_values():
    # The 5-fold quintic map sends [0.01, 1] into roughly [0.68, 1.14]:
    # NS_5 output is near-orthogonal but not orthogonal.
    lo, hi = P.quintic_band()
    assert 0.67 < lo < 0.70 and 1.12 < hi < 1.15


def test_token_block_sum_equals_whole_chunk():
    r = np.random.default_rng(20)
    W = P.rand_weights(r, 16, 32)
    K, V = r.normal(size=(1000, 16)), r.normal(size=(1000, 16))
    eta = np.abs(r.normal(size=1000))
    a = oracle.swiglu_grad(*W, K, V, eta)
    b = oracle.swiglu_grad(*W, K, V, eta, token_block=97)
    assert max(P.rel_err(x, y) for x, y in zip(b, a)) < 1e-12


def test_batched_entry_points_match_pairwise():
    import lact_synth as S
    w = S.WORKLOADS["tiny"].replace(B=2, H=2, T_kv=128, T_q=128, chunk_kv=32, chunk_q=32,
                                    d=8, h=16, opt="momentum", beta=0.9)
    st = S.gen_weights(w)
    x = S.gen_inputs(w)
    hp = oracle.Hyper(opt=w.opt, beta=w.beta)
    O, new = oracle.lact_chunked_forward(st, x["Q"], x["K"], x["V"], x["eta"],
                                         w.chunk_kv, w.chunk_q, w.order, hp)
    for b in range(2):
        for h in range(2):
            W = tuple(st[n][b, h].astype(np.float64) for n in ("W1", "W2", "W3"))
            M = tuple(np.zeros_like(m) for m in W)
            Op, Wp, Mp = oracle.chunked_forward_pair(
                W, M, x["Q"][b, h].astype(np.float64), x["K"][b, h].astype(np.float64),
                x["V"][b, h].astype(np.float64), x["eta"][b, h].astype(np.float64),
                w.chunk_kv, w.chunk_q, w.order, hp)
            assert np.array_equal(O[b, h], Op)
            for n, v in zip(("W1", "W2", "W3"), Wp):
                assert np.array_equal(new[n][b, h], v)
            for n, v in zip(("M1", "M2", "M3"), Mp):
                assert np.array_equal(new[n][b, h], v)
    # update / apply entry points reproduce one chunk of the scan
    st1 = oracle.lact_update(st, x["K"][:, :, :32], x["V"][:, :, :32], x["eta"][:, :, :32], hp)
    O1 = oracle.lact_apply(st, x["Q"][:, :, :32])
    O_ref, new_ref = oracle.lact_chunked_forward(st, x["Q"][:, :, :32], x["K"][:, :, :32],
                                                 x["V"][:, :, :32], x["eta"][:, :, :32],
                                                 32, 32, "apply_then_update", hp)
    assert np.array_equal(O1, O_ref)
    for n in ("W1", "W2", "W3", "M1", "M2", "M3"):
        assert np.array_equal(st1[n], new_ref[n])


def test_float32_twin_close_to_float64():
    import lact_synth as S
    w = S.WORKLOADS["tiny"]
    st = S.gen_weights(w)
    x = S.gen_inputs(w)
    hp = oracle.Hyper(opt=w.opt)
    O64, W64 = oracle.lact_chunked_forward(st, x["Q"], x["K"], x["V"], x["eta"],
                                           w.chunk_kv, w.chunk_q, w.order, hp)
    O32, W32 = oracle.lact_chunked_forward(st, x["Q"], x["K"], x["V"], x["eta"],
                                           w.chunk_kv, w.chunk_q, w.order, hp,
                                           dtype=np.float32)
    assert O32.dtype == np.float32
    assert P.rel_err(O32, O64) < 1e-5
    for n in ("W1", "W2", "W3"):
        assert P.rel_err(W32[n], W64[n]) < 1e-5


def test_batched_linear_net_matches_pairwise_and_closed_form():
    """The batched entry point with the linear net (state W1 [B, H, d, d]) runs
    each pair's scan; without normalisation it is the chunk-causal linear
    attention closed form (both orders)."""
    r = np.random.default_rng(31)
    B, H, d, T, chunk = 2, 2, 8, 48, 8
    W0 = r.normal(size=(B, H, d, d)) / np.sqrt(d)
    Q, K, V = (r.normal(size=(B, H, T, d)) for _ in range(3))
    eta = np.abs(r.normal(size=(B, H, T))) * 0.1
    for order in ("apply_then_update", "update_then_apply"):
        for opt, beta in (("gd", 0.0), ("momentum", 0.6), ("muon", 0.0)):
            hp = oracle.Hyper(opt=opt, beta=beta, net="linear", normalize=opt == "muon")
            O, new = oracle.lact_chunked_forward({"W1": W0}, Q, K, V, eta, chunk, chunk, order, hp)
            assert set(new) == ({"W1", "M1"} if hp.uses_momentum() else {"W1"})
            for b in range(B):
                for h in range(H):
                    M = (np.zeros((d, d)),) if hp.uses_momentum() else None
                    Op, Wp, _ = oracle.chunked_forward_pair((W0[b, h],), M, Q[b, h], K[b, h], V[b, h],
                                                            eta[b, h], chunk, chunk, order, hp)
                    assert np.array_equal(O[b, h], Op) and np.array_equal(new["W1"][b, h], Wp[0])
                    if opt != "muon":
                        ref = P.linear_closed_form(W0[b, h], Q[b, h], K[b, h], V[b, h], eta[b, h],
                                                   chunk, order, beta)
                        assert P.rel_err(O[b, h], ref) < 1e-12
