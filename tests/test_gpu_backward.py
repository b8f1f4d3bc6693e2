"""GPU parity of the backward pass (lact_chunked_backward) against the
float64 backward oracle (``oracle.lact_chunked_backward``, pinned by
torch.autograd and finite differences).  Every cotangent (dQ, dK, dV, deta,
dW1, dW2, dW3) is compared per tensor with max |x - y| / max |y|, against the
layer's bars: 1e-4 in fp32 I/O mode, 2e-2 in bf16 mode."""

import numpy as np
import pytest

import lact_synth as S
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu

NAMES = ("dQ", "dK", "dV", "deta", "dW1", "dW2", "dW3")


def cotangent_inputs(w, seed=77):
    """dO like Q and cotangents of the final weights (seeded normal draws)."""
    r = np.random.default_rng(seed)
    dO = r.standard_normal((w.B, w.H, w.T_q, w.d)).astype(np.float32)
    if w.io_dtype == "bf16":
        dO = S.round_bf16(dO)
    st = S.gen_weights(w)
    dWf = {n: (0.1 * r.standard_normal(st[n].shape)).astype(np.float32) for n in ("W1", "W2", "W3")}
    return dO, dWf


def run_backward_gpu(w, x, st, dO, dWf):
    import torch
    import chunk_test_amd as L
    cfg = G.config_of(w)
    dst = {n: G.to_dev(st[n], w, io=False) for n in ("W1", "W2", "W3")}
    Q, K, V, dOt = (G.to_dev(a, w) for a in (x["Q"], x["K"], x["V"], dO))
    eta = G.to_dev(x["eta"], w, io=False)
    fin = None if dWf is None else {n: G.to_dev(dWf[n], w, io=False) for n in ("W1", "W2", "W3")}
    out = L.lact_chunked_backward(cfg, dst, Q, K, V, eta, dOt, w.chunk_kv, w.chunk_q, w.order,
                                  dW_final=fin)
    torch.cuda.synchronize()
    # the initial weights are read only
    for n in ("W1", "W2", "W3"):
        assert np.array_equal(dst[n].cpu().numpy(), st[n]), n
    return {k: v.float().cpu().numpy() for k, v in out.items()}


def run_backward_oracle(w, x, st, dO, dWf, pairs=None):
    import oracle
    hp = oracle.Hyper(opt=w.opt, beta=w.beta, ns_iters=w.ns_iters)
    return oracle.lact_chunked_backward(st, x["Q"], x["K"], x["V"], x["eta"], dO, w.chunk_kv,
                                        w.chunk_q, w.order, hp, dW_final=dWf, pairs=pairs)


def compare(w, got, ref, pairs=None):
    tol = G.tol_of(w)
    sel = (lambda a: a) if pairs is None else (lambda a: np.stack([a[b, h] for b, h in pairs]))
    errs = {n: G.rel_err(sel(got[n]), sel(ref[n])) for n in NAMES}
    G.say(f"  {w.name}: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()) + f" (tol {tol:.0e})")
    return {k: v for k, v in errs.items() if not v <= tol}


SMALL = S.WORKLOADS["tiny"].replace(name="bw", B=1, H=2, d=32, h=64, T_kv=192, chunk_kv=64, T_q=48,
                                    chunk_q=16)
CASES = [SMALL.replace(name=f"bw-{opt}{'-b' if beta else ''}-{order[:1]}", opt=opt, beta=beta, order=order)
         for opt, beta in (("gd", 0.0), ("momentum", 0.9), ("muon", 0.0), ("muon", 0.5))
         for order in ("apply_then_update", "update_then_apply")]
CASES += [
    SMALL.replace(name="bw-d64-h128-ragged", d=64, h=128, T_kv=3 * 300, chunk_kv=300, T_q=3 * 50,
                  chunk_q=50, opt="momentum", beta=0.5),
    SMALL.replace(name="bw-d128-h256", B=2, H=1, d=128, h=256, T_kv=2 * 256, chunk_kv=256, T_q=2 * 64,
                  chunk_q=64, opt="muon", order="update_then_apply"),
    S.WORKLOADS["posed"].replace(name="bw-posed-bf16", H=2, T_kv=4096, chunk_kv=4096, T_q=256,
                                 chunk_q=256),
    S.WORKLOADS["lm"].replace(name="bw-lm-bf16", B=1, H=2, T_kv=4096, chunk_kv=1024, T_q=4096,
                              chunk_q=1024),
    S.WORKLOADS["video"].replace(name="bw-video-split", H=1, T_kv=3 * 1024, chunk_kv=1024,
                                 T_q=3 * 1024, chunk_q=1024),
    # bf16 at d = 128 with chunks that are no multiple of the 32-token stages
    # (ragged last stage and split in the matrix-core contractions)
    S.WORKLOADS["lm"].replace(name="bw-lm-bf16-ragged", B=1, H=2, T_kv=3 * 1000, chunk_kv=1000,
                              T_q=3 * 200, chunk_q=200, order="update_then_apply"),
    # the same at d = 64 (posed and million-token shapes), Muon, both orders
    S.WORKLOADS["posed"].replace(name="bw-posed-bf16-ragged", H=2, T_kv=3 * 700, chunk_kv=700,
                                 T_q=3 * 100, chunk_q=100, products="auto"),
    S.WORKLOADS["posed"].replace(name="bw-posed-bf16-a", H=3, T_kv=2 * 2048, chunk_kv=2048,
                                 T_q=2 * 256, chunk_q=256, order="apply_then_update", opt="momentum",
                                 beta=0.9),
    # hidden sizes that are multiples of 32 but not of 128: matrix-core token
    # kernels with the fp32 contraction kernel
    S.WORKLOADS["lm"].replace(name="bw-d128-h96-bf16", B=1, H=2, h=96, T_kv=2 * 512, chunk_kv=512,
                              T_q=2 * 128, chunk_q=128, opt="muon", products="auto"),
    S.WORKLOADS["posed"].replace(name="bw-d64-h64-bf16", H=2, h=64, T_kv=2 * 600, chunk_kv=600,
                                 T_q=2 * 100, chunk_q=100, opt="gd", products="bf16"),
]


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_backward_parity(w):
    G.say(f"case {w.name}")
    st = S.gen_weights(w)
    x = S.gen_inputs(w)
    dO, dWf = cotangent_inputs(w)
    got = run_backward_gpu(w, x, st, dO, dWf)
    ref = run_backward_oracle(w, x, st, dO, dWf)
    bad = compare(w, got, ref)
    assert not bad, bad


def test_backward_without_final_cotangent():
    w = CASES[2]
    st = S.gen_weights(w)
    x = S.gen_inputs(w)
    dO, _ = cotangent_inputs(w)
    got = run_backward_gpu(w, x, st, dO, None)
    ref = run_backward_oracle(w, x, st, dO, None)
    assert not compare(w, got, ref)


def test_backward_lm_full_size_sampled():
    """The language-model workload at full size (8 x 8 pairs, 16 chunks of
    2048, d = 128, h = 256, momentum 0.9, bf16), two sampled pairs against the
    oracle; every pair's cotangents finite."""
    w = S.WORKLOADS["lm"]
    pairs = [(0, 0), (5, 3)]
    G.say(f"case {w.name} backward, oracle pairs {pairs}")
    st = S.gen_weights(w)
    x = S.gen_inputs(w)
    dO, dWf = cotangent_inputs(w)
    got = run_backward_gpu(w, x, st, dO, dWf)
    ref = run_backward_oracle(w, x, st, dO, dWf, pairs=pairs)
    bad = compare(w, got, ref, pairs=pairs)
    assert not bad, bad
    for n in NAMES:
        assert np.all(np.isfinite(got[n])), n


@pytest.mark.parametrize("name", ["bw-posed-bf16", "bw-lm-bf16"])
def test_backward_repeat_is_bitwise_equal(name):
    """The matrix-core contraction sums its token splits in the workgroup that
    finishes last; the sum runs in split order whichever that is, so two runs
    give the same bits."""
    w = next(c for c in CASES if c.name == name)
    G.say(f"case {w.name} twice")
    st = S.gen_weights(w)
    x = S.gen_inputs(w)
    dO, dWf = cotangent_inputs(w)
    a = run_backward_gpu(w, x, st, dO, dWf)
    b = run_backward_gpu(w, x, st, dO, dWf)
    for n in NAMES:
        assert np.array_equal(a[n], b[n]), n
