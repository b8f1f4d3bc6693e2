"""GPU parity of the LaCT block's window attention (lact_window_attention)
and of the whole block (lact_block_forward: attention + TTT layer on shared
Q, K, V) against the float64 oracle (``oracle.window_attention``,
``oracle.block_forward``).  Bars: 1e-4 fp32, 2e-2 bf16, on O (and on the
block's final weights)."""

import numpy as np
import pytest

import lact_synth as S
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu


def attention_case(B, H, T, d, io, seed):
    w = S.WORKLOADS["tiny"].replace(name="attn", B=B, H=H, d=d, h=2 * d, T_kv=T, T_q=T, chunk_kv=T,
                                    chunk_q=T, io_dtype=io, seed=seed)
    return w, S.gen_inputs(w)


@pytest.mark.parametrize("B,H,T,d,io,window,scale", [
    (1, 2, 300, 64, "fp32", 1, 0.0),
    (1, 2, 300, 64, "fp32", 37, 0.0),
    (2, 1, 257, 32, "fp32", 64, 0.9),
    (1, 2, 200, 128, "fp32", 1000, 0.0),   # window longer than the sequence: causal attention
    (1, 2, 3000, 128, "bf16", 2048, 0.0),  # the 760M language model's window
    (1, 3, 1100, 64, "bf16", 129, 2.0),
    # the matrix-core kernel (bf16, d = 128): ragged lengths, windows shorter than a
    # 32-key sub-tile, the identity window, a window longer than the sequence
    (1, 2, 1000, 128, "bf16", 1, 0.0),
    (1, 2, 777, 128, "bf16", 33, 0.5),
    (2, 1, 300, 128, "bf16", 100000, 0.0),
    (1, 1, 4100, 128, "bf16", 4096, 0.0),
    # scores of tens of units (scale 40 on unit rows): a query's running maximum
    # moves by more than the kernel's lazy-rescale margin many times
    (1, 2, 2000, 128, "bf16", 512, 40.0),
])
def test_window_attention_parity(B, H, T, d, io, window, scale):
    import torch
    import chunk_test_amd as L
    import oracle
    w, x = attention_case(B, H, T, d, io, seed=T + window)
    cfg = G.config_of(w)
    Q, K, V = (G.to_dev(x[n], w) for n in ("Q", "K", "V"))
    O = torch.empty_like(Q)
    L.lact_window_attention(cfg, Q, K, V, O, window, scale)
    torch.cuda.synchronize()
    got = O.float().cpu().numpy()
    sc = None if scale <= 0 else scale
    for b in range(B):
        for h in range(H):
            ref = oracle.window_attention(x["Q"][b, h].astype(np.float64), x["K"][b, h].astype(np.float64),
                                          x["V"][b, h].astype(np.float64), window, sc)
            err = G.rel_err(got[b, h], ref)
            assert err <= G.tol_of(w), (b, h, err)
    # accumulate adds into what O holds
    O2 = torch.ones_like(Q)
    L.lact_window_attention(cfg, Q, K, V, O2, window, scale, accumulate=True)
    torch.cuda.synchronize()
    assert G.rel_err(O2.float().cpu().numpy() - 1.0, got) <= 2 * G.tol_of(w)


@pytest.mark.parametrize("window", [700, 4096])
def test_window_attention_rising_scores(window):
    """Keys whose length grows along the sequence (0.2 to 6 times unit length,
    scale 4): every query's maximum keeps rising across its window, so the
    softmax reference moves (and the output is rescaled) again and again,
    with probabilities both near the lazy margin and far below it."""
    import torch
    import chunk_test_amd as L
    import oracle
    B, H, T, d = 1, 2, 3000, 128
    w, x = attention_case(B, H, T, d, "bf16", seed=11 + window)
    # (scaled in float32, then rounded to the bf16 the kernel reads; the
    # oracle sees the same rounded values)
    ramp = np.linspace(0.2, 6.0, T, dtype=np.float32)[None, None, :, None]
    x["K"] = S.round_bf16(x["K"].astype(np.float32) * ramp)
    cfg = G.config_of(w)
    Q, K, V = (G.to_dev(x[n], w) for n in ("Q", "K", "V"))
    O = torch.empty_like(Q)
    L.lact_window_attention(cfg, Q, K, V, O, window, 4.0)
    torch.cuda.synchronize()
    got = O.float().cpu().numpy()
    for h in range(H):
        ref = oracle.window_attention(x["Q"][0, h].astype(np.float64), x["K"][0, h].astype(np.float64),
                                      x["V"][0, h].astype(np.float64), window, 4.0)
        err = G.rel_err(got[0, h], ref)
        assert err <= G.tol_of(w), (h, err)


@pytest.mark.parametrize("w,window", [
    (S.WORKLOADS["tiny"].replace(name="block-tiny", H=2, opt="momentum", beta=0.9), 100),
    (S.WORKLOADS["lm"].replace(name="block-lm", B=1, H=2, T_kv=4096, T_q=4096, chunk_kv=1024,
                               chunk_q=1024), 2048),
    (S.WORKLOADS["video"].replace(name="block-video", H=1, T_kv=2 * 4096, T_q=2 * 4096), 4096),
], ids=["block-tiny", "block-lm", "block-video"])
def test_block_parity(w, window):
    import torch
    import chunk_test_amd as L
    import oracle
    G.say(f"case {w.name} window {window}")
    st = S.gen_weights(w)
    x = S.gen_inputs(w)
    # shared Q, K, V: the queries are the keys' tokens
    x["Q"] = x["K"].copy()
    cfg = G.config_of(w)
    dst = G.device_state(w, st)
    Q, K, V = (G.to_dev(x[n], w) for n in ("Q", "K", "V"))
    eta = G.to_dev(x["eta"], w, io=False)
    O = torch.empty_like(Q)
    ws = L.alloc_workspace(cfg, w.chunk_kv, w.chunk_q)
    L.lact_block_forward(cfg, dst, Q, K, V, eta, O, w.chunk_kv, window, ws)
    torch.cuda.synchronize()
    hp = oracle.Hyper(opt=w.opt, beta=w.beta, ns_iters=w.ns_iters, token_block=65536)
    O_ref, st_ref = oracle.block_forward(st, x["Q"], x["K"], x["V"], x["eta"], w.chunk_kv, window, hp)
    s_gpu = {n: t.cpu().numpy() for n, t in dst.items()}
    _, bad = G.compare(w, O.float().cpu().numpy(), s_gpu, O_ref, st_ref)
    assert not bad, bad
