"""Pins of the window-attention oracle and of the block's sum (CPU, float64).

* a window as long as the sequence is plain causal attention: torch's
  scaled_dot_product_attention with is_causal (a library routine);
* a window of one token returns the values;
* every other window equals masked full attention written as one matrix
  expression (mask t - w < s <= t), a different formulation;
* attention weights are a softmax: outputs of constant values are that
  constant; outputs are convex combinations (inside the values' range);
* the block is the TTT layer's output plus the attention output.
"""

import numpy as np
import pytest

import oracle
import lact_synth as S


def rand_qkv(seed, T=40, d=8):
    r = np.random.default_rng(seed)
    return r.normal(size=(T, d)), r.normal(size=(T, d)), r.normal(size=(T, d))


def test_full_window_is_causal_attention():
    torch = pytest.importorskip("torch")
    Q, K, V = rand_qkv(1)
    O = oracle.window_attention(Q, K, V, window=len(Q))
    t = lambda x: torch.tensor(x)[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(t(Q), t(K), t(V), is_causal=True)[0, 0].numpy()
    assert np.max(np.abs(O - ref)) < 1e-12


def test_window_one_returns_values():
    Q, K, V = rand_qkv(2)
    assert np.max(np.abs(oracle.window_attention(Q, K, V, window=1) - V)) < 1e-15


@pytest.mark.parametrize("window,scale", [(5, None), (17, 0.7), (39, None)])
def test_window_equals_masked_matrix_form(window, scale):
    Q, K, V = rand_qkv(3)
    T, d = Q.shape
    sc = 1 / np.sqrt(d) if scale is None else scale
    s = (Q @ K.T) * sc
    i, j = np.arange(T)[:, None], np.arange(T)[None, :]
    s = np.where((j <= i) & (j > i - window), s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    assert np.max(np.abs(oracle.window_attention(Q, K, V, window, scale) - p @ V)) < 1e-12


def test_softmax_weights_are_convex():
    Q, K, _ = rand_qkv(4)
    V = np.full_like(Q, 2.5)
    assert np.max(np.abs(oracle.window_attention(Q, K, V, 7) - 2.5)) < 1e-12
    _, _, V = rand_qkv(5)
    O = oracle.window_attention(Q, K, V, 7)
    assert np.all(O <= V.max(axis=0) + 1e-12) and np.all(O >= V.min(axis=0) - 1e-12)


def test_block_is_ttt_plus_attention():
    w = S.WORKLOADS["tiny"].replace(B=1, H=2, T_kv=64, T_q=64, chunk_kv=16, chunk_q=16, d=8, h=16,
                                    opt="momentum", beta=0.9)
    st = S.gen_weights(w)
    x = S.gen_inputs(w)
    hp = oracle.Hyper(opt=w.opt, beta=w.beta)
    O, new = oracle.block_forward(st, x["Q"], x["K"], x["V"], x["eta"], 16, 12, hp)
    O_t, new_t = oracle.lact_chunked_forward(st, x["Q"], x["K"], x["V"], x["eta"], 16, 16,
                                             "apply_then_update", hp)
    for h in range(2):
        att = oracle.window_attention(x["Q"][0, h].astype(np.float64), x["K"][0, h].astype(np.float64),
                                      x["V"][0, h].astype(np.float64), 12)
        assert np.max(np.abs(O[0, h] - O_t[0, h] - att)) < 1e-12
    for n in new:
        assert np.array_equal(new[n], new_t[n])
