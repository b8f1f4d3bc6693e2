"""GPU parity of the linear fast net f_W(x) = W x on the chunk scan (the
linear state the pages compare the SwiGLU fast net against: "LaCT: Large
Chunk Test-Time Training" review, "Large chunks alone do not explain the
gains").  Against the float64 oracle in both orders, with GD, momentum and
Muon and every row rule; without normalisation also against the
chunk-causal linear-attention closed form directly.  Bars as for the layer:
1e-4 in fp32 mode, 2e-2 in bf16 mode."""

import numpy as np
import pytest

import lact_synth as S
from tests import gpu_helpers as G
from tests import oracle_pins as P

pytestmark = pytest.mark.gpu

BASE = S.WORKLOADS["tiny"].replace(name="lin", net="linear", h=64, norm="none")

CASES = [
    BASE.replace(name="lin-gd-none-atu"),
    BASE.replace(name="lin-gd-none-uta", order="update_then_apply"),
    BASE.replace(name="lin-mom-none-atu", opt="momentum", beta=0.9),
    BASE.replace(name="lin-mom-none-uta", opt="momentum", beta=0.6, order="update_then_apply"),
    BASE.replace(name="lin-gd-unit", norm="unit"),
    BASE.replace(name="lin-muon-unit-atu", opt="muon", norm="unit"),
    BASE.replace(name="lin-muon-unit-uta", opt="muon", norm="unit", order="update_then_apply"),
    BASE.replace(name="lin-muon-mom-keep", opt="muon", beta=0.5, norm="keep"),
    BASE.replace(name="lin-d128-mom-keep", B=2, H=2, d=128, h=128, opt="momentum", beta=0.9,
                 norm="keep"),
    BASE.replace(name="lin-d16-muon", H=3, d=16, h=16, opt="muon", norm="unit"),
    BASE.replace(name="lin-d32-ragged", H=2, d=32, h=32, T_kv=3 * 300, chunk_kv=300, T_q=3 * 70,
                 chunk_q=70, norm="unit", opt="momentum", beta=0.5),
    BASE.replace(name="lin-bf16-muon", io_dtype="bf16", H=4, T_kv=2 * 4096, chunk_kv=4096,
                 T_q=2 * 512, chunk_q=512, opt="muon", norm="unit"),
    BASE.replace(name="lin-bf16-d128-gd-uta", io_dtype="bf16", B=2, H=3, d=128, h=128,
                 T_kv=3 * 1000, chunk_kv=1000, T_q=3 * 100, chunk_q=100, norm="unit",
                 order="update_then_apply"),
    BASE.replace(name="lin-chunk1", T_kv=5, chunk_kv=1, T_q=5, chunk_q=1, opt="muon", norm="unit"),
]


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_linear_net_parity(w):
    G.say(f"case {w.name}")
    st = S.gen_weights(w)
    assert set(st) == {"W1"} and st["W1"].shape == (w.B, w.H, w.d, w.d)
    x = S.gen_inputs(w)
    O, st_gpu = G.run_gpu(w, x, st)
    O_ref, st_ref = G.run_oracle(w, x, st)
    _, bad = G.compare(w, O, st_gpu, O_ref, st_ref)
    assert not bad, bad
    if w.norm == "unit":
        assert np.max(np.abs(np.linalg.norm(st_gpu["W1"], axis=-1) - 1)) < 1e-5
    if w.norm == "keep":
        want = np.linalg.norm(st["W1"], axis=-1)
        assert np.max(np.abs(np.linalg.norm(st_gpu["W1"], axis=-1) - want)) < 1e-4


@pytest.mark.parametrize("w", [c for c in CASES if c.norm == "none"], ids=lambda w: w.name)
def test_linear_net_matches_linear_attention_closed_form(w):
    """Without normalisation the scan is chunk-causal linear attention:
    o_t = W0 q_t + sum over earlier (or, update-then-apply, also the same)
    chunks of eta_i (k_i . q_t) v_i, with heavy-ball momentum weighting a
    chunk's gradient by the partial geometric sums of beta."""
    st = S.gen_weights(w)
    x = S.gen_inputs(w)
    O, _ = G.run_gpu(w, x, st)
    for b in range(w.B):
        for h in range(w.H):
            ref = P.linear_closed_form(st["W1"][b, h].astype(np.float64), x["Q"][b, h].astype(np.float64),
                                       x["K"][b, h].astype(np.float64), x["V"][b, h].astype(np.float64),
                                       x["eta"][b, h].astype(np.float64), w.chunk_kv, w.order,
                                       w.beta if w.opt == "momentum" else 0.0)
            assert G.rel_err(O[b, h], ref) <= G.FP32_TOL, (b, h)
