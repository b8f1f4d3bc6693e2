"""The allocation-free entry point (lact_chunked_forward_noalloc) against
lact_chunked_forward with a caller workspace: the same kernels on the same
inputs, so the same bits; two calls in a row, the second on a smaller input
(the scratch array keeps the first call's contents), and a size above the
array refused before anything runs."""

import numpy as np
import pytest

import lact_synth as S
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu


def _run_noalloc(w, x, st_np):
    import torch
    import chunk_test_amd as L
    cfg = G.config_of(w)
    st = G.device_state(w, st_np)
    Q, K, V = (G.to_dev(x[n], w) for n in ("Q", "K", "V"))
    eta = G.to_dev(x["eta"], w, io=False)
    O = torch.empty_like(Q)
    L.lact_chunked_forward_noalloc(cfg, st, Q, K, V, eta, O, w.chunk_kv, w.chunk_q, w.order)
    torch.cuda.synchronize()
    return O.float().cpu().numpy(), {n: t.cpu().numpy() for n, t in st.items()}


CASES = [
    # bf16 Muon at d = 64 (split partials + reduction + MFMA Newton-Schulz tail), then a
    # smaller momentum run at d = 128 and a tiny fp32 run, all through the one array
    S.WORKLOADS["posed"].replace(name="noalloc-posed", H=4, T_kv=65536, T_q=1024,
                                 chunk_kv=65536, chunk_q=1024),
    S.WORKLOADS["lm"].replace(name="noalloc-lm", B=1, H=2, T_kv=4096, T_q=4096, chunk_kv=1024,
                              chunk_q=1024),
    S.WORKLOADS["tiny"],
]


def test_noalloc_matches_workspace_entry_point_on_consecutive_calls():
    import chunk_test_amd as L
    assert L.noalloc_scratch_bytes() == 64 << 20
    for w in CASES:
        G.say(f"case {w.name}")
        need = L.workspace_bytes(G.config_of(w), w.chunk_kv, w.chunk_q)
        assert need <= L.noalloc_scratch_bytes()
        st = S.gen_weights(w)
        x = S.gen_inputs(w)
        O_ref, s_ref = G.run_gpu(w, x, st)
        O, s = _run_noalloc(w, x, st)
        assert np.array_equal(O, O_ref), w.name
        for n in s_ref:
            assert np.array_equal(s[n], s_ref[n]), (w.name, n)
    # and the first case again after the smaller ones
    w = CASES[0]
    st = S.gen_weights(w)
    x = S.gen_inputs(w)
    O_ref, s_ref = G.run_gpu(w, x, st)
    O, s = _run_noalloc(w, x, st)
    assert np.array_equal(O, O_ref)
    for n in s_ref:
        assert np.array_equal(s[n], s_ref[n]), n


def test_noalloc_refuses_chunks_beyond_its_scratch():
    import torch
    import chunk_test_amd as L
    w = S.WORKLOADS["video"]  # 127.5 MiB of workspace per chunk
    cfg = G.config_of(w)
    assert L.workspace_bytes(cfg, w.chunk_kv, w.chunk_q) > L.noalloc_scratch_bytes()
    st = {n: torch.zeros((1, w.H) + ((w.d, w.h) if n[1] == "2" else (w.h, w.d)), device="cuda")
          for n in ("W1", "W2", "W3")}
    Q = torch.zeros(1, w.H, 4096, w.d, dtype=torch.bfloat16, device="cuda")
    eta = torch.zeros(1, w.H, 4096, device="cuda")
    with pytest.raises(L.LactError) as e:
        L.lact_chunked_forward_noalloc(cfg, st, Q, Q, Q, eta, torch.empty_like(Q), 4096, 4096,
                                       "apply_then_update")
    assert e.value.status == -3 and "scratch" in str(e.value)
